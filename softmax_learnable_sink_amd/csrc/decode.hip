// Paged decode with a learnable per-head sink and optional first/last window.
//
// Split-K: each sequence's selected tokens are cut into pieces, each with its
// own partial: for large work, equal token ranges of the whole batch's
// concatenated selections, one per resident workgroup (a range may cross
// sequence boundaries); otherwise chunks of `chunk` tokens.  A workgroup takes
// one range or chunk and NW (4, or 2 for small grids) KV heads of it; wave w
// computes the scores of all query heads of its KV head (GQA group, up to 16
// per wave), so every K/V byte is read from HBM once:
//   * the slots of the chunk's tokens are computed once into LDS from the
//     block table and the window rule (sglang PR #12504 "To implement
//     attention-sink": first W1 tokens followed by the last W2 tokens of each
//     sequence, or the whole prefix when it is not longer than W1 + W2) and
//     shared by the workgroup's waves;
//   * each wave walks the chunk in steps of 32 tokens: S^T (16 tokens x 16
//     heads) = K Q^T on 16x16x32 bf16 MFMA with K rows loaded straight from
//     the paged cache, a running max / sum per head WITHOUT the sink, and
//     O^T += V^T P^T with V staged in a wave-private LDS tile and read back
//     transposed;
//   * each wave writes one partial (acc[D], m, l) per (sequence, head, piece).
// The combine kernel merges the pieces and folds the sink into the
// denominator exactly once (sglang PR #8825, Summary of Changes: the decode
// path receives the per-head sink; flash-attention PR #1819 review thread:
// decoding with a sink through the KV-cache entry point was reported wrong,
// so the merge is where the sink must enter, once).
#include <algorithm>
#include <atomic>
#include <climits>
#include <mutex>
#include <type_traits>

#include "checks.h"
#include "common.h"
#include "launch.h"

namespace attn_sink {
namespace {

constexpr int kThreads = 256;

constexpr int kSub = 2048;  // selected tokens whose slots are staged in LDS at once

template <int D>
constexpr int vrow() { return D + 8; }  // V staging row stride: D + 16 B padding

template <int D, int NW>
struct DecLds {
  int slot[kSub];               // slot of each selected token of the current block
  __bf16 v[NW][32 * vrow<D>()]; // per-wave V staging tiles, natural [token][d]
  int wsum[NW];                 // per-wave counts (compaction of listed tokens)
};

template <int D>
struct KVRegs {
  static constexpr int KS = D / 32;       // k-steps of the score MFMA
  static constexpr int TPL = D / 16;      // V tokens per lane
  static constexpr int NTG = 32 / TPL;    // lanes sharing one d-chunk
  uint4 kr[2][KS];
  uint4 vr[TPL];
  uint32_t vvalid;  // bit t: V row t holds a selected token

  // K rows (score MFMA operand) and V rows (for the transposed LDS tile) of
  // step tokens base .. base+31, slots taken from the LDS slot table (-1 = no
  // token).  A token without a slot reads row 0 of the cache; its K score is
  // masked and its V row is replaced by zeros when the tile is staged (not
  // here, so that no register with a load in flight is overwritten).
  __device__ __forceinline__ void load(const int* slot, int base, const __bf16* kbase,
                                       const __bf16* vbase, size_t rs, int lane) {
    const int kg = lane >> 4, r = lane & 15;
    const int tg = lane % NTG, c = lane / NTG;
    int ks[2], vs[TPL];
#pragma unroll
    for (int G = 0; G < 2; ++G)
      // MFMA row r of token group G holds token 8*(r/4) + 4*G + r%4 of the step
      ks[G] = slot[base + 8 * (r >> 2) + 4 * G + (r & 3)];
#pragma unroll
    for (int t = 0; t < TPL; ++t) vs[t] = slot[base + TPL * tg + t];
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      const __bf16* row = kbase + (size_t)max(ks[G], 0) * rs + 8 * kg;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) kr[G][s2] = *reinterpret_cast<const uint4*>(row + 32 * s2);
    }
    vvalid = 0;
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      vr[t] = *reinterpret_cast<const uint4*>(vbase + (size_t)max(vs[t], 0) * rs + 8 * c);
      vvalid |= (vs[t] >= 0 ? 1u : 0u) << t;
    }
  }
  // The same through buffer resources over the K and V caches (each below
  // 4 GiB): 32-bit byte offsets, no 64-bit address per row.
  __device__ __forceinline__ void load(const int* slot, int base, __amdgpu_buffer_rsrc_t rk,
                                       __amdgpu_buffer_rsrc_t rv, uint32_t rs_bytes, int lane) {
    const int kg = lane >> 4, r = lane & 15;
    const int tg = lane % NTG, c = lane / NTG;
    int ks[2], vs[TPL];
#pragma unroll
    for (int G = 0; G < 2; ++G) ks[G] = slot[base + 8 * (r >> 2) + 4 * G + (r & 3)];
#pragma unroll
    for (int t = 0; t < TPL; ++t) vs[t] = slot[base + TPL * tg + t];
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      const uint32_t row = (uint32_t)max(ks[G], 0) * rs_bytes + 16 * kg;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) kr[G][s2] = buf_load16(rk, row + 64 * s2);
    }
    vvalid = 0;
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      vr[t] = buf_load16(rv, (uint32_t)max(vs[t], 0) * rs_bytes + 16 * c);
      vvalid |= (vs[t] >= 0 ? 1u : 0u) << t;
    }
  }
};

// A operand (16 d x 32 tokens) of O^T += V^T P^T read from the natural V tile:
// lane l gets d = 16*db + l%16 and tokens 8*(l/16) .. +7.  ds_read_b64_tr_b16
// hands lane i of each 16-lane group element i%4 of the 4-element vectors that
// lanes 4j + i/4 (j = 0..3) of the group addressed, in order of j; so lane s of
// group G addresses token 8G + 4h + s/4, columns 16*db + 4*(s%4) .. +3, for
// the two loads h = 0, 1.
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ bf16x8 vt_frag16(const __bf16* vtile, int db, int lane) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int sl = lane & 15, G = lane >> 4;
  const __bf16* p0 = vtile + (8 * G + (sl >> 2)) * vrow<D>() + 16 * db + 4 * (sl & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * vrow<D>()));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The partial kernel's grid is sized by the longest possible sequence, so many
// of its (sequence, split) slots hold no selected token.  Workgroups that exit
// at once, interleaved with the working ones, cost a third of the read rate
// (a read probe of this access pattern: 5.8 -> 4.0 TB/s), so workgroup j takes
// the j-th chunk that does hold tokens, in sequence order, and the workgroups
// without work all sit at the end of the grid.  Chunk counts per sequence:
// Whole chunks of a sequence, and whether a shorter last one follows.  The
// chunks are taken whole ones first (in sequence order), then the shorter
// last ones, so that the shortest work runs at the end of the grid.
__device__ __forceinline__ int full_chunks(int nsel, int chunk, int max_splits) {
  return min(max_splits, nsel / chunk);
}
__device__ __forceinline__ int part_chunk(int nsel, int chunk, int max_splits) {
  return (nsel / chunk < max_splits && nsel % chunk != 0) ? 1 : 0;
}

// Wave-wide search: the first of 64 counts c (one per lane) whose inclusive
// prefix sum exceeds rem.  On a hit, lane `first` holds it and `before` is
// the sum of the counts ahead of it; otherwise rem drops by the total.
__device__ __forceinline__ bool wave_find(int c, int& rem, int lane, int& first, int& before) {
  int x = c;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  const int tot = __shfl(x, 63, 64);
  if (rem >= tot) {  // uniform over the wave
    rem -= tot;
    return false;
  }
  first = __builtin_ctzll(__ballot(x > rem));
  before = __shfl(x - c, first, 64);
  return true;
}

// Up to kScanSeqs sequences, every wave finds its workgroup's chunk itself
// (all lengths loaded at once).
constexpr int kScanSeqs = 256;
__device__ __forceinline__ bool find_chunk(const int32_t* seqlens, int B, int w1, int w2,
                                           int chunk, int max_splits, int j, int lane, int& b,
                                           int& split, int& L) {
  constexpr int R = kScanSeqs / 64;
  int len[R], nsel[R];
#pragma unroll
  for (int r = 0; r < R; ++r) len[r] = seqlens[min(64 * r + lane, B - 1)];
#pragma unroll
  for (int r = 0; r < R; ++r) nsel[r] = 64 * r + lane < B ? n_selected(len[r], w1, w2) : 0;
  int rem = j, first, before;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (wave_find(full_chunks(nsel[r], chunk, max_splits), rem, lane, first, before)) {
      b = 64 * r + first;
      split = rem - before;
      L = __shfl(len[r], first, 64);
      return true;
    }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (wave_find(part_chunk(nsel[r], chunk, max_splits), rem, lane, first, before)) {
      b = 64 * r + first;
      split = full_chunks(__shfl(nsel[r], first, 64), chunk, max_splits);
      L = __shfl(len[r], first, 64);
      return true;
    }
  return false;
}

// More sequences: decode_plan_kernel lists the chunks in the same order once
// (one workgroup scanning the sequences 256 at a time, whole chunks in a
// first pass, last ones in a second) and workgroup j reads entry j.
__global__ __launch_bounds__(256) void decode_plan_kernel(const int32_t* __restrict__ seqlens,
                                                          int B, int w1, int w2, int chunk,
                                                          int max_splits,
                                                          int32_t* __restrict__ items,
                                                          int32_t* __restrict__ count) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int b0 = 0; b0 < B; b0 += 256) {
      const int b = b0 + tid;
      const int nsel = b < B ? n_selected(seqlens[b], w1, w2) : 0;
      const int nf = full_chunks(nsel, chunk, max_splits);
      const int ns = pass == 0 ? nf : part_chunk(nsel, chunk, max_splits);
      int x = ns;  // inclusive scan over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (lane == 63) wsum[wave] = x;
      __syncthreads();
      int off = base + x - ns;
      for (int w = 0; w < wave; ++w) off += wsum[w];
      for (int t = 0; t < ns; ++t) items[off + t] = b * max_splits + (pass == 0 ? t : nf);
      base += (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
      __syncthreads();  // wsum is rewritten by the next round
    }
  if (tid == 0) *count = base;
}

// 1-D grid of ceil(units / NW) workgroups per chunk slot (B * splits slots),
// NW waves per workgroup; the chunk of slot j is found as above (`items` NULL:
// by the scan; else from the list).  A unit is one KV head and up to 16 of its
// query heads; wave w owns unit (blockIdx.x % ceil(units/NW))*NW + w and walks
// every token of the workgroup's chunk, so the NW waves of a workgroup read
// adjacent heads' slices of the same token rows together and share one slot
// table.  Each wave writes its own partials.
//
// LIST: per-query index lists instead of whole sequences.  "Sequence" b is then
// packed query row b (B rows) of sequence row_seq[b]; its tokens are the
// entries of kv_index row b (topk of them) that lie in [0, L) and at or before
// the row's position L - nq + i; each chunk covers `chunk` list entries, every
// slot of the grid is real, and a chunk's valid entries are compacted into the
// slot table.
struct ListArgs {
  const int32_t* kv_index;  // [B, topk]
  const int32_t* row_seq;   // [B]: sequence of each packed row
  const int32_t* cu_q;      // [sequences + 1]
  int topk;
};

// Work assignment of decode_partial_kernel.
enum : int {
  kModeChunks = 0,  // workgroup j: the j-th chunk that holds tokens
  kModeList = 1,    // per-query index lists (see ListArgs)
  kModeEven = 2,    // equal token ranges (see EvenArgs)
};

// kModeEven: the selected tokens of all sequences, concatenated in sequence
// order (T of them), are cut into G equal ranges per column of KV-head units;
// workgroup i of a column takes tokens [i*T/G, (i+1)*T/G) and writes one
// partial per sequence its range touches, at piece index i + b of the head's
// row of `pstride` = G + B partials (unique: for a sequence the pieces are
// consecutive workgroups, and a workgroup's pieces consecutive sequences).
// With every range equally long and the grid one round of resident
// workgroups, no short tail of lone workgroups ends the launch.  G shrinks
// to min(G, ceil(T / kEvenMinTokens)) on the device so that every range
// holds tokens.  Workgroup 0 also writes the sequences' first concatenated
// token (starts[b], starts[B] = T) for the combine.
constexpr int kEvenMinTokens = 64;
constexpr int kEvenMaxG = kDecodeEvenMaxG;  // workgroups per column the workspace has room for
struct EvenArgs {
  int G;
  int pstride;
  int32_t* starts;  // [B + 1]
};
__host__ __device__ __forceinline__ int even_groups(int G, int T) {
  return max(1, min(G, (T + kEvenMinTokens - 1) / kEvenMinTokens));
}
// Workgroup (of Ge) whose range holds concatenated token t < T.
__host__ __device__ __forceinline__ int even_owner(long long t, int Ge, int T) {
  return (int)(((t + 1) * Ge + T - 1) / T) - 1;
}

template <int D, int NW, int MODE, bool BUF>
__global__ __launch_bounds__(64 * NW) void decode_partial_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seqlens, float* __restrict__ part,
    const int32_t* __restrict__ items, const int32_t* __restrict__ count, int B, int Hq, int Hkv,
    int hgroups, int page_shift, int max_pages, float sl2, int w1, int w2, int chunk,
    int max_splits, ListArgs la, EvenArgs ev, uint32_t kv_bytes) {
  ATTN_SINK_CHECK_GUARD();
  constexpr bool LIST = MODE == kModeList;
  __shared__ DecLds<D, NW> s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int kg = lane >> 4, hl = lane & 15;
  const int nxu = (Hkv * hgroups + NW - 1) / NW;
  const int j = blockIdx.x / nxu;
  const int unit = (blockIdx.x % nxu) * NW + wave;
  const bool active = unit < Hkv * hgroups;
  const int kvh = active ? unit / hgroups : 0, hgi = active ? unit % hgroups : 0;
  const int g = Hq / Hkv;
  const int g_eff = min(16, g - 16 * hgi);
  const int h0 = kvh * g + 16 * hgi;
  const size_t rs = (size_t)Hkv * D;
  const __bf16* kbase = kc + (size_t)kvh * D;
  const __bf16* vbase = vc + (size_t)kvh * D;
  const uint32_t head_bytes = (uint32_t)(kvh * D * 2);
  const auto rk = make_rsrc(kbase, kv_bytes - head_bytes);
  const auto rv = make_rsrc(vbase, kv_bytes - head_bytes);
  const uint32_t rs_bytes = (uint32_t)(rs * 2);
  auto load_step = [&](KVRegs<D>& regs, int base) {
    if constexpr (BUF)
      regs.load(s.slot, base, rk, rv, rs_bytes, lane);
    else
      regs.load(s.slot, base, kbase, vbase, rs, lane);
  };
  constexpr int TPL = KVRegs<D>::TPL, NTG = KVRegs<D>::NTG;
  __bf16* vt = s.v[wave];

  // One piece: selected tokens u0 .. u1-1 of sequence b (L cached tokens;
  // LIST: packed row b of sequence seq at position pos), with its partial
  // (acc, m, l) for head h written at index pbase + h * pstride.
  auto run = [&](int b, int seq, int L, int pos, int u0, int u1, size_t pbase, size_t pstride) {
    const int32_t* bt_row = bt + (size_t)(LIST ? seq : b) * max_pages;
    // Q^T fragments (B operand): column = head hl, k = d = 32*s + 8*kg ..
    bf16x8 qf[D / 32];
#pragma unroll
    for (int s2 = 0; s2 < D / 32; ++s2)
      qf[s2] = (active && hl < g_eff)
                   ? *reinterpret_cast<const bf16x8*>(q + ((size_t)b * Hq + h0 + hl) * D + 32 * s2 + 8 * kg)
                   : bf16x8{};

    float m = kNegInf, l = 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc[db] = f32x4{};

    // One 32-token step of this wave: scores, online softmax, V^T staging, P.V.
    auto step = [&](const KVRegs<D>& cur, int base, int nsub) {
      f32x4 sc[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int s2 = 0; s2 < D / 32; ++s2)
          sc[G] = mfma16(__builtin_bit_cast(bf16x8, cur.kr[G][s2]), qf[s2], sc[G]);
      float x[8];
#pragma unroll
      for (int G = 0; G < 2; ++G)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[4 * G + j] = (base + 8 * kg + 4 * G + j < nsub) ? sc[G][j] : kNegInf;
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m, mx * sl2);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      m = m_new;
      float p[8], rsum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2_fast(__builtin_fmaf(x[e], sl2, -m_use));
        rsum += p[e];
      }
      l = l * alpha + rsum;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) acc[db] *= alpha;
      const bf16x8 pf = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);

      // V staging, natural rows: token TPL*tg + t, d-chunk c; rows without a
      // selected token are written as zeros
      {
        const int tg = lane % NTG, c = lane / NTG;
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
          const bool ok = (cur.vvalid >> t) & 1u;
          const uint4 x = cur.vr[t];
          *reinterpret_cast<uint4*>(vt + (TPL * tg + t) * vrow<D>() + 8 * c) =
              uint4{ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u};
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int db = 0; db < D / 16; ++db) acc[db] = mfma16(vt_frag16<D>(vt, db, lane), pf, acc[db]);
      wave_lds_sync();
    };

    for (int sub0 = u0; sub0 < u1; sub0 += kSub) {
      constexpr int kPer = kSub / (64 * NW);
      int nsub, nsteps, npad;
      if constexpr (LIST) {
        // thread t takes list entries t*kPer .. +kPer-1 of the block; the valid
        // ones are compacted in entry order (a workgroup-wide exclusive scan of
        // the per-thread counts), the rest of the table up to npad holds -1
        const int ne = min(kSub, u1 - sub0);
        const int32_t* lrow = la.kv_index + (size_t)b * la.topk + sub0;
        int tv[kPer], sv[kPer], cnt = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int x = tid * kPer + i;
          const int t = lrow[min(x, ne - 1)];
          const bool ok = (x < ne) & (t >= 0) & (t < L) & (t <= pos);
          tv[i] = ok ? t : -1;
          cnt += ok ? 1 : 0;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) sv[i] = slot_of(bt_row, max(tv[i], 0), page_shift);
#pragma unroll
        for (int i = 0; i < kPer; ++i) asm volatile("" : "+v"(sv[i]));
        int x = cnt;  // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(x, d, 64);
          if (lane >= d) x += y;
        }
        if (lane == 63) s.wsum[wave] = x;
        __syncthreads();
        int off = x - cnt, total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          off += w < wave ? s.wsum[w] : 0;
          total += s.wsum[w];
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (tv[i] >= 0) s.slot[off++] = sv[i];
        nsub = total;
        nsteps = (nsub + 31) >> 5;
        npad = min(kSub, 64 * max(1, (nsteps + 1) >> 1));
        for (int y = nsub + tid; y < npad; y += 64 * NW) s.slot[y] = -1;
      } else {
        nsub = min(kSub, u1 - sub0);
        nsteps = (nsub + 31) >> 5;
        // slot table of this block, padded with -1 up to an even number of steps;
        // every block-table load of a thread is issued before its first LDS write,
        // so the table costs one memory latency (overlapping the Q loads)
        npad = min(kSub, 64 * ((nsteps + 1) >> 1));
        int sv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i)  // index clamped to a selected token
          sv[i] = slot_of(bt_row, token_of(sub0 + min(tid + i * 64 * NW, nsub - 1), L, w1, w2),
                          page_shift);
        // keep the loads unconditional and issued together (otherwise the compiler
        // sinks each one into the branch that uses it and waits for it there)
#pragma unroll
        for (int i = 0; i < kPer; ++i) asm volatile("" : "+v"(sv[i]));
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int x = tid + i * 64 * NW;
          if (x < npad) s.slot[x] = x < nsub ? sv[i] : -1;
        }
      }
      __syncthreads();
      // start the step loop with no VMEM load pending, so that the compiler's
      // wait tracking does not hold a step's MFMAs on the next step's prefetch
      __builtin_amdgcn_s_waitcnt(0);
      if (active) {
        // Two register sets in turn, two steps per iteration with no exit in
        // between (so the compiler cannot sink the prefetch below a branch); an
        // odd last step runs on padding slots and is fully masked.
        // sched_barrier keeps each prefetch issued ahead of the step it overlaps
        KVRegs<D> ra, rb;
        load_step(ra, 0);
        for (int st = 0; st < nsteps; st += 2) {
          load_step(rb, 32 * (st + 1));
          __builtin_amdgcn_sched_barrier(0);
          step(ra, 32 * st, nsub);
          load_step(ra, 32 * min(st + 2, npad / 32 - 1));
          __builtin_amdgcn_sched_barrier(0);
          step(rb, 32 * (st + 1), nsub);
        }
      }
      __syncthreads();
    }
    if (!active) return;

    // ---- partial (acc, m, l) of this wave's heads: lane (kg, hl) holds head hl,
    // d = 16*db + 4*kg + j
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (hl < g_eff) {
      float* dst = part + (pbase + (size_t)(h0 + hl) * pstride) * (D + 2);
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * kg) = acc[db];
      if (kg == 0) {
        dst[D] = m;
        dst[D + 1] = l;
      }
    }
  };  // run

  if constexpr (MODE == kModeEven) {
    // every wave scans the selected-token counts itself (B <= kScanSeqs;
    // T < 2^31 is checked by the host)
    constexpr int R = kScanSeqs / 64;
    int len[R], nsel[R], st[R];
#pragma unroll
    for (int r = 0; r < R; ++r) len[r] = seqlens[min(64 * r + lane, B - 1)];
    int T = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      nsel[r] = 64 * r + lane < B ? n_selected(len[r], w1, w2) : 0;
      int x = nsel[r];  // inclusive scan over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      st[r] = T + x - nsel[r];
      T += __shfl(x, 63, 64);
    }
    if (blockIdx.x == 0 && wave == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (64 * r + lane < B) ev.starts[64 * r + lane] = st[r];
      if (lane == 0) ev.starts[B] = T;
    }
    if (T == 0) return;  // uniform over the workgroup
    const int Ge = even_groups(ev.G, T);
    if (j >= Ge) return;  // uniform over the workgroup
    const int lo = (int)((long long)j * T / Ge), hi = (int)((long long)(j + 1) * T / Ge);
    // first sequence whose tokens reach past lo, then every one starting before hi
    int rem = lo, first = 0, before = 0, b = -1;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (b < 0 && wave_find(nsel[r], rem, lane, first, before)) b = 64 * r + first;
    b = __builtin_amdgcn_readfirstlane(b);
    for (; b < B; ++b) {
      int sb = 0, nb = 0, Lb = 0;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if ((b >> 6) == r) {
          sb = __shfl(st[r], b & 63, 64);
          nb = __shfl(nsel[r], b & 63, 64);
          Lb = __shfl(len[r], b & 63, 64);
        }
      sb = __builtin_amdgcn_readfirstlane(sb);
      nb = __builtin_amdgcn_readfirstlane(nb);
      Lb = __builtin_amdgcn_readfirstlane(Lb);
      if (sb >= hi) break;
      if (nb == 0) continue;
      run(b, 0, Lb, 0, max(lo, sb) - sb, min(hi, sb + nb) - sb, (size_t)j + b,
          (size_t)ev.pstride);
    }
  } else {
    int b, split, L, seq = 0, pos = 0;
    if constexpr (LIST) {
      split = j % max_splits;
      b = j / max_splits;
      seq = la.row_seq[b];
      L = seqlens[seq];
      const int qs = la.cu_q[seq];
      pos = L - (la.cu_q[seq + 1] - qs) + (b - qs);
      seq = __builtin_amdgcn_readfirstlane(seq);
      pos = __builtin_amdgcn_readfirstlane(pos);
    } else if (items) {
      if (j >= *count) return;  // uniform over the workgroup
      const int item = items[j];
      split = item % max_splits;
      b = item / max_splits;
      L = seqlens[b];
    } else if (!find_chunk(seqlens, B, w1, w2, chunk, max_splits, j, lane, b, split, L)) {
      return;  // uniform over the workgroup
    }
    b = __builtin_amdgcn_readfirstlane(b);
    split = __builtin_amdgcn_readfirstlane(split);
    L = __builtin_amdgcn_readfirstlane(L);
    const int nsel = LIST ? la.topk : n_selected(L, w1, w2);
    const int u0 = split * chunk;
    if (u0 >= nsel) return;  // uniform over the workgroup
    run(b, seq, L, pos, u0, min(nsel, u0 + chunk), (size_t)b * Hq * max_splits + split,
        (size_t)max_splits);
  }
}

// One wave per (sequence, query head): merge the chunk partials and fold the
// sink in once: M = max(sink', m_k), Z = 2^(sink'-M) + sum 2^(m_k-M) l_k,
// O = sum 2^(m_k-M) acc_k / Z, LSE = (M + log2 Z) ln 2.
template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ seqlens,
    const float* __restrict__ sink, __bf16* __restrict__ o, float* __restrict__ lse, int B, int Hq,
    int w1, int w2, int chunk, int max_splits, EvenArgs ev) {
  ATTN_SINK_CHECK_GUARD();
  constexpr bool LIST = MODE == kModeList;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= B * Hq) return;
  const int b = bh / Hq, h = bh % Hq;
  int nsp = max_splits;  // LIST: every chunk of every row holds a partial
  const float* base = part + (size_t)bh * max_splits * (D + 2);
  if constexpr (MODE == kModeEven) {
    // pieces i0 .. i1: the workgroups whose ranges hold this sequence's tokens
    const int sb = ev.starts[b], nb = ev.starts[b + 1] - sb, T = ev.starts[B];
    nsp = 0;
    if (nb > 0) {
      const int Ge = even_groups(ev.G, T);
      const int i0 = even_owner(sb, Ge, T), i1 = even_owner((long long)sb + nb - 1, Ge, T);
      nsp = i1 - i0 + 1;
      base = part + ((size_t)h * ev.pstride + i0 + b) * (D + 2);
    }
  } else if constexpr (!LIST) {
    const int nsel = n_selected(seqlens[b], w1, w2);
    nsp = nsel > 0 ? min(max_splits, (nsel + chunk - 1) / chunk) : 0;
  }
  const float sig2 = sink ? sink[h] * kLog2e : kNegInf;
  constexpr int DPL = D / 64;
  float od[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) od[i] = 0.f;
  float M = sig2, z = 0.f;

  if (nsp <= 8) {
    // up to 8 pieces (the equal-range grids have about B_total/B + 1 per
    // sequence): every lane loads every piece's (m, l) and its own d of the
    // accumulators at once, one memory round trip instead of three
    float mk[8], lk[8], ak[8][DPL];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mk[j] = kNegInf;
      lk[j] = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) ak[j][i] = 0.f;
      if (j < nsp) {  // wave-uniform
        const float* pk = base + (size_t)j * (D + 2);
        mk[j] = pk[D];
        lk[j] = pk[D + 1];
#pragma unroll
        for (int i = 0; i < DPL; ++i) ak[j][i] = pk[lane + 64 * i];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) M = fmaxf(M, mk[j]);
    const float Mu = M == kNegInf ? 0.f : M;  // nothing visible and no sink
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = exp2_fast(mk[j] - Mu);  // 0 for pieces past the end
      z += f * lk[j];
#pragma unroll
      for (int i = 0; i < DPL; ++i) od[i] += f * ak[j][i];
    }
    if (sig2 != kNegInf) z += exp2_fast(sig2 - Mu);
    const float inv = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[(size_t)bh * D + lane + 64 * i] = (__bf16)(od[i] * inv);
    if (lse && lane == 0)
      lse[LIST ? (size_t)h * B + b : (size_t)bh] = z > 0.f ? (Mu + log2_fast(z)) * kLn2 : kNegInf;
    return;
  }

  // pass 1: lane k reads chunk k's (m, l); the max and the weighted sum of l
  // are wave reductions, so no load waits on another
  for (int k = lane; k < nsp; k += 64) M = fmaxf(M, base[(size_t)k * (D + 2) + D]);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) M = wave_max_xor(M, x);
  const float Mu = M == kNegInf ? 0.f : M;  // nothing visible and no sink
  for (int k = lane; k < nsp; k += 64) {
    const float* pk = base + (size_t)k * (D + 2);
    z += exp2_fast(pk[D] - Mu) * pk[D + 1];
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) z += __shfl_xor(z, x, 64);

  // pass 2: lane = d; chunks in groups of 8 with all loads issued first
  for (int k0 = 0; k0 < nsp; k0 += 8) {
    float mk[8], ak[8][DPL];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = min(k0 + j, nsp - 1);
      const float* pk = base + (size_t)k * (D + 2);
      mk[j] = k0 + j < nsp ? pk[D] : kNegInf;
#pragma unroll
      for (int i = 0; i < DPL; ++i) ak[j][i] = pk[lane + 64 * i];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = exp2_fast(mk[j] - Mu);  // 0 for chunks past the end
#pragma unroll
      for (int i = 0; i < DPL; ++i) od[i] += f * ak[j][i];
    }
  }
  if (sig2 != kNegInf) z += exp2_fast(sig2 - Mu);
  const float inv = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[(size_t)bh * D + lane + 64 * i] = (__bf16)(od[i] * inv);
  // LSE [B, Hq], or [Hq, B] for packed rows (LIST)
  if (lse && lane == 0)
    lse[LIST ? (size_t)h * B + b : (size_t)bh] = z > 0.f ? (Mu + log2_fast(z)) * kLn2 : kNegInf;
}

__global__ void select_slots_kernel(const int32_t* __restrict__ bt,
                                    const int32_t* __restrict__ seqlens, int max_pages,
                                    int page_shift, int w1, int w2, int64_t* __restrict__ slots,
                                    int32_t* __restrict__ counts, int max_sel) {
  const int b = blockIdx.x;
  const int L = seqlens[b];
  const int nsel = n_selected(L, w1, w2);
  const int32_t* bt_row = bt + (size_t)b * max_pages;
  for (int u = threadIdx.x; u < max_sel; u += blockDim.x)
    slots[(size_t)b * max_sel + u] =
        u < nsel ? (int64_t)slot_of(bt_row, token_of(u, L, w1, w2), page_shift) : -1;
  if (threadIdx.x == 0) counts[b] = nsel;
}

// One workgroup per (selected index, sequence); copies Hkv*D elements.
__global__ void gather_kv_kernel(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                                 const int32_t* __restrict__ bt,
                                 const int32_t* __restrict__ seqlens, int row_elems,
                                 int max_pages, int page_shift, int w1, int w2,
                                 uint16_t* __restrict__ ko, uint16_t* __restrict__ vo,
                                 int max_sel, int elem_halves) {
  const int u = blockIdx.x, b = blockIdx.y;
  const int L = seqlens[b];
  const int nsel = n_selected(L, w1, w2);
  const size_t n = (size_t)row_elems * elem_halves;  // row length in 16-bit words
  uint16_t* kd = ko + ((size_t)b * max_sel + u) * n;
  uint16_t* vd = vo + ((size_t)b * max_sel + u) * n;
  if (u >= nsel) {
    for (size_t x = threadIdx.x; x < n; x += blockDim.x) kd[x] = vd[x] = 0;
    return;
  }
  const size_t slot = (size_t)slot_of(bt + (size_t)b * max_pages, token_of(u, L, w1, w2), page_shift);
  for (size_t x = threadIdx.x; x < n; x += blockDim.x) {
    kd[x] = kc[slot * n + x];
    vd[x] = vc[slot * n + x];
  }
}

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace

DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int page_size, int max_pages, int w1, int w2,
                       int num_splits) {
  DecodePlan p{0, 0, 0, false};
  const long long maxL = (long long)max_pages * page_size;
  const long long max_sel = (w2 > 0) ? std::min<long long>(maxL, (long long)w1 + w2) : maxL;
  const int g = Hq / Hkv;
  const long long units = (long long)B * Hkv * ((g + 15) / 16);
  // Equal token ranges (kModeEven) unless a split count is asked for, the
  // sequences are too many for the in-kernel scan, their total could overflow
  // int32, or the work is small: with fewer than 1024 units x 2048-token
  // chunks, equal ranges become short pieces that each pay a workgroup's
  // start and a partial (the single-sequence 1024 + 7168 window decode:
  // 24 -> 32 us), and the chunks below serve better.
  if (num_splits == 0 && B <= kScanSeqs && (long long)B * max_sel <= INT32_MAX &&
      units * ((max_sel + 2047) / 2048) >= 1024) {
    p.even = true;
    p.chunk = 0;
    p.max_splits = 0;
    p.workspace_bytes = (size_t)Hq * (kEvenMaxG + B) * (D + 2) * sizeof(float) +
                        ((size_t)B + 1) * sizeof(int32_t);
    return p;
  }
  long long chunk;
  if (num_splits > 0) {
    chunk = (max_sel + num_splits - 1) / num_splits;
    chunk = (chunk + 31) / 32 * 32;
  } else {
    // Long chunks amortise each workgroup's start (slot table, first loads);
    // shorter ones only when long ones leave too few waves in flight.
    chunk = 2048;
    if (units * ((max_sel + chunk - 1) / chunk) < 1024) {
      chunk = 1024;
      while (chunk > 128 && units * ((max_sel + chunk - 1) / chunk) < 2048) chunk /= 2;
    }
  }
  if (chunk < 32) chunk = 32;
  p.chunk = (int)chunk;
  p.max_splits = (int)((max_sel + chunk - 1) / chunk);
  if (p.max_splits < 1) p.max_splits = 1;
  // partials, then the chunk list and its length
  p.workspace_bytes = (size_t)B * Hq * p.max_splits * (D + 2) * sizeof(float) +
                      ((size_t)B * p.max_splits + 1) * sizeof(int32_t);
  return p;
}

namespace {
// Workgroups of decode_partial_kernel<D, 4, kModeEven, BUF> resident on the
// whole device at once (CUs x workgroups per CU), per device, computed once.
template <int D, bool BUF>
int even_capacity() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, decode_partial_kernel<D, 4, kModeEven, BUF>, 256, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  c = cus * per_cu;
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}
}  // namespace

// ---------------------------------------------------------------------------
// Library-held scratch of attn_sink_fwd_decode_paged_noalloc, for callers that
// cannot allocate: the split partials and their bookkeeping of one call (the
// workspace of attn_sink_fwd_decode_paged).  Each device that runs the entry
// point holds its own copy until the process ends; host code reaches it only
// through the device address hipGetSymbolAddress returns for that device.
// ---------------------------------------------------------------------------
namespace {
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // once per device, with that device current
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<float*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const int hgroups = (g + 15) / 16;
  const int units = a.Hkv * hgroups;
  const int page_shift = log2_exact(a.page_size);
  const float sl2 = a.scale * kLog2e;
  const auto* q = static_cast<const __bf16*>(a.q);
  const auto* kc = static_cast<const __bf16*>(a.k_cache);
  const auto* vc = static_cast<const __bf16*>(a.v_cache);
  auto* o = static_cast<__bf16*>(a.o);
  const dim3 cgrid((a.B * a.Hq + 3) / 4);
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using W2 = std::integral_constant<int, 2>;
  using W4 = std::integral_constant<int, 4>;

  // caches below 4 GiB (each of K and V) are read through buffer resources
  const long long kv_bytes = (long long)a.num_pages * a.page_size * a.Hkv * a.D * 2;
  const bool buf = kv_bytes > 0 && kv_bytes < (1LL << 32);
  const uint32_t kvb = buf ? (uint32_t)kv_bytes : 0u;
  using T = std::true_type;
  using F = std::false_type;
#ifdef ATTN_SINK_DEVICE_CHECKS
  // sequence lengths in [1, max_pages * page_size], block-table entries of the
  // selected tokens' pages in [0, num_pages)
  check_paged_kernel<<<a.B, 256, 0, stream>>>(a.block_table, a.seqlens, nullptr, a.B, 0, 0,
                                               a.max_pages, a.page_size, a.num_pages, 1, a.w1,
                                               a.w2, 1);
#endif

  if (a.even) {
    // one round of resident workgroups (measured: two rounds of half-length
    // ranges are 1-4 % slower), split evenly over the columns of 4 KV-head
    // units
    const int ncols = (units + 3) / 4;
    auto run = [&](auto d, auto use_buf) {
      constexpr int D = decltype(d)::value;
      constexpr bool BUF = decltype(use_buf)::value;
      const int cap = even_capacity<D, BUF>();
      const int G = std::max(1, std::min(kEvenMaxG, cap / ncols));
      const EvenArgs ev{G, G + a.B,
                        reinterpret_cast<int32_t*>(a.partials +
                                                   (size_t)a.Hq * (kEvenMaxG + a.B) * (a.D + 2))};
      decode_partial_kernel<D, 4, kModeEven, BUF>
          <<<dim3((unsigned)(ncols * G)), 256, 0, stream>>>(
              q, kc, vc, a.block_table, a.seqlens, a.partials, nullptr, nullptr, a.B, a.Hq,
              a.Hkv, hgroups, page_shift, a.max_pages, sl2, a.w1, a.w2, 0, 0, ListArgs{}, ev,
              kvb);
      decode_combine_kernel<D, kModeEven><<<cgrid, kThreads, 0, stream>>>(
          a.partials, a.seqlens, a.sink, o, a.lse, a.B, a.Hq, a.w1, a.w2, 0, 0, ev);
    };
    if (a.D == 64)
      buf ? run(I64{}, T{}) : run(I64{}, F{});
    else
      buf ? run(I128{}, T{}) : run(I128{}, F{});
    return hipGetLastError();
  }

  int32_t* items = reinterpret_cast<int32_t*>(a.partials + (size_t)a.B * a.Hq * a.max_splits *
                                                               (a.D + 2));
  int32_t* count = items + (size_t)a.B * a.max_splits;
  if (a.B > kScanSeqs) {
    decode_plan_kernel<<<1, 256, 0, stream>>>(a.seqlens, a.B, a.w1, a.w2, a.chunk, a.max_splits,
                                               items, count);
  } else {
    items = nullptr;
    count = nullptr;
  }
  // 4 waves per workgroup (4 KV heads of one chunk sharing a slot table),
  // unless that leaves CUs without a workgroup: then 2, which doubles the
  // workgroups (the single-sequence window decode: 24 -> 19 us).
  const long long slots = (long long)a.B * a.max_splits;
  const bool narrow = ((units + 3) / 4) * slots < 256;
  auto partial = [&](auto d, auto nw) {
    constexpr int D = decltype(d)::value, NW = decltype(nw)::value;
    const dim3 grid((unsigned)(((units + NW - 1) / NW) * slots));
    if (buf)
      decode_partial_kernel<D, NW, kModeChunks, true><<<grid, 64 * NW, 0, stream>>>(
          q, kc, vc, a.block_table, a.seqlens, a.partials, items, count, a.B, a.Hq, a.Hkv,
          hgroups, page_shift, a.max_pages, sl2, a.w1, a.w2, a.chunk, a.max_splits, ListArgs{},
          EvenArgs{}, kvb);
    else
      decode_partial_kernel<D, NW, kModeChunks, false><<<grid, 64 * NW, 0, stream>>>(
          q, kc, vc, a.block_table, a.seqlens, a.partials, items, count, a.B, a.Hq, a.Hkv,
          hgroups, page_shift, a.max_pages, sl2, a.w1, a.w2, a.chunk, a.max_splits, ListArgs{},
          EvenArgs{}, 0u);
  };
  if (a.D == 64) {
    if (narrow)
      partial(I64{}, W2{});
    else
      partial(I64{}, W4{});
    decode_combine_kernel<64, kModeChunks><<<cgrid, kThreads, 0, stream>>>(
        a.partials, a.seqlens, a.sink, o, a.lse, a.B, a.Hq, a.w1, a.w2, a.chunk, a.max_splits,
        EvenArgs{});
  } else {
    if (narrow)
      partial(I128{}, W2{});
    else
      partial(I128{}, W4{});
    decode_combine_kernel<128, kModeChunks><<<cgrid, kThreads, 0, stream>>>(
        a.partials, a.seqlens, a.sink, o, a.lse, a.B, a.Hq, a.w1, a.w2, a.chunk, a.max_splits,
        EvenArgs{});
  }
  return hipGetLastError();
}

// Packed row -> its sequence, for the per-query list mode.
__global__ __launch_bounds__(256) void row_seq_kernel(const int32_t* __restrict__ cu_q,
                                                      int32_t* __restrict__ row_seq) {
  ATTN_SINK_CHECK_GUARD();
  const int b = blockIdx.x;
  for (int r = cu_q[b] + threadIdx.x; r < cu_q[b + 1]; r += 256) row_seq[r] = b;
}

DecodePlan plan_index_rows(int total_q, int Hq, int Hkv, int D, int topk) {
  // the decode plan with the list length as every row's selection and the
  // rows as its sequences
  (void)D;
  DecodePlan p{0, 0, 0};
  const int g = Hq / Hkv;
  const long long units = (long long)total_q * Hkv * ((g + 15) / 16);
  long long chunk = 2048;
  if (units * ((topk + chunk - 1) / chunk) < 1024) {
    chunk = 1024;
    while (chunk > 128 && units * ((topk + chunk - 1) / chunk) < 2048) chunk /= 2;
  }
  p.chunk = (int)chunk;
  p.max_splits = (int)((topk + chunk - 1) / chunk);
  if (p.max_splits < 1) p.max_splits = 1;
  p.workspace_bytes = (size_t)total_q * Hq * p.max_splits * (D + 2) * sizeof(float) +
                      (size_t)total_q * sizeof(int32_t);
  return p;
}

hipError_t launch_index_rows_bf16(const IndexRowsArgs& a, hipStream_t stream) {
  const DecodePlan plan = plan_index_rows(a.total_q, a.Hq, a.Hkv, a.D, a.topk);
  const int g = a.Hq / a.Hkv;
  const int hgroups = (g + 15) / 16;
  const int units = a.Hkv * hgroups;
  const int page_shift = log2_exact(a.page_size);
  const float sl2 = a.scale * kLog2e;
  const auto* q = static_cast<const __bf16*>(a.q);
  const auto* kc = static_cast<const __bf16*>(a.k_cache);
  const auto* vc = static_cast<const __bf16*>(a.v_cache);
  auto* o = static_cast<__bf16*>(a.o);
  float* part = static_cast<float*>(a.workspace);
  int32_t* row_seq = reinterpret_cast<int32_t*>(part + (size_t)a.total_q * a.Hq *
                                                            plan.max_splits * (a.D + 2));
#ifdef ATTN_SINK_DEVICE_CHECKS
  // query offsets, lengths in [0, max_pages * page_size] and every page of [0, L)
  check_paged_kernel<<<a.B, 256, 0, stream>>>(
      a.block_table, a.seqlens_k, a.cu_seqlens_q, a.B, a.total_q, a.total_q, a.max_pages,
      a.page_size, (int)(a.kv_rows / a.page_size), 0, -1, -1, 0);
#endif
  row_seq_kernel<<<a.B, 256, 0, stream>>>(a.cu_seqlens_q, row_seq);
  const ListArgs la{a.kv_index, row_seq, a.cu_seqlens_q, a.topk};
  const long long slots = (long long)a.total_q * plan.max_splits;
  const bool narrow = ((units + 3) / 4) * slots < 256;
  // caches below 4 GiB (each of K and V) are read through buffer resources
  const long long kv_bytes = a.kv_rows * a.Hkv * a.D * 2;
  const bool buf = kv_bytes > 0 && kv_bytes < (1LL << 32);
  auto partial = [&](auto d, auto nw) {
    constexpr int D = decltype(d)::value, NW = decltype(nw)::value;
    const dim3 grid((unsigned)(((units + NW - 1) / NW) * slots));
    if (buf)
      decode_partial_kernel<D, NW, kModeList, true><<<grid, 64 * NW, 0, stream>>>(
          q, kc, vc, a.block_table, a.seqlens_k, part, nullptr, nullptr, a.total_q, a.Hq, a.Hkv,
          hgroups, page_shift, a.max_pages, sl2, -1, -1, plan.chunk, plan.max_splits, la,
          EvenArgs{}, (uint32_t)kv_bytes);
    else
      decode_partial_kernel<D, NW, kModeList, false><<<grid, 64 * NW, 0, stream>>>(
          q, kc, vc, a.block_table, a.seqlens_k, part, nullptr, nullptr, a.total_q, a.Hq, a.Hkv,
          hgroups, page_shift, a.max_pages, sl2, -1, -1, plan.chunk, plan.max_splits, la,
          EvenArgs{}, 0u);
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using W2 = std::integral_constant<int, 2>;
  using W4 = std::integral_constant<int, 4>;
  const dim3 cgrid((a.total_q * a.Hq + 3) / 4);
  if (a.D == 64) {
    if (narrow)
      partial(I64{}, W2{});
    else
      partial(I64{}, W4{});
    decode_combine_kernel<64, kModeList><<<cgrid, kThreads, 0, stream>>>(
        part, a.seqlens_k, a.sink, o, a.lse, a.total_q, a.Hq, -1, -1, plan.chunk,
        plan.max_splits, EvenArgs{});
  } else {
    if (narrow)
      partial(I128{}, W2{});
    else
      partial(I128{}, W4{});
    decode_combine_kernel<128, kModeList><<<cgrid, kThreads, 0, stream>>>(
        part, a.seqlens_k, a.sink, o, a.lse, a.total_q, a.Hq, -1, -1, plan.chunk,
        plan.max_splits, EvenArgs{});
  }
  return hipGetLastError();
}

hipError_t launch_select_slots(const int32_t* bt, const int32_t* seqlens, int B, int max_pages,
                               int page_size, int w1, int w2, int64_t* slots, int32_t* counts,
                               int max_sel, hipStream_t stream) {
  select_slots_kernel<<<B, 256, 0, stream>>>(bt, seqlens, max_pages, log2_exact(page_size), w1, w2,
                                             slots, counts, max_sel);
  return hipGetLastError();
}

hipError_t launch_gather_kv(const void* kc, const void* vc, const int32_t* bt,
                            const int32_t* seqlens, int B, int Hkv, int D, int page_size,
                            int max_pages, int w1, int w2, void* k_out, void* v_out, int max_sel,
                            int elem_bytes, hipStream_t stream) {
  const dim3 grid(max_sel, B);
  gather_kv_kernel<<<grid, 256, 0, stream>>>(
      static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), bt, seqlens, Hkv * D,
      max_pages, log2_exact(page_size), w1, w2, static_cast<uint16_t*>(k_out),
      static_cast<uint16_t*>(v_out), max_sel, elem_bytes / 2);
  return hipGetLastError();
}

#ifdef ATTN_SINK_DEVICE_CHECKS
ATTN_SINK_DEFINE_CHECK_READER(read_check_word_decode)
#endif

}  // namespace attn_sink
