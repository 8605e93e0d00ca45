// Backward of attention with a learnable per-head sink (bf16, fp32 accumulate).
//
// With P_ij = exp(s_ij - LSE_i) (LSE from the forward, sink included) and
// Di = <dO_i, O_i>:
//   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (<dO_i, v_j> - Di),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dSink_h = -sum_{b,i} exp(sink_h - LSE_i) Di
// (flash-attention PR #1819 "feat: Implement Sink Attention", Description:
// the backward returns the sink's gradient).  Because the sink has no value
// row and LSE already contains it, the sink needs no term in the main
// kernels: its gradient is a by-product of the Di pass.
//
// Kernels (all deterministic, no atomics):
//   bwd_preprocess   -Di, LSE * log2(e) and per-(b, h, 64-row block) dSink
//                    partials
//   bwd_dkdv         KV-stationary: a wave owns 32 keys and accumulates dK/dV
//                    over all query heads of its GQA group and all query tiles
//                    that can see them
//   bwd_dq           Q-stationary (the forward's frame): recomputes S and dP
//                    and accumulates dQ in registers
//   bwd_main         (D 64) the dK/dV and dQ blocks in one launch
//   bwd_dsink_reduce fixed-order sum of the dSink partials
#include <cstddef>
#include <type_traits>

#include "checks.h"
#include "common.h"
#include "launch.h"

namespace attn_sink {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;  // rows per query tile / keys per KV tile
constexpr int kPad = 8;    // LDS row padding (elements, 16 B)


__device__ __forceinline__ uint32_t pick16(const uint4& x, int e) {
  const uint32_t w = e < 2 ? x.x : (e < 4 ? x.y : (e < 6 ? x.z : x.w));
  return (w >> (16 * (e & 1))) & 0xffffu;
}

// A operand (32 d x 16 rows) of an MFMA that contracts over tile rows, read
// from a natural-layout tile (rows permuted within 32-blocks by perm_row):
// lane l gets d = 32*db + l%32 and logical rows r0 + 16*(l/32) .. +7 (r0 a
// multiple of 8).  ds_read_b64_tr_b16 hands lane i of each 16-lane group
// element i%4 of the 4-element vectors that lanes 4j + i/4 (j = 0..3) of the
// group addressed, in order of j; so lane s of a group addresses logical row
// (r0 + 16*hh + 4h + s/4), columns (32*db + 16*gg + 4*(s%4)) .. +3, for the
// two loads h = 0, 1.  Under perm_row those rows sit at LDS rows
// (r0 & ~31) + 2*(r0 & 31) + 4*hh + s/4 + 8h.  The lane's part and the
// constant part of the address are added once, so that the compiler keeps
// the read tied to its LDS buffer (see the tile loads in common.h).
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* nat, int r0, int db, int lane) {
  constexpr int NS = D + kPad;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int sl = lane & 15, gg = (lane >> 4) & 1, hh = lane >> 5;
  const int ol = (4 * hh + (sl >> 2)) * NS + 16 * gg + 4 * (sl & 3);
  const int oc = ((r0 & ~31) + 2 * (r0 & 31)) * NS + 32 * db;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(nat + (ol + oc)));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(nat + (ol + oc + 8 * NS)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Rows [0, NR) of a wave's LDS region `stage` (rows of D + 8 elements) to
// global memory, 16 bytes per lane, eight lanes per row at D = 64: every store
// instruction writes whole rows instead of 8-byte pieces of 32 rows.  row_ptr(r)
// is row r's destination, NULL to skip it.  The caller has written the rows.
template <int D, int NR, typename RowPtr>
__device__ __forceinline__ void store_staged(const __bf16* stage, int lane, RowPtr row_ptr) {
  constexpr int SS = D + kPad, CPR = D / 8;
  static_assert((NR * CPR) % 64 == 0, "whole store instructions");
  // the wave's own LDS writes are in order before its reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int c0 = 0; c0 < NR * CPR; c0 += 64) {
    const int r = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * SS + 8 * ch);
    __bf16* dst = row_ptr(r);
    if (dst) *reinterpret_cast<u32x4*>(dst + 8 * ch) = v;
  }
}

// LDS tile buffers per pass: K/V or Q/dO tiles are loaded straight into LDS
// one tile (two buffers) or two tiles (three) ahead of the one in use.  D = 64
// runs two workgroups per CU and keeps two buffers (three measured 1.3 %
// slower on training: the longer unrolled loop spills); D = 128 runs one
// workgroup per CU and takes three (backward 3 % faster).
template <int D>
constexpr int bwd_bufs() { return D == 64 ? 2 : 3; }

// Rows of sequence b.  A dense batch (cu_q == NULL) has Sq query and Sk key
// rows per sequence and LSE laid out [B, Hq, Sq]; a packed variable-length
// batch takes its rows from the cumulative lengths and lays LSE out
// [Hq, total_q].  Di follows the LSE layout.
struct SeqRows {
  int q0, nq;     // first packed query row, query count
  int k0, nk;     // first packed key row, key count
  size_t l0, lh;  // LSE / Di index of (head 0, row 0), stride between heads
};
__device__ __forceinline__ SeqRows seq_rows(const int32_t* cu_q, const int32_t* cu_k, int b,
                                            int Sq, int Sk, int Hq, int total_q) {
  if (!cu_q) return SeqRows{b * Sq, Sq, b * Sk, Sk, (size_t)b * Hq * Sq, (size_t)Sq};
  const int q0 = cu_q[b], k0 = cu_k[b];
  return SeqRows{q0, cu_q[b + 1] - q0, k0, cu_k[b + 1] - k0, (size_t)q0, (size_t)total_q};
}

// ---------------------------------------------------------------------------
// Di = <dO_i, O_i> (stored negated: the dK/dV pass starts its dP
// accumulators from it), LSE_i * log2(e) (the exponent offset of the base-2
// probabilities) and dSink partials.  Grid (ceil(Sq/64), Hq, B); 4 threads per
// row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(
    const __bf16* __restrict__ o, const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ sink, float* __restrict__ ndi, float* __restrict__ lse2,
    float* __restrict__ dsink_part, const int32_t* __restrict__ cu_q, int Sq, int Hq,
    int total_q) {
  ATTN_SINK_CHECK_GUARD();
  constexpr int PER = D / 4;  // elements per thread
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const SeqRows sr = seq_rows(cu_q, cu_q, b, Sq, 0, Hq, total_q);
  const int row = blockIdx.x * 64 + tid / 4;
  const int part = tid % 4;
  float acc = 0.f;
  if (row < sr.nq) {
    const size_t off = ((size_t)(sr.q0 + row) * Hq + h) * D + part * PER;
#pragma unroll
    for (int c = 0; c < PER / 8; ++c) {
      const uint4 a = *reinterpret_cast<const uint4*>(o + off + 8 * c);
      const uint4 g = *reinterpret_cast<const uint4*>(dout + off + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc = __builtin_fmaf(bf16_bits_to_f32(pick16(a, e)), bf16_bits_to_f32(pick16(g, e)), acc);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  float contrib = 0.f;
  if (row < sr.nq && part == 0) {
    const size_t x = sr.l0 + h * sr.lh + row;
    const float L = lse[x];
    ndi[x] = -acc;
    lse2[x] = L * kLog2e;
    if (sink) {
      // a head whose sink is -inf contributes nothing, also on rows that see
      // no key (LSE = -inf there, and -inf - -inf would be NaN)
      const float sh = sink[h];
      contrib = sh == kNegInf ? 0.f : -exp2_fast((sh - L) * kLog2e) * acc;
    }
  }
  if (!sink) return;
  // fixed-order block sum: wave tree, then waves in order
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) contrib += __shfl_xor(contrib, x, 64);
  __shared__ float ws[4];
  if ((tid & 63) == 0) ws[tid >> 6] = contrib;
  __syncthreads();
  if (tid == 0)
    dsink_part[((size_t)b * Hq + h) * gridDim.x + blockIdx.x] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
}

// dSink_h: one workgroup per head.  Thread t sums partials t, t + 256, ...
// of the head (over sequences, then row blocks), then the 256 sums are added
// by a fixed tree: the order depends only on B and nblk, never on timing.
__global__ __launch_bounds__(kThreads) void bwd_dsink_reduce_kernel(
    const float* __restrict__ part, float* __restrict__ dsink, int Hq, int B, int nblk) {
  ATTN_SINK_CHECK_GUARD();
  const int h = blockIdx.x, tid = threadIdx.x;
  const int n = B * nblk;
  float acc = 0.f;
  for (int i = tid; i < n; i += kThreads) {
    const int b = i / nblk, k = i - b * nblk;
    acc += part[((size_t)b * Hq + h) * nblk + k];
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) acc += __shfl_xor(acc, x, 64);
  __shared__ float ws[kThreads / 64];
  if ((tid & 63) == 0) ws[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) dsink[h] = (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

// ---------------------------------------------------------------------------
// dK / dV.  Grid (Hkv, B, ceil(max Sk/128)).  Wave w owns keys k0 + 32w .. +31,
// held as MFMA B operands (K^T, V^T) in registers.  Per (head, query tile):
//   S  = Q K^T,  dP = dO V^T        (A = Q, dO from LDS, natural layout)
//   P = 2^(S*sl2 - LSE*log2e), dS = P (dP - Di)
//   dV^T += dO^T P,  dK^T += Q^T dS (A = dO^T, Q^T from LDS, transposed)
// Lane (hh, l32) holds key l32 and query rows 32*qb + 16*hh + i.
// ---------------------------------------------------------------------------
// One tile buffer of the dK/dV pass: 64 rows of Q and of dO (rows permuted,
// the tile-load layout) and the rows' LSE * log2(e) and -Di (the first 64 of
// each row vector; one 1 KB load fills it, zeros past the rows).
template <int D>
struct DkdvTile {
  __bf16 q[kTile * (D + kPad)];
  __bf16 dO[kTile * (D + kPad)];
  alignas(16) float lse2[4 * kTile];
  alignas(16) float ndi[4 * kTile];
};

#define DKDV_PARAMS                                                                             \
  const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,     \
      const __bf16 *__restrict__ dout, const float *__restrict__ lse2,                          \
      const float *__restrict__ ndi, __bf16 *__restrict__ dk, __bf16 *__restrict__ dv,          \
      const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int Sq, int Sk, int Hq, \
      int Hkv, int total_q, float scale, float sl2, int causal, int w1, int w2

// Work block (kvh, b, kb): (KV head, sequence, block of 128 keys); t0 .. t2
// are the LDS tile buffers (NB of them; t2 unused when NB = 2).
template <int D, int NB>
__device__ __forceinline__ void dkdv_block(DkdvTile<D>& t0, DkdvTile<D>& t1, DkdvTile<D>& t2,
                                           int kvh, int b, int kb, DKDV_PARAMS) {
  constexpr int NS = D + kPad;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loads and LDS bases
  const int hh = lane >> 5, l32 = lane & 31;
  const int g = Hq / Hkv;
  const SeqRows sr = seq_rows(cu_q, cu_k, b, Sq, Sk, Hq, total_q);
  const int nq = sr.nq, nk = sr.nk;
  const int k0 = kb * 128;
  if (k0 >= nk) return;  // uniform over the workgroup
  const int k1 = min(nk, k0 + 128);
  const int key = k0 + 32 * wave + l32;
  const int off = nk - nq;

  // K^T / V^T B operands: column key, k = d = 16*ks + 8*hh ..
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (key < nk) {
      const size_t base = ((size_t)(sr.k0 + key) * Hkv + kvh) * D + 16 * ks + 8 * hh;
      kf[ks] = *reinterpret_cast<const bf16x8*>(k + base);
      vf[ks] = *reinterpret_cast<const bf16x8*>(v + base);
    } else {
      kf[ks] = bf16x8{};
      vf[ks] = bf16x8{};
    }
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  // query rows that can see keys [k0, k1)
  int i_lo = 0, i_hi = nq;
  if (causal) i_lo = max(0, k0 - off);
  if (w2 > 0 && k0 >= w1) i_hi = min(nq, (k1 - 1) + w2 - 1 - off + 1);
  const int t_lo = i_lo / kTile;
  const int t_hi = i_hi > i_lo ? (i_hi + kTile - 1) / kTile : t_lo;
  const int ntq = t_hi - t_lo;
  const int niter = ntq * g;

  const size_t rs = (size_t)Hq * D;
  // iteration -> (query head, query tile): the last query tile first, all heads
  // of the group for each tile.  Every key block's range of tiles ends at the
  // sequence's last tile, so the key blocks of one KV head that run together
  // (all on one XCD: the grid's fastest index is the KV head) walk the same
  // Q/dO tiles at the same time and share them in L2.  Training workload
  // (B2 S8192 64/8 heads): 6.6 -> 1.6 GB of HBM reads per launch against the
  // first tile first, head by head; the time is the same.
  // The iterations are requested and computed in order, so both walk the
  // (head, tile) sequence with counters instead of dividing by g (fewer scalar
  // instructions per step: training -0.9 %).

  // Tile loads straight into LDS: SP 1 KB loads of Q and SP of dO (rows
  // permuted), and the 64 rows' LSE * log2(e) and -Di.  Waves 0 and 1 load Q,
  // waves 2 and 3 dO, each every other load j = (wave & 1) + 2u; SP is odd,
  // so the odd waves' last load (j = SP) is the row vector instead (wave 1
  // the LSE, wave 3 -Di).  Every wave issues U loads per tile, all of the
  // same kind with no branch between them: a branch there made the compiler
  // hold the first LDS read of each step on the loads of the tile after next.
  constexpr int SP = kDmaSlots(D), U = (SP + 1) / 2;
  static_assert(SP % 2 == 1, "odd slot count per row");
  const bool wq = wave < 2;
  uint32_t doff[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = (wave & 1) + 2 * u;
    doff[u] = j < SP ? dma_offset<D>(j, lane, (uint32_t)(rs * 2), true) : 16u * lane;
  }
  // the next iteration to request: its head (within the group), its first
  // row and the rows' addresses; past the last iteration the loads read an
  // empty resource, so that every step issues the same loads
  int rq_h = 0, rq_i0 = (t_hi - 1) * kTile, rq_left = niter;
  const __bf16* rq_t = (wq ? q : dout) + ((size_t)sr.q0 * Hq + kvh * g) * D + (size_t)rq_i0 * rs;
  const float* rq_r = (wq ? lse2 : ndi) + sr.l0 + (size_t)(kvh * g) * sr.lh + rq_i0;
  auto request = [&](DkdvTile<D>& t) {
    const int nrow = rq_left > 0 ? nq - rq_i0 : 0;
    const auto rt = make_rsrc(rq_t, (uint32_t)((size_t)nrow * rs * 2));
    const auto rr = make_rsrc(rq_r, (uint32_t)nrow * 4u);
    // destinations as byte offsets from the buffer
    char* tb = reinterpret_cast<char*>(&t);
    const uint32_t fo = wq ? offsetof(DkdvTile<D>, q) : offsetof(DkdvTile<D>, dO);
    const uint32_t ro = wq ? offsetof(DkdvTile<D>, lse2) : offsetof(DkdvTile<D>, ndi);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (wave & 1) + 2 * u;
      const bool row = j >= SP;
      dma16(row ? rr : rt, tb + (row ? ro : fo + 1024u * j), doff[u]);
    }
    --rq_left;
    if (++rq_h == g) {  // past the group's last head: head 0 of the previous tile
      rq_h = 0;
      rq_i0 -= kTile;
      rq_t -= (size_t)(g - 1) * D + (size_t)kTile * rs;
      rq_r -= (size_t)(g - 1) * sr.lh + kTile;
    } else {
      rq_t += D;
      rq_r += sr.lh;
    }
  };
  int st_h = 0, st_i0 = (t_hi - 1) * kTile;  // the same walk for the steps

  // One step: wait until iteration it's tile has landed (the next NB - 2
  // tiles' loads may stay in flight); after the barrier it has for every
  // wave, and every wave is done with the previous tile's buffer, which the
  // request overwrites.  Steps past the last iteration only keep the loads and
  // waits uniform.
  auto step = [&](int it, DkdvTile<D>& cur, DkdvTile<D>& ahead) {
    wait_vmcnt<(NB - 2) * U>();
    tile_barrier();
    request(ahead);
    if (it >= niter) return;
    const int i0 = st_i0;
    if (++st_h == g) {
      st_h = 0;
      st_i0 -= kTile;
    }
    const int p0 = off + i0;
    const bool need_mask = (i0 + kTile > nq) || (causal && p0 < k1 - 1) ||
                           (w2 > 0 && k1 - 1 >= w1 && p0 + kTile - 1 - w2 >= k0);

    // S and dP of both 32-row blocks first (four independent MFMA chains), then
    // per row block P = 2^(S sl2 - LSE log2 e), dS = P (dP - Di) (rounded to
    // bf16 operands) and dV^T += dO^T P, dK^T += Q^T dS, so the exps of one
    // row block can run under the other's MFMAs.  Lane (hh, l32): key l32,
    // rows 32*qb + 16*hh + i.  The dV/dK A operands are read transposed from
    // the natural tiles; k-step (qb, c) covers rows 32*qb + 16*hh + 8*c .. +7.
    // Only the P / dS arithmetic sits on one of two straight-line paths (mask
    // or not, chosen per row block); the accumulating MFMAs are common code.
    // (With the whole tile in each arm, the join of the two arms' dK/dV
    // accumulators cost 64 register copies per tile.)
    // dP accumulators start at -Di (the rows' element i = row rbase + i), so
    // that dS = P (dP - Di) is one multiply per score
    f32x16 sa[2], pa[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sa[qb] = f32x16{};
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f32x4 d2 =
            *reinterpret_cast<const f32x4*>(&cur.ndi[32 * qb + 16 * hh + 4 * c4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) pa[qb][4 * c4 + e] = d2[e];
      }
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int r = (32 * qb + l32) * NS + 16 * ks + 8 * hh;
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&cur.q[r]);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(&cur.dO[r]);
        sa[qb] = mfma32(qa, kf[ks], sa[qb]);
        pa[qb] = mfma32(da, vf[ks], pa[qb]);
      }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int rbase = 32 * qb + 16 * hh;
      bf16x8 pb[2], sb[2];
      // masked: element i (row i0 + rbase + i) is visible iff lo <= i < hi,
      // from the causal bound (key <= the row's position), the last window
      // (the row's position < key + w2 when key >= w1), the rows past nq and
      // the keys past nk
      auto grads = [&](auto masked) {
        int lo = 0, hi = 16;
        if constexpr (decltype(masked)::value) {
          const int rb = i0 + rbase;
          lo = causal ? key - off - rb : -16;
          hi = nq - rb;
          if (w2 > 0 && key >= w1) hi = min(hi, key + w2 - off - rb);
          if (key >= nk) hi = -16;
        }
        float pv[16], dsv[16];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&cur.lse2[rbase + 4 * c4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * c4 + e;
            float p = exp2_fast(__builtin_fmaf(sa[qb][i], sl2, -a[e]));
            if constexpr (decltype(masked)::value) p = ((i >= lo) & (i < hi)) ? p : 0.f;
            pv[i] = p;
            dsv[i] = p * pa[qb][i];
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          pb[c] = to_bf16x8(pv[8 * c], pv[8 * c + 1], pv[8 * c + 2], pv[8 * c + 3],
                            pv[8 * c + 4], pv[8 * c + 5], pv[8 * c + 6], pv[8 * c + 7]);
          sb[c] = to_bf16x8(dsv[8 * c], dsv[8 * c + 1], dsv[8 * c + 2], dsv[8 * c + 3],
                            dsv[8 * c + 4], dsv[8 * c + 5], dsv[8 * c + 6], dsv[8 * c + 7]);
        }
      };
      // D = 64 (two waves per SIMD): the dV/dK A operands are read before the
      // P/dS arithmetic, so their LDS latency is spent under it (training
      // fwd+bwd -0.5 %, packed training -0.8 %).  At D = 128 the 64 extra
      // registers measured 4 % slower; there they are read just in time.
      constexpr bool kEarly = D == 64;
      bf16x8 dot[D / 32][2], qt[D / 32][2];
      auto read_ops = [&](int db, int c) {
        dot[db][c] = tr_frag<D>(cur.dO, 32 * qb + 8 * c, db, lane);
        qt[db][c] = tr_frag<D>(cur.q, 32 * qb + 8 * c, db, lane);
      };
      if constexpr (kEarly) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int c = 0; c < 2; ++c) read_ops(db, c);
      }
      if (need_mask)
        grads(std::true_type{});
      else
        grads(std::false_type{});
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if constexpr (!kEarly) read_ops(db, c);
          dva[db] = mfma32(dot[db][c], pb[c], dva[db]);
          dka[db] = mfma32(qt[db][c], sb[c], dka[db]);
        }
      }
    }
  };

  __builtin_amdgcn_s_waitcnt(0);  // the K^T / V^T fragments
  request(t0);
  if constexpr (NB == 3) {
    request(t1);
    for (int it = 0; it < niter; it += 3) {
      step(it, t0, t2);
      step(it + 1, t1, t0);
      step(it + 2, t2, t1);
    }
  } else {
    for (int it = 0; it < niter; it += 2) {
      step(it, t0, t1);
      step(it + 1, t1, t0);
    }
  }
  // no load may still write this workgroup's LDS; then the tile buffers stage
  // dK (rows 0 .. 31 of the wave's region) and dV (rows 32 .. 63)
  wait_vmcnt<0>();
  __syncthreads();
  constexpr int NS2 = D + kPad;
  __bf16* stage = wave < 2 ? (wave == 0 ? t0.q : t0.dO) : (wave == 2 ? t1.q : t1.dO);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d = 32 * db + 8 * a + 4 * hh;
      *reinterpret_cast<bf16x4*>(stage + l32 * NS2 + d) =
          to_bf16x4(dka[db][4 * a] * scale, dka[db][4 * a + 1] * scale,
                    dka[db][4 * a + 2] * scale, dka[db][4 * a + 3] * scale);
      *reinterpret_cast<bf16x4*>(stage + (32 + l32) * NS2 + d) =
          to_bf16x4(dva[db][4 * a], dva[db][4 * a + 1], dva[db][4 * a + 2], dva[db][4 * a + 3]);
    }
  store_staged<D, 64>(stage, lane, [&](int r) -> __bf16* {
    const int kr = k0 + 32 * wave + (r & 31);
    if (kr >= nk) return nullptr;
    return (r < 32 ? dk : dv) + ((size_t)(sr.k0 + kr) * Hkv + kvh) * D;
  });
}

// grid: (Hkv, B, key blocks) with the key block slowest, so the key blocks
// that see the most query rows (the first ones under a causal mask) start first
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_dkdv_kernel(DKDV_PARAMS) {
  ATTN_SINK_CHECK_GUARD();
  // one LDS variable per tile buffer, so that the compiler can tell the
  // buffer a load in flight writes from the one being read
  __shared__ DkdvTile<D> t0, t1;
  if constexpr (bwd_bufs<D>() == 3) {
    __shared__ DkdvTile<D> t2;
    dkdv_block<D, 3>(t0, t1, t2, blockIdx.x, blockIdx.y, blockIdx.z, q, k, v, dout, lse2, ndi, dk,
                     dv, cu_q, cu_k, Sq, Sk, Hq, Hkv, total_q, scale, sl2, causal, w1, w2);
  } else {
    dkdv_block<D, 2>(t0, t1, t0, blockIdx.x, blockIdx.y, blockIdx.z, q, k, v, dout, lse2, ndi, dk,
                     dv, cu_q, cu_k, Sq, Sk, Hq, Hkv, total_q, scale, sl2, causal, w1, w2);
  }
}

// ---------------------------------------------------------------------------
// dQ.  Same frame and schedule as the forward: 4 waves = 4 query heads of one
// GQA group (or 4 row blocks when the group size is not a multiple of 4), 32
// query rows per wave.  Per KV tile:
//   S^T = K Q^T, dP^T = V dO^T (A = K, V from LDS natural layout)
//   dS^T = P^T (dP^T - Di),  dQ^T += K^T dS^T (A = K^T from LDS transposed)
// ---------------------------------------------------------------------------
// One tile buffer of the dQ pass: 64 keys of K and V (rows permuted, the
// tile-load layout).
template <int D>
struct DqTile {
  __bf16 k[kTile * (D + kPad)];
  __bf16 v[kTile * (D + kPad)];
};

struct QRange {
  int n1, b_start, n2;
  __device__ __forceinline__ int count() const { return n1 + n2; }
  __device__ __forceinline__ int tile(int it) const { return it < n1 ? it : b_start + (it - n1); }
};

__device__ __forceinline__ QRange kv_tiles(int Sk, int p_min, int p_max, int causal, int w1, int w2) {
  QRange r{0, 0, 0};
  const int kend = causal ? min(Sk, p_max + 1) : Sk;
  if (kend <= 0) return r;
  const int tend = (kend + kTile - 1) / kTile;
  if (w2 <= 0) {
    r.n1 = tend;
    return r;
  }
  const int a_end = (min(w1, kend) + kTile - 1) / kTile;
  const int b_beg = max(0, p_min - w2 + 1) / kTile;
  if (b_beg <= a_end) {
    r.n1 = tend;
    return r;
  }
  r.n1 = a_end;
  r.b_start = b_beg;
  r.n2 = tend - b_beg;
  return r;
}

#define DQ_PARAMS                                                                               \
  const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,     \
      const __bf16 *__restrict__ dout, const float *__restrict__ lse2,                          \
      const float *__restrict__ ndi, __bf16 *__restrict__ dq, const int32_t *__restrict__ cu_q, \
      const int32_t *__restrict__ cu_k, int B, int Sq, int Sk, int Hq, int Hkv, int total_q,     \
      int hpw, float scale, float sl2, int causal, int w1, int w2

// Work block w of the forward's XCD-aware order (row tile of one head group).
// A wave owns 32*QB rows of one head: with QB = 2 every K, V and K^T fragment
// read from LDS feeds two MFMAs (one per 32-row block), which halves the LDS
// traffic per MFMA; the transposing K^T reads are the slowest LDS reads.
template <int D, int QB, int NB>
__device__ __forceinline__ void dq_block(DqTile<D>& t0, DqTile<D>& t1, DqTile<D>& t2, int w,
                                         DQ_PARAMS) {
  constexpr int NS = D + kPad;
  constexpr int RW = 32 * QB;  // rows per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loads and LDS bases
  const int hh = lane >> 5, l32 = lane & 31;
  const int g = Hq / Hkv;
  const int groups = g / hpw;
  const int R = RW * (4 / hpw);
  const WorkItem wi = work_item(w, B * Hkv, groups, (Sq + R - 1) / R);
  const int kvh = wi.pair % Hkv, b = wi.pair / Hkv;
  const SeqRows sr = seq_rows(cu_q, cu_k, b, Sq, Sk, Hq, total_q);
  const int nq = sr.nq, nk = sr.nk;
  const int row0 = wi.tile * R;
  if (row0 >= nq) return;  // uniform over the workgroup
  const int h = kvh * g + wi.grp * hpw + (wave % hpw);
  const int rb = wave / hpw;
  const int wrow0 = row0 + rb * RW;
  const int off = nk - nq;
  const int p_min = off + row0;
  const int p_max = off + min(nq, row0 + R) - 1;

  // per row block qb: this lane's row wrow0 + 32*qb + l32, its Q / dO
  // fragments, LSE (log2 units) and -Di
  bf16x8 qf[QB][D / 16], of[QB][D / 16];
  float l2r[QB], ndi_r[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 32 * qb + l32;
    ndi_r[qb] = 0.f;
    l2r[qb] = 0.f;
    if (row < nq) {
      const size_t base = ((size_t)(sr.q0 + row) * Hq + h) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(q + base + 16 * ks);
        of[qb][ks] = *reinterpret_cast<const bf16x8*>(dout + base + 16 * ks);
      }
      l2r[qb] = lse2[sr.l0 + h * sr.lh + row];
      ndi_r[qb] = ndi[sr.l0 + h * sr.lh + row];
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        qf[qb][ks] = bf16x8{};
        of[qb][ks] = bf16x8{};
      }
    }
  }
  f32x16 dqa[D / 32][QB];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) dqa[db][qb] = f32x16{};

  const QRange tr = kv_tiles(nk, p_min, p_max, causal, w1, w2);
  const int ntiles = tr.count();
  const size_t rs = (size_t)Hkv * D;
  const __bf16* kbase = k + ((size_t)sr.k0 * Hkv + kvh) * D;
  const __bf16* vbase = v + ((size_t)sr.k0 * Hkv + kvh) * D;
  // K/V tiles straight into LDS (rows permuted): waves 0 and 1 load K, waves
  // 2 and 3 V, every other 1 KB load j = (wave & 1) + 2u; SP is odd, so the
  // odd waves repeat their last load (same data to the same slots) and every
  // wave issues U loads per tile.
  constexpr int SP = kDmaSlots(D), U = (SP + 1) / 2;
  static_assert(SP % 2 == 1, "odd slot count per row");
  const bool wk = wave < 2;
  uint32_t doff[U], dlds[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = (wave & 1) + 2 * u < SP ? (wave & 1) + 2 * u : (wave & 1) + 2 * u - 2;
    doff[u] = dma_offset<D>(j, lane, (uint32_t)(rs * 2), true);
    dlds[u] = 512 * j;  // elements
  }
  // tile it into buffer t; past the last tile the loads read an empty
  // resource, so that every step issues the same loads
  auto request = [&](int it, DqTile<D>& t) {
    const int key0 = it < ntiles ? tr.tile(it) * kTile : 0;
    const uint32_t bytes = it < ntiles ? (uint32_t)((size_t)(nk - key0) * rs * 2) : 0u;
    const auto r = make_rsrc((wk ? kbase : vbase) + (size_t)key0 * rs, bytes);
    __bf16* dst = wk ? t.k : t.v;
#pragma unroll
    for (int u = 0; u < U; ++u) dma16(r, dst + dlds[u], doff[u]);
  };
  // One step: as in the dK/dV pass.
  auto step = [&](int it, DqTile<D>& cur, DqTile<D>& ahead) {
    wait_vmcnt<(NB - 2) * U>();
    tile_barrier();
    request(it + NB - 1, ahead);
    if (it >= ntiles) return;
    const int key0 = tr.tile(it) * kTile;
    const bool need_mask = (key0 + kTile > nk) || (causal && key0 + kTile - 1 > p_min) ||
                           (w2 > 0 && key0 + kTile - 1 >= w1 && key0 <= p_max - w2) ||
                           (row0 + R > nq);
    // one 32-key block at a time: S^T and dP^T of every row block, dS^T, then
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st[QB], dp[QB];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int r = (32 * kb + l32) * NS + 16 * ks + 8 * hh;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&cur.k[r]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&cur.v[r]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          st[qb] = mfma32(ka, qf[qb][ks], ks == 0 ? f32x16{} : st[qb]);
          dp[qb] = mfma32(va, of[qb][ks], ks == 0 ? f32x16{} : dp[qb]);
        }
      }
      // dS^T = P^T (dP^T - Di); masked (one of two straight-line paths chosen
      // per tile): element i (key jb + i) of row block qb is visible iff i <= hi
      // (the causal bound, the keys past nk, the rows past nq) and, with a
      // window, i < a (first window) or i > bnd (last window)
      bf16x8 sb[QB][2];
      auto grad_scores = [&](auto masked) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int row = wrow0 + 32 * qb + l32;
          const int p = off + row;
          const int jb = key0 + 32 * kb + 16 * hh;
          int hi = 15, a = 16, bnd = -1;
          if constexpr (decltype(masked)::value) {
            hi = min(causal ? p - jb : 15, nk - 1 - jb);
            if (row >= nq) hi = -1;
            if (w2 > 0) {
              a = w1 - jb;
              bnd = p - w2 - jb;
            }
          }
          float dsv[16];
          if (w2 > 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float pr = exp2_fast(__builtin_fmaf(st[qb][i], sl2, -l2r[qb]));
              if constexpr (decltype(masked)::value)
                pr = ((i <= hi) & ((i < a) | (i > bnd))) ? pr : 0.f;
              dsv[i] = pr * (dp[qb][i] + ndi_r[qb]);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float pr = exp2_fast(__builtin_fmaf(st[qb][i], sl2, -l2r[qb]));
              if constexpr (decltype(masked)::value) pr = i <= hi ? pr : 0.f;
              dsv[i] = pr * (dp[qb][i] + ndi_r[qb]);
            }
          }
#pragma unroll
          for (int c = 0; c < 2; ++c)
            sb[qb][c] = to_bf16x8(dsv[8 * c], dsv[8 * c + 1], dsv[8 * c + 2], dsv[8 * c + 3],
                                  dsv[8 * c + 4], dsv[8 * c + 5], dsv[8 * c + 6],
                                  dsv[8 * c + 7]);
        }
      };
      if (need_mask)
        grad_scores(std::true_type{});
      else
        grad_scores(std::false_type{});
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 ka = tr_frag<D>(cur.k, 32 * kb + 8 * c, db, lane);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) dqa[db][qb] = mfma32(ka, sb[qb][c], dqa[db][qb]);
        }
    }
  };

  __builtin_amdgcn_s_waitcnt(0);  // the Q / dO fragments, LSE and Di
  request(0, t0);
  if constexpr (NB == 3) {
    request(1, t1);
    for (int it = 0; it < ntiles; it += 3) {
      step(it, t0, t2);
      step(it + 1, t1, t0);
      step(it + 2, t2, t1);
    }
  } else {
    for (int it = 0; it < ntiles; it += 2) {
      step(it, t0, t1);
      step(it + 1, t1, t0);
    }
  }
  // no load may still write this workgroup's LDS; then the tile buffers stage dQ
  wait_vmcnt<0>();
  __syncthreads();
  __bf16* stage = wave < 2 ? (wave == 0 ? t0.k : t0.v) : (wave == 2 ? t1.k : t1.v);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<bf16x4*>(stage + (32 * qb + l32) * NS + 32 * db + 8 * a + 4 * hh) =
            to_bf16x4(dqa[db][qb][4 * a] * scale, dqa[db][qb][4 * a + 1] * scale,
                      dqa[db][qb][4 * a + 2] * scale, dqa[db][qb][4 * a + 3] * scale);
  store_staged<D, RW>(stage, lane, [&](int r) -> __bf16* {
    return wrow0 + r < nq ? dq + ((size_t)(sr.q0 + wrow0 + r) * Hq + h) * D : nullptr;
  });
}

// Rows per wave of the dQ blocks: two 32-row blocks at D = 64, one at D = 128
// (registers).
template <int D>
constexpr int dq_qb() { return D == 64 ? 2 : 1; }

template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_dq_kernel(DQ_PARAMS) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ DqTile<D> t0, t1;  // one LDS variable per tile buffer
  if constexpr (bwd_bufs<D>() == 3) {
    __shared__ DqTile<D> t2;
    dq_block<D, dq_qb<D>(), 3>(t0, t1, t2, blockIdx.x, q, k, v, dout, lse2, ndi, dq, cu_q, cu_k,
                               B, Sq, Sk, Hq, Hkv, total_q, hpw, scale, sl2, causal, w1, w2);
  } else {
    dq_block<D, dq_qb<D>(), 2>(t0, t1, t0, blockIdx.x, q, k, v, dout, lse2, ndi, dq, cu_q, cu_k,
                               B, Sq, Sk, Hq, Hkv, total_q, hpw, scale, sl2, causal, w1, w2);
  }
}

// One tile buffer of the one-launch backward: a workgroup runs either pass.
template <int D>
union BwdTile {
  DkdvTile<D> kv;
  DqTile<D> q;
};

// dK/dV and dQ in one launch: workgroups [0, nkv) are the dK/dV blocks in the
// order of bwd_dkdv_kernel's grid (KV head fastest, key block slowest), the
// rest the dQ blocks in their own order.  The two passes are independent, so
// the dQ blocks fill the CUs that the dK/dV pass's last, uneven blocks leave.
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_main_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ ndi, __bf16* __restrict__ dq, __bf16* __restrict__ dk,
    __bf16* __restrict__ dv, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    int B, int Sq, int Sk, int Hq, int Hkv, int total_q, int hpw, float scale, float sl2,
    int causal, int w1, int w2, int nkv) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ BwdTile<D> t0, t1;  // one LDS variable per tile buffer
  const int w = blockIdx.x;
  if constexpr (bwd_bufs<D>() == 3) {
    __shared__ BwdTile<D> t2;
    if (w < nkv)
      dkdv_block<D, 3>(t0.kv, t1.kv, t2.kv, w % Hkv, (w / Hkv) % B, w / (Hkv * B), q, k, v, dout,
                       lse2, ndi, dk, dv, cu_q, cu_k, Sq, Sk, Hq, Hkv, total_q, scale, sl2,
                       causal, w1, w2);
    else
      dq_block<D, dq_qb<D>(), 3>(t0.q, t1.q, t2.q, w - nkv, q, k, v, dout, lse2, ndi, dq, cu_q,
                                 cu_k, B, Sq, Sk, Hq, Hkv, total_q, hpw, scale, sl2, causal, w1,
                                 w2);
  } else {
    if (w < nkv)
      dkdv_block<D, 2>(t0.kv, t1.kv, t0.kv, w % Hkv, (w / Hkv) % B, w / (Hkv * B), q, k, v, dout,
                       lse2, ndi, dk, dv, cu_q, cu_k, Sq, Sk, Hq, Hkv, total_q, scale, sl2,
                       causal, w1, w2);
    else
      dq_block<D, dq_qb<D>(), 2>(t0.q, t1.q, t0.q, w - nkv, q, k, v, dout, lse2, ndi, dq, cu_q,
                                 cu_k, B, Sq, Sk, Hq, Hkv, total_q, hpw, scale, sl2, causal, w1,
                                 w2);
  }
}

}  // namespace

size_t backward_workspace_bytes(int B, int max_sq, int Hq, size_t rows) {
  const size_t nblk = (size_t)(max_sq + 63) / 64;
  const size_t di = (size_t)Hq * rows;  // -Di, and as many LSE * log2(e)
  const size_t part = (size_t)B * Hq * nblk;
  return (2 * di + part) * sizeof(float);
}

// Dense batches: Sq, Sk are every sequence's lengths and cu arrays are NULL.
// Packed batches: Sq, Sk are upper bounds of the lengths (they size the grids)
// and rows come from the cu arrays.  Grids that would be empty are skipped.
hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const int hpw = heads_per_wg(g);
  const float sl2 = a.scale * kLog2e;
  const int nblk = (a.Sq + 63) / 64;
  const size_t rows = a.cu_seqlens_q ? (size_t)a.total_q : (size_t)a.B * a.Sq;
  // workspace: -Di and LSE * log2(e) ([Hq, rows] each, in the LSE layout),
  // then the dSink partials
  float* ndi = static_cast<float*>(a.workspace);
  float* lse2 = ndi + (size_t)a.Hq * rows;
  float* part = lse2 + (size_t)a.Hq * rows;
  const auto* q = static_cast<const __bf16*>(a.q);
  const auto* k = static_cast<const __bf16*>(a.k);
  const auto* v = static_cast<const __bf16*>(a.v);
  const auto* o = static_cast<const __bf16*>(a.o);
  const auto* dout = static_cast<const __bf16*>(a.dout);
  auto* dq = static_cast<__bf16*>(a.dq);
  auto* dk = static_cast<__bf16*>(a.dk);
  auto* dv = static_cast<__bf16*>(a.dv);
  const int32_t* cq = a.cu_seqlens_q;
  const int32_t* ck = a.cu_seqlens_k;
  const int tq = a.total_q;
  const dim3 pgrid(nblk, a.Hq, a.B);
  const dim3 kgrid(a.Hkv, a.B, (a.Sk + 127) / 128);
  const dim3 qgrid((unsigned)bwd_dq_workgroups(a.B, a.Sq, a.Hq, a.Hkv, a.D));
  const bool rows_q = a.Sq > 0, rows_k = a.Sk > 0;
#ifdef ATTN_SINK_DEVICE_CHECKS
  if (cq)  // packed query and key offsets
    check_cu_kernel<<<(a.B + 255) / 256, 256, 0, stream>>>(cq, ck, a.B, a.total_q, a.total_k,
                                                            a.Sq, a.Sk);
#endif
  if (a.D == 64) {
    if (rows_q)
      bwd_preprocess_kernel<64><<<pgrid, kThreads, 0, stream>>>(o, dout, a.lse, a.sink, ndi, lse2,
                                                                part, cq, a.Sq, a.Hq, tq);
    // one launch for both passes (D 64; training workloads 3 % faster than two
    // launches); the D 128 path keeps two launches
    if (rows_k && rows_q) {
      const int nkv = (int)(kgrid.x * kgrid.y * kgrid.z);
      bwd_main_kernel<64><<<dim3(nkv + qgrid.x), kThreads, 0, stream>>>(
          q, k, v, dout, lse2, ndi, dq, dk, dv, cq, ck, a.B, a.Sq, a.Sk, a.Hq, a.Hkv, tq, hpw,
          a.scale, sl2, a.causal, a.w1, a.w2, nkv);
    } else {
      if (rows_k)
        bwd_dkdv_kernel<64><<<kgrid, kThreads, 0, stream>>>(q, k, v, dout, lse2, ndi, dk, dv, cq,
                                                            ck, a.Sq, a.Sk, a.Hq, a.Hkv, tq,
                                                            a.scale, sl2, a.causal, a.w1, a.w2);
      if (rows_q)
        bwd_dq_kernel<64><<<qgrid, kThreads, 0, stream>>>(q, k, v, dout, lse2, ndi, dq, cq, ck,
                                                          a.B, a.Sq, a.Sk, a.Hq, a.Hkv, tq, hpw,
                                                          a.scale, sl2, a.causal, a.w1, a.w2);
    }
  } else {
    if (rows_q)
      bwd_preprocess_kernel<128><<<pgrid, kThreads, 0, stream>>>(o, dout, a.lse, a.sink, ndi,
                                                                 lse2, part, cq, a.Sq, a.Hq, tq);
    if (rows_k)
      bwd_dkdv_kernel<128><<<kgrid, kThreads, 0, stream>>>(q, k, v, dout, lse2, ndi, dk, dv, cq,
                                                           ck, a.Sq, a.Sk, a.Hq, a.Hkv, tq,
                                                           a.scale, sl2, a.causal, a.w1, a.w2);
    if (rows_q)
      bwd_dq_kernel<128><<<qgrid, kThreads, 0, stream>>>(q, k, v, dout, lse2, ndi, dq, cq, ck,
                                                         a.B, a.Sq, a.Sk, a.Hq, a.Hkv, tq, hpw,
                                                         a.scale, sl2, a.causal, a.w1, a.w2);
  }
  if (a.sink && a.dsink)
    bwd_dsink_reduce_kernel<<<a.Hq, kThreads, 0, stream>>>(part, a.dsink, a.Hq, a.B, nblk);
  return hipGetLastError();
}

#ifdef ATTN_SINK_DEVICE_CHECKS
ATTN_SINK_DEFINE_CHECK_READER(read_check_word_backward)
#endif

}  // namespace attn_sink
