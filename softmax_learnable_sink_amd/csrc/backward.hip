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
//   bwd_preprocess   Di and per-(b, h, 64-row block) dSink partials
//   bwd_dkdv         KV-stationary: a wave owns 32 keys and accumulates dK/dV
//                    over all query heads of its GQA group and all query tiles
//                    that can see them
//   bwd_dq           Q-stationary (the forward's frame): recomputes S and dP
//                    and accumulates dQ in registers
//   bwd_main         (D 64) the dK/dV and dQ blocks in one launch
//   bwd_dsink_reduce fixed-order sum of the dSink partials
#include <type_traits>

#include "checks.h"
#include "common.h"
#include "launch.h"

namespace attn_sink {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;  // rows per query tile / keys per KV tile
constexpr int kPad = 8;    // LDS row padding (elements, 16 B)

__device__ __forceinline__ int perm_row(int j) { return ((j & 15) >> 2) * 8 + (j >> 4) * 4 + (j & 3); }
__device__ __forceinline__ int lds_row(int j) { return (j & ~31) + perm_row(j & 31); }

__device__ __forceinline__ uint32_t pick16(const uint4& x, int e) {
  const uint32_t w = e < 2 ? x.x : (e < 4 ? x.y : (e < 6 ? x.z : x.w));
  return (w >> (16 * (e & 1))) & 0xffffu;
}

// A operand (32 d x 16 rows) of an MFMA that contracts over tile rows, read
// from a natural-layout tile (rows permuted within 32-blocks, see lds_row):
// lane l gets d = 32*db + l%32 and logical rows r0 + 16*(l/32) .. +7.
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element i%4 of the
// 4-element vectors that lanes 4j + i/4 (j = 0..3) of the group addressed, in
// order of j; so lane s of a group addresses logical row (base + 4h + s/4),
// columns (dbase + 4*(s%4)) .. +3, for the two loads h = 0, 1.
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* nat, int r0, int db, int lane) {
  constexpr int NS = D + kPad;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int sl = lane & 15, gg = (lane >> 4) & 1, hh = lane >> 5;
  const int col = 32 * db + 16 * gg + 4 * (sl & 3);
  const int ra = r0 + 16 * hh + (sl >> 2);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(nat + lds_row(ra) * NS + col));
  const i16x4 b =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(nat + lds_row(ra + 4) * NS + col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 64 rows x D tile stored in natural layout only (rows permuted).
template <int D>
struct RowTile {
  static constexpr int CH = D / 8;
  static constexpr int N = kTile * CH / kThreads;
  uint4 r[N];
  uint32_t off[N];
  __device__ __forceinline__ void init(size_t rs, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * kThreads;
      off[i] = (uint32_t)(((size_t)(idx / CH) * rs + 8 * (idx % CH)) * 2);
    }
  }
  __device__ __forceinline__ void load(const __bf16* base, size_t rs, int row0, int nrows) {
    const auto rsrc = make_rsrc(base + (size_t)row0 * rs, (uint32_t)((size_t)(nrows - row0) * rs * 2));
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = buf_load16(rsrc, off[i]);
  }
  __device__ __forceinline__ void store(__bf16* nat, int tid) const {
    constexpr int NS = D + kPad;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * kThreads;
      *reinterpret_cast<uint4*>(nat + lds_row(idx / CH) * NS + 8 * (idx % CH)) = r[i];
    }
  }
};

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
// Di = <dO_i, O_i> and dSink partials.  Grid (ceil(Sq/64), Hq, B); 4 threads
// per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(
    const __bf16* __restrict__ o, const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ sink, float* __restrict__ di, float* __restrict__ dsink_part,
    const int32_t* __restrict__ cu_q, int Sq, int Hq, int total_q) {
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
    di[x] = acc;
    if (sink) {
      // a head whose sink is -inf contributes nothing, also on rows that see
      // no key (LSE = -inf there, and -inf - -inf would be NaN)
      const float sh = sink[h];
      const float L = lse[x];
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
template <int D>
struct DkdvLds {
  __bf16 q[2][kTile * (D + kPad)];
  __bf16 dO[2][kTile * (D + kPad)];
  alignas(16) float lse2[2][kTile];
  alignas(16) float di[2][kTile];  // -Di of the tile's rows
};

#define DKDV_PARAMS                                                                             \
  const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,     \
      const __bf16 *__restrict__ dout, const float *__restrict__ lse,                           \
      const float *__restrict__ di, __bf16 *__restrict__ dk, __bf16 *__restrict__ dv,           \
      const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int Sq, int Sk, int Hq, \
      int Hkv, int total_q, float scale, float sl2, int causal, int w1, int w2

// Work block (kvh, b, kb): (KV head, sequence, block of 128 keys).
template <int D>
__device__ __forceinline__ void dkdv_block(DkdvLds<D>& s, int kvh, int b, int kb, DKDV_PARAMS) {
  constexpr int NS = D + kPad;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  RowTile<D> tq, tdo;
  tq.init(rs, tid);
  tdo.init(rs, tid);
  float lse_r = 0.f, di_r = 0.f;
  // iteration -> (query head, query tile): the last query tile first, all heads
  // of the group for each tile.  Every key block's range of tiles ends at the
  // sequence's last tile, so the key blocks of one KV head that run together
  // (all on one XCD: the grid's fastest index is the KV head) walk the same
  // Q/dO tiles at the same time and share them in L2.  Training workload
  // (B2 S8192 64/8 heads): 6.6 -> 1.6 GB of HBM reads per launch against the
  // first tile first, head by head; the time is the same.
  auto head_of = [&](int it) { return kvh * g + it % g; };
  auto row_of = [&](int it) { return (t_hi - 1 - it / g) * kTile; };
  auto load_iter = [&](int it) {
    const int h = head_of(it);
    const int i0 = row_of(it);
    const size_t base = ((size_t)sr.q0 * Hq + h) * D;
    tq.load(q + base, rs, i0, nq);
    tdo.load(dout + base, rs, i0, nq);
    // per-row LSE and Di of the tile (zero past the last row)
    const size_t x = sr.l0 + h * sr.lh + i0;
    const uint32_t nb = (uint32_t)(nq - i0) * 4;
    lse_r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                          make_rsrc(lse + x, nb), (tid & 63) * 4, 0, 0));
    di_r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         make_rsrc(di + x, nb), (tid & 63) * 4, 0, 0));
  };
  auto store_iter = [&](int buf) {
    tq.store(s.q[buf], tid);
    tdo.store(s.dO[buf], tid);
    if (tid < kTile) {
      s.lse2[buf][tid] = lse_r * kLog2e;
      s.di[buf][tid] = -di_r;  // the dP accumulators start at -Di
    }
  };

  __builtin_amdgcn_s_waitcnt(0);
  if (niter > 0) {
    load_iter(0);
    store_iter(0);
  }
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int buf = it & 1;
    const int i0 = row_of(it);
    if (it + 1 < niter) load_iter(it + 1);
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
            *reinterpret_cast<const f32x4*>(&s.di[buf][32 * qb + 16 * hh + 4 * c4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) pa[qb][4 * c4 + e] = d2[e];
      }
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int r = (32 * qb + l32) * NS + 16 * ks + 8 * hh;
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&s.q[buf][r]);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(&s.dO[buf][r]);
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
          const f32x4 a = *reinterpret_cast<const f32x4*>(&s.lse2[buf][rbase + 4 * c4]);
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
      if (need_mask)
        grads(std::true_type{});
      else
        grads(std::false_type{});
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 dot = tr_frag<D>(s.dO[buf], 32 * qb + 8 * c, db, lane);
          const bf16x8 qt = tr_frag<D>(s.q[buf], 32 * qb + 8 * c, db, lane);
          dva[db] = mfma32(dot, pb[c], dva[db]);
          dka[db] = mfma32(qt, sb[c], dka[db]);
        }
      }
    }

    if (it + 1 < niter) store_iter(buf ^ 1);
    __syncthreads();
  }

  if (key < nk) {
    const size_t base = ((size_t)(sr.k0 + key) * Hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * db + 8 * a + 4 * hh;
        *reinterpret_cast<bf16x4*>(dk + base + d) =
            to_bf16x4(dka[db][4 * a] * scale, dka[db][4 * a + 1] * scale,
                      dka[db][4 * a + 2] * scale, dka[db][4 * a + 3] * scale);
        *reinterpret_cast<bf16x4*>(dv + base + d) =
            to_bf16x4(dva[db][4 * a], dva[db][4 * a + 1], dva[db][4 * a + 2], dva[db][4 * a + 3]);
      }
  }
}

// grid: (Hkv, B, key blocks) with the key block slowest, so the key blocks
// that see the most query rows (the first ones under a causal mask) start first
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_dkdv_kernel(DKDV_PARAMS) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ DkdvLds<D> s;
  dkdv_block<D>(s, blockIdx.x, blockIdx.y, blockIdx.z, q, k, v, dout, lse, di, dk, dv, cu_q, cu_k,
                Sq, Sk, Hq, Hkv, total_q, scale, sl2, causal, w1, w2);
}

// ---------------------------------------------------------------------------
// dQ.  Same frame and schedule as the forward: 4 waves = 4 query heads of one
// GQA group (or 4 row blocks when the group size is not a multiple of 4), 32
// query rows per wave.  Per KV tile:
//   S^T = K Q^T, dP^T = V dO^T (A = K, V from LDS natural layout)
//   dS^T = P^T (dP^T - Di),  dQ^T += K^T dS^T (A = K^T from LDS transposed)
// ---------------------------------------------------------------------------
template <int D>
struct DqLds {
  __bf16 k[2][kTile * (D + kPad)];
  __bf16 v[2][kTile * (D + kPad)];
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
      const __bf16 *__restrict__ dout, const float *__restrict__ lse,                           \
      const float *__restrict__ di, __bf16 *__restrict__ dq, const int32_t *__restrict__ cu_q,  \
      const int32_t *__restrict__ cu_k, int B, int Sq, int Sk, int Hq, int Hkv, int total_q,     \
      int hpw, float scale, float sl2, int causal, int w1, int w2

// Work block w of the forward's XCD-aware order (row tile of one head group).
// A wave owns 32*QB rows of one head: with QB = 2 every K, V and K^T fragment
// read from LDS feeds two MFMAs (one per 32-row block), which halves the LDS
// traffic per MFMA; the transposing K^T reads are the slowest LDS reads.
template <int D, int QB>
__device__ __forceinline__ void dq_block(DqLds<D>& s, int w, DQ_PARAMS) {
  constexpr int NS = D + kPad;
  constexpr int RW = 32 * QB;  // rows per wave
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  // fragments, LSE (log2 units) and Di
  bf16x8 qf[QB][D / 16], of[QB][D / 16];
  float lse2[QB], di_r[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 32 * qb + l32;
    di_r[qb] = 0.f;
    lse2[qb] = 0.f;
    if (row < nq) {
      const size_t base = ((size_t)(sr.q0 + row) * Hq + h) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(q + base + 16 * ks);
        of[qb][ks] = *reinterpret_cast<const bf16x8*>(dout + base + 16 * ks);
      }
      lse2[qb] = lse[sr.l0 + h * sr.lh + row] * kLog2e;
      di_r[qb] = di[sr.l0 + h * sr.lh + row];
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
  RowTile<D> tk, tv;
  tk.init(rs, tid);
  tv.init(rs, tid);
  __builtin_amdgcn_s_waitcnt(0);
  if (ntiles > 0) {
    tk.load(kbase, rs, tr.tile(0) * kTile, nk);
    tv.load(vbase, rs, tr.tile(0) * kTile, nk);
    tk.store(s.k[0], tid);
    tv.store(s.v[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int key0 = tr.tile(it) * kTile;
    if (it + 1 < ntiles) {
      tk.load(kbase, rs, tr.tile(it + 1) * kTile, nk);
      tv.load(vbase, rs, tr.tile(it + 1) * kTile, nk);
    }
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
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&s.k[buf][r]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&s.v[buf][r]);
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
              float pr = exp2_fast(__builtin_fmaf(st[qb][i], sl2, -lse2[qb]));
              if constexpr (decltype(masked)::value)
                pr = ((i <= hi) & ((i < a) | (i > bnd))) ? pr : 0.f;
              dsv[i] = pr * (dp[qb][i] - di_r[qb]);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float pr = exp2_fast(__builtin_fmaf(st[qb][i], sl2, -lse2[qb]));
              if constexpr (decltype(masked)::value) pr = i <= hi ? pr : 0.f;
              dsv[i] = pr * (dp[qb][i] - di_r[qb]);
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
          const bf16x8 ka = tr_frag<D>(s.k[buf], 32 * kb + 8 * c, db, lane);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) dqa[db][qb] = mfma32(ka, sb[qb][c], dqa[db][qb]);
        }
    }
    if (it + 1 < ntiles) {
      tk.store(s.k[buf ^ 1], tid);
      tv.store(s.v[buf ^ 1], tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 32 * qb + l32;
    if (row < nq) {
      __bf16* dst = dq + ((size_t)(sr.q0 + row) * Hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<bf16x4*>(dst + 32 * db + 8 * a + 4 * hh) =
              to_bf16x4(dqa[db][qb][4 * a] * scale, dqa[db][qb][4 * a + 1] * scale,
                        dqa[db][qb][4 * a + 2] * scale, dqa[db][qb][4 * a + 3] * scale);
    }
  }
}

// Rows per wave of the dQ blocks: two 32-row blocks at D = 64, one at D = 128
// (registers).
template <int D>
constexpr int dq_qb() { return D == 64 ? 2 : 1; }

template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_dq_kernel(DQ_PARAMS) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ DqLds<D> s;
  dq_block<D, dq_qb<D>()>(s, blockIdx.x, q, k, v, dout, lse, di, dq, cu_q, cu_k, B, Sq, Sk, Hq,
                          Hkv, total_q, hpw, scale, sl2, causal, w1, w2);
}

// dK/dV and dQ in one launch: workgroups [0, nkv) are the dK/dV blocks in the
// order of bwd_dkdv_kernel's grid (KV head fastest, key block slowest), the
// rest the dQ blocks in their own order.  The two passes are independent, so
// the dQ blocks fill the CUs that the dK/dV pass's last, uneven blocks leave.
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_main_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ di,
    __bf16* __restrict__ dq, __bf16* __restrict__ dk, __bf16* __restrict__ dv,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int B, int Sq, int Sk,
    int Hq, int Hkv, int total_q, int hpw, float scale, float sl2, int causal, int w1, int w2,
    int nkv) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ union {
    DkdvLds<D> kv;
    DqLds<D> q;
  } s;
  const int w = blockIdx.x;
  if (w < nkv) {
    dkdv_block<D>(s.kv, w % Hkv, (w / Hkv) % B, w / (Hkv * B), q, k, v, dout, lse, di, dk, dv,
                  cu_q, cu_k, Sq, Sk, Hq, Hkv, total_q, scale, sl2, causal, w1, w2);
  } else {
    dq_block<D, dq_qb<D>()>(s.q, w - nkv, q, k, v, dout, lse, di, dq, cu_q, cu_k, B, Sq, Sk, Hq,
                            Hkv, total_q, hpw, scale, sl2, causal, w1, w2);
  }
}

}  // namespace

size_t backward_workspace_bytes(int B, int max_sq, int Hq, size_t rows) {
  const size_t nblk = (size_t)(max_sq + 63) / 64;
  const size_t di = (size_t)Hq * rows;
  const size_t part = (size_t)B * Hq * nblk;
  return (di + part) * sizeof(float);
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
  float* di = static_cast<float*>(a.workspace);
  float* part = di + (size_t)a.Hq * rows;
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
      bwd_preprocess_kernel<64><<<pgrid, kThreads, 0, stream>>>(o, dout, a.lse, a.sink, di, part,
                                                                cq, a.Sq, a.Hq, tq);
    // one launch for both passes (D 64; training workloads 3 % faster than two
    // launches); the D 128 path keeps two launches
    if (rows_k && rows_q) {
      const int nkv = (int)(kgrid.x * kgrid.y * kgrid.z);
      bwd_main_kernel<64><<<dim3(nkv + qgrid.x), kThreads, 0, stream>>>(
          q, k, v, dout, a.lse, di, dq, dk, dv, cq, ck, a.B, a.Sq, a.Sk, a.Hq, a.Hkv, tq, hpw,
          a.scale, sl2, a.causal, a.w1, a.w2, nkv);
    } else {
      if (rows_k)
        bwd_dkdv_kernel<64><<<kgrid, kThreads, 0, stream>>>(q, k, v, dout, a.lse, di, dk, dv, cq,
                                                            ck, a.Sq, a.Sk, a.Hq, a.Hkv, tq,
                                                            a.scale, sl2, a.causal, a.w1, a.w2);
      if (rows_q)
        bwd_dq_kernel<64><<<qgrid, kThreads, 0, stream>>>(q, k, v, dout, a.lse, di, dq, cq, ck,
                                                          a.B, a.Sq, a.Sk, a.Hq, a.Hkv, tq, hpw,
                                                          a.scale, sl2, a.causal, a.w1, a.w2);
    }
  } else {
    if (rows_q)
      bwd_preprocess_kernel<128><<<pgrid, kThreads, 0, stream>>>(o, dout, a.lse, a.sink, di,
                                                                 part, cq, a.Sq, a.Hq, tq);
    if (rows_k)
      bwd_dkdv_kernel<128><<<kgrid, kThreads, 0, stream>>>(q, k, v, dout, a.lse, di, dk, dv, cq,
                                                           ck, a.Sq, a.Sk, a.Hq, a.Hkv, tq,
                                                           a.scale, sl2, a.causal, a.w1, a.w2);
    if (rows_q)
      bwd_dq_kernel<128><<<qgrid, kThreads, 0, stream>>>(q, k, v, dout, a.lse, di, dq, cq, ck,
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
