// Forward prefill of attention with a learnable per-head sink logit.
//
// bf16 path (gfx950 MFMA): one workgroup = 4 waves sharing one KV head.  When
// the GQA group size is a multiple of 4 the 4 waves are 4 query heads of the
// same group over the same query rows, so every K/V tile staged in LDS feeds 4
// heads and all waves have the same causal extent.  Each wave owns 32*QB query
// rows and works in the transposed frame
//     S^T = K Q^T   (A = K tile from LDS, B = Q^T from registers)
//     O^T += V^T P^T (A = V^T tile from LDS, B = P^T from registers)
// so every lane owns one query row: the running max / sum are per-lane scalars
// and the softmax needs a single cross-lane exchange (lane l <-> l^32).
// The sink seeds the running max (m = sink * log2 e) and is added to the
// denominator once, at the end (flash-attention PR #1819 "feat: Implement
// Sink Attention", Description: one extra logit per head before the softmax;
// sglang PR #8825, Summary of Changes: an additional value per head in the
// softmax denominator).
//
// The same per-wave tile steps (WaveRows) also drive extend_kernel (packed
// variable-length queries against a paged cache or packed K/V, with K/V rows
// gathered per tile) and index_kernel (each block of query rows against the
// tokens of one index list).
//
// fp32 path: a plain VALU kernel, one thread per query row, K/V tiles in LDS.
#include <atomic>
#include <climits>
#include <type_traits>

#include "checks.h"
#include "common.h"
#include "launch.h"

namespace attn_sink {
namespace {

constexpr int kBN = 64;        // keys per KV tile
constexpr int kThreads = 256;  // 4 waves of 64

// K rows sit in LDS in the order perm_row (common.h): the MFMA reading row r
// then sees key dma_row(r) = 16*((r>>2)&1) + 4*(r>>3) + (r&3) of its 32-key
// block, which puts keys 16h .. 16h+15 of the block, in order, into
// accumulator half h.
template <int D>
struct Lds {
  static constexpr int KS = D + 8;   // K row stride (elements), 16 B of padding
  static constexpr int VS = D + 8;   // V row stride (elements), 16 B of padding
  __bf16 k[2][kBN * KS];
  __bf16 v[2][kBN * VS];             // natural [key][d]; read transposed (ds_read_b64_tr_b16)
};
// One K/V tile buffer in the same layout (the prefill keeps each buffer in an
// LDS variable of its own).
template <int D>
struct KvTile {
  __bf16 k[kBN * Lds<D>::KS];
  __bf16 v[kBN * Lds<D>::VS];
};

// A operand of O^T += V^T P^T for d block db and the 16 keys of k-step (kb, c):
// lane l gets d = 32*db + l%32 and keys 32*kb + 16*(l/32) + 8*c .. +7, read
// from the natural V tile with two transpose loads.  ds_read_b64_tr_b16 hands
// lane i of each 16-lane group element i%4 of the 4-element vectors that lanes
// 4j + i/4 (j = 0..3) of the group addressed, in order of j; so lane s of a
// group addresses row (base + 4h + s/4), columns (dbase + 4*(s%4)) .. +3.
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ bf16x8 vt_frag(const __bf16* vtile, int db, int kb, int c, int lane) {
  const int sl = lane & 15, gg = (lane >> 4) & 1, hh = lane >> 5;
  // the lane's part of the address, then the constant part: each read's
  // address is then at most two steps from the tile (see dma_offset)
  const int ol = (16 * hh + (sl >> 2)) * Lds<D>::VS + 16 * gg + 4 * (sl & 3);
  const int oc = (32 * kb + 8 * c) * Lds<D>::VS + 32 * db;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtile + (ol + oc)));
  const i16x4 b =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtile + (ol + oc + 4 * Lds<D>::VS)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Tile schedule of one workgroup: tiles [0, n1) then [b_start, b_start + n2).
struct TileRange {
  int n1, b_start, n2;
  __device__ __forceinline__ int count() const { return n1 + n2; }
  __device__ __forceinline__ int tile(int it) const { return it < n1 ? it : b_start + (it - n1); }
};

__device__ __forceinline__ TileRange tile_range(int Sk, int p_min, int p_max, int causal, int w1,
                                                int w2) {
  TileRange r{0, 0, 0};
  const int kend = causal ? min(Sk, p_max + 1) : Sk;
  if (kend <= 0) return r;
  const int tend = (kend + kBN - 1) / kBN;
  if (w2 <= 0) {
    r.n1 = tend;
    return r;
  }
  // first window: keys [0, w1); last window: keys (p - w2, p] for p in [p_min, p_max]
  const int a_end = (min(w1, kend) + kBN - 1) / kBN;
  const int b_beg = max(0, p_min - w2 + 1) / kBN;
  if (b_beg <= a_end) {
    r.n1 = tend;
    return r;
  }
  r.n1 = a_end;
  r.b_start = b_beg;
  r.n2 = tend - b_beg;
  return r;
}

// Where a wave's query rows sit (absolute positions, bottom-right causal).
struct RowGeom {
  int Sk, causal, w1, w2;
  int p_min, p_max;  // first / last absolute position of the workgroup's rows
  int p_lane;        // absolute position of this lane's row in query block 0
};

// The running state of one wave: 32*QB query rows of one head, Q^T fragments,
// running max / sum per row (one row per lane) and the O^T accumulators.  The
// tile steps below are shared by every forward kernel here, so all of them
// compute the same arithmetic in the same order.
template <int D, int QB>
struct WaveRows {
  bf16x8 qf[QB][D / 16];
  float m[QB], l[QB];
  f32x16 acc[D / 32][QB];
  float sig2;

  // qrow0: row 0 of this sequence in a [rows, Hq, D] layout; rows >= Sq are zero.
  // NTQ: read Q non-temporally (it is read once; the L2 is kept for K/V).
  template <bool NTQ = false>
  __device__ __forceinline__ void init(const __bf16* qrow0, const float* sink, int Sq, int Hq,
                                       int h, int wrow0, int hh, int l32) {
    // Q^T fragments (B operand): query row wrow0 + 32*qb + l32, d = 16*ks + 8*hh ..
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wrow0 + 32 * qb + l32;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        if (row < Sq) {
          const bf16x8* src = reinterpret_cast<const bf16x8*>(
              qrow0 + ((size_t)row * Hq + h) * D + 16 * ks + 8 * hh);
          if constexpr (NTQ)
            qf[qb][ks] = __builtin_nontemporal_load(src);
          else
            qf[qb][ks] = *src;
        } else {
          qf[qb][ks] = bf16x8{};
        }
      }
    }
    sig2 = sink ? sink[h] * kLog2e : kNegInf;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m[qb] = sig2 == kNegInf ? kMaxFloor : sig2;
      l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db][qb] = f32x16{};
    }
  }

  // S^T = K Q^T over one 64-key tile: 2 key blocks x QB query blocks of 32x32.
  __device__ __forceinline__ void scores(const __bf16* kl, f32x16 (&st)[2][QB], int l32,
                                         int hh) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) st[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            kl + (32 * kb + l32) * Lds<D>::KS + 16 * ks + 8 * hh);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) st[kb][qb] = mfma32(kf, qf[qb][ks], st[kb][qb]);
      }
    }
  }

  // Does the 64-key tile at key0 straddle a mask boundary of these rows?  Only
  // such tiles are masked.  Callers issue the score MFMAs inside both arms of
  // the mask branch: with the branch after them, the unmasked arm had to copy
  // all score registers (24 v_mov_b64 per tile) to where the masked arm left
  // its results.
  __device__ __forceinline__ static bool needs_mask(int key0, const RowGeom& g) {
    return (key0 + kBN > g.Sk) || (g.causal && key0 + kBN - 1 > g.p_min) ||
           (g.w2 > 0 && key0 + kBN - 1 >= g.w1 && key0 <= g.p_max - g.w2);
  }

  // Keys named by a list: element i of key block kb is tile key 32*kb + 16*hh + i,
  // whose token position is tok[that key] (INT_MAX for an empty entry); it is
  // visible to the lane's row at position p iff token <= p.
  __device__ __forceinline__ void mask_tokens(f32x16 (&st)[2][QB], const int* tok, int p_lane,
                                              int hh) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int4 x = *reinterpret_cast<const int4*>(tok + 32 * kb + 16 * hh + 4 * c);
        const int t[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int p = p_lane + 32 * qb;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st[kb][qb][4 * c + e] = t[e] <= p ? st[kb][qb][4 * c + e] : kNegInf;
        }
      }
  }

  __device__ __forceinline__ void mask(f32x16 (&st)[2][QB], int key0, const RowGeom& g,
                                       int hh) const {
    // Per lane and key block, element i (key j = base + i) is visible iff
    // i <= hi (causal bound and j < Sk) and, with a window, i < a (first
    // window) or i > bnd (last window).
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int p = g.p_lane + 32 * qb;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int base = key0 + 32 * kb + 16 * hh;
        const int hi = min(g.causal ? p - base : 15, g.Sk - 1 - base);
        if (g.w2 > 0) {
          const int a = g.w1 - base, bnd = p - g.w2 - base;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const bool vis = (i <= hi) & ((i < a) | (i > bnd));
            st[kb][qb][i] = vis ? st[kb][qb][i] : kNegInf;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) st[kb][qb][i] = i <= hi ? st[kb][qb][i] : kNegInf;
        }
      }
    }
  }

  // Online softmax in base 2 with the exact running max of the tile, P rounded
  // to bf16 for P V.  The running max never is -inf (a row without a sink
  // starts at kMaxFloor, below every score), so it needs no guard before it
  // is subtracted: a row that has seen no key keeps p = 0 and alpha = 1.
  __device__ __forceinline__ void online(f32x16 (&st)[2][QB], bf16x8 (&pf)[2][QB][2], float sl2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kb][qb][i]);
      mx = max_xor32(mx);
      const float m_new = max_no_quiet(m[qb], mx * sl2);
      const float alpha = exp2_fast(m[qb] - m_new);
      m[qb] = m_new;
      float rsum;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(__builtin_fmaf(st[kb][qb][i], sl2, -m_new));
          st[kb][qb][i] = p;
          rsum = kb == 0 && i == 0 ? p : rsum + p;
        }
      l[qb] = l[qb] * alpha + rsum;
      // alpha == 1 exactly when no row of this block's max grew
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db][qb] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const f32x16& x = st[kb][qb];
          pf[kb][qb][c] = to_bf16x8(x[8 * c + 0], x[8 * c + 1], x[8 * c + 2], x[8 * c + 3],
                                    x[8 * c + 4], x[8 * c + 5], x[8 * c + 6], x[8 * c + 7]);
        }
    }
  }

  // O^T += V^T P^T: k-steps of 16 keys (key block kb, half c).
  __device__ __forceinline__ void pv(const __bf16* vl, const bf16x8 (&pf)[2][QB][2], int lane) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, c = t & 1;
        const bf16x8 vf = vt_frag<D>(vl, db, kb, c, lane);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[db][qb] = mfma32(vf, pf[kb][qb][c], acc[db][qb]);
      }
    }
  }

  // Fold the sink into the denominator once, normalise, store O and LSE.
  // orow0: row 0 of this sequence in O [rows, Hq, D]; lse_row0: this head's
  // LSE of row 0 (rows contiguous), or NULL.  The wave's O rows pass through
  // its LDS region `stage` (rows of D + 8 elements), so that every store
  // instruction writes whole lines of O (the prefill and index-list kernels
  // 1.5 % faster than with each lane storing its 8-byte pieces).  NTO: write
  // O non-temporally, which only whole-line stores make cheap.
  template <bool NTO = false>
  __device__ __forceinline__ void finish(__bf16* orow0, float* lse_row0, int Sq, int Hq, int h,
                                         int wrow0, int hh, int l32, __bf16* stage, int lane) {
    constexpr int SS = D + 8, RW = 32 * QB, CPR = D / 8;  // stage stride, rows, chunks per row
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wrow0 + 32 * qb + l32;
      float lt = l[qb] + __shfl_xor(l[qb], 32, 64);
      if (sig2 != kNegInf) lt += exp2_fast(sig2 - m[qb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16& x = acc[db][qb];
          *reinterpret_cast<bf16x4*>(stage + (32 * qb + l32) * SS + 32 * db + 8 * a + 4 * hh) =
              to_bf16x4(x[4 * a] * inv, x[4 * a + 1] * inv, x[4 * a + 2] * inv,
                        x[4 * a + 3] * inv);
        }
      if (lse_row0 && hh == 0 && row < Sq)
        lse_row0[row] = lt > 0.f ? (m[qb] + log2_fast(lt)) * kLn2 : kNegInf;
    }
    // the wave's own LDS writes are in order before its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c0 = 0; c0 < RW * CPR; c0 += 64) {
      const int r = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * SS + 8 * ch);
      if (wrow0 + r < Sq) {
        u32x4* dst =
            reinterpret_cast<u32x4*>(orow0 + ((size_t)(wrow0 + r) * Hq + h) * D + 8 * ch);
        if constexpr (NTO)
          __builtin_nontemporal_store(v, dst);
        else
          *dst = v;
      }
    }
  }
};

// 4 waves: 4 query heads of one GQA group (or 4 row blocks) over the same rows.
template <int D, int QB>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ sink, __bf16* __restrict__ o, float* __restrict__ lse, int B, int Sq,
    int Sk, int Hq, int Hkv, int hpw, float sl2, int causal, int w1, int w2) {
  constexpr int NB = D == 64 ? 3 : 2;  // LDS tile buffers
  __shared__ KvTile<D> s0, s1;
  constexpr int RW = 32 * QB;  // query rows per wave
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;

  const int g = Hq / Hkv;
  const int groups = g / hpw;  // workgroups per KV head
  const int R = RW * (4 / hpw);
  const WorkItem wi = work_item(blockIdx.x, B * Hkv, groups, (Sq + R - 1) / R);
  const int kvh = wi.pair % Hkv, b = wi.pair / Hkv;
  const int h = kvh * g + wi.grp * hpw + (wave % hpw);
  const int rb = wave / hpw;   // row block of this wave inside the workgroup
  const int row0 = wi.tile * R;
  const int wrow0 = row0 + rb * RW;
  const int off = Sk - Sq;  // bottom-right alignment
  const RowGeom geom{Sk, causal, w1, w2, off + row0, off + min(Sq, row0 + R) - 1,
                     off + wrow0 + l32};

  WaveRows<D, QB> wr;
  wr.init(q + (size_t)b * Sq * Hq * D, sink, Sq, Hq, h, wrow0, hh, l32);

  const size_t rs = (size_t)Hkv * D;
  const __bf16* kbase = k + ((size_t)b * Sk * Hkv + kvh) * D;
  const __bf16* vbase = v + ((size_t)b * Sk * Hkv + kvh) * D;
  const TileRange tr = tile_range(Sk, geom.p_min, geom.p_max, causal, w1, w2);
  const int ntiles = tr.count();

  // K/V tiles go straight into LDS, NB - 1 tiles ahead of the one in use
  // (three buffers at D = 64; two at D = 128, where three would not leave room
  // for two workgroups per CU).  A tile is SP 1 KB loads of K (rows permuted)
  // and SP of V (natural rows): waves 0 and 1 load K, waves 2 and 3 V, each
  // taking every other load j = (wave & 1) + 2u.  SP is odd, so the odd wave
  // repeats its last load (same data to the same slots): every wave then
  // issues U loads per tile and the waits below are the same static count
  // for all (the compiler's own wait tracking needs that to see which buffer
  // a load in flight may still be writing).  Tile i sits in buffer
  // i % NB; each buffer is an LDS variable of its own and the loop is unrolled
  // by NB, so that every LDS read names a buffer no load in flight writes
  // (otherwise the compiler waits for all loads in flight before such reads).
  constexpr int SP = kDmaSlots(D), U = (SP + 1) / 2;
  static_assert(SP % 2 == 1, "odd slot count per row");
  const bool wk = wave < 2;
  uint32_t doff[U], dlds[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = (wave & 1) + 2 * u < SP ? (wave & 1) + 2 * u : (wave & 1) + 2 * u - 2;
    doff[u] = dma_offset<D>(j, lane, (uint32_t)(rs * 2), wk);
    dlds[u] = 512 * j;  // elements
  }
  // Tile it into dst_buf; past the last tile the loads read an empty
  // resource (they write zeros to a buffer nobody reads), so that every step
  // issues the same loads.
  auto request = [&](int it, KvTile<D>& dst_buf) {
    const int key0 = it < ntiles ? tr.tile(it) * kBN : 0;
    const uint32_t bytes = it < ntiles ? (uint32_t)((size_t)(Sk - key0) * rs * 2) : 0u;
    const auto r = make_rsrc((wk ? kbase : vbase) + (size_t)key0 * rs, bytes);
    __bf16* dst = wk ? dst_buf.k : dst_buf.v;
#pragma unroll
    for (int u = 0; u < U; ++u) dma16(r, dst + dlds[u], doff[u]);
  };
  // One step: wait until tile it has landed (the next NB - 2 tiles' loads may
  // stay in flight); after the barrier it has for every wave, and every wave
  // is done with tile it - 1's buffer, which the request overwrites.  The loop
  // runs whole groups of NB steps; steps past the last tile only keep the
  // loads and waits uniform.
  auto step = [&](int it, KvTile<D>& cur, KvTile<D>& ahead) {
    wait_vmcnt<(NB - 2) * U>();
    tile_barrier();
    request(it + NB - 1, ahead);
    if (it < ntiles) {
      const int key0 = tr.tile(it) * kBN;
      f32x16 st[2][QB];
      bf16x8 pf[2][QB][2];
      if (WaveRows<D, QB>::needs_mask(key0, geom)) {
        wr.scores(cur.k, st, l32, hh);
        wr.mask(st, key0, geom, hh);
      } else {
        wr.scores(cur.k, st, l32, hh);
      }
      wr.online(st, pf, sl2);
      wr.pv(cur.v, pf, lane);
    }
  };

  // Q and the sink are loaded before the first tile request, so that the
  // vector-memory counter holds tile loads only.
  __builtin_amdgcn_s_waitcnt(0);
  request(0, s0);
  if constexpr (NB == 3) {
    __shared__ KvTile<D> s2;
    request(1, s1);
    for (int it = 0; it < ntiles; it += 3) {
      step(it, s0, s2);
      step(it + 1, s1, s0);
      step(it + 2, s2, s1);
    }
  } else {
    for (int it = 0; it < ntiles; it += 2) {
      step(it, s0, s1);
      step(it + 1, s1, s0);
    }
  }
  // no load may still write this workgroup's LDS; then the tile buffers stage O
  wait_vmcnt<0>();
  __syncthreads();
  __bf16* stage = wave < 2 ? (wave == 0 ? s0.k : s0.v) : (wave == 2 ? s1.k : s1.v);
  wr.finish(o + (size_t)b * Sq * Hq * D, lse ? lse + ((size_t)b * Hq + h) * Sq : nullptr, Sq, Hq,
            h, wrow0, hh, l32, stage, lane);
}

// ---------------------------------------------------------------------------
// Chunked prefill (extend) against a paged KV cache.  Sequence b's nq new
// queries are rows cu_q[b] .. cu_q[b+1]-1 of a packed [total_q, Hq, D] tensor
// and the last nq tokens of its L = seqlens[b] cached tokens, so row i sits at
// position L - nq + i (sglang PR #8825, Summary of Changes: the extend path
// takes the same sink; flash-attention PR #1819, Description: so do the
// variable-length functions).  The same 4-wave tile steps as the prefill run
// on K/V tiles gathered from the cache through the block table.
// ---------------------------------------------------------------------------

// One 64-key tile of K or V gathered row by row straight into LDS, in the
// prefill's tile layout (K rows permuted, V natural).  Waves 0 and 1 load K,
// waves 2 and 3 V, each every other 1 KB load of the tile (the odd wave
// repeating its last, so that every wave issues U loads); this lane's slot in
// load u is tile row row[u], chunk offset cb[u].  slot[u] is the cache row (or
// packed K/V row) behind it, -1 for none (a key past the context, an empty
// list entry): that slot reads zeros, from an offset past the buffer resource
// or from a zero row.
__device__ __align__(16) uint4 g_zero_row[1];  // 16 zero bytes

constexpr uint32_t kNoRow = 0xFFFFFF00u;  // past any resource of these kernels

template <int D, bool BUF>
struct GatherDma {
  static constexpr int SP = kDmaSlots(D), U = (SP + 1) / 2;
  int row[U];
  uint32_t cb[U];
  int dl[U];      // LDS element offset of load u
  int page[U];    // block-table entries behind row[u] of the tile fetched ahead
  int slot[U];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (wave & 1) + 2 * u < SP ? (wave & 1) + 2 * u : (wave & 1) + 2 * u - 2;
      const int s = 64 * j + lane, p = s / SP, c = s % SP;
      row[u] = wave < 2 ? dma_row(p) : p;
      cb[u] = (uint32_t)(c == SP - 1 ? 0 : c) * 16u;
      dl[u] = 512 * j;
    }
  }
  // Tiles of consecutive keys (the chunked-prefill and packed paths): key
  // key0 + row of a tile (key0 a multiple of 64) sits in block-table entry
  // (key0 >> shift) + (row >> shift) at in-page position (key0 & mask) +
  // (row & mask), for every power-of-two page size.  The lane's parts of
  // those are fixed: rp4 (its entry offset in bytes) and rin (its byte
  // offset inside the page, plus the 16-byte chunk); with no block table the
  // key is a packed row and rin is row * rs_bytes plus the chunk.
  uint32_t rp4[U], rin[U];
  __device__ __forceinline__ void init_contiguous(bool paged, int page_shift, uint32_t rs_bytes) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      rp4[u] = (uint32_t)(row[u] >> page_shift) * 4u;
      rin[u] = (uint32_t)(paged ? row[u] & ((1 << page_shift) - 1) : row[u]) * rs_bytes + cb[u];
    }
  }
  // one tile of consecutive keys at byte offsets off[u] into r (BUF)
  __device__ __forceinline__ void issue_at(__bf16* dst, __amdgpu_buffer_rsrc_t r,
                                           const uint32_t (&off)[U]) const {
#pragma unroll
    for (int u = 0; u < U; ++u) dma16(r, dst + dl[u], off[u]);
  }
  // the loads of one tile into dst (this wave's K or V buffer); r covers the
  // wave's array from its KV head (BUF), base is the same array otherwise
  __device__ __forceinline__ void issue(__bf16* dst, __amdgpu_buffer_rsrc_t r, const __bf16* base,
                                        uint32_t rs_bytes) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (BUF) {
        dma16(r, dst + dl[u], slot[u] >= 0 ? (uint32_t)slot[u] * rs_bytes + cb[u] : kNoRow);
      } else {
        const void* src = slot[u] >= 0 ? (const void*)(reinterpret_cast<const char*>(base) +
                                                       (size_t)slot[u] * rs_bytes + cb[u])
                                       : (const void*)g_zero_row;
        dma16_global(src, dst + dl[u]);
      }
    }
  }
};

// Packed variable-length queries against either a paged cache (bt != NULL:
// K/V rows are cache slots, L = seqlens[b]) or packed variable-length K/V
// (bt == NULL: sequence b's keys are rows cu_k[b] .. cu_k[b+1]-1, L = their
// count).  Row i of sequence b sits at position L - nq + i.
template <int D, int QB, bool BUF>
__global__ __launch_bounds__(kThreads, 2) void extend_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ cu_k,
    const float* __restrict__ sink, __bf16* __restrict__ o, float* __restrict__ lse, int B,
    int total_q, int max_sq, int Hq, int Hkv, int hpw, int page_shift, int max_pages, float sl2,
    int causal, int w1, int w2, uint32_t kv_bytes, int round_wgs) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ KvTile<D> s0, s1;  // one LDS variable per tile buffer
  constexpr int RW = 32 * QB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;

  const int g = Hq / Hkv;
  const int groups = g / hpw;
  const int R = RW * (4 / hpw);
  const WorkItem wi = work_item(blockIdx.x, B * Hkv, groups, (max_sq + R - 1) / R);
  const int kvh = wi.pair % Hkv, b = wi.pair / Hkv;
  const int qbase = cu_q[b], nq = cu_q[b + 1] - qbase;
  const int row0 = wi.tile * R;
  if (row0 >= nq) return;  // uniform over the workgroup
  const int h = kvh * g + wi.grp * hpw + (wave % hpw);
  const int rb = wave / hpw;
  const int wrow0 = row0 + rb * RW;
  const int kbase = bt ? 0 : cu_k[b];
  const int L = bt ? seqlens[b] : cu_k[b + 1] - kbase;
  const int off = L - nq;
  const RowGeom geom{L, causal, w1, w2, off + row0, off + min(nq, row0 + R) - 1,
                     off + wrow0 + l32};

  // Q is read and O written non-temporally: with them out of the L2, more of
  // the pair's context stays there between the rounds below (chunked-prefill
  // workload: 1.35 -> 1.06x the algorithmic HBM bytes, the same time).
  WaveRows<D, QB> wr;
  wr.template init<true>(q + (size_t)qbase * Hq * D, sink, nq, Hq, h, wrow0, hh, l32);

  // K/V tiles gathered straight into LDS one tile ahead; the block-table
  // entries of a tile are read a tile before that
  const uint32_t rs_bytes = (uint32_t)(Hkv * D * 2);
  const bool wk = wave < 2;
  const __bf16* base = (wk ? kc : vc) + (size_t)kvh * D;
  const auto rsrc = make_rsrc(base, kv_bytes - (uint32_t)(kvh * D * 2));
  const int32_t* bt_row = bt ? bt + (size_t)b * max_pages : nullptr;
  const int pmask = (1 << page_shift) - 1;
  const TileRange tr = tile_range(L, geom.p_min, geom.p_max, causal, w1, w2);
  const int nt = tr.count();
  // Key order.  With the XCD-aware order each XCD walks its pairs' workgroups
  // in sequence, round_wgs at a time (those resident on it at once), and every
  // round streams the whole context of its pair.  Odd rounds walk the keys
  // backwards, so they start on the keys the round before them read last,
  // which are still in that XCD's L2 (chunked-prefill workload: 1.56 -> 1.36x
  // the algorithmic HBM bytes).  The softmax does not depend on the order.
  const bool rev = round_wgs > 0 && (B * Hkv) % 8 == 0 && ((blockIdx.x / 8) / round_wgs) % 2 == 1;
  auto tile_at = [&](int it) { return rev ? tr.tile(nt - 1 - it) : tr.tile(it); };
  constexpr int GU = GatherDma<D, BUF>::U;
  GatherDma<D, BUF> gd;
  gd.init(wave, lane);
  // With buffer resources (the host picks them only for pages of under
  // 16 MB) the per-tile address work is an add and a clamp per block-table
  // read and a 24-bit multiply-add per load, the lanes' row parts being fixed
  // (init_contiguous): chunked-prefill workload -4.5 %, packed training -1.8 %.
  // With 64-bit addresses each lane forms its key, page and slot.
  const uint32_t page_bytes = (uint32_t)rs_bytes << page_shift;
  constexpr bool fast = BUF;
  if constexpr (fast) gd.init_contiguous(bt_row != nullptr, page_shift, rs_bytes);
  auto fetch = [&](int it) {  // block-table entries of tile it's rows (clamped to the context)
    if (bt_row) {
      const int key0 = tile_at(it) * kBN;
      if constexpr (fast) {
        const uint32_t e0 = (uint32_t)(key0 >> page_shift) * 4u;
        const uint32_t emax = (uint32_t)((L - 1) >> page_shift) * 4u;
#pragma unroll
        for (int u = 0; u < GU; ++u)
          gd.page[u] = *reinterpret_cast<const int32_t*>(
              reinterpret_cast<const char*>(bt_row) + min(e0 + gd.rp4[u], emax));
      } else {
#pragma unroll
        for (int u = 0; u < GU; ++u)
          gd.page[u] = bt_row[min(key0 + gd.row[u], L - 1) >> page_shift];
      }
    }
  };
  auto request = [&](int it, KvTile<D>& dst) {  // slots of tile it's rows, then the loads
    const int key0 = tile_at(it) * kBN;
    if constexpr (fast) {
      {
        const int lim = L - key0;  // rows at or past it have no key
        uint32_t off[GU];
        if (bt_row) {
          const uint32_t u0 = (uint32_t)(key0 & pmask) * rs_bytes;
#pragma unroll
          for (int u = 0; u < GU; ++u)
            off[u] = gd.row[u] < lim ? __umul24((uint32_t)gd.page[u], page_bytes) + u0 + gd.rin[u]
                                     : kNoRow;
        } else {
          const uint32_t u0 = (uint32_t)(kbase + key0) * rs_bytes;
#pragma unroll
          for (int u = 0; u < GU; ++u) off[u] = gd.row[u] < lim ? u0 + gd.rin[u] : kNoRow;
        }
        gd.issue_at(wk ? dst.k : dst.v, rsrc, off);
        return;
      }
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int key = key0 + gd.row[u];
      gd.slot[u] = key >= L ? -1 : bt_row ? (gd.page[u] << page_shift) | (key & pmask) : kbase + key;
    }
    gd.issue(wk ? dst.k : dst.v, rsrc, base, rs_bytes);
  };
  // one tile: wait until it has landed (and the entries of the next one);
  // after the barrier it has for every wave, and every wave is done with the
  // previous tile's buffer, which the next tile's loads overwrite
  auto step = [&](int it, KvTile<D>& cur, KvTile<D>& ahead) {
    wait_vmcnt<0>();
    tile_barrier();
    if (it + 1 < nt) request(it + 1, ahead);
    if (it + 2 < nt) fetch(it + 2);
    const int key0 = tile_at(it) * kBN;
    f32x16 st[2][QB];
    bf16x8 pf[2][QB][2];
    if (WaveRows<D, QB>::needs_mask(key0, geom)) {
      wr.scores(cur.k, st, l32, hh);
      wr.mask(st, key0, geom, hh);
    } else {
      wr.scores(cur.k, st, l32, hh);
    }
    wr.online(st, pf, sl2);
    wr.pv(cur.v, pf, lane);
  };

  if (nt > 0) {
    fetch(0);
    __builtin_amdgcn_s_waitcnt(0);  // Q, the sink and tile 0's entries
    request(0, s0);
    if (nt > 1) fetch(1);
    for (int it = 0; it < nt; it += 2) {
      step(it, s0, s1);
      if (it + 1 < nt) step(it + 1, s1, s0);
    }
    // no load may still write this workgroup's LDS
    wait_vmcnt<0>();
  }
  __syncthreads();  // the tile buffers stage O
  __bf16* stage = wave < 2 ? (wave == 0 ? s0.k : s0.v) : (wave == 2 ? s1.k : s1.v);
  wr.template finish<true>(o + (size_t)qbase * Hq * D,
                           lse ? lse + (size_t)h * total_q + qbase : nullptr, nq, Hq, h, wrow0,
                           hh, l32, stage, lane);
}

// ---------------------------------------------------------------------------
// Index-list selection: the keys of a block of query rows are the tokens named
// by one list (positions in the sequence, read through the block table).  The
// list is staged in LDS once; per 64-entry tile the block-table pages are
// fetched two tiles ahead and the K/V rows one tile ahead.
// ---------------------------------------------------------------------------
constexpr int kMaxList = 2048;  // longest list (LDS-resident, 8 KB)

// Packed new queries against a paged cache (as extend_kernel); the rows of
// each block of block_q rows of a sequence attend to the tokens of one list
// (kv_index row cu_blocks[b] + row / block_q) at or before their positions.
template <int D, int QB, bool BUF>
__global__ __launch_bounds__(kThreads, 2) void index_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ kv_index,
    const int32_t* __restrict__ cu_blocks, const float* __restrict__ sink, __bf16* __restrict__ o,
    float* __restrict__ lse, int B, int total_q, int max_sq, int Hq, int Hkv, int page_shift,
    int max_pages, int block_q, int topk, float sl2, uint32_t kv_bytes) {
  ATTN_SINK_CHECK_GUARD();
  __shared__ KvTile<D> s0, s1;  // one LDS variable per tile buffer
  __shared__ __attribute__((aligned(16))) int tokl[kMaxList];
  __shared__ int tmax[kMaxList / kBN];  // largest token of each tile (INT_MAX if one is empty)
  constexpr int RW = 32 * QB;  // rows per wave = rows per workgroup (4 heads of a group)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;

  const int g = Hq / Hkv;
  const WorkItem wi = work_item(blockIdx.x, B * Hkv, g / 4, (max_sq + RW - 1) / RW);
  const int kvh = wi.pair % Hkv, b = wi.pair / Hkv;
  const int qbase = cu_q[b], nq = cu_q[b + 1] - qbase;
  const int row0 = wi.tile * RW;
  if (row0 >= nq) return;  // uniform over the workgroup
  const int h = kvh * g + wi.grp * 4 + wave;
  const int L = seqlens[b];
  const int p_lane = L - nq + row0 + l32;
  const int nt = (topk + kBN - 1) / kBN;

  // The block's list -> LDS, padded to whole tiles, entries outside [0, L)
  // empty (INT_MAX), with the tokens that every row of the workgroup sees (at
  // or before its first row) moved in front of the others.  The attention does
  // not depend on the order of the keys, and then only the tiles after those
  // tokens need the mask, whatever order the list comes in (a top-k list
  // ordered by score, not by position).  Thread i partitions entries
  // [i EPT, (i + 1) EPT) after a scan of the counts.  Then each tile's largest
  // token is recorded, so tiles whose tokens all precede the first row skip
  // the mask.
  const int p_first = L - nq + row0;
  {
    constexpr int EPT = kMaxList / kThreads;
    __shared__ int wsum[kThreads / 64];
    const int32_t* list = kv_index + (size_t)(cu_blocks[b] + row0 / block_q) * topk;
    const int n = nt * kBN;
    int tk[EPT], ne = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      const int x = e < topk ? list[e] : -1;
      tk[i] = ((x >= 0) & (x < L)) ? x : INT_MAX;
      ne += (e < n) & (tk[i] <= p_first);
    }
    int incl = ne;  // inclusive scan of the early counts over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = incl - ne, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      before += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      if (e < n) {
        const bool early = tk[i] <= p_first;
        tokl[early ? before : total + (e - before)] = tk[i];
        before += early;
      }
    }
    __syncthreads();
    for (int e = tid; e < n; e += kThreads) {
      int mx = tokl[e];
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d, 64));
      if (lane == 0) tmax[e / kBN] = mx;
    }
  }

  WaveRows<D, QB> wr;
  wr.init(q + (size_t)qbase * Hq * D, sink, nq, Hq, h, row0, hh, l32);

  // K/V tiles gathered straight into LDS one tile ahead; the block-table
  // entries of a tile are read a tile before that
  const uint32_t rs_bytes = (uint32_t)(Hkv * D * 2);
  const bool wk = wave < 2;
  const __bf16* base = (wk ? kc : vc) + (size_t)kvh * D;
  const auto rsrc = make_rsrc(base, kv_bytes - (uint32_t)(kvh * D * 2));
  const int32_t* bt_row = bt + (size_t)b * max_pages;
  const int pmask = (1 << page_shift) - 1;
  constexpr int GU = GatherDma<D, BUF>::U;
  GatherDma<D, BUF> gd;
  gd.init(wave, lane);
  auto fetch = [&](int it) {  // block-table entries of tile it's tokens
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int t = tokl[it * kBN + gd.row[u]];
      gd.page[u] = bt_row[(t == INT_MAX ? 0 : t) >> page_shift];
    }
  };
  auto request = [&](int it, KvTile<D>& dst) {  // slots of tile it's tokens, then the loads
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int t = tokl[it * kBN + gd.row[u]];
      gd.slot[u] = t == INT_MAX ? -1 : (gd.page[u] << page_shift) | (t & pmask);
    }
    gd.issue(wk ? dst.k : dst.v, rsrc, base, rs_bytes);
  };
  // one tile, as in extend_kernel
  auto step = [&](int it, KvTile<D>& cur, KvTile<D>& ahead) {
    wait_vmcnt<0>();
    tile_barrier();
    if (it + 1 < nt) request(it + 1, ahead);
    if (it + 2 < nt) fetch(it + 2);
    f32x16 st[2][QB];
    bf16x8 pf[2][QB][2];
    if (__builtin_amdgcn_readfirstlane(tmax[it]) > p_first) {
      wr.scores(cur.k, st, l32, hh);
      wr.mask_tokens(st, tokl + it * kBN, p_lane, hh);
    } else {
      wr.scores(cur.k, st, l32, hh);
    }
    wr.online(st, pf, sl2);
    wr.pv(cur.v, pf, lane);
  };

  __syncthreads();  // the list
  fetch(0);
  __builtin_amdgcn_s_waitcnt(0);  // Q, the sink and tile 0's entries
  request(0, s0);
  if (nt > 1) fetch(1);
  for (int it = 0; it < nt; it += 2) {
    step(it, s0, s1);
    if (it + 1 < nt) step(it + 1, s1, s0);
  }
  // no load may still write this workgroup's LDS; then the tile buffers stage O
  wait_vmcnt<0>();
  __syncthreads();
  __bf16* stage = wave < 2 ? (wave == 0 ? s0.k : s0.v) : (wave == 2 ? s1.k : s1.v);
  wr.finish(o + (size_t)qbase * Hq * D, lse ? lse + (size_t)h * total_q + qbase : nullptr, nq,
            Hq, h, row0, hh, l32, stage, lane);
}

// ---------------------------------------------------------------------------
// fp32 VALU path: one thread per query row, 32-key tiles of K and V in LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ sink, float* __restrict__ o, float* __restrict__ lse, int Sq, int Sk,
    int Hq, int Hkv, float sl2, int causal, int w1, int w2) {
  constexpr int TK = 32;
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (Hq / Hkv);
  const int row = blockIdx.x * 64 + tid;
  const int off = Sk - Sq;
  const int p = off + row;
  const int p_max = off + min(Sq, (int)blockIdx.x * 64 + 64) - 1;
  const int kend = causal ? max(0, min(Sk, p_max + 1)) : Sk;

  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = row < Sq ? q[(((size_t)b * Sq + row) * Hq + h) * D + d] : 0.f;
    acc[d] = 0.f;
  }
  const float sig2 = sink ? sink[h] * kLog2e : kNegInf;
  float m = sig2, l = 0.f;

  for (int key0 = 0; key0 < kend; key0 += TK) {
    for (int x = tid; x < TK * D; x += 64) {
      const int j = key0 + x / D, d = x % D;
      const size_t src = (((size_t)b * Sk + j) * Hkv + kvh) * D + d;
      ks[x / D][d] = j < Sk ? k[src] : 0.f;
      vs[x / D][d] = j < Sk ? v[src] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < TK; ++jj) {
      const int j = key0 + jj;
      if (j >= kend || !key_visible(j, p, causal, w1, w2)) continue;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = __builtin_fmaf(qr[d], ks[jj][d], dot);
      const float sc = dot * sl2;
      if (sc > m) {
        const float alpha = exp2_fast(m - sc);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
        m = sc;
      }
      const float pj = exp2_fast(sc - m);
      l += pj;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(pj, vs[jj][d], acc[d]);
    }
    __syncthreads();
  }
  if (row >= Sq) return;
  if (sig2 != kNegInf) l += exp2_fast(sig2 - m);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* orow = o + (((size_t)b * Sq + row) * Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
  if (lse) lse[((size_t)b * Hq + h) * Sq + row] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const int hpw = heads_per_wg(g);
  const float sl2 = a.scale * kLog2e;
  const dim3 block(kThreads);
  const auto* q = static_cast<const __bf16*>(a.q);
  const auto* k = static_cast<const __bf16*>(a.k);
  const auto* v = static_cast<const __bf16*>(a.v);
  auto* o = static_cast<__bf16*>(a.o);
  const dim3 grid((unsigned)fwd_workgroups(a.B, a.Sq, a.Hq, a.Hkv, a.D));
  if (a.D == 64) {
    prefill_bf16_kernel<64, 2><<<grid, block, 0, stream>>>(q, k, v, a.sink, o, a.lse, a.B, a.Sq,
                                                           a.Sk, a.Hq, a.Hkv, hpw, sl2, a.causal,
                                                           a.w1, a.w2);
  } else {
    prefill_bf16_kernel<128, 1><<<grid, block, 0, stream>>>(q, k, v, a.sink, o, a.lse, a.B,
                                                            a.Sq, a.Sk, a.Hq, a.Hkv, hpw, sl2,
                                                            a.causal, a.w1, a.w2);
  }
  return hipGetLastError();
}

namespace {
// Workgroups of extend_kernel<D, QB, BUF> resident on one XCD at once (the
// device's CUs / 8 x workgroups per CU), per device, computed on the first
// call; 0 (keys in order everywhere) if HIP cannot tell.
template <int D, int QB, bool BUF>
int extend_round_wgs() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, extend_kernel<D, QB, BUF>, kThreads,
                                                   0) != hipSuccess ||
      cus < 8 || per_cu <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  c = cus / 8 * per_cu;
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}
}  // namespace

hipError_t launch_extend_bf16(const ExtendArgs& a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const int hpw = heads_per_wg(g);
  const float sl2 = a.scale * kLog2e;
  int shift = 0;
  while ((1 << shift) < a.page_size) ++shift;
  const auto* q = static_cast<const __bf16*>(a.q);
  const auto* kc = static_cast<const __bf16*>(a.k);
  const auto* vc = static_cast<const __bf16*>(a.v);
  auto* o = static_cast<__bf16*>(a.o);
#ifdef ATTN_SINK_DEVICE_CHECKS
  if (a.block_table)  // query offsets, lengths, every page of [0, L)
    check_paged_kernel<<<a.B, 256, 0, stream>>>(
        a.block_table, a.seqlens_k, a.cu_seqlens_q, a.B, a.total_q, a.max_seqlen_q, a.max_pages,
        a.page_size, (int)(a.kv_rows / a.page_size), 0, -1, -1, 0);
  else  // packed query and key offsets
    check_cu_kernel<<<(a.B + 255) / 256, 256, 0, stream>>>(
        a.cu_seqlens_q, a.cu_seqlens_k, a.B, a.total_q, (int)a.kv_rows, a.max_seqlen_q, INT_MAX);
#endif
  // K/V arrays below 4 GiB are read through buffer resources with 32-bit
  // offsets (chunked-prefill workload: 2.33 -> 2.07 ms against 64-bit
  // addresses per 16-byte chunk); larger ones through global addresses
  // (and pages of under 16 MB, for 24-bit page offsets)
  const long long kv_bytes = a.kv_rows * a.Hkv * a.D * 2;
  const bool buf = kv_bytes > 0 && kv_bytes <= (long long)kNoRow &&
                   (!a.block_table || (((long long)a.Hkv * a.D * 2) << shift) < (1LL << 24));
  auto run = [&](auto d, auto qb, auto use_buf) {
    constexpr int D = decltype(d)::value, QB = decltype(qb)::value;
    constexpr bool BUF = decltype(use_buf)::value;
    const dim3 grid((unsigned)fwd_workgroups(a.B, a.max_seqlen_q, a.Hq, a.Hkv, D));
    extend_kernel<D, QB, BUF><<<grid, kThreads, 0, stream>>>(
        q, kc, vc, a.block_table, a.cu_seqlens_q, a.seqlens_k, a.cu_seqlens_k, a.sink, o, a.lse,
        a.B, a.total_q, a.max_seqlen_q, a.Hq, a.Hkv, hpw, shift, a.max_pages, sl2, a.causal, a.w1,
        a.w2, (uint32_t)(buf ? kv_bytes : 0), extend_round_wgs<D, QB, BUF>());
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using T = std::true_type;
  using F = std::false_type;
  if (a.D == 64) {
    if (buf)
      run(I64{}, I2{}, T{});
    else
      run(I64{}, I2{}, F{});
  } else {
    if (buf)
      run(I128{}, I1{}, T{});
    else
      run(I128{}, I1{}, F{});
  }
  return hipGetLastError();
}

hipError_t launch_index_bf16(const IndexArgs& a, hipStream_t stream) {
  const float sl2 = a.scale * kLog2e;
  int shift = 0;
  while ((1 << shift) < a.page_size) ++shift;
  const auto* q = static_cast<const __bf16*>(a.q);
  const auto* kc = static_cast<const __bf16*>(a.k_cache);
  const auto* vc = static_cast<const __bf16*>(a.v_cache);
  auto* o = static_cast<__bf16*>(a.o);
#ifdef ATTN_SINK_DEVICE_CHECKS
  check_paged_kernel<<<a.B, 256, 0, stream>>>(
      a.block_table, a.seqlens_k, a.cu_seqlens_q, a.B, a.total_q, a.max_seqlen_q, a.max_pages,
      a.page_size, (int)(a.kv_rows / a.page_size), 0, -1, -1, 0);
#endif
  // caches below 4 GiB through buffer resources, as in launch_extend_bf16
  const long long kv_bytes = a.kv_rows * a.Hkv * a.D * 2;
  const bool buf = kv_bytes > 0 && kv_bytes <= (long long)kNoRow;
  auto run = [&](auto d, auto qb, auto use_buf) {
    constexpr int D = decltype(d)::value, QB = decltype(qb)::value;
    const dim3 grid((unsigned)index_workgroups(a.B, a.max_seqlen_q, a.Hq, a.Hkv, D));
    index_kernel<D, QB, decltype(use_buf)::value><<<grid, kThreads, 0, stream>>>(
        q, kc, vc, a.block_table, a.cu_seqlens_q, a.seqlens_k, a.kv_index, a.cu_blocks, a.sink, o,
        a.lse, a.B, a.total_q, a.max_seqlen_q, a.Hq, a.Hkv, shift, a.max_pages, a.block_q, a.topk,
        sl2, (uint32_t)(buf ? kv_bytes : 0));
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using T = std::true_type;
  using F = std::false_type;
  if (a.D == 64) {
    if (buf)
      run(I64{}, I2{}, T{});
    else
      run(I64{}, I2{}, F{});
  } else {
    if (buf)
      run(I128{}, I1{}, T{});
    else
      run(I128{}, I1{}, F{});
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  const float sl2 = a.scale * kLog2e;
  const dim3 grid((a.Sq + 63) / 64, a.Hq, a.B);
  const auto* q = static_cast<const float*>(a.q);
  const auto* k = static_cast<const float*>(a.k);
  const auto* v = static_cast<const float*>(a.v);
  auto* o = static_cast<float*>(a.o);
  if (a.D == 64)
    prefill_f32_kernel<64><<<grid, 64, 0, stream>>>(q, k, v, a.sink, o, a.lse, a.Sq, a.Sk, a.Hq,
                                                    a.Hkv, sl2, a.causal, a.w1, a.w2);
  else
    prefill_f32_kernel<128><<<grid, 64, 0, stream>>>(q, k, v, a.sink, o, a.lse, a.Sq, a.Sk,
                                                     a.Hq, a.Hkv, sl2, a.causal, a.w1, a.w2);
  return hipGetLastError();
}

#ifdef ATTN_SINK_DEVICE_CHECKS
ATTN_SINK_DEFINE_CHECK_READER(read_check_word_prefill)
#endif

}  // namespace attn_sink
