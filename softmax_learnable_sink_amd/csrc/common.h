// Device helpers shared by the sink-attention kernels (gfx950 / CDNA4).
//
// Numerics: every score is kept in the base-2 domain, s' = s * scale * log2(e),
// so one v_exp_f32 (2^x) per probability suffices; the sink logit enters the
// same domain as sink * log2(e) (it is not multiplied by the softmax scale:
// it is an extra logit next to the already-scaled scores -- flash-attention
// PR #1819 "feat: Implement Sink Attention", Description).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_sink {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Start of a running max that has seen nothing: finite, below every score.
constexpr float kMaxFloor = -3.4028234663852886e38f;  // -FLT_MAX

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32); only called with x >= 1.
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Lane l holds A row l%32 and B column l%32, k = 8*(l/32) .. +7; the result
// element (row 8a + 4*(l/32) + b, column l%32) sits in acc[4a + b].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16). Lane l holds A row l%16 / B column l%16,
// k = 8*(l/16) .. +7; result (row 4*(l/16) + j, column l%16) in acc[j].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  f32x8 v = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ bf16x4 to_bf16x4(float a0, float a1, float a2, float a3) {
  f32x4 v = {a0, a1, a2, a3};
  return __builtin_convertvector(v, bf16x4);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// without a branch.  Word 3 is the gfx9-family default (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// ---------------------------------------------------------------------------
// Tiles loaded straight into LDS (buffer_load_dwordx4 ... lds).  Lane l of
// one such load writes its 16 bytes to LDS at base + 16 l, and a lane
// past the resource's end writes zeros.  The data never passes through VGPRs
// and the waves write nothing to LDS themselves, so a tile can be requested
// several tiles ahead at no register cost.
//
// A tile is 64 rows of D bf16 stored in LDS rows of D + 8 elements (16 bytes of
// padding against bank conflicts): kDmaSlots(D) = D/8 + 1 16-byte slots per
// row, the last one padding.  Load j of a tile fills slots 64 j .. 64 j + 63,
// so a tile takes kDmaSlots(D) loads of 1 KB each; a lane whose slot is padding
// reads its row's first chunk again.  Rows may be permuted inside 32-row
// blocks (the layout the score MFMA's operand reads want, perm_row below).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDmaSlots(int D) { return D / 8 + 1; }

// Row permutation inside a 32-row block: logical row j is stored at LDS row
// perm_row(j), so that the four rows an MFMA result register group covers are
// contiguous.  dma_row inverts it.
__device__ __forceinline__ int perm_row(int j) {
  return ((j & 15) >> 2) * 8 + (j >> 4) * 4 + (j & 3);
}
__device__ __forceinline__ int dma_row(int p) {
  return (p & ~31) + 16 * ((p >> 2) & 1) + 4 * ((p >> 3) & 3) + (p & 3);
}

// Byte offset (from the tile's first row, rows rs_bytes apart) that lane
// `lane` reads for load j of a tile.
template <int D>
__device__ __forceinline__ uint32_t dma_offset(int j, int lane, uint32_t rs_bytes, bool permuted) {
  constexpr int SP = kDmaSlots(D);
  const int slot = 64 * j + lane;
  const int p = slot / SP, c = slot % SP;
  const int row = permuted ? dma_row(p) : p;
  return (uint32_t)row * rs_bytes + (uint32_t)(c == SP - 1 ? 0 : c) * 16u;
}

// One 16-byte-per-lane (1 KB) load into LDS at lds (wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
// The same from a 64-bit address per lane (global_load_lds_dwordx4).
typedef __attribute__((address_space(1))) void global_void;
__device__ __forceinline__ void dma16_global(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)lds, 16, 0, 0);
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier that orders the compiler's LDS accesses but leaves the
// vector-memory counter alone: the tiles requested ahead stay in flight.  The
// caller waits for the tile it is about to read (wait_vmcnt) and for its own
// LDS reads (lgkmcnt) first.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// max(x, x of lane ^ 32) without an LDS round trip.  v_permlane32_swap swaps
// the upper half of its first operand with the lower half of its second; fed
// two copies of x it leaves, per lane, x and its partner's x (in some order).
// Written as one asm block: the compiler's own folding of the builtin's two
// results is not reliable when both operands hold the same value.  The s_nops
// give the permlane the wait states it needs around the VALU copy.
__device__ __forceinline__ float max_xor32(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b;
  asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(a), "=&v"(b));
  return __builtin_bit_cast(float, a);
}

// max(a, b) as one v_max_f32 for operands that are never NaN: fmaxf adds an
// instruction that quiets a loop-carried operand first (the compiler cannot
// see that it is already quiet), and it turns v_med3 with +inf back into that
// pair.
__device__ __forceinline__ float max_no_quiet(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float wave_max_xor(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}

// Workgroup -> (batch x KV head pair, head group, row tile).  Workgroups are
// handed to the 8 XCDs round robin by id.  When the pair count is a multiple
// of 8, XCD x owns pairs x, x + 8, ... and walks them one after another (all
// row tiles and head groups of a pair together), so the K/V a pair's
// workgroups share stays in that XCD's L2; with pairs numbered b * Hkv + kvh
// and Hkv a multiple of 8, every XCD holds one KV head of every sequence, so
// sequences of different lengths still give every XCD the same work.  Other
// pair counts are walked tile-major over all pairs.  Within a pair the row
// tile runs backwards so that the tiles with the most keys under a causal
// mask start first.
struct WorkItem {
  int pair, grp, tile;
};
__device__ __forceinline__ WorkItem work_item(int w, int npairs, int groups, int ntiles) {
  constexpr int kXcds = 8;
  int pair, grp, z;
  if (npairs % kXcds == 0) {
    const int local = w / kXcds, per_pair = groups * ntiles;
    pair = w % kXcds + kXcds * (local / per_pair);
    z = (local % per_pair) / groups;
    grp = local % groups;
  } else {
    const int col = w % (npairs * groups);
    pair = col / groups;
    grp = col % groups;
    z = w / (npairs * groups);
  }
  return WorkItem{pair, grp, ntiles - 1 - z};
}

// ---------------------------------------------------------------------------
// Visibility and the first/last-window selection (sglang PR #12504 "To
// implement attention-sink": keep the first W1 and the last W2 tokens of each
// sequence; the window applies only when the sequence is longer than W1+W2).
// The window is on iff w2 > 0 (the host passes -1, -1 for "off").
// ---------------------------------------------------------------------------

// Key j visible to a query at absolute position p (bottom-right causal).
// Written without short-circuit operators so it compiles to selects.
__device__ __forceinline__ bool key_visible(int j, int p, int causal, int w1, int w2) {
  const bool c_ok = (causal == 0) | (j <= p);
  const bool w_ok = (w2 <= 0) | (j < w1) | (j > p - w2);
  return c_ok & w_ok;
}

// Number of selected tokens of a sequence of length L.
__host__ __device__ __forceinline__ int n_selected(int L, int w1, int w2) {
  return (w2 > 0 && L > w1 + w2) ? w1 + w2 : L;
}

// Token index of the u-th selected token of a sequence of length L.
__device__ __forceinline__ int token_of(int u, int L, int w1, int w2) {
  return (w2 > 0 && L > w1 + w2 && u >= w1) ? L - w2 + (u - w1) : u;
}

// Physical slot of token t: page block_table[t / P] at offset t % P.
__device__ __forceinline__ int slot_of(const int32_t* bt_row, int t, int page_shift) {
  const int page = bt_row[t >> page_shift];
  return (page << page_shift) | (t & ((1 << page_shift) - 1));
}

}  // namespace attn_sink
