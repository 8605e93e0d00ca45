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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

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
