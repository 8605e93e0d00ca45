// Host-side launchers of the sink-attention kernels.  Arguments are already
// validated by the C-ABI layer (api.hip); these only pick a kernel and a grid
// and enqueue it on `stream`.  They return the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn_sink {

// ---------------------------------------------------------------------------
// Grid sizes of the launches that grow with the problem, shared by the
// launchers and the C ABI's size checks.  A dispatch's work-item count (per
// grid dimension) must fit 32 bits.
// ---------------------------------------------------------------------------
// Query heads per wave group of the forward and dQ workgroups (4 waves).
inline int heads_per_wg(int g) { return (g % 4 == 0) ? 4 : (g % 2 == 0 ? 2 : 1); }
// Forward prefill / extend / variable-length workgroups over `rows` rows.
inline long long fwd_workgroups(int B, int rows, int Hq, int Hkv, int D) {
  const int g = Hq / Hkv, hpw = heads_per_wg(g);
  const long long R = (long long)(D == 64 ? 64 : 32) * (4 / hpw);
  return (long long)B * Hkv * (g / hpw) * ((rows + R - 1) / R);
}
// Index-list workgroups (4 query heads per workgroup, 32*QB rows).
inline long long index_workgroups(int B, int rows, int Hq, int Hkv, int D) {
  const long long R = D == 64 ? 64 : 32;
  return (long long)B * Hkv * (Hq / Hkv / 4) * ((rows + R - 1) / R);
}
// Backward dQ and dK/dV workgroups.
inline long long bwd_dq_workgroups(int B, int Sq, int Hq, int Hkv, int D) {
  const int g = Hq / Hkv, hpw = heads_per_wg(g);
  const long long R = (D == 64 ? 64LL : 32LL) * (4 / hpw);  // rows per workgroup
  return (long long)B * Hkv * (g / hpw) * ((Sq + R - 1) / R);
}
inline long long bwd_dkdv_workgroups(int B, int Sk, int Hkv) {
  return (long long)Hkv * B * ((Sk + 127) / 128);
}
inline bool dispatch_fits(long long workgroups, int threads) {
  return workgroups >= 0 && workgroups * threads <= 0xffffffffLL;
}

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sink;
  void* o;
  float* lse;
  int B, Sq, Sk, Hq, Hkv, D;
  float scale;
  int causal, w1, w2;
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

// Packed variable-length queries against K/V that are either a paged cache
// (block_table != NULL; sequence lengths in seqlens_k) or packed
// variable-length tensors (block_table == NULL; rows cu_seqlens_k[b] ..).
struct ExtendArgs {
  const void* q;  // packed [total_q, Hq, D]
  const void* k;  // [num_pages, page_size, Hkv, D] or [total_k, Hkv, D]
  const void* v;
  const int32_t* block_table;
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  const int32_t* cu_seqlens_k;
  const float* sink;
  void* o;
  float* lse;  // [Hq, total_q] or NULL
  int B, total_q, max_seqlen_q, Hq, Hkv, D, page_size, max_pages;
  float scale;
  int causal, w1, w2;
  long long kv_rows;  // rows of k and v: num_pages * page_size, or total_k
};

hipError_t launch_extend_bf16(const ExtendArgs& a, hipStream_t stream);

// Packed new queries against a paged cache; each block of block_q query rows
// of a sequence attends to the tokens of one list (row cu_blocks[b] + i /
// block_q of kv_index [*, topk]).  Needs Hq / Hkv % 4 == 0 and block_q a
// multiple of 64.
struct IndexArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  const int32_t* kv_index;
  const int32_t* cu_blocks;
  const float* sink;
  void* o;
  float* lse;  // [Hq, total_q] or NULL
  int B, total_q, max_seqlen_q, Hq, Hkv, D, page_size, max_pages, block_q, topk;
  float scale;
  long long kv_rows;  // num_pages * page_size
};

hipError_t launch_index_bf16(const IndexArgs& a, hipStream_t stream);

// Workgroups per column of 4 KV-head units in the equal-range decode grid (the
// workspace has room for this many partials per head and sequence).
constexpr int kDecodeEvenMaxG = 1024;

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seqlens;
  const float* sink;
  void* o;
  float* lse;
  int B, Hq, Hkv, D, page_size, max_pages, num_pages;
  float scale;
  int w1, w2;
  int chunk;       // selected tokens per split
  int max_splits;  // grid extent over splits
  float* partials; // workspace: [B, Hq, max_splits, D + 2] fp32 partials, then the
                   // chunk list (B * max_splits int32) and its length (int32);
                   // equal ranges: [Hq, G + B, D + 2] partials (room for
                   // G <= 1024), then the sequences' starts (B + 1 int32)
  bool even;       // equal token ranges instead of chunks
};

// Split plan shared by the workspace query and the launch.
struct DecodePlan {
  int chunk;
  int max_splits;
  size_t workspace_bytes;
  bool even;  // equal token ranges per workgroup (chunk, max_splits unused)
};
DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int page_size, int max_pages, int w1,
                       int w2, int num_splits);

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);

// Size of the library-held decode scratch (one copy per device) and this
// device's address of it, looked up on the first call per device.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;  // ATTN_SINK_DECODE_SCRATCH_BYTES
hipError_t decode_scratch(float** ptr);

// Per-query index lists: packed query rows against a paged cache, row r
// attending to the tokens of kv_index row r (topk entries) at or before its
// position.  Runs the paged-decode kernels with the rows as their sequences.
struct IndexRowsArgs {
  const void* q;  // [total_q, Hq, D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  const int32_t* kv_index;  // [total_q, topk]
  const float* sink;
  void* o;
  float* lse;  // [Hq, total_q] or NULL
  int B, total_q, Hq, Hkv, D, page_size, max_pages, topk;
  float scale;
  void* workspace;
  long long kv_rows;  // num_pages * page_size
};
DecodePlan plan_index_rows(int total_q, int Hq, int Hkv, int D, int topk);
hipError_t launch_index_rows_bf16(const IndexRowsArgs& a, hipStream_t stream);

hipError_t launch_select_slots(const int32_t* bt, const int32_t* seqlens, int B, int max_pages,
                               int page_size, int w1, int w2, int64_t* slots, int32_t* counts,
                               int max_sel, hipStream_t stream);
hipError_t launch_gather_kv(const void* kc, const void* vc, const int32_t* bt,
                            const int32_t* seqlens, int B, int Hkv, int D, int page_size,
                            int max_pages, int w1, int w2, void* k_out, void* v_out, int max_sel,
                            int elem_bytes, hipStream_t stream);

struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const float* sink;
  void* dq;
  void* dk;
  void* dv;
  float* dsink;
  // Dense: cu arrays NULL, Sq / Sk the lengths, LSE [B, Hq, Sq].  Packed
  // variable-length: cu arrays [B+1], Sq / Sk upper bounds of the lengths,
  // total_q packed query rows, LSE [Hq, total_q].
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int B, Sq, Sk, total_q, total_k, Hq, Hkv, D;
  float scale;
  int causal, w1, w2;
  void* workspace;
};
// Di for `rows` query rows per head plus dSink partials of B sequences of at
// most max_sq rows.
size_t backward_workspace_bytes(int B, int max_sq, int Hq, size_t rows);
hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream);

#ifdef ATTN_SINK_DEVICE_CHECKS
// Error words of the files with device checks (ORed kCheck* flags), read after
// the stream's work and cleared if asked.
hipError_t read_check_word_decode(unsigned* word, bool clear, hipStream_t stream);
hipError_t read_check_word_prefill(unsigned* word, bool clear, hipStream_t stream);
hipError_t read_check_word_backward(unsigned* word, bool clear, hipStream_t stream);
#endif

}  // namespace attn_sink
