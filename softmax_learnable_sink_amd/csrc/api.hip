// C ABI of libattn_sink.so (declared in include/attn_sink.h).
//
// Every entry point validates all host-visible arguments before it makes any
// HIP call, so invalid input never reaches the device; device-resident values
// (sequence lengths, block-table entries) are documented preconditions.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "attn_sink.h"
#include "checks.h"
#include "launch.h"

using namespace attn_sink;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return ATTN_SINK_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_SINK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

// Window arguments: both -1 (off) or w1 >= 0 and w2 >= 1.
int check_window(int w1, int w2) {
  const bool off = (w1 == -1 && w2 == -1);
  REQUIRE(off || (w1 >= 0 && w2 >= 1), ATTN_SINK_ERR_INVALID_ARG,
          "window_first/window_last must both be -1 (no window) or satisfy "
          "window_first >= 0 and window_last >= 1 (got %d, %d)", w1, w2);
  return ATTN_SINK_OK;
}

int check_heads(int Hq, int Hkv, int D) {
  REQUIRE(Hq >= 1 && Hkv >= 1, ATTN_SINK_ERR_INVALID_ARG, "Hq and Hkv must be >= 1 (got %d, %d)",
          Hq, Hkv);
  REQUIRE(Hq % Hkv == 0, ATTN_SINK_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq,
          Hkv);
  REQUIRE(D == 64 || D == 128, ATTN_SINK_ERR_UNSUPPORTED, "head dim D must be 64 or 128 (got %d)",
          D);
  return ATTN_SINK_OK;
}

int check_scale(float scale) {
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_SINK_ERR_INVALID_ARG,
          "softmax_scale must be finite and > 0 (got %g)", (double)scale);
  return ATTN_SINK_OK;
}

bool fits_int32(long long x) { return x >= 0 && x <= INT_MAX; }

// Largest grid extent in y and z, and the largest byte range one 32-bit buffer
// resource addresses (the kernels address a batch's K/V or Q/dO slice through one).
constexpr long long kMaxGridYZ = 65535;
constexpr long long kMaxSlice = 0xffffffffLL;
constexpr const char* kGridMsg =
    "the problem is too large for one launch (a grid's work-items must fit 32 bits and its "
    "y/z extents 65535)";

}  // namespace

extern "C" {

int attn_sink_abi_version(void) { return ATTN_SINK_ABI_VERSION; }

const char* attn_sink_last_error(void) { return g_last_error.c_str(); }

int attn_sink_fwd_prefill(const void* q, const void* k, const void* v, const float* sink, void* o,
                          float* lse, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                          float softmax_scale, int causal, int window_first, int window_last,
                          int dtype, void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16 || dtype == ATTN_SINK_F32, ATTN_SINK_ERR_UNSUPPORTED,
          "unknown dtype %d", dtype);
  REQUIRE(B >= 1 && Sq >= 1 && Sk >= 0, ATTN_SINK_ERR_INVALID_ARG,
          "need B >= 1, Sq >= 1, Sk >= 0 (got %d, %d, %d)", B, Sq, Sk);
  if (int r = check_heads(Hq, Hkv, D)) return r;
  if (int r = check_scale(softmax_scale)) return r;
  if (int r = check_window(window_first, window_last)) return r;
  REQUIRE(causal == 0 || causal == 1, ATTN_SINK_ERR_INVALID_ARG, "causal must be 0 or 1");
  REQUIRE(window_last < 0 || causal, ATTN_SINK_ERR_UNSUPPORTED,
          "the first/last window needs causal = 1");
  REQUIRE(q && o && (Sk == 0 || (k && v)), ATTN_SINK_ERR_INVALID_ARG,
          "q, k, v and o must not be NULL");
  REQUIRE(aligned16(q) && aligned16(o) && aligned16(k) && aligned16(v), ATTN_SINK_ERR_INVALID_ARG,
          "q, k, v and o must be 16-byte aligned");
  REQUIRE(aligned4(sink) && aligned4(lse), ATTN_SINK_ERR_INVALID_ARG,
          "sink and lse must be 4-byte aligned");
  REQUIRE(fits_int32((long long)B * Sq * Hq) && fits_int32((long long)B * Sk * Hkv),
          ATTN_SINK_ERR_UNSUPPORTED, "too many rows for 32-bit row indices");
  REQUIRE(B <= kMaxGridYZ, ATTN_SINK_ERR_UNSUPPORTED, "B must be <= %lld (got %d)", kMaxGridYZ,
          B);
  REQUIRE(dtype != ATTN_SINK_BF16 || (long long)Sk * Hkv * D * 2 <= kMaxSlice,
          ATTN_SINK_ERR_UNSUPPORTED, "one batch's K or V slice exceeds 4 GiB");
  REQUIRE(dtype == ATTN_SINK_BF16 ? dispatch_fits(fwd_workgroups(B, Sq, Hq, Hkv, D), 256)
                                  : Hq <= kMaxGridYZ,
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  PrefillArgs a{q, k, v, sink, o, lse, B, Sq, Sk, Hq, Hkv, D, softmax_scale, causal,
                window_first, window_last};
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  return hip_status(dtype == ATTN_SINK_BF16 ? launch_prefill_bf16(a, st) : launch_prefill_f32(a, st),
                    "attn_sink_fwd_prefill launch");
}

int attn_sink_fwd_extend_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* cu_seqlens_q,
                               const int32_t* seqlens_k, const float* sink, void* o, float* lse,
                               int B, int total_q, int max_seqlen_q, int Hq, int Hkv, int D,
                               int page_size, int max_pages_per_seq, int num_pages,
                               float softmax_scale, int window_first, int window_last, int dtype,
                               void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16, ATTN_SINK_ERR_UNSUPPORTED,
          "paged extend supports bf16 only (dtype %d)", dtype);
  REQUIRE(B >= 1 && total_q >= 0 && max_seqlen_q >= 0, ATTN_SINK_ERR_INVALID_ARG,
          "need B >= 1, total_q >= 0, max_seqlen_q >= 0 (got %d, %d, %d)", B, total_q,
          max_seqlen_q);
  if (int r = check_heads(Hq, Hkv, D)) return r;
  if (int r = check_scale(softmax_scale)) return r;
  if (int r = check_window(window_first, window_last)) return r;
  REQUIRE(pow2(page_size) && page_size <= 256, ATTN_SINK_ERR_UNSUPPORTED,
          "page_size must be a power of two in [1, 256] (got %d)", page_size);
  REQUIRE(max_pages_per_seq >= 1 && num_pages >= 1, ATTN_SINK_ERR_INVALID_ARG,
          "max_pages_per_seq and num_pages must be >= 1");
  REQUIRE(fits_int32((long long)num_pages * page_size) &&
              fits_int32((long long)max_pages_per_seq * page_size),
          ATTN_SINK_ERR_UNSUPPORTED, "num_pages or max_pages_per_seq times page_size exceeds 2^31 - 1");
  REQUIRE(fits_int32((long long)total_q * Hq), ATTN_SINK_ERR_UNSUPPORTED,
          "too many rows for 32-bit row indices");
  REQUIRE(q && k_cache && v_cache && block_table && cu_seqlens_q && seqlens_k && o,
          ATTN_SINK_ERR_INVALID_ARG,
          "q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k and o must not be NULL");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(o),
          ATTN_SINK_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  REQUIRE(aligned4(block_table) && aligned4(cu_seqlens_q) && aligned4(seqlens_k) &&
              aligned4(sink) && aligned4(lse),
          ATTN_SINK_ERR_INVALID_ARG,
          "block_table, cu_seqlens_q, seqlens_k, sink and lse must be 4-byte aligned");
  REQUIRE(dispatch_fits(fwd_workgroups(B, max_seqlen_q, Hq, Hkv, D), 256),
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  if (total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;  // nothing to compute
  ExtendArgs a{q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, nullptr, sink, o, lse,
               B, total_q, max_seqlen_q, Hq, Hkv, D, page_size, max_pages_per_seq,
               softmax_scale, 1, window_first, window_last,
               (long long)num_pages * page_size};
  return hip_status(launch_extend_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_fwd_extend_paged launch");
}

int attn_sink_fwd_index_paged(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* cu_seqlens_q,
                              const int32_t* seqlens_k, const int32_t* kv_index,
                              const int32_t* cu_blocks, const float* sink, void* o, float* lse,
                              int B, int total_q, int max_seqlen_q, int Hq, int Hkv, int D,
                              int page_size, int max_pages_per_seq, int num_pages, int block_q,
                              int topk, float softmax_scale, int dtype, void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16, ATTN_SINK_ERR_UNSUPPORTED,
          "index-list attention supports bf16 only (dtype %d)", dtype);
  REQUIRE(B >= 1 && total_q >= 0 && max_seqlen_q >= 0, ATTN_SINK_ERR_INVALID_ARG,
          "need B >= 1, total_q >= 0, max_seqlen_q >= 0 (got %d, %d, %d)", B, total_q,
          max_seqlen_q);
  if (int r = check_heads(Hq, Hkv, D)) return r;
  REQUIRE((Hq / Hkv) % 4 == 0, ATTN_SINK_ERR_UNSUPPORTED,
          "index-list attention needs Hq / Hkv to be a multiple of 4 (got %d)", Hq / Hkv);
  REQUIRE(block_q >= 64 && block_q % 64 == 0, ATTN_SINK_ERR_UNSUPPORTED,
          "block_q must be a positive multiple of 64 (got %d)", block_q);
  REQUIRE(topk >= 1 && topk <= 2048, ATTN_SINK_ERR_UNSUPPORTED,
          "topk must be in [1, 2048] (got %d)", topk);
  if (int r = check_scale(softmax_scale)) return r;
  REQUIRE(pow2(page_size) && page_size <= 256, ATTN_SINK_ERR_UNSUPPORTED,
          "page_size must be a power of two in [1, 256] (got %d)", page_size);
  REQUIRE(max_pages_per_seq >= 1 && num_pages >= 1, ATTN_SINK_ERR_INVALID_ARG,
          "max_pages_per_seq and num_pages must be >= 1");
  REQUIRE(fits_int32((long long)num_pages * page_size) &&
              fits_int32((long long)max_pages_per_seq * page_size),
          ATTN_SINK_ERR_UNSUPPORTED, "num_pages or max_pages_per_seq times page_size exceeds 2^31 - 1");
  REQUIRE(fits_int32((long long)total_q * Hq), ATTN_SINK_ERR_UNSUPPORTED,
          "too many rows for 32-bit row indices");
  REQUIRE(q && k_cache && v_cache && block_table && cu_seqlens_q && seqlens_k && kv_index &&
              cu_blocks && o,
          ATTN_SINK_ERR_INVALID_ARG,
          "q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, kv_index, cu_blocks and o "
          "must not be NULL");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(o),
          ATTN_SINK_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  REQUIRE(aligned4(block_table) && aligned4(cu_seqlens_q) && aligned4(seqlens_k) &&
              aligned4(kv_index) && aligned4(cu_blocks) && aligned4(sink) && aligned4(lse),
          ATTN_SINK_ERR_INVALID_ARG, "int32 and fp32 arrays must be 4-byte aligned");
  REQUIRE(dispatch_fits(index_workgroups(B, max_seqlen_q, Hq, Hkv, D), 256),
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  if (total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;  // nothing to compute
  IndexArgs a{q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, kv_index, cu_blocks,
              sink, o, lse, B, total_q, max_seqlen_q, Hq, Hkv, D, page_size, max_pages_per_seq,
              block_q, topk, softmax_scale, (long long)num_pages * page_size};
  return hip_status(launch_index_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_fwd_index_paged launch");
}

size_t attn_sink_index_rows_workspace_bytes(int total_q, int Hq, int Hkv, int D, int topk) {
  if (total_q < 0 || topk < 1 || check_heads(Hq, Hkv, D) != ATTN_SINK_OK) return 0;
  return plan_index_rows(total_q, Hq, Hkv, D, topk).workspace_bytes;
}

int attn_sink_fwd_index_rows_paged(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* cu_seqlens_q,
                                   const int32_t* seqlens_k, const int32_t* kv_index,
                                   const float* sink, void* o, float* lse, int B, int total_q,
                                   int Hq, int Hkv, int D, int page_size, int max_pages_per_seq,
                                   int num_pages, int topk, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, int dtype, void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16, ATTN_SINK_ERR_UNSUPPORTED,
          "index-list attention supports bf16 only (dtype %d)", dtype);
  REQUIRE(B >= 1 && total_q >= 0, ATTN_SINK_ERR_INVALID_ARG,
          "need B >= 1, total_q >= 0 (got %d, %d)", B, total_q);
  if (int r = check_heads(Hq, Hkv, D)) return r;
  REQUIRE(topk >= 1, ATTN_SINK_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", topk);
  if (int r = check_scale(softmax_scale)) return r;
  REQUIRE(pow2(page_size) && page_size <= 256, ATTN_SINK_ERR_UNSUPPORTED,
          "page_size must be a power of two in [1, 256] (got %d)", page_size);
  REQUIRE(max_pages_per_seq >= 1 && num_pages >= 1, ATTN_SINK_ERR_INVALID_ARG,
          "max_pages_per_seq and num_pages must be >= 1");
  REQUIRE(fits_int32((long long)num_pages * page_size) &&
              fits_int32((long long)max_pages_per_seq * page_size),
          ATTN_SINK_ERR_UNSUPPORTED, "num_pages or max_pages_per_seq times page_size exceeds 2^31 - 1");
  REQUIRE(fits_int32((long long)total_q * Hq), ATTN_SINK_ERR_UNSUPPORTED,
          "too many rows for 32-bit row indices");
  REQUIRE(q && k_cache && v_cache && block_table && cu_seqlens_q && seqlens_k && kv_index && o,
          ATTN_SINK_ERR_INVALID_ARG,
          "q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, kv_index and o must not be "
          "NULL");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(o),
          ATTN_SINK_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  REQUIRE(aligned4(block_table) && aligned4(cu_seqlens_q) && aligned4(seqlens_k) &&
              aligned4(kv_index) && aligned4(sink) && aligned4(lse),
          ATTN_SINK_ERR_INVALID_ARG, "int32 and fp32 arrays must be 4-byte aligned");
  if (total_q == 0) return ATTN_SINK_OK;  // nothing to compute
  const DecodePlan plan = plan_index_rows(total_q, Hq, Hkv, D, topk);
  REQUIRE(dispatch_fits((long long)total_q * plan.max_splits * (Hkv * ((Hq / Hkv + 15) / 16) + 3),
                        64) &&
              dispatch_fits(((long long)total_q * Hq + 3) / 4, 256),
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  REQUIRE(workspace && aligned16(workspace), ATTN_SINK_ERR_WORKSPACE,
          "a 16-byte aligned workspace of %zu bytes is required", plan.workspace_bytes);
  REQUIRE(workspace_bytes >= plan.workspace_bytes, ATTN_SINK_ERR_WORKSPACE,
          "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
          plan.workspace_bytes);
  IndexRowsArgs a{q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, kv_index, sink, o,
                  lse, B, total_q, Hq, Hkv, D, page_size, max_pages_per_seq, topk,
                  softmax_scale, workspace, (long long)num_pages * page_size};
  return hip_status(launch_index_rows_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_fwd_index_rows_paged launch");
}

int attn_sink_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, const float* sink, void* o, float* lse,
                         int B, int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv,
                         int D, float softmax_scale, int causal, int window_first,
                         int window_last, int dtype, void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16, ATTN_SINK_ERR_UNSUPPORTED,
          "the variable-length forward supports bf16 only (dtype %d)", dtype);
  REQUIRE(B >= 1 && total_q >= 0 && total_k >= 0 && max_seqlen_q >= 0,
          ATTN_SINK_ERR_INVALID_ARG,
          "need B >= 1, total_q >= 0, total_k >= 0, max_seqlen_q >= 0 (got %d, %d, %d, %d)", B,
          total_q, total_k, max_seqlen_q);
  if (int r = check_heads(Hq, Hkv, D)) return r;
  if (int r = check_scale(softmax_scale)) return r;
  if (int r = check_window(window_first, window_last)) return r;
  REQUIRE(causal == 0 || causal == 1, ATTN_SINK_ERR_INVALID_ARG, "causal must be 0 or 1");
  REQUIRE(window_last < 0 || causal, ATTN_SINK_ERR_UNSUPPORTED,
          "the first/last window needs causal = 1");
  REQUIRE(fits_int32((long long)total_q * Hq) && fits_int32((long long)total_k * Hkv),
          ATTN_SINK_ERR_UNSUPPORTED, "too many rows for 32-bit row indices");
  REQUIRE(cu_seqlens_q && cu_seqlens_k && (total_q == 0 || (q && o)) &&
              (total_k == 0 || (k && v)),
          ATTN_SINK_ERR_INVALID_ARG,
          "cu_seqlens_q, cu_seqlens_k and the tensors of non-empty sides must not be NULL");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o), ATTN_SINK_ERR_INVALID_ARG,
          "q, k, v and o must be 16-byte aligned");
  REQUIRE(aligned4(cu_seqlens_q) && aligned4(cu_seqlens_k) && aligned4(sink) && aligned4(lse),
          ATTN_SINK_ERR_INVALID_ARG,
          "cu_seqlens_q, cu_seqlens_k, sink and lse must be 4-byte aligned");
  REQUIRE(dispatch_fits(fwd_workgroups(B, max_seqlen_q, Hq, Hkv, D), 256),
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  if (total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;  // nothing to compute
  ExtendArgs a{q, k, v, nullptr, cu_seqlens_q, nullptr, cu_seqlens_k, sink, o, lse, B, total_q,
               max_seqlen_q, Hq, Hkv, D, 1, 0, softmax_scale, causal, window_first, window_last,
               (long long)total_k};
  return hip_status(launch_extend_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_fwd_varlen launch");
}

static int check_decode_common(int B, int Hq, int Hkv, int D, int page_size, int max_pages,
                               int w1, int w2, int num_splits) {
  REQUIRE(B >= 1, ATTN_SINK_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
  if (int r = check_heads(Hq, Hkv, D)) return r;
  REQUIRE(pow2(page_size) && page_size <= 256, ATTN_SINK_ERR_UNSUPPORTED,
          "page_size must be a power of two in [1, 256] (got %d)", page_size);
  REQUIRE(max_pages >= 1, ATTN_SINK_ERR_INVALID_ARG, "max_pages_per_seq must be >= 1");
  REQUIRE(fits_int32((long long)max_pages * page_size), ATTN_SINK_ERR_UNSUPPORTED,
          "max_pages_per_seq * page_size exceeds 2^31 - 1");
  REQUIRE(num_splits >= 0, ATTN_SINK_ERR_INVALID_ARG, "num_splits must be >= 0");
  return check_window(w1, w2);
}

size_t attn_sink_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int page_size,
                                        int max_pages_per_seq, int window_first, int window_last,
                                        int num_splits) {
  if (check_decode_common(B, Hq, Hkv, D, page_size, max_pages_per_seq, window_first, window_last,
                          num_splits) != ATTN_SINK_OK)
    return 0;
  return plan_decode(B, Hq, Hkv, D, page_size, max_pages_per_seq, window_first, window_last,
                     num_splits)
      .workspace_bytes;
}

}  // extern "C"

// Validation shared by the two paged-decode entry points; fills the plan.
static int check_decode_call(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seqlens_k,
                             const float* sink, const void* o, const float* lse, int B, int Hq,
                             int Hkv, int D, int page_size, int max_pages_per_seq, int num_pages,
                             float softmax_scale, int window_first, int window_last,
                             int num_splits, int dtype, DecodePlan* plan) {
  REQUIRE(dtype == ATTN_SINK_BF16, ATTN_SINK_ERR_UNSUPPORTED,
          "paged decode supports bf16 only (dtype %d)", dtype);
  if (int r = check_decode_common(B, Hq, Hkv, D, page_size, max_pages_per_seq, window_first,
                                  window_last, num_splits))
    return r;
  if (int r = check_scale(softmax_scale)) return r;
  REQUIRE(num_pages >= 1, ATTN_SINK_ERR_INVALID_ARG, "num_pages must be >= 1");
  REQUIRE(fits_int32((long long)num_pages * page_size), ATTN_SINK_ERR_UNSUPPORTED,
          "num_pages * page_size exceeds 2^31 - 1");
  REQUIRE(q && k_cache && v_cache && block_table && seqlens_k && o, ATTN_SINK_ERR_INVALID_ARG,
          "q, k_cache, v_cache, block_table, seqlens_k and o must not be NULL");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(o),
          ATTN_SINK_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  REQUIRE(aligned4(block_table) && aligned4(seqlens_k) && aligned4(sink) && aligned4(lse),
          ATTN_SINK_ERR_INVALID_ARG, "block_table, seqlens_k, sink and lse must be 4-byte aligned");
  *plan = plan_decode(B, Hq, Hkv, D, page_size, max_pages_per_seq, window_first, window_last,
                      num_splits);
  REQUIRE(B <= kMaxGridYZ && plan->max_splits <= kMaxGridYZ, ATTN_SINK_ERR_UNSUPPORTED,
          "B (%d) and the split count (%d) must each be <= %lld", B, plan->max_splits, kMaxGridYZ);
  // chunk grid: ceil(units / NW) workgroups of 64 * NW threads per slot (NW 2 or 4); the
  // equal-range grid is at most 1024 workgroups per column of 4 units
  REQUIRE(dispatch_fits((long long)B * plan->max_splits * (Hkv * ((Hq / Hkv + 15) / 16) + 3), 64) &&
              dispatch_fits((long long)kDecodeEvenMaxG *
                                ((Hkv * ((Hq / Hkv + 15) / 16) + 3) / 4), 256) &&
              dispatch_fits(((long long)B * Hq + 3) / 4, 256),
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  return ATTN_SINK_OK;
}

extern "C" {

int attn_sink_fwd_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seqlens_k,
                               const float* sink, void* o, float* lse, int B, int Hq, int Hkv,
                               int D, int page_size, int max_pages_per_seq, int num_pages,
                               float softmax_scale, int window_first, int window_last,
                               int num_splits, void* workspace, size_t workspace_bytes, int dtype,
                               void* hip_stream) {
  DecodePlan plan{};
  if (int r = check_decode_call(q, k_cache, v_cache, block_table, seqlens_k, sink, o, lse, B, Hq,
                                Hkv, D, page_size, max_pages_per_seq, num_pages, softmax_scale,
                                window_first, window_last, num_splits, dtype, &plan))
    return r;
  REQUIRE(workspace && aligned16(workspace), ATTN_SINK_ERR_WORKSPACE,
          "a 16-byte aligned workspace of %zu bytes is required", plan.workspace_bytes);
  REQUIRE(workspace_bytes >= plan.workspace_bytes, ATTN_SINK_ERR_WORKSPACE,
          "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
          plan.workspace_bytes);
  DecodeArgs a{q, k_cache, v_cache, block_table, seqlens_k, sink, o, lse, B, Hq, Hkv, D,
               page_size, max_pages_per_seq, num_pages, softmax_scale, window_first, window_last,
               plan.chunk, plan.max_splits, static_cast<float*>(workspace), plan.even};
  return hip_status(launch_decode_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_fwd_decode_paged launch");
}

int attn_sink_fwd_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seqlens_k,
                                       const float* sink, void* o, float* lse, int B, int Hq,
                                       int Hkv, int D, int page_size, int max_pages_per_seq,
                                       int num_pages, float softmax_scale, int window_first,
                                       int window_last, int num_splits, int dtype,
                                       void* hip_stream) {
  DecodePlan plan{};
  if (int r = check_decode_call(q, k_cache, v_cache, block_table, seqlens_k, sink, o, lse, B, Hq,
                                Hkv, D, page_size, max_pages_per_seq, num_pages, softmax_scale,
                                window_first, window_last, num_splits, dtype, &plan))
    return r;
  REQUIRE(plan.workspace_bytes <= kDecodeScratchBytes, ATTN_SINK_ERR_UNSUPPORTED,
          "this decode needs %zu bytes of scratch; the library's scratch holds %zu (use "
          "attn_sink_fwd_decode_paged with a workspace)",
          plan.workspace_bytes, kDecodeScratchBytes);
  float* ws = nullptr;
  if (int r = hip_status(decode_scratch(&ws), "attn_sink_fwd_decode_paged_noalloc scratch"))
    return r;
  DecodeArgs a{q, k_cache, v_cache, block_table, seqlens_k, sink, o, lse, B, Hq, Hkv, D,
               page_size, max_pages_per_seq, num_pages, softmax_scale, window_first, window_last,
               plan.chunk, plan.max_splits, ws, plan.even};
  return hip_status(launch_decode_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_fwd_decode_paged_noalloc launch");
}

size_t attn_sink_bwd_workspace_bytes(int B, int Sq, int Sk, int Hq, int Hkv, int D) {
  if (B < 1 || Sq < 1 || Sk < 0 || check_heads(Hq, Hkv, D) != ATTN_SINK_OK) return 0;
  return backward_workspace_bytes(B, Sq, Hq, (size_t)B * Sq);
}

size_t attn_sink_bwd_varlen_workspace_bytes(int B, int total_q, int max_seqlen_q, int Hq) {
  if (B < 1 || total_q < 0 || max_seqlen_q < 0 || Hq < 1) return 0;
  return backward_workspace_bytes(B, max_seqlen_q, Hq, (size_t)total_q);
}

int attn_sink_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, const float* sink, void* dq, void* dk, void* dv, float* dsink,
                  int B, int Sq, int Sk, int Hq, int Hkv, int D, float softmax_scale, int causal,
                  int window_first, int window_last, void* workspace, size_t workspace_bytes,
                  int dtype, void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16, ATTN_SINK_ERR_UNSUPPORTED,
          "the backward supports bf16 only (dtype %d)", dtype);
  REQUIRE(B >= 1 && Sq >= 1 && Sk >= 1, ATTN_SINK_ERR_INVALID_ARG,
          "need B, Sq, Sk >= 1 (got %d, %d, %d)", B, Sq, Sk);
  if (int r = check_heads(Hq, Hkv, D)) return r;
  if (int r = check_scale(softmax_scale)) return r;
  if (int r = check_window(window_first, window_last)) return r;
  REQUIRE(causal == 0 || causal == 1, ATTN_SINK_ERR_INVALID_ARG, "causal must be 0 or 1");
  REQUIRE(window_last < 0 || causal, ATTN_SINK_ERR_UNSUPPORTED,
          "the first/last window needs causal = 1");
  REQUIRE(q && k && v && o && dout && lse && dq && dk && dv, ATTN_SINK_ERR_INVALID_ARG,
          "q, k, v, o, dout, lse, dq, dk and dv must not be NULL");
  REQUIRE(!sink || dsink, ATTN_SINK_ERR_INVALID_ARG, "dsink is required when sink is given");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) && aligned16(dout) &&
              aligned16(dq) && aligned16(dk) && aligned16(dv),
          ATTN_SINK_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(aligned4(lse) && aligned4(sink) && aligned4(dsink), ATTN_SINK_ERR_INVALID_ARG,
          "lse, sink and dsink must be 4-byte aligned");
  REQUIRE(fits_int32((long long)B * Sq * Hq) && fits_int32((long long)B * Sk * Hkv),
          ATTN_SINK_ERR_UNSUPPORTED, "too many rows for 32-bit row indices");
  REQUIRE(B <= kMaxGridYZ && (Sk + 127) / 128 <= kMaxGridYZ, ATTN_SINK_ERR_UNSUPPORTED,
          "B (%d) and ceil(Sk / 128) (%d) must each be <= %lld", B, (Sk + 127) / 128, kMaxGridYZ);
  REQUIRE((long long)Sk * Hkv * D * 2 <= kMaxSlice && (long long)Sq * Hq * D * 2 <= kMaxSlice,
          ATTN_SINK_ERR_UNSUPPORTED, "one batch's K/V or Q/dO slice exceeds 4 GiB");
  REQUIRE(Hq <= kMaxGridYZ &&
              dispatch_fits(bwd_dkdv_workgroups(B, Sk, Hkv) + bwd_dq_workgroups(B, Sq, Hq, Hkv, D),
                            256),
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  const size_t need = backward_workspace_bytes(B, Sq, Hq, (size_t)B * Sq);
  REQUIRE(workspace && aligned16(workspace), ATTN_SINK_ERR_WORKSPACE,
          "a 16-byte aligned workspace of %zu bytes is required", need);
  REQUIRE(workspace_bytes >= need, ATTN_SINK_ERR_WORKSPACE,
          "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  BackwardArgs a{q,  k,  v,      o,      dout, lse, sink, dq, dk, dv, dsink, nullptr, nullptr, B,
                 Sq, Sk, B * Sq, B * Sk, Hq,   Hkv, D,    softmax_scale, causal, window_first,
                 window_last, workspace};
  return hip_status(launch_backward_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_bwd launch");
}

int attn_sink_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, const float* sink,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq,
                         void* dk, void* dv, float* dsink, int B, int total_q, int total_k,
                         int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int D,
                         float softmax_scale, int causal, int window_first, int window_last,
                         void* workspace, size_t workspace_bytes, int dtype, void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16, ATTN_SINK_ERR_UNSUPPORTED,
          "the backward supports bf16 only (dtype %d)", dtype);
  REQUIRE(B >= 1 && total_q >= 0 && total_k >= 0 && max_seqlen_q >= 0 && max_seqlen_k >= 0,
          ATTN_SINK_ERR_INVALID_ARG,
          "need B >= 1 and total_q, total_k, max_seqlen_q, max_seqlen_k >= 0");
  if (int r = check_heads(Hq, Hkv, D)) return r;
  if (int r = check_scale(softmax_scale)) return r;
  if (int r = check_window(window_first, window_last)) return r;
  REQUIRE(causal == 0 || causal == 1, ATTN_SINK_ERR_INVALID_ARG, "causal must be 0 or 1");
  REQUIRE(window_last < 0 || causal, ATTN_SINK_ERR_UNSUPPORTED,
          "the first/last window needs causal = 1");
  REQUIRE(cu_seqlens_q && cu_seqlens_k && (total_q == 0 || (q && o && dout && lse && dq)) &&
              (total_k == 0 || (k && v && dk && dv)),
          ATTN_SINK_ERR_INVALID_ARG,
          "cu_seqlens_q, cu_seqlens_k and the tensors of non-empty sides must not be NULL");
  REQUIRE(!sink || dsink, ATTN_SINK_ERR_INVALID_ARG, "dsink is required when sink is given");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) && aligned16(dout) &&
              aligned16(dq) && aligned16(dk) && aligned16(dv),
          ATTN_SINK_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(aligned4(lse) && aligned4(sink) && aligned4(dsink) && aligned4(cu_seqlens_q) &&
              aligned4(cu_seqlens_k),
          ATTN_SINK_ERR_INVALID_ARG, "lse, sink, dsink and cu_seqlens must be 4-byte aligned");
  REQUIRE(fits_int32((long long)total_q * Hq) && fits_int32((long long)total_k * Hkv),
          ATTN_SINK_ERR_UNSUPPORTED, "too many rows for 32-bit row indices");
  REQUIRE(B <= kMaxGridYZ && (max_seqlen_k + 127) / 128 <= kMaxGridYZ, ATTN_SINK_ERR_UNSUPPORTED,
          "B (%d) and ceil(max_seqlen_k / 128) (%d) must each be <= %lld", B,
          (max_seqlen_k + 127) / 128, kMaxGridYZ);
  REQUIRE((long long)max_seqlen_k * Hkv * D * 2 <= kMaxSlice &&
              (long long)max_seqlen_q * Hq * D * 2 <= kMaxSlice,
          ATTN_SINK_ERR_UNSUPPORTED, "one sequence's K/V or Q/dO slice exceeds 4 GiB");
  REQUIRE(Hq <= kMaxGridYZ &&
              dispatch_fits(bwd_dkdv_workgroups(B, max_seqlen_k, Hkv) +
                                bwd_dq_workgroups(B, max_seqlen_q, Hq, Hkv, D),
                            256),
          ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  const size_t need = backward_workspace_bytes(B, max_seqlen_q, Hq, (size_t)total_q);
  REQUIRE(workspace && aligned16(workspace), ATTN_SINK_ERR_WORKSPACE,
          "a 16-byte aligned workspace of %zu bytes is required", need);
  REQUIRE(workspace_bytes >= need, ATTN_SINK_ERR_WORKSPACE,
          "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  BackwardArgs a{q,  k,  v,  o,  dout, lse, sink, dq, dk, dv, dsink, cu_seqlens_q, cu_seqlens_k,
                 B,  max_seqlen_q, max_seqlen_k, total_q, total_k, Hq, Hkv, D, softmax_scale,
                 causal, window_first, window_last, workspace};
  return hip_status(launch_backward_bf16(a, static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_bwd_varlen launch");
}

int attn_sink_decode_select_slots(const int32_t* block_table, const int32_t* seqlens_k, int B,
                                  int max_pages_per_seq, int page_size, int window_first,
                                  int window_last, int64_t* slots, int32_t* counts, int max_sel,
                                  void* hip_stream) {
  REQUIRE(B >= 1 && max_pages_per_seq >= 1 && max_sel >= 1, ATTN_SINK_ERR_INVALID_ARG,
          "need B, max_pages_per_seq, max_sel >= 1");
  REQUIRE(pow2(page_size) && page_size <= 256, ATTN_SINK_ERR_UNSUPPORTED,
          "page_size must be a power of two in [1, 256] (got %d)", page_size);
  if (int r = check_window(window_first, window_last)) return r;
  REQUIRE(block_table && seqlens_k && slots && counts, ATTN_SINK_ERR_INVALID_ARG,
          "block_table, seqlens_k, slots and counts must not be NULL");
  REQUIRE(aligned4(block_table) && aligned4(seqlens_k) && aligned4(counts) &&
              (reinterpret_cast<uintptr_t>(slots) & 7u) == 0,
          ATTN_SINK_ERR_INVALID_ARG, "misaligned pointer");
  REQUIRE(dispatch_fits(B, 256), ATTN_SINK_ERR_UNSUPPORTED, "%s", kGridMsg);
  return hip_status(launch_select_slots(block_table, seqlens_k, B, max_pages_per_seq, page_size,
                                        window_first, window_last, slots, counts, max_sel,
                                        static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_decode_select_slots launch");
}

int attn_sink_gather_kv(const void* k_cache, const void* v_cache, const int32_t* block_table,
                        const int32_t* seqlens_k, int B, int Hkv, int D, int page_size,
                        int max_pages_per_seq, int window_first, int window_last, void* k_out,
                        void* v_out, int max_sel, int dtype, void* hip_stream) {
  REQUIRE(dtype == ATTN_SINK_BF16 || dtype == ATTN_SINK_F32, ATTN_SINK_ERR_UNSUPPORTED,
          "unknown dtype %d", dtype);
  REQUIRE(B >= 1 && Hkv >= 1 && D >= 1 && max_pages_per_seq >= 1 && max_sel >= 1,
          ATTN_SINK_ERR_INVALID_ARG, "sizes must be >= 1");
  REQUIRE(pow2(page_size) && page_size <= 256, ATTN_SINK_ERR_UNSUPPORTED,
          "page_size must be a power of two in [1, 256] (got %d)", page_size);
  if (int r = check_window(window_first, window_last)) return r;
  REQUIRE(k_cache && v_cache && block_table && seqlens_k && k_out && v_out,
          ATTN_SINK_ERR_INVALID_ARG, "pointers must not be NULL");
  REQUIRE(aligned4(block_table) && aligned4(seqlens_k) && aligned4(k_cache) && aligned4(v_cache) &&
              aligned4(k_out) && aligned4(v_out),
          ATTN_SINK_ERR_INVALID_ARG, "misaligned pointer");
  REQUIRE(dispatch_fits(max_sel, 256) && B <= kMaxGridYZ, ATTN_SINK_ERR_UNSUPPORTED, "%s",
          kGridMsg);
  return hip_status(launch_gather_kv(k_cache, v_cache, block_table, seqlens_k, B, Hkv, D,
                                     page_size, max_pages_per_seq, window_first, window_last,
                                     k_out, v_out, max_sel, dtype == ATTN_SINK_BF16 ? 2 : 4,
                                     static_cast<hipStream_t>(hip_stream)),
                    "attn_sink_gather_kv launch");
}

int attn_sink_device_check_flags(unsigned* flags, int clear, void* hip_stream) {
  REQUIRE(flags, ATTN_SINK_ERR_INVALID_ARG, "flags must not be NULL");
#ifdef ATTN_SINK_DEVICE_CHECKS
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  unsigned a = 0, b = 0, c = 0;
  if (int r = hip_status(read_check_word_decode(&a, clear != 0, st), "device check word")) return r;
  if (int r = hip_status(read_check_word_prefill(&b, clear != 0, st), "device check word")) return r;
  if (int r = hip_status(read_check_word_backward(&c, clear != 0, st), "device check word"))
    return r;
  *flags = a | b | c;
  return ok();
#else
  (void)clear;
  (void)hip_stream;
  *flags = 0;
  return fail(ATTN_SINK_ERR_UNSUPPORTED,
              "this library was built without device checks (libattn_sink_debug.so has them)");
#endif
}

int attn_sink_check_paged_inputs(const int32_t* block_table, const int32_t* seqlens_k,
                                 const int32_t* cu_seqlens_q, int B, int total_q,
                                 int max_seqlen_q, int max_pages_per_seq, int page_size,
                                 int num_pages, int window_first, int window_last, int decode,
                                 unsigned* flags) {
  REQUIRE(block_table && seqlens_k && flags, ATTN_SINK_ERR_INVALID_ARG,
          "block_table, seqlens_k and flags must not be NULL");
  REQUIRE(B >= 1 && max_pages_per_seq >= 1 && num_pages >= 1, ATTN_SINK_ERR_INVALID_ARG,
          "B, max_pages_per_seq and num_pages must be >= 1");
  REQUIRE(pow2(page_size) && page_size <= 256, ATTN_SINK_ERR_UNSUPPORTED,
          "page_size must be a power of two in [1, 256] (got %d)", page_size);
  if (int r = check_window(window_first, window_last)) return r;
  unsigned f = 0;
  for (int b = 0; b < B; ++b) {
    if (cu_seqlens_q && !cu_ok(cu_seqlens_q, b, B, total_q, max_seqlen_q)) f |= kCheckCuSeqlens;
    const int L = seqlens_k[b];
    if (!seqlen_ok(L, decode ? 1 : 0, max_pages_per_seq, page_size)) {
      f |= kCheckSeqlen;
      continue;
    }
    const PageRanges r = page_ranges(L, page_size, window_first, window_last, decode != 0);
    const int32_t* row = block_table + (size_t)b * max_pages_per_seq;
    for (int i = 0; i < r.n_first; ++i)
      if (!page_ok(row[i], num_pages)) f |= kCheckPage;
    for (int i = r.last0; i < r.n_pages; ++i)
      if (!page_ok(row[i], num_pages)) f |= kCheckPage;
  }
  *flags = f;
  return ok();
}

}  // extern "C"
