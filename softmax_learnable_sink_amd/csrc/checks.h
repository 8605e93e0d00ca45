// Device-side preconditions of the paged and packed entry points.
//
// The C ABI validates every host-visible argument; values that live on the
// device (sequence lengths, block-table entries, cumulative sequence offsets)
// are documented preconditions.  A debug build (ATTN_SINK_DEVICE_CHECKS)
// checks them on the device: a check kernel runs ahead of each launch that
// reads them and ORs the violations into this source file's error word, and
// every kernel of the file returns at once while the word is set, so bad
// values are reported instead of read through.  The predicates below are
// host/device functions: the host-side checker of the C ABI applies the same
// ones to host arrays.
#pragma once

#include "common.h"

namespace attn_sink {

enum : unsigned {
  kCheckSeqlen = 1u,     // seqlens_k[b] outside [min_len, max_pages * page_size]
  kCheckPage = 2u,       // a block-table entry the call reads outside [0, num_pages)
  kCheckCuSeqlens = 4u,  // cu_seqlens not 0 = cu[0] <= ... <= cu[B] = total, or a length
                         // above its stated maximum
};

__host__ __device__ inline bool seqlen_ok(int L, int min_len, int max_pages, int page_size) {
  return L >= min_len && (long long)L <= (long long)max_pages * page_size;
}

// Block-table entries a sequence of L tokens has read: pages [0, n_first) and
// [last0, n_pages).  The decode reads exactly the pages of its selected
// tokens (the first W1 and the last W2 when the window applies); the other
// paged kernels read whole key tiles, so every page of [0, L) is checked.
struct PageRanges {
  int n_first, last0, n_pages;
};
__host__ __device__ inline PageRanges page_ranges(int L, int page_size, int w1, int w2,
                                                  bool exact_selection) {
  const int np = (L + page_size - 1) / page_size;
  if (exact_selection && w2 > 0 && L > w1 + w2)
    return PageRanges{(w1 + page_size - 1) / page_size, (L - w2) / page_size, np};
  return PageRanges{np, np, np};
}

__host__ __device__ inline bool page_ok(int page, int num_pages) {
  return page >= 0 && page < num_pages;
}

// Sequence b of a cumulative-offset array of B + 1 entries.
__host__ __device__ inline bool cu_ok(const int32_t* cu, int b, int B, int total, int max_len) {
  const int a = cu[b], e = cu[b + 1];
  return a <= e && e - a <= max_len && (b > 0 || a == 0) && (b < B - 1 || e == total);
}

#ifdef ATTN_SINK_DEVICE_CHECKS
namespace {
__device__ unsigned g_check_word;  // this source file's violations so far

// One workgroup per sequence: its length, the block-table entries it reads and
// (cu_q != NULL) its query offsets.
__global__ __launch_bounds__(256) void check_paged_kernel(
    const int32_t* __restrict__ bt, const int32_t* __restrict__ seqlens,
    const int32_t* __restrict__ cu_q, int B, int total_q, int max_sq, int max_pages,
    int page_size, int num_pages, int min_len, int w1, int w2, int exact_selection) {
  const int b = blockIdx.x;
  unsigned f = 0;
  if (cu_q && threadIdx.x == 0 && !cu_ok(cu_q, b, B, total_q, max_sq)) f |= kCheckCuSeqlens;
  const int L = seqlens[b];
  if (!seqlen_ok(L, min_len, max_pages, page_size)) {
    f |= kCheckSeqlen;
  } else {
    const PageRanges r = page_ranges(L, page_size, w1, w2, exact_selection != 0);
    const int32_t* row = bt + (size_t)b * max_pages;
    for (int i = threadIdx.x; i < r.n_first; i += blockDim.x)
      if (!page_ok(row[i], num_pages)) f |= kCheckPage;
    for (int i = r.last0 + threadIdx.x; i < r.n_pages; i += blockDim.x)
      if (!page_ok(row[i], num_pages)) f |= kCheckPage;
  }
  if (f) atomicOr(&g_check_word, f);
}

// Packed variable-length offsets: one thread per sequence.
__global__ __launch_bounds__(256) void check_cu_kernel(const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ cu_k, int B,
                                                       int total_q, int total_k, int max_sq,
                                                       int max_sk) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  if (!cu_ok(cu_q, b, B, total_q, max_sq) || !cu_ok(cu_k, b, B, total_k, max_sk))
    atomicOr(&g_check_word, kCheckCuSeqlens);
}
}  // namespace

// Kernels of a file with device checks return at once once a violation is recorded.
#define ATTN_SINK_CHECK_GUARD() \
  do {                          \
    if (g_check_word) return;   \
  } while (0)

// This file's error word (host side): read it after the stream's work, and
// clear it if asked.
#define ATTN_SINK_DEFINE_CHECK_READER(name)                                           \
  hipError_t name(unsigned* word, bool clear, hipStream_t stream) {                   \
    void* p = nullptr;                                                                \
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_check_word));                 \
    if (e == hipSuccess) e = hipMemcpyAsync(word, p, sizeof(unsigned),                \
                                            hipMemcpyDeviceToHost, stream);           \
    if (e == hipSuccess) e = hipStreamSynchronize(stream);                            \
    if (e == hipSuccess && clear) e = hipMemsetAsync(p, 0, sizeof(unsigned), stream); \
    if (e == hipSuccess && clear) e = hipStreamSynchronize(stream);                   \
    return e;                                                                         \
  }
#else
#define ATTN_SINK_CHECK_GUARD() \
  do {                          \
  } while (0)
#endif

}  // namespace attn_sink
