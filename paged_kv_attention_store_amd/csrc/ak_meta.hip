// Device-side batch metadata: the CSR page table from a 2-D block table, and the
// flat cache slot of every new token.
//
// "vLLM attention backend", "From a 2-D block table to a CSR page table":
// request r's pages are the first ceil(L_r / B) entries of its block-table row;
// kv_indptr is the running sum of those counts, kv_indices their concatenation
// and last_page_len = L_r - (pages_r - 1) * B.  The worked example of the same
// page and "Write the KV first": token j of the n_r new tokens of request r sits
// at position p = L_r - n_r + j and is written to slot page[p / B] * B + p % B.
//
// "vLLM attention backend", "Hybrid KV and virtual kernel blocks": when the
// cache manager's block holds M = ratio * B tokens and the kernel takes B-token
// pages, manager block b is kernel pages b * ratio .. b * ratio + ratio - 1 of the
// same cache viewed as [P * ratio, B, Hkv, D]; the CSR lists kernel pages.
//
// Integer work only.  The running sum is one workgroup (the batch is at most a
// few thousand requests); the copy of page ids and the slot computation are
// spread over the machine.

#include "ak_launch.h"

namespace ak {

namespace {

constexpr int kScanThreads = 1024;

// a length is clamped into [0, row_stride * ratio * B] so that its pages stay inside the row
__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t B, int64_t row_stride, int32_t ratio) {
  const int64_t cap = row_stride * ratio * (int64_t)B;
  return L <= 0 ? 0 : (int32_t)((int64_t)L < cap ? (int64_t)L : cap);
}

// kv_indptr and last_page_len: chunks of 1024 requests, each an inclusive scan
// (within a wave by shuffles up, across the 16 waves through LDS) plus
// the running carry of the chunks before it
__global__ __launch_bounds__(kScanThreads) void csr_scan_kernel(const int32_t* __restrict__ seq_lens,
                                                                int32_t R, int32_t B, int64_t row_stride,
                                                                int32_t ratio,
                                                                int32_t* __restrict__ kv_indptr,
                                                                int32_t* __restrict__ last_page_len) {
  __shared__ int32_t wsum[kScanThreads / 64];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    kv_indptr[0] = 0;
    carry_s = 0;
  }
  __syncthreads();
  for (int32_t base = 0; base < R; base += kScanThreads) {
    const int32_t r = base + tid;
    const int32_t L = r < R ? clamp_len(seq_lens[r], B, row_stride, ratio) : 0;
    const int32_t pg = (int32_t)(((int64_t)L + B - 1) / B);
    int32_t v = pg;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const int32_t u = __shfl_up(v, k, 64);
      if (lane >= k) v += u;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int32_t carry = carry_s;
    if (r < R) {
      kv_indptr[r + 1] = carry + before + v;
      last_page_len[r] = pg > 0 ? L - (pg - 1) * B : 0;
    }
    __syncthreads();   // every thread has read carry_s and wsum
    if (tid == kScanThreads - 1) carry_s = carry + before + v;
    __syncthreads();
  }
}

// kv_indices: workgroup r writes the kernel pages of request r
__global__ __launch_bounds__(256) void csr_copy_kernel(const int32_t* __restrict__ block_table,
                                                       int64_t row_stride, int32_t ratio,
                                                       const int32_t* __restrict__ kv_indptr,
                                                       int32_t* __restrict__ kv_indices,
                                                       int64_t capacity) {
  const int32_t r = blockIdx.x;
  const int64_t a = kv_indptr[r], b = kv_indptr[r + 1];
  const int32_t* row = block_table + (int64_t)r * row_stride;
  if (ratio == 1) {
    for (int64_t i = threadIdx.x; i < b - a; i += 256)
      if (a + i < capacity) kv_indices[a + i] = row[i];
  } else {
    for (int64_t i = threadIdx.x; i < b - a; i += 256)
      if (a + i < capacity) kv_indices[a + i] = row[i / ratio] * ratio + (int32_t)(i % ratio);
  }
}

// slot_mapping: one thread per new token; its request by binary search in qo_indptr
__global__ __launch_bounds__(256) void slots_kernel(const int32_t* __restrict__ block_table,
                                                    int64_t row_stride,
                                                    const int32_t* __restrict__ qo_indptr,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int32_t R, int32_t B,
                                                    int64_t* __restrict__ slot_mapping, int64_t N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  int32_t lo = 0, hi = R;   // first r with qo_indptr[r + 1] > i
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    if (qo_indptr[mid + 1] > i) hi = mid; else lo = mid + 1;
  }
  int64_t slot = -1;
  if (lo < R) {
    const int64_t j = i - qo_indptr[lo];
    const int64_t n = (int64_t)qo_indptr[lo + 1] - qo_indptr[lo];
    const int64_t p = (int64_t)seq_lens[lo] - n + j;
    if (p >= 0 && p / B < row_stride) slot = (int64_t)block_table[lo * row_stride + p / B] * B + p % B;
  }
  slot_mapping[i] = slot;
}

}  // namespace

hipError_t launch_csr_from_block_table(const int32_t* block_table, int64_t row_stride,
                                       const int32_t* seq_lens, int32_t R, int32_t B, int32_t ratio,
                                       int32_t* kv_indptr, int32_t* kv_indices, int64_t capacity,
                                       int32_t* last_page_len, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, seq_lens, R, B, row_stride,
                     ratio, kv_indptr, last_page_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || R == 0) return e;
  hipLaunchKernelGGL(csr_copy_kernel, dim3((unsigned)R), dim3(256), 0, s, block_table, row_stride,
                     ratio, kv_indptr, kv_indices, capacity);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* block_table, int64_t row_stride, const int32_t* qo_indptr,
                               const int32_t* seq_lens, int32_t R, int32_t B, int64_t* slot_mapping,
                               int64_t N, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(slots_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, block_table,
                     row_stride, qo_indptr, seq_lens, R, B, slot_mapping, N);
  return hipGetLastError();
}

}  // namespace ak
