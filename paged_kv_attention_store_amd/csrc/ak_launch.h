// Host-side launchers of the gfx950 kernels (one translation unit per kernel family).
#pragma once

#include <hip/hip_runtime.h>

#include "ak_device.h"

namespace ak {

struct StoreArgs {
  const void* src[2];       // k, v rows  [N, Hkv, D]
  void* dst[2];             // k, v caches [P, B, Hkv, D]
  const int64_t* slots;     // [N]
  int64_t s_st[2], s_sh[2]; // source strides (elements): token, head
  int64_t d_sp[2], d_sb[2], d_sh[2];  // cache strides (elements): page, slot, head
  float scale[2];           // fp8 per-tensor scales
  int64_t num_slots;        // P * B (slots >= this are ignored)
  int32_t N, Hkv, D, B;
};

// src/dst dtypes are ak_dtype values.
hipError_t launch_store_kv(const StoreArgs& a, int src_dtype, int dst_dtype, hipStream_t s);

// addressing: 0 = the decode / fp32 kernels' row offsets, 1 = the prefill
// kernels' copy offsets, 2 = their 32-bit form (page ids below 2^24)
hipError_t launch_gather_slots(const Req* reqs, const int64_t* kv_off, const int32_t* kv_indices,
                               int32_t R, int32_t log2B, int64_t num_pages, int32_t addressing,
                               int64_t* slots, hipStream_t s);

hipError_t launch_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, hipStream_t s);

// kv dtype: AK_BF16 or AK_FP8_E4M3 for bf16 queries.
// n_wg > 0: a persistent launch of n_wg workgroups, each running its items
// a.wg_first[g] .. a.wg_first[g+1]-1 (stream-K plans); else one workgroup per item.
hipError_t launch_attn_small(const AttnArgs& a, int n_items, int D, int kv_dtype, bool shared_pages,
                             int n_wg, hipStream_t s);
hipError_t launch_attn_large(const AttnArgs& a, int n_items, int D, int kv_dtype, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, int n_items, int D, hipStream_t s);

// out dtype: AK_F32 or AK_BF16.
hipError_t launch_merge(const MergeArgs& a, int D, int out_dtype, hipStream_t s);
hipError_t launch_merge2(const Merge2Args& a, int D, int dtype, hipStream_t s);
hipError_t launch_csr_from_block_table(const int32_t* block_table, int64_t row_stride,
                                       const int32_t* seq_lens, int32_t R, int32_t B, int32_t ratio,
                                       int32_t* kv_indptr, int32_t* kv_indices, int64_t capacity,
                                       int32_t* last_page_len, hipStream_t s);
hipError_t launch_slot_mapping(const int32_t* block_table, int64_t row_stride, const int32_t* qo_indptr,
                               const int32_t* seq_lens, int32_t R, int32_t B, int64_t* slot_mapping,
                               int64_t N, hipStream_t s);

// ---- K/V row addressing shared by the attention kernels and ak_gather_slots
// (which runs these same functions with page stride B and slot stride 1, so the
// offset they produce is the flat cache slot page * B + t % B).

// A page id clamped into the pool, so a corrupt table cannot address outside it.
__device__ __forceinline__ int32_t clamp_page(int32_t page, int64_t num_pages) {
  const int32_t pmax = (int32_t)min(num_pages - 1, (int64_t)INT32_MAX);
  return min(max(page, 0), pmax);
}

// Index into kv_indices of the page holding KV position t of a request whose
// page list starts at page_off.
__device__ __forceinline__ int32_t kv_page_index(int32_t page_off, int32_t t, int32_t log2B) {
  return page_off + (t >> log2B);
}

// The (clamped) physical page holding KV position t of a request.
__device__ __forceinline__ int32_t kv_page_id(const int32_t* __restrict__ kv_indices, int32_t page_off,
                                              int32_t t, int32_t log2B, int64_t num_pages) {
  return clamp_page(kv_indices[kv_page_index(page_off, t, log2B)], num_pages);
}

// Offset of KV position t's row in page `page`, for a page stride and a slot
// stride in any unit (bytes in the kernels).
__device__ __forceinline__ int64_t kv_row_offset(int32_t page, int32_t t, int32_t log2B,
                                                 int64_t page_stride, int64_t slot_stride) {
  return (int64_t)page * page_stride + (int64_t)(t & ((1 << log2B) - 1)) * slot_stride;
}

// The same for the load-to-LDS copies, with the offset inside the page formed in
// 32 bits (slot stride times the page size below 2 GiB, checked on the host) and
// a byte offset within the row added to it.
__device__ __forceinline__ uint64_t kv_copy_offset(uint32_t page, int32_t t, int32_t log2B,
                                                   uint32_t page_stride, uint32_t slot_stride,
                                                   uint32_t in_row) {
  const uint32_t slot = (uint32_t)(t & ((1 << log2B) - 1));
  return (uint64_t)page * page_stride + (slot * slot_stride + in_row);
}

// The same offset formed entirely in 32 bits with 24-bit multiplies, for pools
// that satisfy kv_copy32_ok: every page id below 2^24, page and slot strides
// below 2^24 bytes and the whole pool (from the head's base) within 4 GiB, so
// the address is a uniform 64-bit base plus this per-lane 32-bit offset.
__device__ __forceinline__ uint32_t kv_copy_offset32(uint32_t page, int32_t t, int32_t log2B,
                                                     uint32_t page_stride, uint32_t slot_stride,
                                                     uint32_t in_row) {
  const uint32_t slot = (uint32_t)(t & ((1 << log2B) - 1));
  return __umul24(page, page_stride) + __umul24(slot, slot_stride) + in_row;
}

// Host check for kv_copy_offset32: num_pages pages of page_stride bytes with
// slots of slot_stride bytes (B per page) and rows of row_bytes.
inline bool kv_copy32_ok(int64_t num_pages, int64_t page_stride, int64_t slot_stride, int32_t B,
                         int64_t row_bytes) {
  constexpr int64_t k24 = int64_t(1) << 24;
  if (num_pages < 1 || num_pages > k24 || page_stride >= k24 || slot_stride >= k24) return false;
  const int64_t span = (num_pages - 1) * page_stride + (int64_t)(B - 1) * slot_stride + row_bytes;
  return span <= (int64_t(1) << 32) - 1;
}

}  // namespace ak
