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

hipError_t launch_gather_slots(const Req* reqs, const int64_t* kv_off, const int32_t* kv_indices,
                               int32_t R, int32_t log2B, int64_t num_pages, int64_t* slots,
                               hipStream_t s);

hipError_t launch_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, hipStream_t s);

// kv dtype: AK_BF16 or AK_FP8_E4M3 for bf16 queries.
hipError_t launch_attn_small(const AttnArgs& a, int n_items, int D, int kv_dtype, bool shared_pages,
                             hipStream_t s);
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

// Physical page holding KV position t of a request whose pages start at
// kv_indices[page_off]; the position's row inside the page is t & (B - 1).
// Page ids are clamped into the pool so a corrupt table cannot address outside it.
__device__ __forceinline__ int64_t kv_page(const int32_t* __restrict__ kv_indices, int32_t page_off,
                                           int32_t t, int32_t log2B, int64_t num_pages) {
  int64_t page = (int64_t)kv_indices[page_off + (t >> log2B)];
  return page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
}

}  // namespace ak
