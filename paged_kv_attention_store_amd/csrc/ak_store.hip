// store_kv: scatter this step's K/V rows into the paged cache by slot, and the
// debug gather of the plan's slot arithmetic.
//
// "vLLM attention backend", "Write the KV first": the step's K/V are written
// into the paged cache by slot_mapping before attention reads the cache.
// Memory-bound: one wave per token moves its row in 16-byte (or wider) vector
// accesses; K and V are the two planes of blockIdx.y.

#include "ak_launch.h"

namespace ak {

namespace {

template <int SRC>
struct Load8;

template <>
struct Load8<AK_F32> {
  __device__ static void run(const void* p, float (&x)[8]) {
    const f32x4* v = reinterpret_cast<const f32x4*>(p);
    f32x4 a = __builtin_nontemporal_load(v), b = __builtin_nontemporal_load(v + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
};

template <>
struct Load8<AK_BF16> {
  __device__ static void run(const void* p, float (&x)[8]) {
    u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
};

template <int DST>
struct Store8;

template <>
struct Store8<AK_F32> {
  __device__ static void run(void* p, const float (&x)[8], float) {
    f32x4* v = reinterpret_cast<f32x4*>(p);
    v[0] = f32x4{x[0], x[1], x[2], x[3]};
    v[1] = f32x4{x[4], x[5], x[6], x[7]};
  }
};

template <>
struct Store8<AK_BF16> {
  __device__ static void run(void* p, const float (&x)[8], float) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
};

template <>
struct Store8<AK_FP8_E4M3> {
  __device__ static void run(void* p, const float (&x)[8], float scale) {
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = f32_to_e4m3(x[i] / scale);   // IEEE binary32 quotient
    u32x2 w;
    w[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    *reinterpret_cast<u32x2*>(p) = w;
  }
};

constexpr int elem_size(int dt) { return dt == AK_F32 ? 4 : (dt == AK_BF16 ? 2 : 1); }

template <int SRC, int DST>
__device__ __forceinline__ void move8(const char* sp, char* dp, float scale) {
  float x[8];
  Load8<SRC>::run(sp, x);
  Store8<DST>::run(dp, x, scale);
}

// One wave per token: the token's slot is read once (a scalar load) and its
// Hkv * D elements move as 8-element groups, 64 consecutive groups per
// instruction, so every load and store instruction covers contiguous memory when
// the token's heads are contiguous in both the source and the cache (the usual
// layout); other head strides split the group index into (head, column).
template <int SRC, int DST>
__global__ __launch_bounds__(256) void store_kv_kernel(StoreArgs a) {
  constexpr int ES = elem_size(SRC), ED = elem_size(DST);
  const int plane = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gph = a.D >> 3;                  // groups per head
  const int gpt = a.Hkv * gph;               // groups per token
  const int64_t s_sh = a.s_sh[plane], d_sh = a.d_sh[plane];
  const bool flat = s_sh == a.D && d_sh == a.D;
  const char* src = static_cast<const char*>(a.src[plane]);
  char* dst = static_cast<char*>(a.dst[plane]);
  const float scale = a.scale[plane];
  auto offs = [&](int j, int64_t& so, int64_t& dof) {
    if (flat) {
      so = dof = (int64_t)j << 3;
    } else {
      const int h = j / gph, d0 = (j - h * gph) << 3;
      so = h * s_sh + d0;
      dof = h * d_sh + d0;
    }
  };
  for (int tok = blockIdx.x * 4 + wave; tok < a.N; tok += gridDim.x * 4) {
    const int64_t slot = a.slots[tok];
    if (slot < 0 || slot >= a.num_slots) continue;   // uniform over the wave
    const int64_t page = slot / a.B;
    const int64_t off = slot - page * a.B;
    const char* sp = src + (int64_t)tok * a.s_st[plane] * ES;
    char* dp = dst + (page * a.d_sp[plane] + off * a.d_sb[plane]) * ED;
    int j = lane;
    for (; j + 64 < gpt; j += 128) {   // two groups in flight per lane
      int64_t so0, do0, so1, do1;
      offs(j, so0, do0);
      offs(j + 64, so1, do1);
      float x0[8], x1[8];
      Load8<SRC>::run(sp + so0 * ES, x0);
      Load8<SRC>::run(sp + so1 * ES, x1);
      Store8<DST>::run(dp + do0 * ED, x0, scale);
      Store8<DST>::run(dp + do1 * ED, x1, scale);
    }
    if (j < gpt) {
      int64_t so, dof;
      offs(j, so, dof);
      move8<SRC, DST>(sp + so * ES, dp + dof * ED, scale);
    }
  }
}

// The flat slot of every KV position of every request, through the addressing
// functions the attention kernels use for their K/V rows, with page stride B and
// slot stride 1 in place of the cache's byte strides.
template <int ADDRESSING>
__global__ __launch_bounds__(256) void gather_slots_kernel(const Req* __restrict__ reqs,
                                                           const int64_t* __restrict__ kv_off,
                                                           const int32_t* __restrict__ kv_indices,
                                                           int32_t log2B, int64_t num_pages,
                                                           int64_t* __restrict__ slots) {
  const Req rq = reqs[blockIdx.y];
  const int64_t base = kv_off[blockIdx.y];
  const int32_t B = 1 << log2B;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < rq.L; t += gridDim.x * blockDim.x) {
    if (ADDRESSING == 0) {
      // decode and fp32 kernels: clamped page id, then the row offset
      const int32_t page = kv_page_id(kv_indices, rq.page_off, t, log2B, num_pages);
      slots[base + t] = kv_row_offset(page, t, log2B, B, 1);
    } else if (ADDRESSING == 1) {
      // prefill kernels: raw page id loaded ahead, clamped at the copy, copy offset
      const int32_t raw = kv_indices[kv_page_index(rq.page_off, t, log2B)];
      slots[base + t] = (int64_t)kv_copy_offset((uint32_t)clamp_page(raw, num_pages), t, log2B,
                                                (uint32_t)B, 1u, 0u);
    } else {
      // prefill kernels on pools within kv_copy_offset32's bounds: the same, in 32 bits
      const int32_t raw = kv_indices[kv_page_index(rq.page_off, t, log2B)];
      slots[base + t] = (int64_t)kv_copy_offset32((uint32_t)clamp_page(raw, num_pages), t, log2B,
                                                  (uint32_t)B, 1u, 0u);
    }
  }
}

__global__ __launch_bounds__(256) void fp8_to_bf16_kernel(const uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ out, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const u32x2 w = reinterpret_cast<const u32x2*>(codes)[i];
    reinterpret_cast<u32x4*>(out)[i] = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(w[0], w[1]));
  }
}

}  // namespace

hipError_t launch_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, out, n8);
  return hipGetLastError();
}

hipError_t launch_store_kv(const StoreArgs& a, int src_dtype, int dst_dtype, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  int64_t blocks = ((int64_t)a.N + 3) / 4;   // four tokens (waves) per block
  if (blocks > 8192) blocks = 8192;
  dim3 grid((unsigned)blocks, 2);
#define AK_STORE_CASE(S, D)                                                 \
  if (src_dtype == S && dst_dtype == D) {                                   \
    hipLaunchKernelGGL((store_kv_kernel<S, D>), grid, dim3(256), 0, s, a); \
    return hipGetLastError();                                               \
  }
  AK_STORE_CASE(AK_F32, AK_F32)
  AK_STORE_CASE(AK_F32, AK_BF16)
  AK_STORE_CASE(AK_F32, AK_FP8_E4M3)
  AK_STORE_CASE(AK_BF16, AK_BF16)
  AK_STORE_CASE(AK_BF16, AK_FP8_E4M3)
#undef AK_STORE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gather_slots(const Req* reqs, const int64_t* kv_off, const int32_t* kv_indices,
                               int32_t R, int32_t log2B, int64_t num_pages, int32_t addressing,
                               int64_t* slots, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  if (R <= 0) return hipSuccess;
  dim3 grid(64, (unsigned)R);
  if (addressing == 0) {
    hipLaunchKernelGGL(gather_slots_kernel<0>, grid, dim3(256), 0, s, reqs, kv_off, kv_indices,
                       log2B, num_pages, slots);
  } else if (addressing == 1) {
    hipLaunchKernelGGL(gather_slots_kernel<1>, grid, dim3(256), 0, s, reqs, kv_off, kv_indices,
                       log2B, num_pages, slots);
  } else {
    hipLaunchKernelGGL(gather_slots_kernel<2>, grid, dim3(256), 0, s, reqs, kv_off, kv_indices,
                       log2B, num_pages, slots);
  }
  return hipGetLastError();
}

}  // namespace ak
