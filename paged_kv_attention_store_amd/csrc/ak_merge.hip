// Merge of split-KV partial attention states.
//
// "SGLang attention backend", "The two forms of extend": two attention states
// over disjoint key sets combine exactly through their log-sum-exp; with
// m = max_s lse_s, out = sum_s e^(lse_s - m) out_s / sum_s e^(lse_s - m) and
// lse = m + ln sum_s e^(lse_s - m).  Partials hold each part's normalised
// output (fp32) and its LSE in base 2; the final LSE is written in base e.
//
// One wavefront per (query token, query head) job, each lane owning D/64
// consecutive columns; bandwidth-bound (reads S * (D + 1) floats per job).

#include "ak_launch.h"

namespace ak {

namespace {

template <int D, int OUT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int PER = D / 64;
  const int job = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (job >= a.n_jobs) return;
  const MergeJob jb = a.jobs[job];
  float m = -INFINITY;
  for (int s = 0; s < jb.count; ++s) m = fmaxf(m, a.part_lse[jb.pfirst + (int64_t)s * jb.pstride]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < jb.count; ++s) {
      const int64_t prow = jb.pfirst + (int64_t)s * jb.pstride;
      const float w = exp2f(a.part_lse[prow] - m);   // -inf parts weigh 0
      const float* po = a.part_o + prow * D + lane * PER;
      if (PER == 2) {
        const float2 v = *reinterpret_cast<const float2*>(po);
        acc[0] += w * v.x;
        acc[PER - 1] += w * v.y;
      } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += w * po[i];
      }
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t obase = jb.token * a.o_st + jb.head * a.o_sh + lane * PER;
  if (OUT == AK_F32) {
    float* o = static_cast<float*>(a.out) + obase;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = acc[i] * inv;
  } else {
    uint16_t* o = static_cast<uint16_t*>(a.out) + obase;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = (uint16_t)f32_to_bf16_bits(acc[i] * inv);
  }
  if (a.lse && lane == 0)
    a.lse[jb.token * a.l_st + jb.head * a.l_sh] =
        wsum > 0.f ? (m + log2f(wsum)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int D, int out_dtype, hipStream_t s) {
  if (a.n_jobs <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.n_jobs + 3) / 4));
#define AK_MERGE_CASE(DD, O)                                                \
  if (D == DD && out_dtype == O) {                                          \
    hipLaunchKernelGGL((merge_kernel<DD, O>), grid, dim3(256), 0, s, a);    \
    return hipGetLastError();                                               \
  }
  AK_MERGE_CASE(64, AK_F32)
  AK_MERGE_CASE(128, AK_F32)
  AK_MERGE_CASE(64, AK_BF16)
  AK_MERGE_CASE(128, AK_BF16)
#undef AK_MERGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace ak
