// Merge of split-KV partial attention states.
//
// "SGLang attention backend", "The two forms of extend": two attention states
// over disjoint key sets combine exactly through their log-sum-exp; with
// m = max_s lse_s, out = sum_s e^(lse_s - m) out_s / sum_s e^(lse_s - m) and
// lse = m + ln sum_s e^(lse_s - m).  Partials hold each part's normalised
// output (fp32) and its LSE in base 2; the final LSE is written in base e.
//
// One wavefront per (query token, query head) job, each lane owning D/64
// consecutive columns; bandwidth-bound (reads S * (D + 1) floats per job) once
// the part loads overlap.
// The same combination of two states given as tensors backs ak_merge_states.

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
  if (jb.count == 0) return;   // padding job
  // The parts' LSEs are read 64 at a time, one per lane, and reduced across the
  // wave; lane j then holds part (chunk + j)'s weight, which the weighted sum
  // takes by a lane broadcast.  The sum runs over the parts in order with four
  // row loads in flight (the same arithmetic, part by part, as one load at a time).
  float m = -INFINITY;
  for (int s = lane; s < jb.count; s += 64) m = fmaxf(m, a.part_lse[jb.pfirst + (int64_t)s * jb.pstride]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int c0 = 0; c0 < jb.count; c0 += 64) {
      const int n = min(64, jb.count - c0);
      const float wl = lane < n ? exp2f(a.part_lse[jb.pfirst + (int64_t)(c0 + lane) * jb.pstride] - m)
                                : 0.f;   // -inf parts weigh 0
      const float* pbase = a.part_o + ((int64_t)jb.pfirst + (int64_t)c0 * jb.pstride) * D + lane * PER;
      const int64_t pstep = (int64_t)jb.pstride * D;
      int j = 0;
      for (; j + 4 <= n; j += 4) {
        float v[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < PER; ++i) v[u][i] = pbase[(j + u) * pstep + i];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = __shfl(wl, j + u, 64);
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] += w * v[u][i];
          wsum += w;
        }
      }
      for (; j < n; ++j) {
        const float w = __shfl(wl, j, 64);
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += w * pbase[j * pstep + i];
        wsum += w;
      }
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

// Two states given as tensors (the public merge): one wavefront per (token,
// head), lane owning D/64 consecutive columns; LSEs in base e.
template <int D, int DT>
__global__ __launch_bounds__(256) void merge2_kernel(Merge2Args a) {
  constexpr int PER = D / 64;
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (job >= (int64_t)a.T * a.H) return;
  const int64_t t = job / a.H, h = job - t * a.H;
  const float la = a.la[t * a.la_st + h * a.la_sh];
  const float lb = a.lb[t * a.lb_st + h * a.lb_sh];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f;
  if (m != -INFINITY) {
    wa = __expf(la - m);   // exactly 1 for the larger state; 0 for a -inf state
    wb = __expf(lb - m);
  }
  const float wsum = wa + wb;
  const float ia = wsum > 0.f ? wa / wsum : 0.f, ib = wsum > 0.f ? wb / wsum : 0.f;
  float va[PER], vb[PER];
  const int64_t ca = t * a.a_st + h * a.a_sh + lane * PER;
  const int64_t cb = t * a.b_st + h * a.b_sh + lane * PER;
  if (DT == AK_F32) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      va[i] = static_cast<const float*>(a.oa)[ca + i];
      vb[i] = static_cast<const float*>(a.ob)[cb + i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      va[i] = bf16_bits_to_f32(static_cast<const uint16_t*>(a.oa)[ca + i]);
      vb[i] = bf16_bits_to_f32(static_cast<const uint16_t*>(a.ob)[cb + i]);
    }
  }
  const int64_t co = t * a.o_st + h * a.o_sh + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    // a weight of 0 drops its state even where that state holds no finite data
    const float v = (ia > 0.f ? ia * va[i] : 0.f) + (ib > 0.f ? ib * vb[i] : 0.f);
    if (DT == AK_F32)
      static_cast<float*>(a.out)[co + i] = v;
    else
      static_cast<uint16_t*>(a.out)[co + i] = (uint16_t)f32_to_bf16_bits(v);
  }
  if (a.lse && lane == 0) a.lse[t * a.l_st + h * a.l_sh] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_merge2(const Merge2Args& a, int D, int dtype, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  const int64_t jobs = (int64_t)a.T * a.H;
  if (jobs <= 0) return hipSuccess;
  dim3 grid((unsigned)((jobs + 3) / 4));
  if (D == 64 && dtype == AK_F32) hipLaunchKernelGGL((merge2_kernel<64, AK_F32>), grid, dim3(256), 0, s, a);
  else if (D == 128 && dtype == AK_F32) hipLaunchKernelGGL((merge2_kernel<128, AK_F32>), grid, dim3(256), 0, s, a);
  else if (D == 64 && dtype == AK_BF16) hipLaunchKernelGGL((merge2_kernel<64, AK_BF16>), grid, dim3(256), 0, s, a);
  else if (D == 128 && dtype == AK_BF16) hipLaunchKernelGGL((merge2_kernel<128, AK_BF16>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int D, int out_dtype, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
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
