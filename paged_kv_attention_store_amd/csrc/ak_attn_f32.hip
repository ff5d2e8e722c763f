// fp32 paged attention on the vector ALU (no fp32 MFMA needed at the sizes the
// fp32 path serves).  Handles any work item: up to 128 rows of one
// (request, KV head) against one KV range.
//
// Method: mini-sglang "GPU attention", CPU reference paged attention; masks as
// in "SGLang attention backend", "Where masks come from".
//
// Each wave takes rows w, w+4, ... of the item.  For a row, 64 keys at a time:
// lane i scores key tb+i against the row's query (held in LDS and broadcast),
// the wave takes the block max and rescales its running state (base-2 online
// softmax), and each lane accumulates D/64 output columns over the block's
// keys with the probabilities broadcast by shuffles.

#include "ak_launch.h"

namespace ak {

namespace {

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int PER = D / 64;
  __shared__ __align__(16) float qs[4][D];
  const Item it = a.items[blockIdx.x];
  if (it.nrows == 0) return;   // padding item (uniform over the workgroup)
  const Req rq = a.reqs[it.r];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int G = a.G;
  const float* kc = static_cast<const float*>(a.k_cache) + (int64_t)it.hk * a.k_sh;
  const float* vc = static_cast<const float*>(a.v_cache) + (int64_t)it.hk * a.v_sh;

  for (int rl = wave; rl < it.nrows; rl += 4) {
    const int rho = it.row0 + rl;
    const int jq = rho / G;
    const int head = it.hk * G + (rho - jq * G);
    const int64_t qtok = (int64_t)rq.q_off + jq;
    const int qpos = rq.L - rq.n + jq;
    int lo = it.kv_begin, hi = it.kv_end;
    if (a.window >= 0) lo = max(lo, qpos - a.window);
    if (a.causal) hi = min(hi, qpos + 1);
    const float* qp = static_cast<const float*>(a.q) + qtok * a.q_st + (int64_t)head * a.q_sh;
#pragma unroll
    for (int i = 0; i < PER; ++i) qs[wave][lane + 64 * i] = qp[lane + 64 * i];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the row's query is in LDS

    float m = -INFINITY, l = 0.f, o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    for (int tb = lo; tb < hi; tb += 64) {
      const int t = tb + lane;
      const bool vis = t < hi;
      const int tc = vis ? t : hi - 1;
      const int32_t page = kv_page_id(a.kv_indices, rq.page_off, tc, a.log2B, a.num_pages);
      const float* kr = kc + kv_row_offset(page, tc, a.log2B, a.k_sp, a.k_sb);
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + d);
        const f32x4 qv = *reinterpret_cast<const f32x4*>(&qs[wave][d]);
        s = fmaf(kv[0], qv[0], s);
        s = fmaf(kv[1], qv[1], s);
        s = fmaf(kv[2], qv[2], s);
        s = fmaf(kv[3], qv[3], s);
      }
      s = vis ? s * a.score_scale : -INFINITY;
      float mb = s;
#pragma unroll
      for (int k = 32; k >= 1; k >>= 1) mb = fmaxf(mb, shfl_xor_f(mb, k));
      const float m_new = fmaxf(m, mb);           // finite: key tb is visible
      const float alpha = fast_exp2(m - m_new);
      const float p = fast_exp2(s - m_new);
      float ps = p;
#pragma unroll
      for (int k = 32; k >= 1; k >>= 1) ps += shfl_xor_f(ps, k);
      l = l * alpha + ps;
      m = m_new;
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] *= alpha;
      const int nt = min(64, hi - tb);
      const int64_t voff = kv_row_offset(page, tc, a.log2B, a.v_sp, a.v_sb);
      for (int k = 0; k < nt; ++k) {
        const float pk = __shfl(p, k, 64);
        const int64_t vo = __shfl(voff, k, 64);
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] = fmaf(pk, vc[vo + lane + 64 * i], o[i]);
      }
    }
    const bool any = l > 0.f;
    const float inv = any ? a.v_scale / l : 0.f;
    const float lse2 = any ? m + log2f(l) : -INFINITY;
    if (it.pbase < 0) {
      float* op = static_cast<float*>(a.out) + qtok * a.o_st + (int64_t)head * a.o_sh;
#pragma unroll
      for (int i = 0; i < PER; ++i) op[lane + 64 * i] = o[i] * inv;
      if (a.lse && lane == 0) a.lse[qtok * a.l_st + (int64_t)head * a.l_sh] = lse2 * kLn2;
    } else {
      const int64_t prow = (int64_t)it.pbase + rl;
#pragma unroll
      for (int i = 0; i < PER; ++i) a.part_o[prow * D + lane + 64 * i] = o[i] * inv;
      if (lane == 0) a.part_lse[prow] = lse2;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // qs reused by the next row
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int n_items, int D, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  if (n_items <= 0) return hipSuccess;
  dim3 grid((unsigned)n_items);
  if (D == 128) {
    hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(256), 0, s, a);
  } else if (D == 64) {
    hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ak
