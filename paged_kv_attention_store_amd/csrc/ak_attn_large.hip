// Large-tile paged attention: 128 query rows of one (request, KV head) -- the
// extend/prefill shape, where the rows are (query token, head of the group)
// pairs packed token-major so GQA heads share every K/V tile.
//
// Method: mini-sglang "GPU attention", CPU reference paged attention; causal
// mask aligned to the sequence end; "SGLang attention backend", "Where masks
// come from" (causal bit and window_left, never a materialised mask); the GQA
// head-group fusion figure of "Why metadata is built once per step".
//
// gfx950 mapping.  One workgroup of 4 waves per 128-row tile, wave w owning rows
// 32w .. 32w+31.  The KV range is walked in 64-token blocks:
//   * the block's K rows are gathered through the page table into LDS (16-byte
//     chunks, XOR-swizzled by token so MFMA operand reads are conflict-free);
//     V rows are gathered and written transposed (d-major, 4-token groups
//     XOR-swizzled by d) so PV operands are two 8-byte reads;
//   * S^T (64 tokens x 32 rows) = K Q^T with 32x32x16 bf16 MFMA, Q held in
//     registers for the whole tile;
//   * online softmax per row in base 2: a row lives in lanes n and n+32, so the
//     block max needs one xor-shuffle;
//   * O^T (D x 32 rows) += V^T P^T, P taken from the S^T registers as produced.
// FP8 caches are widened to bf16 while staging (exact).

#include "ak_launch.h"

namespace ak {

namespace {

constexpr int kKB = 64;       // tokens per KV block
constexpr int kRows = 128;    // rows per tile

template <int D>
__device__ __forceinline__ int k_pos(int t, int c) {
  // position of 16-byte chunk c of token t's K row in the staged tile (in chunks)
  return t * (D / 8) + (D == 128 ? (c ^ (t & 15)) : (c ^ ((t >> 1) & 7)));
}

__device__ __forceinline__ int vt_pos(int d, int tg) {
  // position (in bf16) of 4-token group tg of column d in the transposed V tile
  return d * kKB + ((tg ^ (d & 15)) << 2);
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void attn_large_kernel(AttnArgs a) {
  constexpr int NS = D / 16;      // S^T k-steps (16 d each)
  constexpr int NDT = D / 32;     // O^T d-tiles (32 d each)
  constexpr int CPR = D / 8;      // 16-byte bf16 chunks per row
  __shared__ __align__(16) __bf16 ks[kKB * D];
  __shared__ __align__(16) __bf16 vt[D * kKB];
  __shared__ int64_t s_koff[kKB], s_voff[kKB];

  const Item it = a.items[blockIdx.x];
  const Req rq = a.reqs[it.r];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n32 = lane & 31;
  const int hf = lane >> 5;
  const int G = a.G;

  // ---- this lane's row
  const int rl = wave * 32 + n32;
  const bool rvalid = rl < it.nrows;
  const int rho = it.row0 + rl;
  const int jq = rho / G;
  const int head = it.hk * G + (rho - jq * G);
  const int64_t qtok = (int64_t)rq.q_off + jq;
  const int qpos = rq.L - rq.n + jq;
  int row_lo = it.kv_begin, row_hi = it.kv_end;
  if (a.window >= 0) row_lo = max(row_lo, qpos - a.window);
  if (a.causal) row_hi = min(row_hi, qpos + 1);
  if (!rvalid) row_lo = row_hi = 0;

  bf16x8 qop[NS];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + qtok * a.q_st + (int64_t)head * a.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qop[s] = rvalid ? *reinterpret_cast<const bf16x8*>(qp + 16 * s + 8 * hf)
                      : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int ebytes = FP8 ? 1 : 2;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)it.hk * a.k_sh * ebytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)it.hk * a.v_sh * ebytes;
  const int32_t bmask = (1 << a.log2B) - 1;
  const int tid = threadIdx.x;

  for (int tb = it.kv_begin; tb < it.kv_end; tb += kKB) {
    __syncthreads();   // the previous block's LDS reads are done
    if (tid < kKB) {
      const int t = min(tb + tid, it.kv_end - 1);
      const int64_t page = kv_page(a.kv_indices, rq.page_off, t, a.log2B, a.num_pages);
      const int64_t slot = t & bmask;
      s_koff[tid] = (page * a.k_sp + slot * a.k_sb) * ebytes;
      s_voff[tid] = (page * a.v_sp + slot * a.v_sb) * ebytes;
    }
    __syncthreads();
    // ---- K: 64 rows x CPR chunks of 16 bytes (bf16) into the swizzled tile
    if (FP8) {
      // source chunk = 16 codes = two bf16 chunks
      for (int q = tid; q < kKB * (CPR / 2); q += 256) {
        const int t = q / (CPR / 2), c = q % (CPR / 2);
        const u32x4 w = *reinterpret_cast<const u32x4*>(kbase + s_koff[t] + c * 16);
        *reinterpret_cast<bf16x8*>(ks + 8 * k_pos<D>(t, 2 * c)) = e4m3x8_to_bf16x8(w[0], w[1]);
        *reinterpret_cast<bf16x8*>(ks + 8 * k_pos<D>(t, 2 * c + 1)) = e4m3x8_to_bf16x8(w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int q = tid; q < kKB * CPR; q += 256) {
        const int t = q / CPR, c = q % CPR;
        const u32x4 w = *reinterpret_cast<const u32x4*>(kbase + s_koff[t] + c * 16);
        *reinterpret_cast<u32x4*>(ks + 8 * k_pos<D>(t, c)) = w;
      }
    }
    // ---- V: thread (u = 4-token group, c = 8-column chunk) -> 8 transposed 8-byte writes
    for (int q = tid; q < (kKB / 4) * CPR; q += 256) {
      const int u = q & 15, c = q >> 4;
      uint32_t e[4][4];   // e[token][dword] = bf16 pairs of columns 8c .. 8c+7
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const char* src = vbase + s_voff[4 * u + j];
        if (FP8) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(src + c * 8);
          const u32x4 b = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(w[0], w[1]));
#pragma unroll
          for (int k = 0; k < 4; ++k) e[j][k] = b[k];
        } else {
          const u32x4 w = *reinterpret_cast<const u32x4*>(src + c * 16);
#pragma unroll
          for (int k = 0; k < 4; ++k) e[j][k] = w[k];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = 8 * c + i;
        const int sh = (i & 1) * 16;
        const uint32_t v0 = (e[0][i >> 1] >> sh) & 0xffffu, v1 = (e[1][i >> 1] >> sh) & 0xffffu;
        const uint32_t v2 = (e[2][i >> 1] >> sh) & 0xffffu, v3 = (e[3][i >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<u32x2*>(vt + vt_pos(d, u)) = u32x2{v0 | (v1 << 16), v2 | (v3 << 16)};
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: two 32-token tiles
    f32x16 sacc[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[T][i] = 0.f;
      const int t = 32 * T + n32;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(ks + 8 * k_pos<D>(t, 2 * s + hf));
        sacc[T] = mfma32(kop, qop[s], sacc[T]);
      }
    }
    // ---- online softmax; element i of tile T is token 32T + 8(i/4) + 4hf + i%4
    float mb = -INFINITY;
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = tb + 32 * T + 8 * (i >> 2) + 4 * hf + (i & 3);
        const bool vis = (t >= row_lo) & (t < row_hi);
        sacc[T][i] = vis ? sacc[T][i] * a.score_scale : -INFINITY;
        mb = fmaxf(mb, sacc[T][i]);
      }
    mb = fmaxf(mb, shfl_xor_f(mb, 32));
    const float m_new = fmaxf(m_run, mb);
    float alpha = 1.f, psum = 0.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[T][i] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[T][i] = exp2f(sacc[T][i] - m_new);
          psum += sacc[T][i];
        }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    // ---- O^T += V^T P^T over four 16-token k-steps
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int T = kk >> 1, i0 = 8 * (kk & 1);
      u32x4 pw;
#pragma unroll
      for (int h = 0; h < 4; ++h) pw[h] = pack_bf16x2(sacc[T][i0 + 2 * h], sacc[T][i0 + 2 * h + 1]);
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 32 * dt + n32;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vt + vt_pos(d, 4 * kk + hf));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vt + vt_pos(d, 4 * kk + 2 + hf));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[dt] = mfma32(vop, pop, oacc[dt]);
      }
    }
  }

  // ---- finalise: O^T element i of tile dt is column d = 32dt + 8(i/4) + 4hf + i%4
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (!rvalid) return;
  const bool any = l_tot > 0.f;
  const float inv = any ? a.v_scale / l_tot : 0.f;
  const float lse2 = any ? m_run + log2f(l_tot) : -INFINITY;
  if (it.pbase < 0) {
    uint16_t* op = static_cast<uint16_t*>(a.out) + qtok * a.o_st + (int64_t)head * a.o_sh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * hf;
        const u32x2 w{pack_bf16x2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                      pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
    if (a.lse && hf == 0) a.lse[qtok * a.l_st + (int64_t)head * a.l_sh] = lse2 * kLn2;
  } else {
    const int64_t prow = (int64_t)it.pbase + rl;
    float* pp = a.part_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * hf;
        *reinterpret_cast<f32x4*>(pp + d0) =
            f32x4{oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                  oacc[dt][4 * g + 3] * inv};
      }
    if (hf == 0) a.part_lse[prow] = lse2;
  }
}

}  // namespace

hipError_t launch_attn_large(const AttnArgs& a, int n_items, int D, int kv_dtype, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  dim3 grid((unsigned)n_items);
  if (D == 128 && kv_dtype == AK_BF16) {
    hipLaunchKernelGGL((attn_large_kernel<128, false>), grid, dim3(256), 0, s, a);
  } else if (D == 64 && kv_dtype == AK_BF16) {
    hipLaunchKernelGGL((attn_large_kernel<64, false>), grid, dim3(256), 0, s, a);
  } else if (D == 128 && kv_dtype == AK_FP8_E4M3) {
    hipLaunchKernelGGL((attn_large_kernel<128, true>), grid, dim3(256), 0, s, a);
  } else if (D == 64 && kv_dtype == AK_FP8_E4M3) {
    hipLaunchKernelGGL((attn_large_kernel<64, true>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ak
