// Small-tile paged attention: up to 16 query rows of one (request, KV head)
// against one KV range -- the decode shape (G query heads x n queries <= 16),
// including one split of a split-KV partition.
//
// Method: mini-sglang "GPU attention", CPU reference paged attention (gather
// K/V through the page list, queries at the sequence end, GQA); "SGLang
// attention backend", "Where masks come from" (causal bit, window_left) and the
// head-group fusion figure of "Why metadata is built once per step" (query
// heads of one KV head share every K/V byte, so they form one tile).
//
// gfx950 mapping.  One workgroup (4 waves) per work item (or, for a stream-K
// plan, one persistent workgroup per equal share of the batch's decode KV, running
// the share's items one after the other); wave w takes the item's blocks w,
// w+4, ... (16 tokens for bf16 rows, 32 for fp8 rows).  The
// item's page ids are staged once in LDS.  Each wave runs a register pipeline:
// the K and V rows of the next block (bf16, D = 128) or next two blocks (fp8
// rows, D = 64) are in flight into spare register sets while block k is
// computed; the loads are unconditional (clamped addresses) so the compiler's
// memory-counter waits keep them in flight.
// Per block:
//   S^T (tokens x 16 rows) = K * Q^T   16x16x32 bf16 MFMA per 16 tokens; K rows
//     go straight from HBM into the MFMA A operand (each lane loads 16-32
//     contiguous bytes of one token row per step pair);
//   online softmax per row in base 2 (the scale carries log2(e)); a row lives in
//     the 4 lanes l%16 = row, so its max needs two xor-shuffles; the reference
//     max is raised only when a block exceeds it by more than 2^8;
//   O^T (D x 16 rows) += V^T * P^T   per 16 d: one 16x16x16 MFMA (16-token
//     blocks) or 16x16x32 MFMA (32-token blocks); P stays in the registers the
//     S^T tile produced it in, V is staged through LDS and read column-wise.
// The d order inside a 32-wide k-step is permuted identically for K and Q
// (contraction order is free), and the token order inside PV's k-steps follows
// the S^T register layout identically for P and V.  FP8 rows are widened to
// bf16 in registers (exact, two codes per instruction).
// The 4 waves' (m, l, O) states are merged in LDS at the end; the item writes
// the final output or, for a split, its normalised partial and base-2 LSE.

#include <climits>

#include "ak_launch.h"

namespace ak {

namespace {

constexpr int kWaves = 4;
constexpr float kLazy = 8.0f;    // raise the running max only beyond this margin (base 2)

template <int D>
__device__ __forceinline__ int dmap(int s, int g4) {
  // k-step s (0 .. D/32-1), lane group g4 (0..3) -> first of 8 d values
  return 64 * (s >> 1) + 16 * g4 + 8 * (s & 1);
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// D(16x16) += A(16x16) * B(16x16), bf16 inputs: lane l holds A[l%16][4*(l/16) .. +4],
// B[4*(l/16) .. +4][l%16]; D as for the 16x16x32 form.
__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int D, bool FP8>
struct Shape {
  // bf16 rows stream 16 tokens per wave block (halving the registers a block
  // needs), fp8 rows 32 tokens
  static constexpr int BLK = FP8 ? 32 : 16;
  static constexpr int NT = BLK / 16;                           // S^T tiles per block
  static constexpr int NSTEP = D / 32;                          // S^T k-steps
  static constexpr int NDT = D / 16;                            // O^T d-tiles
  static constexpr int EB = FP8 ? 1 : 2;                        // cache bytes per element
  static constexpr int KL = FP8 ? (NSTEP + 1) / 2 : NSTEP;      // 16-byte K loads per tile
  static constexpr int CPR = D * EB / 16;                       // 16-byte chunks per cache row
  static constexpr int TPI = 64 / CPR;                          // tokens per V load instruction
  static constexpr int VL = BLK / TPI;                          // V load instructions per block
  static constexpr int VROW = D + 4;                            // padded row of the V stage
  static constexpr int STAGE = BLK * VROW;                      // bf16 elements per wave stage
};

// s_waitcnt operand that waits for every outstanding vector memory operation
// (vmcnt 0; expcnt and lgkmcnt left at their maxima)
constexpr int kVmcntZero = 0x0F70;

// CPT consecutive fp32 values of one output row as bf16 (8 or 4 columns: one
// 16- or 8-byte store)
template <int CPT>
__device__ __forceinline__ void store_row_bf16(uint16_t* op, const float* o) {
  u32x4 w4;
#pragma unroll
  for (int cc = 0; cc < CPT; cc += 2) w4[cc / 2] = pack_bf16x2(o[cc], o[cc + 1]);
  if (CPT == 8) {
    *reinterpret_cast<u32x4*>(op) = w4;
  } else {
    *reinterpret_cast<u32x2*>(op) = u32x2{w4[0], w4[1]};
  }
}

// kv_load: one 16-byte K/V read, streaming (non-temporal) unless the batch's
// requests share pages
template <bool STREAM>
__device__ __forceinline__ u32x4 kv_load(const void* p) {
  if (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

// LDS of one workgroup: the waves' V stages, reused by the 4-wave combine
template <int D, bool FP8>
struct SmallLds {
  using S = Shape<D, FP8>;
  static constexpr int ORW = D + 4;          // floats per row of the combine buffer
  static constexpr int STAGE_BYTES = kWaves * S::STAGE * 2;
  static constexpr int COMB_BYTES = (2 * kWaves * 16 + kWaves * 16 * ORW) * 4;
  static constexpr int SMEM = STAGE_BYTES > COMB_BYTES ? STAGE_BYTES : COMB_BYTES;
};

// One work item (a KV range of one decode-shaped unit) on one workgroup.
// `smem`, `s_pages` and `s_last` are the workgroup's LDS, `tid` the thread's
// index in the workgroup; every thread returns from here with no barrier
// pending, and the caller separates two items run by one workgroup with a
// barrier (the next item reuses the LDS).
template <int D, bool FP8, bool STREAM, bool PERSIST>
__device__ __forceinline__ void small_item(const AttnArgs& a, const Item& it,
                                           unsigned char (&smem)[SmallLds<D, FP8>::SMEM],
                                           int32_t (&s_pages)[kSmallMaxPages], int32_t& s_last,
                                           int tid) {
  using S = Shape<D, FP8>;
  constexpr int BLK = S::BLK, NT = S::NT, NSTEP = S::NSTEP, NDT = S::NDT, EB = S::EB;
  constexpr int KL = S::KL, CPR = S::CPR, TPI = S::TPI, VL = S::VL, VROW = S::VROW;
  constexpr int ORW = SmallLds<D, FP8>::ORW;
  const Req rq = a.reqs[it.r];
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int G = a.G;

  // ---- the item's page ids, clamped into the pool, staged once in LDS (the
  // loop then reads them from LDS: no global index load sits between two
  // blocks' data loads in the in-order memory counter)
  const int32_t kv_begin = it.kv_begin, kv_end = it.kv_end;
  const int first_page = kv_begin >> a.log2B;
  {
    const int npages = ((kv_end - 1) >> a.log2B) - first_page + 1;   // <= kSmallMaxPages (plan)
    for (int i = tid; i < npages; i += 256)
      s_pages[i] = kv_page_id(a.kv_indices, rq.page_off, (first_page + i) << a.log2B, a.log2B,
                              a.num_pages);
  }

  // ---- this lane's query row (column of S^T and O^T)
  const bool rvalid = n16 < it.nrows;
  const int rho = it.row0 + n16;
  const int jq = rho / G;
  const int head = it.hk * G + (rho - jq * G);
  const int64_t qtok = (int64_t)rq.q_off + jq;
  const int qpos = rq.L - rq.n + jq;
  int row_lo = kv_begin, row_hi = kv_end;
  if (a.window >= 0) row_lo = max(row_lo, qpos - a.window);
  if (a.causal) row_hi = min(row_hi, qpos + 1);
  if (!rvalid) row_lo = row_hi = 0;
  // blocks inside [wave_lo_max, wave_hi_min) need no mask (rows past nrows are never written)
  int wave_lo_max = rvalid ? row_lo : INT_MIN, wave_hi_min = rvalid ? row_hi : INT_MAX;
#pragma unroll
  for (int k = 1; k < 16; k <<= 1) {
    wave_lo_max = max(wave_lo_max, __shfl_xor(wave_lo_max, k, 64));
    wave_hi_min = min(wave_hi_min, __shfl_xor(wave_hi_min, k, 64));
  }

  bf16x8 qop[NSTEP];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + qtok * a.q_st + (int64_t)head * a.q_sh;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (rvalid) {
        qop[s] = *reinterpret_cast<const bf16x8*>(qp + dmap<D>(s, g4));
      } else {
        qop[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      }
    }
  }

  f32x4 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.score_scale;

  const int nblk = (kv_end - kv_begin + BLK - 1) / BLK;
  const int nloc = wave < nblk ? (nblk - wave + kWaves - 1) / kWaves : 0;   // this wave's blocks
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)it.hk * a.k_sh * EB;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)it.hk * a.v_sh * EB;
  const int64_t kps = a.k_sp * EB, kbs = a.k_sb * EB, vps = a.v_sp * EB, vbs = a.v_sb * EB;
  __bf16* vs = reinterpret_cast<__bf16*>(smem) + wave * S::STAGE;

  struct Regs {               // one block's K operands and V rows, as loaded
    u32x4 k[NT][KL];
    u32x4 v[VL];
  };

  // cache row of token t (clamped to the item) -> byte offset of its page/slot
  auto row_off = [&](int t, int64_t ps, int64_t bs) -> int64_t {
    t = min(t, kv_end - 1);
    return kv_row_offset(s_pages[kv_page_index(0, t, a.log2B) - first_page], t, a.log2B, ps, bs);
  };
  // issue the HBM reads of local block k (rows past the item are clamped, so a
  // prefetch past the last block reads valid memory).  When every K/V byte is
  // read once per run the loads are non-temporal: the streamed rows do not evict
  // the page table, Q and partials from the caches (measured: 198 -> 181 us on
  // the 64-request decode batch).  When requests share pages (a common prefix)
  // ordinary loads let the later readers of a page hit the caches.
  auto issue = [&](Regs& rg, int k) {
    const int tb = kv_begin + (wave + kWaves * k) * BLK;
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      const char* row = kbase + row_off(tb + 16 * T + n16, kps, kbs);
#pragma unroll
      for (int p = 0; p < KL; ++p) {
        const int d0 = FP8 ? 64 * p + 16 * g4 : dmap<D>(p, g4);
        rg.k[T][p] = kv_load<STREAM>(row + d0 * EB);
      }
    }
    const int cslot = lane % CPR;
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int r = i * TPI + lane / CPR;
      rg.v[i] = kv_load<STREAM>(vbase + row_off(tb + r, vps, vbs) + cslot * 16);
    }
  };
  // attention over local block k held in `rg`
  auto compute = [&](const Regs& rg, int k) {
    const int tb = kv_begin + (wave + kWaves * k) * BLK;
    // ---- the block's V rows into the wave's stage (bf16; 8-byte pieces, rows are 8-byte aligned)
    {
      const int cslot = lane % CPR;
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int r = i * TPI + lane / CPR;
        u32x2* dst = reinterpret_cast<u32x2*>(vs + r * VROW + cslot * (16 / EB));
        if (FP8) {
          const u32x4 lo = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(rg.v[i][0], rg.v[i][1]));
          const u32x4 hi = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(rg.v[i][2], rg.v[i][3]));
          dst[0] = u32x2{lo[0], lo[1]};
          dst[1] = u32x2{lo[2], lo[3]};
          dst[2] = u32x2{hi[0], hi[1]};
          dst[3] = u32x2{hi[2], hi[3]};
        } else {
          dst[0] = u32x2{rg.v[i][0], rg.v[i][1]};
          dst[1] = u32x2{rg.v[i][2], rg.v[i][3]};
        }
      }
    }
    // ---- S^T = K Q^T
    f32x4 sacc[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      sacc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        bf16x8 kop;
        if (FP8) {
          const u32x4& w = rg.k[T][s >> 1];
          kop = (s & 1) ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
        } else {
          kop = __builtin_bit_cast(bf16x8, rg.k[T][s]);
        }
        sacc[T] = mfma16(kop, qop[s], sacc[T]);
      }
    }
    // ---- online softmax (base 2), rows = lane % 16; element i of tile T is token 16T + 4g4 + i
    if ((tb < wave_lo_max) | (tb + BLK > wave_hi_min)) {
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tb + 16 * T + 4 * g4 + i;
          if (!((t >= row_lo) & (t < row_hi))) sacc[T][i] = -INFINITY;
        }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int T = 0; T < NT; ++T)
      mb = fmaxf(mb, fmaxf(fmaxf(sacc[T][0], sacc[T][1]), fmaxf(sacc[T][2], sacc[T][3])));
    mb = fmaxf(mb, shfl_xor_f(mb, 16));
    mb = fmaxf(mb, shfl_xor_f(mb, 32)) * c;
    const float m_new = (mb > m_run + kLazy) ? mb : m_run;
    if (__any(m_new != m_run)) {
      // rows whose reference stays put keep alpha = 1 (this also covers rows that
      // have seen no visible key yet: -inf - -inf would be NaN); a row leaving
      // -inf gets exp2(-inf) = 0
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha;
      m_run = m_new;
    }
    const float msub = m_run == -INFINITY ? 0.f : m_run;
    float p[NT][4];
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[T][i] = fast_exp2(__builtin_fmaf(sacc[T][i], c, -msub));
        l_run += p[T][i];
      }
    // the stage is private to this wave: make its writes visible to all lanes
    // (and keep the compiler from moving LDS accesses across this point)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const uint16_t* vsu = reinterpret_cast<const uint16_t*>(vs);
    if (NT == 2) {
      // ---- O^T += V^T P^T (16x16x32); k-slot 8*g4 + jj <-> token 16*(jj/4) + 4*g4 + jj%4
      u32x4 pw;
      pw[0] = pack_bf16x2(p[0][0], p[0][1]);
      pw[1] = pack_bf16x2(p[0][2], p[0][3]);
      pw[2] = pack_bf16x2(p[NT - 1][0], p[NT - 1][1]);
      pw[3] = pack_bf16x2(p[NT - 1][2], p[NT - 1][3]);
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + n16;
        u32x4 vw;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int jj0 = 2 * h, jj1 = 2 * h + 1;
          const int t0 = 16 * (jj0 >> 2) + 4 * g4 + (jj0 & 3);
          const int t1 = 16 * (jj1 >> 2) + 4 * g4 + (jj1 & 3);
          vw[h] = (uint32_t)vsu[t0 * VROW + d] | ((uint32_t)vsu[t1 * VROW + d] << 16);
        }
        oacc[dt] = mfma16(__builtin_bit_cast(bf16x8, vw), pop, oacc[dt]);
      }
    } else {
      // ---- O^T += V^T P^T (16x16x16); k-slot 4*g4 + jj <-> token 4*g4 + jj
      const u32x2 pw{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3])};
      const s16x4 pop = __builtin_bit_cast(s16x4, pw);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + n16;
        const int t0 = 4 * g4;
        const u32x2 vw{(uint32_t)vsu[t0 * VROW + d] | ((uint32_t)vsu[(t0 + 1) * VROW + d] << 16),
                       (uint32_t)vsu[(t0 + 2) * VROW + d] | ((uint32_t)vsu[(t0 + 3) * VROW + d] << 16)};
        oacc[dt] = mfma16k16(__builtin_bit_cast(s16x4, vw), pop, oacc[dt]);
      }
    }
    // the next block's stage writes must not pass this block's reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  __syncthreads();   // page table staged

  // ---- register pipeline over this wave's blocks: the reads of the next one
  // (bf16 rows, D = 128) or two (otherwise) blocks are in flight while block k is
  // computed.  Reads are issued unconditionally, so the compiler's memory-counter
  // waits stay exact: each compute waits only for its own block.  (A third
  // register set does not fit beside bf16 D = 128 operands without spills.)
  if (nloc > 0) {
    // (the persistent loop of a stream-K launch holds a little more live state,
    // which two sets leave room for with fp8 rows at D = 128)
    constexpr bool kThree = (FP8 || D == 64) && !(PERSIST && FP8 && D == 128);
    Regs ra, rb, rc;
    issue(ra, 0);
    if (kThree) {
      issue(rb, 1);
      for (int k = 0;; k += 3) {
        issue(rc, k + 2);
        compute(ra, k);
        if (k + 1 >= nloc) break;
        issue(ra, k + 3);
        compute(rb, k + 1);
        if (k + 2 >= nloc) break;
        issue(rb, k + 4);
        compute(rc, k + 2);
        if (k + 3 >= nloc) break;
      }
    } else {
      for (int k = 0;; k += 2) {
        issue(rb, k + 1);
        compute(ra, k);
        if (k + 1 >= nloc) break;
        issue(ra, k + 2);
        compute(rb, k + 1);
        if (k + 2 >= nloc) break;
      }
    }
  }

  // ---- combine the 4 waves' states
  float l_tot = l_run + shfl_xor_f(l_run, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  __syncthreads();
  float* cm = reinterpret_cast<float*>(smem);
  float* cl = cm + kWaves * 16;
  float* co = cl + kWaves * 16;
  if (g4 == 0) {
    cm[wave * 16 + n16] = m_run;
    cl[wave * 16 + n16] = l_tot;
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) co[(wave * 16 + n16) * ORW + 16 * dt + 4 * g4 + i] = oacc[dt][i];
  __syncthreads();

  constexpr int CPT = D / 16;   // columns per thread
  const int row = tid >> 4;
  const int c0 = (tid & 15) * CPT;
  const bool active = row < it.nrows;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cm[w * 16 + (active ? row : 0)]);
  float o[CPT];
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) o[cc] = 0.f;
  float lse2 = -INFINITY;
  if (active && M != -INFINITY) {
    float den = 0.f;
    float wt[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wt[w] = fast_exp2(cm[w * 16 + row] - M);
      den += wt[w] * cl[w * 16 + row];
    }
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) o[cc] += wt[w] * co[(w * 16 + row) * ORW + c0 + cc];
    const float inv = a.v_scale / den;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) o[cc] *= inv;
    lse2 = M + log2f(den);
  }
  if (it.pbase < 0) {   // an unsplit unit: the final output
    if (!active) return;
    const int rrho = it.row0 + row;
    const int rj = rrho / G;
    const int rhead = it.hk * G + (rrho - rj * G);
    const int64_t rtok = (int64_t)rq.q_off + rj;
    store_row_bf16<CPT>(static_cast<uint16_t*>(a.out) + rtok * a.o_st + (int64_t)rhead * a.o_sh + c0, o);
    if (a.lse && (tid & 15) == 0) a.lse[rtok * a.l_st + (int64_t)rhead * a.l_sh] = lse2 * kLn2;
    return;
  }
  // ---- a split unit's parts are merged by whichever workgroup finishes last.
  // Each part publishes its partial rows with device-coherent stores (scope
  // "agent": they bypass the non-coherent per-XCD L2 instead of needing a whole
  // L2 write-back), waits until they are complete, then counts itself in; the
  // one that completes the count reads every part with device-coherent loads
  // and merges them in part order, so the result does not depend on which
  // workgroup that is.  Nothing waits on another workgroup.  The counter is
  // reset for the next run.
  if (it.merge0 < 0) {   // split, but merged by the merge kernel
    if (!active) return;
    const int64_t prow = (int64_t)it.pbase + row;
    float* pp = a.part_o + prow * D + c0;
#pragma unroll
    for (int cc = 0; cc < CPT; cc += 4)
      *reinterpret_cast<f32x4*>(pp + cc) = f32x4{o[cc], o[cc + 1], o[cc + 2], o[cc + 3]};
    if ((tid & 15) == 0) a.part_lse[prow] = lse2;
    return;
  }
  if (active) {
    const int64_t prow = (int64_t)it.pbase + row;
    float* pp = a.part_o + prow * D + c0;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc)
      __hip_atomic_store(pp + cc, o[cc], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((tid & 15) == 0)
      __hip_atomic_store(a.part_lse + prow, lse2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(kVmcntZero);   // this thread's partial stores are complete
  __syncthreads();
  if (tid == 0) {
    const int parts = a.merges[it.merge0].count;
    s_last = __hip_atomic_fetch_add(a.counters + it.merge0, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == parts - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (tid == 0)
    __hip_atomic_store(a.counters + it.merge0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!active) return;
  // The row's 16 lanes read its parts' LSEs 16 at a time and reduce the max in
  // their group; lane j of the group then holds part (chunk + j)'s weight, which
  // the weighted sum takes by a lane broadcast, summing the parts in order with
  // four part rows in flight (the same arithmetic as one part at a time).
  const MergeJob jb = a.merges[it.merge0 + row];
  const int sub = tid & 15;          // lane within the row's group
  const int grp = tid & 48;          // first lane of the group in the wave
  auto lse_of = [&](int s) {
    return __hip_atomic_load(a.part_lse + jb.pfirst + (int64_t)s * jb.pstride, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  };
  float m = -INFINITY;
  for (int s = sub; s < jb.count; s += 16) m = fmaxf(m, lse_of(s));
#pragma unroll
  for (int k = 8; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) o[cc] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s0 = 0; s0 < jb.count; s0 += 16) {
      const int n = min(16, jb.count - s0);
      const float wl = sub < n ? exp2f(lse_of(s0 + sub) - m) : 0.f;   // -inf parts weigh 0
      auto row_of = [&](int s) { return a.part_o + (jb.pfirst + (int64_t)s * jb.pstride) * D + c0; };
      int j = 0;
      for (; j + 4 <= n; j += 4) {
        float v[4][CPT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float* po = row_of(s0 + j + u);
#pragma unroll
          for (int cc = 0; cc < CPT; ++cc)
            v[u][cc] = __hip_atomic_load(po + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = __shfl(wl, grp + j + u, 64);
#pragma unroll
          for (int cc = 0; cc < CPT; ++cc) o[cc] += w * v[u][cc];
          wsum += w;
        }
      }
      for (; j < n; ++j) {
        const float w = __shfl(wl, grp + j, 64);
        const float* po = row_of(s0 + j);
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc)
          o[cc] += w * __hip_atomic_load(po + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wsum += w;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) o[cc] *= inv;
  store_row_bf16<CPT>(static_cast<uint16_t*>(a.out) + (int64_t)jb.token * a.o_st + (int64_t)jb.head * a.o_sh + c0, o);
  if (a.lse && (tid & 15) == 0)
    a.lse[(int64_t)jb.token * a.l_st + (int64_t)jb.head * a.l_sh] =
        wsum > 0.f ? (m + log2f(wsum)) * kLn2 : -INFINITY;
}

// One workgroup per item, or (PERSIST, stream-K plans) one persistent
// workgroup per share running its items in order.
template <int D, bool FP8, bool STREAM, bool PERSIST>
__global__ __launch_bounds__(256, 2) void attn_small_kernel(AttnArgs a) {
  __shared__ __align__(16) unsigned char smem[SmallLds<D, FP8>::SMEM];
  __shared__ int32_t s_pages[kSmallMaxPages];
  __shared__ int32_t s_last;   // this workgroup finished its unit's last part
  if constexpr (PERSIST) {
    const int first = a.wg_first[blockIdx.x], last = a.wg_first[blockIdx.x + 1];
    for (int i = first; i < last; ++i) {
      const Item it = a.items[i];
      // the thread index is re-derived per item from a value the compiler cannot
      // see through, so nothing computed from it is hoisted out of the loop and
      // kept live across items (that would cost the item body its registers)
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      small_item<D, FP8, STREAM, true>(a, it, smem, s_pages, s_last, tid);
      __syncthreads();   // the next item reuses the LDS
    }
  } else {
    const Item it = a.items[blockIdx.x];
    if (it.nrows == 0) return;   // padding item (uniform over the workgroup)
    small_item<D, FP8, STREAM, false>(a, it, smem, s_pages, s_last, (int)threadIdx.x);
  }
}

}  // namespace

hipError_t launch_attn_small(const AttnArgs& a, int n_items, int D, int kv_dtype, bool shared_pages,
                             int n_wg, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  if (n_items <= 0) return hipSuccess;
  const bool persist = n_wg > 0;
  dim3 grid((unsigned)(persist ? n_wg : n_items));
#define AK_SMALL_LAUNCH(DD, F8, ST, PE) \
  hipLaunchKernelGGL((attn_small_kernel<DD, F8, ST, PE>), grid, dim3(256), 0, s, a)
#define AK_SMALL_CASE(DD, F8)                                                 \
  if (D == DD && kv_dtype == (F8 ? AK_FP8_E4M3 : AK_BF16)) {                  \
    if (persist) {                                                            \
      if (shared_pages)                                                       \
        AK_SMALL_LAUNCH(DD, F8, false, true);                                 \
      else                                                                    \
        AK_SMALL_LAUNCH(DD, F8, true, true);                                  \
    } else {                                                                  \
      if (shared_pages)                                                       \
        AK_SMALL_LAUNCH(DD, F8, false, false);                                \
      else                                                                    \
        AK_SMALL_LAUNCH(DD, F8, true, false);                                 \
    }                                                                         \
    return hipGetLastError();                                                 \
  }
  AK_SMALL_CASE(128, false)
  AK_SMALL_CASE(64, false)
  AK_SMALL_CASE(128, true)
  AK_SMALL_CASE(64, true)
#undef AK_SMALL_CASE
#undef AK_SMALL_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace ak
