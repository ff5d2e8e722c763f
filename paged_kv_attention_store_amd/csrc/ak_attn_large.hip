// Large-tile paged attention: 256 query rows of one (request, KV head) -- the
// extend/prefill shape, where the rows are (query token, head of the group)
// pairs packed token-major so GQA heads share every K/V tile.
//
// Method: mini-sglang "GPU attention", CPU reference paged attention; causal
// mask aligned to the sequence end; "SGLang attention backend", "Where masks
// come from" (causal bit and window_left, never a materialised mask); the GQA
// head-group fusion figure of "Why metadata is built once per step".
//
// gfx950 mapping.  One workgroup of 8 waves per 256-row segment, wave w owning
// rows 32w .. 32w+31 (one workgroup per CU: <= 256 registers per lane, up to
// 128 KB of LDS).  The KV range is walked in 128-token blocks whose K and V rows
// are copied HBM -> LDS by the load-to-LDS path while the previous block is
// computed.  Two staging policies share one tile loop (`LargeTile`):
//   * bf16 caches: each block is copied straight into the compute layout, two
//     block buffers alternating;
//   * fp8 caches: each block is copied as it sits in the cache (half the bytes)
//     into one of two staging buffers and widened exactly to bf16 into the one
//     compute tile once per block (one more barrier per block).
// Per block and 32-token tile: S^T = K Q^T and O^T += V^T P^T on the 32x32x16
// bf16 MFMA with Q in registers, online softmax in base 2 with the scale folded
// into one FMA per score, the running max raised only when a tile exceeds it by
// more than 2^8 (the normalisation is exact for any reference value; this only
// skips rescaling O, and probabilities stay below 2^8).

#include "ak_launch.h"

namespace ak {

namespace {

constexpr float kLazy = 8.0f;    // raise the running max only beyond this margin (base 2)
constexpr float kLazyP = 256.0f; // 2^kLazy
constexpr int kDmaKB = 128;      // tokens per KV block
constexpr int kLgkmcntZero = 0xC07F;   // s_waitcnt lgkmcnt(0), other counters unconstrained

// Compute-layout swizzles (bf16 tiles in LDS):
//   * K rows: 16-byte chunk c of token t sits at slot c ^ kswz(t) (conflict-free
//     16-byte operand reads for S^T = K Q^T);
//   * V rows stay token-major (chunk c at slot c ^ vswz(t)); the V^T operand of
//     O^T += V^T P^T comes from two transposing 8-byte reads (ds_read_b64_tr_b16),
//     each giving a lane one column of V over 4 consecutive tokens.
template <int D>
__device__ __forceinline__ int kswz(int t) {
  return D == 128 ? (t & 15) : ((t >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int t) {
  return D == 128 ? 4 * (t & 3) : 4 * ((t >> 1) & 1);
}

// The per-wave state and tile loop of one 256-row segment, whatever the staging.
// A block of KB tokens is NT = KB/32 tiles.  Blocks that lie inside every row
// bound of the wave take the fast path: no masks, and the S^T MFMAs of tile T+1
// are issued before the softmax of tile T, so the matrix core works on the next
// tile while the vector ALU exponentiates this one (the two waves of a SIMD,
// kept in step by the block barrier, would otherwise both wait on the same
// unit).  Other blocks go tile by tile with masks, skipping tiles no row of the
// wave can see.
template <int D, int KB>
struct LargeTile {
  static constexpr int NS = D / 16;          // S^T k-steps (16 d each)
  static constexpr int NDT = D / 32;         // O^T d-tiles (32 d each)
  static constexpr int CPR = D / 8;          // 16-byte chunks per bf16 row
  static constexpr int NT = KB / 32;         // 32-token tiles per block
  static constexpr int TILE = KB * D;        // bf16 elements of one K or V block
  static constexpr int NI = KB * CPR / (64 * 8);   // bf16 load-to-LDS instructions per wave per block
  static_assert(NI >= 1 && NI * 64 * 8 == KB * CPR, "tile shape");

  const AttnArgs& a;
  const Item it;
  const Req rq;
  const int wave, lane, n32, hf, G, lgG;
  int row_lo, row_hi;                  // keys this lane's row sees
  int lo_max, hi_min, lo_min, hi_max;  // the wave's common / union key bounds
  bool wave_active;
  bf16x8 qop[NS];
  f32x16 oacc[NDT];
  float m_run, l_run;
  const float c;
  int vr_tok, vr_sw, vr_col;           // V^T operand read geometry of this lane

  __device__ __forceinline__ LargeTile(const AttnArgs& a_, const Item& it_, const Req& rq_, int wave_,
                                       int lane_)
      : a(a_), it(it_), rq(rq_), wave(wave_), lane(lane_), n32(lane_ & 31), hf(lane_ >> 5), G(a_.G),
        lgG(__builtin_ctz(a_.G)), c(a_.score_scale) {
    // ---- this lane's row (G is a power of two)
    const int rl = wave * 32 + n32;
    const bool rvalid = rl < it.nrows;
    const int qpos = rq.L - rq.n + ((it.row0 + rl) >> lgG);
    row_lo = it.kv_begin;
    row_hi = it.kv_end;
    if (a.window >= 0) row_lo = max(row_lo, qpos - a.window);
    if (a.causal) row_hi = min(row_hi, qpos + 1);
    if (!rvalid) row_lo = row_hi = INT_MIN;       // sees nothing; neutral in the bounds below
    // [lo_max, hi_min): every valid row of the wave sees it (no mask needed);
    // outside [lo_min, hi_max): no row of the wave sees it (nothing to compute)
    lo_max = rvalid ? row_lo : INT_MIN;
    hi_min = rvalid ? row_hi : INT_MAX;
    lo_min = rvalid ? row_lo : INT_MAX;
    hi_max = rvalid ? row_hi : INT_MIN;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) {
      lo_max = max(lo_max, __shfl_xor(lo_max, k, 64));
      hi_min = min(hi_min, __shfl_xor(hi_min, k, 64));
      lo_min = min(lo_min, __shfl_xor(lo_min, k, 64));
      hi_max = max(hi_max, __shfl_xor(hi_max, k, 64));
    }
    wave_active = (wave * 32) < it.nrows;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
    // V^T operand reads.  The P^T operand of k-step kk holds, in lane half hf, the
    // probabilities of tokens 16kk + 4hf + 0..3 and 16kk + 8 + 4hf + 0..3 (the order
    // the S^T accumulator produces them in), so V^T must list the same tokens.  Lane
    // l of a 16-lane group g = l >> 4 reads 8 bytes of token row 4hf + (l & 15) / 4
    // (+8 for the second read, +16kk for k-step kk) at column 32dt + 16(g & 1) +
    // 4(l & 3); the transposing read hands lane l column 32dt + (l & 31) over the
    // 4 tokens read by its group.
    vr_tok = 4 * hf + ((lane & 15) >> 2);             // token within a 16-token k-step
    vr_sw = vswz<D>(vr_tok);                           // token & 3 is fixed per lane
    vr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // column within a 32-column d-tile
  }

  // Copy instruction i of wave w carries the block's 16-byte chunks
  // (8i + w)*64 .. (8i + w)*64 + 63, i.e. whole rows of 64 / CPRC consecutive
  // tokens; consecutive instructions of a wave are 8 such groups apart, so a
  // token's position modulo 16 (which the LDS swizzles depend on) is the same in
  // every instruction of a lane.
  __device__ __forceinline__ int copy_chunk0(int i) const { return (i * 8 + wave) * 64; }
  // KV position copied by this lane in copy instruction i of block b, when a
  // block's rows are CPRC 16-byte chunks each (clamped into the segment's range,
  // so a copy past its end reads valid memory)
  template <int CPRC, int NIC>
  __device__ __forceinline__ int copy_token(int b, int i) const {
    return min(it.kv_begin + b * KB + (copy_chunk0(i) + lane) / CPRC, it.kv_end - 1);
  }
  // page ids of this wave's copied tokens of block b, as stored (clamped when used)
  template <int CPRC, int NIC>
  __device__ __forceinline__ void load_pages(int b, int32_t (&raw)[NIC]) const {
#pragma unroll
    for (int i = 0; i < NIC; ++i)
      raw[i] = a.kv_indices[kv_page_index(rq.page_off, copy_token<CPRC, NIC>(b, i), a.log2B)];
  }

  __device__ __forceinline__ int v_elem(int kk, int dt, int second) const {
    const int tok = 16 * kk + vr_tok + 8 * second;
    const int col = 32 * dt + vr_col;
    return tok * D + 8 * ((col >> 3) ^ vr_sw) + (col & 7);
  }

  // ---- tile pieces.  Tile T of a block is block tokens 32T .. 32T+31; S^T element
  // i of a lane is token 32T + 8(i/4) + 4hf + i%4.
  __device__ __forceinline__ void read_k(const __bf16 (&kc)[TILE], int T, bf16x8 (&kop)[NS]) const {
    const int t = 32 * T + n32;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kop[s] = *reinterpret_cast<const bf16x8*>(&kc[8 * (t * CPR + ((2 * s + hf) ^ kswz<D>(t)))]);
  }
  __device__ __forceinline__ f32x16 s_mfma(const bf16x8 (&kop)[NS]) const {
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) sacc = mfma32(kop[s], qop[s], sacc);
    return sacc;
  }
  __device__ __forceinline__ void read_v(const __bf16 (&vc)[TILE], int kk, bf16x8 (&vop)[NDT]) const {
    typedef short v4s __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(&vc[v_elem(kk, dt, 0)]));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(&vc[v_elem(kk, dt, 1)]));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      vop[dt] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
    }
  }
  // tile max (base-2 units); the reference max is raised (rescaling O and l) only
  // when a tile exceeds it by kLazy
  __device__ __forceinline__ float tile_max(const f32x16& sacc) const {
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mb = fmaxf(mb, sacc[i]);
    mb = halves_max(mb) * c;
    return (mb > m_run + kLazy) ? mb : m_run;
  }
  __device__ __forceinline__ void raise_max(float m_new) {
    if (__any(m_new != m_run)) {
      // alpha = 1 where the reference stays (also rows with no visible key yet:
      // -inf - -inf would be NaN); a row leaving -inf gets exp2(-inf) = 0
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      m_run = m_new;
    }
  }
  // probabilities against the current reference max, packed as the P^T operands
  // of the tile's two 16-token k-steps; their sum goes into l
  __device__ __forceinline__ void exp_pack(const f32x16& sacc, bf16x8 (&pop)[2]) {
    const float msub = m_run == -INFINITY ? 0.f : m_run;
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(__builtin_fmaf(sacc[i], c, -msub));
      psum += p[i];
    }
    l_run += psum;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      u32x4 pw;
#pragma unroll
      for (int h = 0; h < 4; ++h) pw[h] = pack_bf16x2(p[8 * kh + 2 * h], p[8 * kh + 2 * h + 1]);
      pop[kh] = __builtin_bit_cast(bf16x8, pw);
    }
  }
  // Fast-path tile: probabilities against the current reference max first; only
  // if some lane's partial sum exceeds 2^kLazy (so one of its probabilities might)
  // or there is no reference yet is the tile max taken, the reference raised by the
  // same rule as tile_max / raise_max and the probabilities recomputed.  A sum
  // within the bound means every probability is, i.e. the tile max does not exceed
  // the reference by kLazy: the same decision without the max.
  __device__ __forceinline__ void exp_sum(const f32x16& sacc, float (&p)[16], float& psum) const {
    const float msub = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(__builtin_fmaf(sacc[i], c, -msub));
    psum = p[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) psum += p[i];
  }
  __device__ __forceinline__ void exp_check_pack(const f32x16& sacc, bf16x8 (&pop)[2]) {
    float p[16];
    float psum;
    exp_sum(sacc, p, psum);
    if (__any((psum > kLazyP) | (m_run == -INFINITY))) {
      raise_max(tile_max(sacc));
      exp_sum(sacc, p, psum);
    }
    l_run += psum;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      u32x4 pw;
#pragma unroll
      for (int h = 0; h < 4; ++h) pw[h] = pack_bf16x2(p[8 * kh + 2 * h], p[8 * kh + 2 * h + 1]);
      pop[kh] = __builtin_bit_cast(bf16x8, pw);
    }
  }
  __device__ __forceinline__ void o_mfma(const bf16x8 (&vop)[NDT], const bf16x8& pop) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = mfma32(vop[dt], pop, oacc[dt]);
  }

  // attention of the wave's rows over the block whose first KV position is tb,
  // held in the compute tiles kc / vc.  LATE_MAX: the fast path forms each tile's
  // probabilities before (and usually instead of) its max (exp_check_pack); else
  // the max of tile T+1 is taken beside the PV MFMAs of tile T.  (Both keep the
  // same reference-max rule; the fp8 staging, whose block starts with the widening
  // pass, schedules better with the max first.)
  template <bool LATE_MAX>
  __device__ __forceinline__ void compute(const __bf16 (&kc)[TILE], const __bf16 (&vc)[TILE], int tb) {
    bf16x8 kop[NS];
    bf16x8 vop[NDT];
    bf16x8 pop[2];
    if (tb >= lo_max && tb + KB <= hi_min) {
      // Fast path (no masks), software-pipelined over the block's tiles: while the
      // probabilities of tile T are formed, the S^T MFMAs of tile T+1 run and the
      // K operands of tile T+2 and the V operands of tile T are in flight.
      read_k(kc, 0, kop);
      f32x16 sa = s_mfma(kop);
      if (NT > 1) read_k(kc, 1, kop);
      if constexpr (!LATE_MAX) raise_max(tile_max(sa));
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        read_v(vc, 2 * T, vop);
        f32x16 sb;
        if (T + 1 < NT) {
          sb = s_mfma(kop);
          if (T + 2 < NT) read_k(kc, T + 2, kop);
        }
        if constexpr (LATE_MAX) {
          exp_check_pack(sa, pop);
          o_mfma(vop, pop[0]);
          read_v(vc, 2 * T + 1, vop);
          o_mfma(vop, pop[1]);
          if (T + 1 < NT) sa = sb;
        } else {
          exp_pack(sa, pop);
          o_mfma(vop, pop[0]);
          read_v(vc, 2 * T + 1, vop);
          const float m_next = T + 1 < NT ? tile_max(sb) : 0.f;
          o_mfma(vop, pop[1]);
          if (T + 1 < NT) {
            raise_max(m_next);
            sa = sb;
          }
        }
      }
    } else {
      for (int T = 0; T < NT; ++T) {
        const int tt0 = tb + 32 * T;
        if ((tt0 >= hi_max) | (tt0 + 32 <= lo_min)) continue;   // no row of the wave sees it
        read_k(kc, T, kop);
        f32x16 sacc = s_mfma(kop);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tk = tt0 + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (!((tk >= row_lo) & (tk < row_hi))) sacc[i] = -INFINITY;
        }
        raise_max(tile_max(sacc));
        exp_pack(sacc, pop);
        read_v(vc, 2 * T, vop);
        o_mfma(vop, pop[0]);
        read_v(vc, 2 * T + 1, vop);
        o_mfma(vop, pop[1]);
      }
    }
  }

  // ---- Q rows.  Each wave copies its 32 rows HBM -> LDS with the load-to-LDS path
  // (whole rows per instruction, 16 bytes per lane), rows 0-15 into q_lo and 16-31
  // into q_hi at this wave's copy region (the NI 1 KB pieces its own block copies
  // fill: piece i at chunk copy_chunk0(i), QPI = 512 / D rows each), chunk c of row
  // r at slot c ^ (r mod CPR); rows past the tile's end fetch its last row (never
  // stored).  Loaded by the lane that owns the row, a load instruction would touch
  // 32 rows 32 bytes at a time.
  static constexpr int QPI = 512 / D;   // Q rows per 1 KB piece
  static_assert(16 * 2 * D == NI * 1024, "a wave's Q half-tile fills its copy region");
  __device__ __forceinline__ void issue_q(__bf16 (&q_lo)[TILE], __bf16 (&q_hi)[TILE]) const {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int o = 1024 * i + 16 * lane;             // byte within the half-tile
        const int r = o / (2 * D), j = (o % (2 * D)) / 16;
        const int rl_c = min(wave * 32 + 16 * pt + r, it.nrows - 1);
        const int rho_c = it.row0 + rl_c;
        const __bf16* src = static_cast<const __bf16*>(a.q) +
                            ((int64_t)rq.q_off + (rho_c >> lgG)) * a.q_st +
                            (int64_t)(it.hk * G + (rho_c & (G - 1))) * a.q_sh +
                            8 * (j ^ (r & (CPR - 1)));
        __bf16* dst = (pt ? q_hi : q_lo) + 8 * copy_chunk0(i);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      }
  }
  __device__ __forceinline__ void read_q(const __bf16 (&q_lo)[TILE], const __bf16 (&q_hi)[TILE]) {
    const int r = n32 & 15;
    const __bf16* qs = (n32 < 16 ? q_lo : q_hi) + 8 * copy_chunk0(r / QPI) + (r % QPI) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qop[s] = *reinterpret_cast<const bf16x8*>(qs + 8 * ((2 * s + hf) ^ (r & (CPR - 1))));
  }

  // ---- finalise: O^T element i of tile dt is column d = 32dt + 8(i/4) + 4hf + i%4.
  // `st` is this wave's private LDS slice (>= 32 padded rows), free once every
  // wave is past the last block's barrier.
  __device__ __forceinline__ void finalize(char* st) {
    const float l_tot = halves_sum(l_run);
    const bool any = l_tot > 0.f;
    const float inv = any ? a.v_scale / l_tot : 0.f;
    const float lse2 = any ? m_run + log2f(l_tot) : -INFINITY;
    // The row's addressing is recomputed here from a lane id the compiler cannot
    // see through, so none of it is kept live (and spilled) across the block loop.
    int le = __lane_id();
    asm volatile("" : "+v"(le));
    const int n32e = le & 31, hfe = le >> 5;
    const int rle = wave * 32 + n32e;
    const bool rvalide = rle < it.nrows;
    const int rho = it.row0 + rle;
    const int64_t qtok = (int64_t)rq.q_off + (rho >> lgG);
    const int head = it.hk * G + (rho & (G - 1));
    if (it.pbase < 0) {
      // Wave w stages its 32 bf16 rows (padded by 16 bytes against bank conflicts)
      // in its own slice, then stores whole rows, 16 bytes per lane and CPR lanes
      // per row.  Stored from the lane that owns the row, a store instruction
      // would touch 32 rows 8 bytes at a time.
      constexpr int RS = 2 * D + 16;              // staged row stride in bytes
      constexpr int RPI = 64 / CPR;               // rows per store instruction
      static_assert(32 * RS <= TILE, "a wave's staged rows fit in its LDS slice");
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dt + 8 * g + 4 * hfe;
          *reinterpret_cast<u32x2*>(st + n32e * RS + 2 * d0) =
              u32x2{pack_bf16x2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                    pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
        }
      if (rvalide && a.lse && hfe == 0) a.lse[qtok * a.l_st + (int64_t)head * a.l_sh] = lse2 * kLn2;
      __syncthreads();
      const int c16 = le % CPR;
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int rr = i * RPI + le / CPR;        // row of the wave
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + rr * RS + 16 * c16);
        const int rl2 = wave * 32 + rr;
        if (rl2 < it.nrows) {
          const int rho2 = it.row0 + rl2;
          const int head2 = it.hk * G + (rho2 & (G - 1));
          uint16_t* op = static_cast<uint16_t*>(a.out) + ((int64_t)rq.q_off + (rho2 >> lgG)) * a.o_st +
                         (int64_t)head2 * a.o_sh;
          *reinterpret_cast<u32x4*>(op + 8 * c16) = v;
        }
      }
    } else {
      if (!rvalide) return;
      const int64_t prow = (int64_t)it.pbase + rle;
      float* pp = a.part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dt + 8 * g + 4 * hfe;
          *reinterpret_cast<f32x4*>(pp + d0) =
              f32x4{oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                    oacc[dt][4 * g + 3] * inv};
        }
      if (hfe == 0) a.part_lse[prow] = lse2;
    }
  }
};

// One kernel for both cache types; FP8 selects the copy-and-widen staging, C32
// the 32-bit copy offsets (kv_copy_offset32; pools within its bounds).
template <int D, int KB, bool FP8, bool C32>
__global__ __launch_bounds__(512, 2) void attn_large_kernel(AttnArgs a) {
  using LT = LargeTile<D, KB>;
  constexpr int TILE = LT::TILE, CPR = LT::CPR, NI = LT::NI;

  const Item it = a.items[blockIdx.x];
  if (it.nrows == 0) return;   // padding item (uniform over the workgroup)
  const Req rq = a.reqs[it.r];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  LT t(a, it, rq, wave, lane);
  const int nb = (it.kv_end - it.kv_begin + KB - 1) / KB;

  if constexpr (!FP8) {
    // ---- bf16 caches: K and V blocks are copied HBM -> LDS by the load-to-LDS
    // path (global_load_lds, 16 bytes per lane), so staging costs neither
    // registers nor VALU work.  Each lane fetches the source chunk that belongs at
    // its LDS slot, which applies the compute layout's swizzle on the gather side.
    // The two LDS buffer pairs are distinct variables and the block loop is
    // unrolled by two, so the compiler can tell that reads of the current buffer
    // never alias the copy in flight into the other one (no memory-counter wait
    // between them).
    __shared__ __align__(16) __bf16 k0s[TILE];
    __shared__ __align__(16) __bf16 v0s[TILE];
    __shared__ __align__(16) __bf16 k1s[TILE];
    __shared__ __align__(16) __bf16 v1s[TILE];
    const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)it.hk * a.k_sh * 2;
    const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)it.hk * a.v_sh * 2;
    const uint32_t kps = (uint32_t)(a.k_sp * 2), kbs = (uint32_t)(a.k_sb * 2);
    const uint32_t vps = (uint32_t)(a.v_sp * 2), vbs = (uint32_t)(a.v_sb * 2);
    // The copy of a block is NI load-to-LDS instructions per wave for K and NI for
    // V; lane l of instruction i carries chunk q = copy_chunk0(i) + l of the
    // block, i.e. block token q / CPR.  Each wave loads the page ids of its own
    // tokens one block ahead of the copy, so the addresses need no shared table.
    auto issue_copy = [&](auto& kd, auto& vd, int b, const int32_t (&raw)[NI]) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int q0 = t.copy_chunk0(i);   // first LDS chunk of this instruction
        const int q = q0 + lane;
        const int tk = q / CPR, j = q % CPR;
        const uint32_t page = (uint32_t)clamp_page(raw[i], a.num_pages);
        const int tok = t.template copy_token<CPR, NI>(b, i);
        const uint32_t ik = 16u * (j ^ kswz<D>(tk)), iv = 16u * (j ^ vswz<D>(tk));
        const char* gk;
        const char* gv;
        if constexpr (C32) {
          gk = kbase + kv_copy_offset32(page, tok, a.log2B, kps, kbs, ik);
          gv = vbase + kv_copy_offset32(page, tok, a.log2B, vps, vbs, iv);
        } else {
          gk = kbase + kv_copy_offset(page, tok, a.log2B, kps, kbs, ik);
          gv = vbase + kv_copy_offset(page, tok, a.log2B, vps, vbs, iv);
        }
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gk),
                                         (__attribute__((address_space(3))) void*)(&kd[8 * q0]),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gv),
                                         (__attribute__((address_space(3))) void*)(&vd[8 * q0]),
                                         16, 0, 0);
      }
    };
    // one block: start the copy of block b+1 (page ids loaded during block b-1)
    // and the page-id loads of block b+2, then compute block b
    int32_t raw[NI];
    auto step = [&](int b, auto& kc, auto& vc, auto& kn, auto& vn) {
      if (b + 1 < nb) issue_copy(kn, vn, b + 1, raw);
      if (b + 2 < nb) t.template load_pages<CPR, NI>(b + 2, raw);
      if (t.wave_active) t.template compute<true>(kc, vc, it.kv_begin + b * KB);
      __builtin_amdgcn_s_waitcnt(0);              // this wave's copies have landed
      __syncthreads();
    };
    // prologue: block 0 and the Q rows copied (Q into the region this wave's own
    // copy of block 1 fills later), page ids of block 1 loaded (an empty KV range
    // -- a non-causal request without pages -- has no blocks)
    if (nb > 0) {
      t.template load_pages<CPR, NI>(0, raw);
      issue_copy(k0s, v0s, 0, raw);
    }
    t.issue_q(k1s, v1s);
    if (nb > 1) t.template load_pages<CPR, NI>(1, raw);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    t.read_q(k1s, v1s);
    // this wave's copy of block 1 lands on its Q rows: the reads complete first
    __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
    for (int b = 0; b < nb; b += 2) {
      step(b, k0s, v0s, k1s, v1s);
      if (b + 1 >= nb) break;
      step(b + 1, k1s, v1s, k0s, v0s);
    }
    // every wave is past the last block's barrier: all LDS is free, each wave
    // stages its output rows in its own half-array
    __bf16* const arr = wave < 2 ? k0s : wave < 4 ? v0s : wave < 6 ? k1s : v1s;
    t.finalize(reinterpret_cast<char*>(arr) + (wave & 1) * TILE);   // TILE bytes = half an array
  } else {
    // ---- fp8 caches: each block's fp8 K and V rows are copied HBM -> LDS as they
    // sit in the cache (16 bytes per lane) into a double-buffered staging area,
    // then all 512 threads widen them exactly to bf16 into the compute tiles in
    // the bf16 layouts.  The staging buffers are distinct variables, so widening
    // one never waits for the copy into the other.
    constexpr int CPR8 = D / 16;                // 16-byte chunks per fp8 row
    constexpr int NI8 = KB * CPR8 / (64 * 8);   // fp8 copy instructions per wave per block
    static_assert(NI8 >= 1 && NI8 * 64 * 8 == KB * CPR8, "fp8 tile shape");
    static_assert(KB * D == TILE, "an fp8 staging buffer holds TILE bytes");
    __shared__ __align__(16) __bf16 kb[TILE];      // the block's K widened to bf16
    __shared__ __align__(16) __bf16 vb[TILE];      // the block's V widened to bf16
    __shared__ __align__(16) uint8_t k8a[KB * D];  // fp8 K/V copies, double-buffered
    __shared__ __align__(16) uint8_t k8b[KB * D];
    __shared__ __align__(16) uint8_t v8a[KB * D];
    __shared__ __align__(16) uint8_t v8b[KB * D];
    const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)it.hk * a.k_sh;
    const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)it.hk * a.v_sh;
    const uint32_t kps = (uint32_t)a.k_sp, kbs = (uint32_t)a.k_sb;
    const uint32_t vps = (uint32_t)a.v_sp, vbs = (uint32_t)a.v_sb;
    // lane l of copy instruction i carries chunk q = copy_chunk0(i) + l of the
    // block (token q / CPR8), into the staging buffer as it sits in the cache row
    auto issue_copy8 = [&](uint8_t* kd, uint8_t* vd, int b, const int32_t (&raw)[NI8]) {
#pragma unroll
      for (int i = 0; i < NI8; ++i) {
        const int q0 = t.copy_chunk0(i);   // first staging chunk of this instruction
        const int j = (q0 + lane) % CPR8;
        const uint32_t page = (uint32_t)clamp_page(raw[i], a.num_pages);
        const int tok = t.template copy_token<CPR8, NI8>(b, i);
        const char* gk;
        const char* gv;
        if constexpr (C32) {
          gk = kbase + kv_copy_offset32(page, tok, a.log2B, kps, kbs, 16u * j);
          gv = vbase + kv_copy_offset32(page, tok, a.log2B, vps, vbs, 16u * j);
        } else {
          gk = kbase + kv_copy_offset(page, tok, a.log2B, kps, kbs, 16u * j);
          gv = vbase + kv_copy_offset(page, tok, a.log2B, vps, vbs, 16u * j);
        }
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gk),
                                         (__attribute__((address_space(3))) void*)(&kd[16 * q0]),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gv),
                                         (__attribute__((address_space(3))) void*)(&vd[16 * q0]),
                                         16, 0, 0);
      }
    };
    // widen the copied block (exact e4m3 -> bf16) into the compute layout: chunk c
    // of token t's K row at slot c ^ kswz(t), of its V row at slot c ^ vswz(t)
    auto widen = [&](const uint8_t* ks, const uint8_t* vs) {
#pragma unroll
      for (int k8 = 0; k8 < KB * CPR8 / 512; ++k8) {
        const int q = tid + 512 * k8;
        const int tk = q / CPR8, j = q % CPR8;
        const u32x4 wk = *reinterpret_cast<const u32x4*>(ks + 16 * q);
        const u32x4 wv = *reinterpret_cast<const u32x4*>(vs + 16 * q);
        *reinterpret_cast<bf16x8*>(&kb[8 * (tk * CPR + ((2 * j) ^ kswz<D>(tk)))]) =
            e4m3x8_to_bf16x8(wk[0], wk[1]);
        *reinterpret_cast<bf16x8*>(&kb[8 * (tk * CPR + ((2 * j + 1) ^ kswz<D>(tk)))]) =
            e4m3x8_to_bf16x8(wk[2], wk[3]);
        *reinterpret_cast<bf16x8*>(&vb[8 * (tk * CPR + ((2 * j) ^ vswz<D>(tk)))]) =
            e4m3x8_to_bf16x8(wv[0], wv[1]);
        *reinterpret_cast<bf16x8*>(&vb[8 * (tk * CPR + ((2 * j + 1) ^ vswz<D>(tk)))]) =
            e4m3x8_to_bf16x8(wv[2], wv[3]);
      }
    };
    // one block: start the copy of block b+1 (page ids loaded during block b-1)
    // and the page-id loads of block b+2, widen block b, then compute it
    int32_t raw[NI8];
    auto step = [&](int b, const uint8_t* kc8, const uint8_t* vc8, uint8_t* kn8, uint8_t* vn8) {
      if (b + 1 < nb) issue_copy8(kn8, vn8, b + 1, raw);
      if (b + 2 < nb) t.template load_pages<CPR8, NI8>(b + 2, raw);
      widen(kc8, vc8);
      __syncthreads();                            // the widened block is complete
      if (t.wave_active) t.template compute<false>(kb, vb, it.kv_begin + b * KB);
      __builtin_amdgcn_s_waitcnt(0);              // this wave's copies have landed
      __syncthreads();                            // and no wave still reads kb / vb
    };
    // prologue: block 0 and the Q rows copied (Q into the compute tiles, read before
    // block 0 is widened over them), page ids of block 1 loaded
    if (nb > 0) {
      t.template load_pages<CPR8, NI8>(0, raw);
      issue_copy8(k8a, v8a, 0, raw);
    }
    t.issue_q(kb, vb);
    if (nb > 1) t.template load_pages<CPR8, NI8>(1, raw);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    t.read_q(kb, vb);
    __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
    __syncthreads();   // every wave holds its Q operands before block 0 is widened over them
    for (int b = 0; b < nb; b += 2) {
      step(b, k8a, v8a, k8b, v8b);
      if (b + 1 >= nb) break;
      step(b + 1, k8b, v8b, k8a, v8a);
    }
    // every wave is past the last block's barrier: waves 0-3 stage their output
    // rows in the compute tiles, waves 4-7 in the staging buffers
    char* const st = wave < 4 ? reinterpret_cast<char*>(wave < 2 ? kb : vb) + (wave & 1) * TILE
                              : reinterpret_cast<char*>(wave == 4 ? k8a : wave == 5 ? k8b
                                                        : wave == 6 ? v8a : v8b);
    t.finalize(st);
  }
}

}  // namespace

hipError_t launch_attn_large(const AttnArgs& a, int n_items, int D, int kv_dtype, hipStream_t s) {
  (void)hipGetLastError();   // a stale error of an earlier call is not this launch's
  if (n_items <= 0) return hipSuccess;
  dim3 grid((unsigned)n_items);
  const int eb = kv_dtype == AK_FP8_E4M3 ? 1 : 2;
  const bool c32 = kv_copy32_ok(a.num_pages, a.k_sp * eb, a.k_sb * eb, 1 << a.log2B, (int64_t)D * eb) &&
                   kv_copy32_ok(a.num_pages, a.v_sp * eb, a.v_sb * eb, 1 << a.log2B, (int64_t)D * eb);
#define AK_LARGE(DD, F8)                                                                          \
  do {                                                                                            \
    if (c32)                                                                                      \
      hipLaunchKernelGGL((attn_large_kernel<DD, kDmaKB, F8, true>), grid, dim3(512), 0, s, a);   \
    else                                                                                          \
      hipLaunchKernelGGL((attn_large_kernel<DD, kDmaKB, F8, false>), grid, dim3(512), 0, s, a);  \
  } while (0)
  if (D == 128 && kv_dtype == AK_BF16) {
    AK_LARGE(128, false);
  } else if (D == 64 && kv_dtype == AK_BF16) {
    AK_LARGE(64, false);
  } else if (D == 128 && kv_dtype == AK_FP8_E4M3) {
    AK_LARGE(128, true);
  } else if (D == 64 && kv_dtype == AK_FP8_E4M3) {
    AK_LARGE(64, true);
  } else {
    return hipErrorInvalidValue;
  }
#undef AK_LARGE
  return hipGetLastError();
}

}  // namespace ak
