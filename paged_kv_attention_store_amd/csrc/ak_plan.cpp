// Host planner: validation, per-request lengths, tiling and the split-KV
// partition.  Plain C++ (no HIP): it reads host arrays only, never the device.
//
// What a plan holds follows "vLLM attention backend", "plan() and run()" and
// "FlashInfer and the backend abstraction", "plan()": the batch's ragged
// structure is turned once per step into a work assignment and split
// temporaries, which every layer's run reuses.  Lengths follow the CSR section
// of the vLLM page: L = (pages - 1) * B + last_page_len, last_page_len in [1, B].

#include <algorithm>
#include <climits>
#include <cmath>
#include <sstream>

#include "ak_internal.h"

namespace ak {

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Guided decode split: a part aims at (decode KV still to cut) / (kGuideShare *
// compute units) tokens (two per resident workgroup slot, two slots per compute
// unit), at least chunk / kGuideFloor.
constexpr int64_t kGuideShare = 4;
constexpr int64_t kGuideFloor = 4;

ak_status fail(ak_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

}  // namespace

ak_status build_plan_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* last_page_len, int32_t R, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t B, int32_t causal, int32_t window,
                          const ak_plan_opts* opts, int32_t num_cus, ak_plan_t* p) {
  if (R < 0) return fail(AK_ERR_INVALID_ARG, "ak_plan: batch_size < 0");
  if (R > 0 && (!qo_indptr || !kv_indptr || !last_page_len))
    return fail(AK_ERR_INVALID_ARG, "ak_plan: null indptr or last_page_len array");
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0)
    return fail(AK_ERR_INVALID_ARG, "ak_plan: head counts, head_dim and page_size must be > 0");
  if (Hq % Hkv != 0)
    return fail(AK_ERR_INVALID_ARG, "ak_plan: num_qo_heads is not a multiple of num_kv_heads");
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(AK_ERR_UNSUPPORTED, "ak_plan: GQA group size must be 1, 2, 4, 8 or 16");
  if (D != 64 && D != 128) return fail(AK_ERR_UNSUPPORTED, "ak_plan: head_dim must be 64 or 128");
  if (!is_pow2(B) || B > 256)
    return fail(AK_ERR_UNSUPPORTED, "ak_plan: page_size must be a power of two <= 256");
  if (causal != 0 && causal != 1) return fail(AK_ERR_INVALID_ARG, "ak_plan: causal must be 0 or 1");
  if (window < -1) return fail(AK_ERR_INVALID_ARG, "ak_plan: window must be -1 or >= 0");
  if (window >= 0 && !causal)
    return fail(AK_ERR_UNSUPPORTED, "ak_plan: a sliding window needs causal = 1");
  if (R > 0 && (qo_indptr[0] != 0 || kv_indptr[0] != 0))
    return fail(AK_ERR_BAD_INDPTR, "ak_plan: qo_indptr[0] and kv_indptr[0] must be 0");

  p->R = R;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->D = D;
  p->B = B;
  p->G = G;
  p->log2B = 0;
  while ((1 << p->log2B) < B) ++p->log2B;
  int lgG = 0;   // G is a power of two (validated above)
  while ((1 << lgG) < G) ++lgG;
  p->causal = causal;
  p->window = window;
  p->num_cus = num_cus > 0 ? num_cus : 256;
  p->sm_scale = (opts && opts->sm_scale > 0.f) ? opts->sm_scale : 1.0f / std::sqrt((float)D);
  const int64_t max_splits = (opts && opts->max_splits > 0) ? opts->max_splits : 64;
  const int64_t min_chunk =
      (opts && opts->min_chunk > 0) ? round_up(opts->min_chunk, kKvAlign) : 256;
  p->merge_in_kernel = opts && (opts->flags & AK_PLAN_MERGE_IN_KERNEL);
  p->shared_pages = opts && (opts->flags & AK_PLAN_SHARED_PAGES);
  p->stream_k = opts && (opts->flags & AK_PLAN_STREAM_K);
  p->wg_first.clear();

  // ---- lengths and validation
  p->kv_lens.assign(R, 0);
  p->reqs.assign(R, Req{});
  for (int32_t r = 0; r < R; ++r) {
    if (qo_indptr[r + 1] < qo_indptr[r] || kv_indptr[r + 1] < kv_indptr[r]) {
      std::ostringstream os;
      os << "ak_plan: indptr decreases at request " << r;
      return fail(AK_ERR_BAD_INDPTR, os.str());
    }
  }
  for (int32_t r = 0; r < R; ++r) {
    const int64_t pages = (int64_t)kv_indptr[r + 1] - kv_indptr[r];
    const int64_t n = (int64_t)qo_indptr[r + 1] - qo_indptr[r];
    int64_t L = 0;
    if (pages > 0) {
      if (last_page_len[r] < 1 || last_page_len[r] > B) {
        std::ostringstream os;
        os << "ak_plan: last_page_len[" << r << "] = " << last_page_len[r] << " outside [1, "
           << B << "]";
        return fail(AK_ERR_BAD_LENGTHS, os.str());
      }
      L = (pages - 1) * B + last_page_len[r];
    }
    if (L > INT32_MAX / 2) return fail(AK_ERR_UNSUPPORTED, "ak_plan: KV length exceeds 2^30");
    if (causal && n > L) {   // the causal diagonal is aligned to the sequence end
      std::ostringstream os;
      os << "ak_plan: request " << r << " has " << n << " queries but only " << L << " KV tokens";
      return fail(AK_ERR_BAD_LENGTHS, os.str());
    }
    if (n * G > INT32_MAX / 2) return fail(AK_ERR_UNSUPPORTED, "ak_plan: too many query rows");
    p->kv_lens[r] = (int32_t)L;
    p->reqs[r] = Req{qo_indptr[r], (int32_t)n, (int32_t)L, kv_indptr[r]};
  }
  p->T = R > 0 ? qo_indptr[R] : 0;
  p->num_kv_pages = R > 0 ? kv_indptr[R] : 0;

  // ---- visible KV range of unit rows [a, b)
  auto kv_range = [&](const Req& q, int64_t a, int64_t b, int32_t& lo, int32_t& hi) {
    const int64_t pa = (int64_t)q.L - q.n + a / G;          // first row's position
    const int64_t pb = (int64_t)q.L - q.n + (b - 1) / G;    // last row's position
    hi = causal ? (int32_t)(pb + 1) : q.L;
    lo = window >= 0 ? (int32_t)std::max<int64_t>(0, pa - window) : 0;
  };

  // ---- small units (<= 16 rows) with their split partition; large tile jobs
  struct Unit {
    int32_t r, hk, rows, lo, hi;
  };
  std::vector<Unit> small;
  std::vector<Item> jobs;   // large tiles, ordered by (request, KV head, first row)
  int64_t small_tokens = 0;
  p->small_items.clear();
  p->large_items.clear();
  p->merges.clear();
  for (int32_t r = 0; r < R; ++r) {
    const Req& q = p->reqs[r];
    if (q.n == 0) continue;
    const int64_t rows = (int64_t)q.n * G;
    if (rows <= kSmallRows) {
      int32_t lo, hi;
      kv_range(q, 0, rows, lo, hi);
      for (int32_t hk = 0; hk < Hkv; ++hk) small.push_back(Unit{r, hk, (int32_t)rows, lo, hi});
      small_tokens += (int64_t)(hi - lo) * Hkv;
    } else {
      for (int32_t hk = 0; hk < Hkv; ++hk)
        for (int64_t row0 = 0; row0 < rows; row0 += kLargeRows) {
          const int64_t nr = std::min<int64_t>(kLargeRows, rows - row0);
          int32_t lo, hi;
          kv_range(q, row0, row0 + nr, lo, hi);
          jobs.push_back(Item{r, hk, (int32_t)row0, (int32_t)nr, lo, hi, -1, 1, -1, {}});
        }
    }
  }

  int64_t prow = 0;
  int64_t split_units = 0;
  if (p->stream_k) {
    // Stream-K: the units' visible KV ranges laid end to end, in unit order, are
    // cut into P equal contiguous shares (cuts on the kKvAlign grid of each
    // unit's positions), one per persistent workgroup; a share's intersection with
    // a unit is one piece (an item), pieces longer than a small tile's page table
    // are cut again, and a unit left in several pieces is merged from their
    // partial states like any split unit.  Items are grouped by workgroup.
    const int64_t P = (int64_t)p->num_cus * kStreamKPerCu;
    const int64_t share =
        std::max<int64_t>(kKvAlign, round_up(ceil_div(std::max<int64_t>(small_tokens, 1), P), kKvAlign));
    const int64_t max_piece =
        std::max<int64_t>(kKvAlign, ((int64_t)(kSmallMaxPages - 2) * B) / kKvAlign * kKvAlign);
    struct Piece {
      int32_t unit, a, b, wg;
    };
    std::vector<Piece> pieces;
    pieces.reserve(small.size() + (size_t)P * 2);
    std::vector<int32_t> npieces(small.size(), 0);
    int64_t flat = 0;   // flattened position of the current unit's first key
    for (size_t ui = 0; ui < small.size(); ++ui) {
      const Unit& u = small[ui];
      int64_t pos = u.lo;
      for (;;) {
        const int64_t g = std::min<int64_t>(P - 1, (flat + pos - u.lo) / share);
        int64_t b = u.hi;
        if (g < P - 1) {   // this share ends at flattened (g + 1) * share
          const int64_t end = (int64_t)u.lo + (g + 1) * share - flat;
          b = std::min<int64_t>(b, std::max<int64_t>(pos + 1, round_up(end, kKvAlign)));
        }
        b = std::min<int64_t>(b, pos + max_piece);
        pieces.push_back(Piece{(int32_t)ui, (int32_t)pos, (int32_t)b, (int32_t)g});
        ++npieces[ui];
        pos = b;
        if (pos >= u.hi) break;
      }
      flat += (int64_t)u.hi - u.lo;
    }
    // partial rows and merge jobs of units left in several pieces
    std::vector<int64_t> ubase(small.size(), -1);
    std::vector<int32_t> umerge(small.size(), -1);
    for (size_t ui = 0; ui < small.size(); ++ui) {
      if (npieces[ui] <= 1) continue;
      const Unit& u = small[ui];
      ubase[ui] = prow;
      umerge[ui] = p->merge_in_kernel ? (int32_t)p->merges.size() : -1;
      const Req& q = p->reqs[u.r];
      for (int32_t rho = 0; rho < u.rows; ++rho) {
        MergeJob m{};
        m.token = q.q_off + (rho >> lgG);
        m.head = u.hk * G + (rho & (G - 1));
        m.pfirst = (int32_t)(prow + rho);
        m.pstride = u.rows;
        m.count = npieces[ui];
        p->merges.push_back(m);
      }
      prow += (int64_t)npieces[ui] * u.rows;
      ++split_units;
      if (prow > INT32_MAX / 2) return fail(AK_ERR_UNSUPPORTED, "ak_plan: split workspace too large");
    }
    p->small_items.reserve(pieces.size());
    p->wg_first.assign((size_t)P + 1, 0);
    std::vector<int32_t> seen(small.size(), 0);
    for (const Piece& pc : pieces) {
      const Unit& u = small[(size_t)pc.unit];
      const int32_t k = seen[(size_t)pc.unit]++;
      const int32_t pb = ubase[(size_t)pc.unit] < 0 ? -1 : (int32_t)(ubase[(size_t)pc.unit] + (int64_t)k * u.rows);
      p->small_items.push_back(Item{u.r, u.hk, 0, u.rows, pc.a, pc.b, pb, 0, umerge[(size_t)pc.unit], {}});
      ++p->wg_first[(size_t)pc.wg + 1];
    }
    for (int64_t g = 0; g < P; ++g) p->wg_first[(size_t)g + 1] += p->wg_first[(size_t)g];
    p->small_merges = (int64_t)p->merges.size();
  } else {
    // Split size: about kPartsPerCu KV chunks per compute unit over the whole batch,
    // between min_chunk and 4096 tokens, in multiples of kKvAlign.
    int64_t chunk = ceil_div(std::max<int64_t>(small_tokens, 1), (int64_t)p->num_cus * kPartsPerCu);
    chunk = std::min<int64_t>(std::max<int64_t>(round_up(chunk, kKvAlign), min_chunk), 4096);
    chunk = std::max<int64_t>(chunk, min_chunk);

    // Units longest first (partial rows and merge jobs follow this order).
    std::vector<int32_t> order(small.size());
    for (size_t i = 0; i < small.size(); ++i) order[i] = (int32_t)i;
    std::sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
      const int32_t lx = small[x].hi - small[x].lo, ly = small[y].hi - small[y].lo;
      return lx != ly ? lx > ly : x < y;
    });
    p->merges.reserve((size_t)small.size() * kSmallRows);
    // parts are at least chunk / kGuideFloor tokens (or min_chunk)
    p->small_items.reserve(small.size() +
                           (size_t)(small_tokens / std::max<int64_t>(min_chunk, chunk / kGuideFloor)) + 16);

    // Guided part size: the units come longest first, and each is cut into parts of
    // about (decode KV still to cut) / (kGuideShare * CUs) tokens, between
    // chunk / kGuideFloor and chunk.  Parts shrink toward the end of the grid, so
    // its last round holds short items and the compute units run out of work
    // nearly together.
    int64_t w_rem = small_tokens;
    const int64_t t_floor = std::max<int64_t>(min_chunk, round_up(chunk / kGuideFloor, kKvAlign));
    for (int32_t ui : order) {
      const Unit& u = small[ui];
      const int64_t len = (int64_t)u.hi - u.lo;
      int64_t t = round_up(ceil_div(std::max<int64_t>(w_rem, 1), kGuideShare * (int64_t)p->num_cus), kKvAlign);
      t = std::min<int64_t>(chunk, std::max<int64_t>(t, t_floor));
      w_rem -= len;
      // S parts with boundaries on a kKvAlign grid anchored below lo, each the grid
      // point nearest to an equal share (parts differ by at most kKvAlign tokens;
      // at least kKvAlign tokens per share keeps every part non-empty)
      const int64_t base = (u.lo / kKvAlign) * kKvAlign;
      const int64_t ext = (int64_t)u.hi - base;
      int64_t S = std::min<int64_t>(max_splits, std::max<int64_t>(1, ceil_div(len, t)));
      for (;;) {
        S = std::max<int64_t>(1, std::min<int64_t>(S, ext / kKvAlign));
        // every part must fit a small tile's page table (only binds for tiny pages)
        const int64_t span = S <= 1 ? (((int64_t)u.hi - 1) >> p->log2B) - (u.lo >> p->log2B) + 1
                                    : (ceil_div(ext, S) + kKvAlign + B - 1) / B + 1;
        if (span <= kSmallMaxPages) break;
        S = std::max<int64_t>(S + 1, ceil_div(S * span, kSmallMaxPages - 1));
      }
      const int64_t nparts = S;
      auto bound = [&](int64_t s) -> int64_t {
        if (s <= 0) return u.lo;
        if (s >= nparts) return u.hi;
        return std::max<int64_t>(u.lo, base + (s * ext + nparts * (kKvAlign / 2)) / (nparts * kKvAlign) * kKvAlign);
      };
      if (nparts <= 1) {
        p->small_items.push_back(Item{u.r, u.hk, 0, u.rows, u.lo, u.hi, -1, 0, -1, {}});
        continue;
      }
      const int64_t ubase = prow;
      // the unit's first merge job, which a part merging in-kernel starts from
      const int32_t m0 = p->merge_in_kernel ? (int32_t)p->merges.size() : -1;
      int32_t a = (int32_t)bound(0);
      for (int64_t s = 0; s < nparts; ++s) {
        const int32_t b = (int32_t)bound(s + 1);
        p->small_items.push_back(
            Item{u.r, u.hk, 0, u.rows, a, b, (int32_t)(ubase + s * u.rows), 0, m0, {}});
        a = b;
      }
      const Req& q = p->reqs[u.r];
      for (int32_t rho = 0; rho < u.rows; ++rho) {
        MergeJob m{};
        m.token = q.q_off + (rho >> lgG);
        m.head = u.hk * G + (rho & (G - 1));
        m.pfirst = (int32_t)(ubase + rho);
        m.pstride = u.rows;
        m.count = (int32_t)nparts;
        p->merges.push_back(m);
      }
      prow += nparts * u.rows;
      ++split_units;
      if (prow > INT32_MAX / 2) return fail(AK_ERR_UNSUPPORTED, "ak_plan: split workspace too large");
    }
    p->small_merges = (int64_t)p->merges.size();
    // Launch order: longest KV range first over all items (a unit's parts are equal
    // slices of it, so unit order alone leaves long items behind short ones), so
    // the dispatcher's earliest-free order approximates longest-processing-time
    // scheduling and the grid ends on the shortest items.  Partial rows, merge jobs
    // and arrival counters are indexed explicitly, so the order is free.
    {
      // a stable counting sort by length when the lengths span a short range (the
      // usual case: parts are at most the 4096-token chunk), else a comparison sort
      const size_t n = p->small_items.size();
      int32_t lmax = 0;
      for (const Item& x : p->small_items) lmax = std::max(lmax, x.kv_end - x.kv_begin);
      std::vector<Item> sorted(n);
      if ((size_t)lmax <= 4 * n + 65536) {
        std::vector<int32_t> start((size_t)lmax + 2, 0);
        for (const Item& x : p->small_items) ++start[(size_t)(lmax - (x.kv_end - x.kv_begin)) + 1];
        for (size_t k = 1; k < start.size(); ++k) start[k] += start[k - 1];
        for (const Item& x : p->small_items) sorted[(size_t)start[(size_t)(lmax - (x.kv_end - x.kv_begin))]++] = x;
      } else {
        std::vector<uint64_t> key(n);
        for (size_t i = 0; i < n; ++i) {
          const Item& x = p->small_items[i];
          key[i] = ((uint64_t)(uint32_t)(lmax - (x.kv_end - x.kv_begin)) << 32) | (uint64_t)i;
        }
        std::sort(key.begin(), key.end());
        for (size_t i = 0; i < n; ++i) sorted[i] = p->small_items[(size_t)(key[i] & 0xFFFFFFFFu)];
      }
      p->small_items.swap(sorted);
    }
  }
  // ---- large tiles: one workgroup per segment, launched longest first so the
  // dispatcher's earliest-free-CU order approximates longest-processing-time
  // scheduling.  The cost of a segment is its 32-token KV tiles plus a fixed
  // start-up cost.  A job longer than an even share of the work over the compute
  // units (at least two minimal parts) would alone set the makespan: it is split
  // along its KV range into parts of about that share, on block boundaries,
  // merged like split small units -- but only when the makespan gain beats the
  // estimated cost of the extra partial traffic.
  if (!jobs.empty()) {
    auto tiles = [](int64_t lo, int64_t hi) { return ceil_div(hi - lo, kLargeTile); };
    const size_t nj = jobs.size();
    int64_t total = 0, longest = 0;
    for (const Item& j : jobs) {
      const int64_t c = tiles(j.kv_begin, j.kv_end) + kSegCost;
      total += c;
      longest = std::max(longest, c);
    }
    const int64_t share = std::max<int64_t>(ceil_div(total, p->num_cus), 2 * kMinPartTiles + kSegCost);
    std::vector<int32_t> nparts(nj, 1);
    if (longest > share) {
      int64_t longest_part = share;
      double split_bytes = 0.0;
      for (size_t i = 0; i < nj; ++i) {
        const int64_t t = tiles(jobs[i].kv_begin, jobs[i].kv_end);
        if (t + kSegCost <= share) continue;
        const int64_t k = std::min<int64_t>(ceil_div(t, share - kSegCost), max_splits);
        if (k < 2) continue;
        nparts[i] = (int32_t)k;
        const int64_t per = round_up(ceil_div(t, k), kBlockTiles);
        longest_part = std::max(longest_part, per + kSegCost);
        // each part writes an fp32 partial row (+ lse) that the merge reads back,
        // and the merge writes the output row
        split_bytes += (double)jobs[i].nrows * ((double)k * 2.0 * (D * 4 + 4) + D * 2);
      }
      const double gain = (double)(longest - longest_part);
      if (gain <= 2.0 * split_bytes / kTileBytes) std::fill(nparts.begin(), nparts.end(), 1);
    }
    struct Seg {
      int32_t job, lo, hi;
      int64_t cost;
    };
    std::vector<Seg> segs;
    segs.reserve(nj * 2);
    for (size_t i = 0; i < nj; ++i) {
      const Item& j = jobs[i];
      if (nparts[i] <= 1) {
        segs.push_back(Seg{(int32_t)i, j.kv_begin, j.kv_end, tiles(j.kv_begin, j.kv_end) + kSegCost});
        continue;
      }
      const int64_t t = tiles(j.kv_begin, j.kv_end);
      const int64_t per = round_up(ceil_div(t, nparts[i]), kBlockTiles) * kLargeTile;
      int64_t parts = 0;
      for (int64_t lo = j.kv_begin; lo < j.kv_end; lo += per) {
        const int64_t hi = std::min<int64_t>(j.kv_end, lo + per);
        segs.push_back(Seg{(int32_t)i, (int32_t)lo, (int32_t)hi, tiles(lo, hi) + kSegCost});
        ++parts;
      }
      nparts[i] = (int32_t)parts;
    }
    // partial rows and merge jobs for split jobs (parts of a job are consecutive)
    std::vector<int32_t> pbase_of(nj, -1);
    for (size_t i = 0; i < nj; ++i) {
      if (nparts[i] <= 1) continue;
      const Item& j = jobs[i];
      pbase_of[i] = (int32_t)prow;
      const Req& q = p->reqs[j.r];
      for (int32_t rl = 0; rl < j.nrows; ++rl) {
        const int32_t rho = j.row0 + rl;
        MergeJob m{};
        m.token = q.q_off + (rho >> lgG);
        m.head = j.hk * G + (rho & (G - 1));
        m.pfirst = (int32_t)(prow + rl);
        m.pstride = j.nrows;
        m.count = nparts[i];
        p->merges.push_back(m);
      }
      prow += (int64_t)nparts[i] * j.nrows;
      ++split_units;
      if (prow > INT32_MAX / 2) return fail(AK_ERR_UNSUPPORTED, "ak_plan: split workspace too large");
    }
    p->large_items.reserve(segs.size());
    int32_t prev = -1, part = 0;
    for (const Seg& g : segs) {
      part = g.job == prev ? part + 1 : 0;
      prev = g.job;
      Item it = jobs[(size_t)g.job];
      it.kv_begin = g.lo;
      it.kv_end = g.hi;
      it.pbase = pbase_of[(size_t)g.job] < 0 ? -1 : pbase_of[(size_t)g.job] + part * it.nrows;
      p->large_items.push_back(it);
    }
    // longest first; ties in layout order
    std::vector<int32_t> order(segs.size());
    for (size_t k = 0; k < segs.size(); ++k) order[k] = (int32_t)k;
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t x, int32_t y) { return segs[(size_t)x].cost > segs[(size_t)y].cost; });
    // The dispatcher hands workgroups to the chip's X dies in turn (workgroup x to
    // die x mod X), and each die has its own L2.  The segments of one (request, KV
    // head) read the same K/V rows, so they are kept on one die: each unit, cut
    // into pieces of at most half a die's share of the work, goes (longest piece
    // first) to the least-loaded die; each die's segments keep the longest-first
    // order; the dies' lists are interleaved, shorter ones padded with empty items
    // (zero rows, which a workgroup leaves at once).  Only for batches of few
    // units (at most two per die, e.g. one long chunk's KV heads): there each
    // unit's segments would otherwise fetch its K/V once per die (measured: 305
    // against 56 MB per launch on a 2048-token chunk, same time); with many units
    // the grouping cut no traffic and its coarser balance cost about 1%.
    const int X = p->xcds;
    size_t units = 0;
    for (size_t i = 0; i < nj; ++i)
      if (i == 0 || jobs[i].r != jobs[i - 1].r || jobs[i].hk != jobs[i - 1].hk) ++units;
    if (X > 1 && segs.size() > (size_t)X && units <= 2 * (size_t)X) {
      int64_t total_cost = 0;
      for (const Seg& g : segs) total_cost += g.cost;
      const int64_t cap = std::max<int64_t>(1, total_cost / (2 * X));
      // pieces: runs of consecutive segments of one unit (segments are in job
      // order, jobs in (request, KV head, first row) order)
      std::vector<int32_t> piece_of(segs.size());
      std::vector<int64_t> piece_cost;
      for (size_t k = 0; k < segs.size(); ++k) {
        const Item& jk = jobs[(size_t)segs[k].job];
        bool same = false;
        if (k > 0) {
          const Item& jp = jobs[(size_t)segs[k - 1].job];
          same = jp.r == jk.r && jp.hk == jk.hk && piece_cost.back() + segs[k].cost <= cap;
        }
        if (!same) piece_cost.push_back(0);
        piece_of[k] = (int32_t)piece_cost.size() - 1;
        piece_cost.back() += segs[k].cost;
      }
      std::vector<int32_t> porder(piece_cost.size());
      for (size_t k = 0; k < porder.size(); ++k) porder[k] = (int32_t)k;
      std::stable_sort(porder.begin(), porder.end(), [&](int32_t x, int32_t y) {
        return piece_cost[(size_t)x] > piece_cost[(size_t)y];
      });
      std::vector<int64_t> load((size_t)X, 0);
      std::vector<int32_t> die_of(piece_cost.size());
      for (int32_t pc : porder) {
        const size_t d = (size_t)(std::min_element(load.begin(), load.end()) - load.begin());
        die_of[(size_t)pc] = (int32_t)d;
        load[d] += piece_cost[(size_t)pc];
      }
      std::vector<std::vector<int32_t>> dies((size_t)X);
      for (int32_t k : order) dies[(size_t)die_of[(size_t)piece_of[(size_t)k]]].push_back(k);
      size_t longest_list = 0;
      for (const auto& d : dies) longest_list = std::max(longest_list, d.size());
      std::vector<int32_t> inter;
      inter.reserve(longest_list * (size_t)X);
      for (size_t i = 0; i < longest_list; ++i)
        for (int d = 0; d < X; ++d) inter.push_back(i < dies[(size_t)d].size() ? dies[(size_t)d][i] : -1);
      while (!inter.empty() && inter.back() < 0) inter.pop_back();
      order.swap(inter);
    }
    std::vector<Item> sorted;
    sorted.reserve(order.size());
    for (int32_t k : order) {
      if (k >= 0) {
        sorted.push_back(p->large_items[(size_t)k]);
      } else {
        Item pad{};
        pad.kind = 1;
        pad.pbase = -1;
        pad.merge0 = -1;
        sorted.push_back(pad);
      }
    }
    p->large_items.swap(sorted);
  }
  p->partial_rows = prow;
  p->split_units = split_units;
  return AK_OK;
}

// Bounds behind a fixed plan's workspace, following the planner above:
//  * small units (<= kSmallRows rows) number at most Hkv * min(batch, tokens); a
//    unit of len KV tokens gets at most ceil(len / t) parts, where the guided part
//    size t is at least min_chunk and at least chunk / kGuideFloor, and the chunk is
//    at least 1/(kPartsPerCu num_cus) of all small-unit KV (which is at most
//    Hkv * pages * B), so all parts together number at most units +
//    min(kGuideFloor kPartsPerCu num_cus, Hkv pages B / min_chunk) (inside the
//    guaranteed range the 4096-token chunk cap and the page-table span never bind);
//  * large jobs number at most Hkv * (ceil(tokens G / kLargeRows) + requests with
//    more than kSmallRows rows); splitting adds at most sum(t) / (share - kSegCost)
//    segments, and share >= max(sum cost / num_cus, 2 kMinPartTiles + kSegCost)
//    bounds that by 19/16 num_cus, which also bounds the split jobs;
//  * partial rows and merge jobs follow from the rows of split units and jobs.
void fixed_capacities(int32_t Hkv, int32_t G, int32_t B, int32_t num_cus, const ak_plan_opts* opts,
                      FixedCaps* c) {
  const int64_t S = (opts && opts->max_splits > 0) ? opts->max_splits : 64;
  const int64_t min_chunk =
      (opts && opts->min_chunk > 0) ? round_up(opts->min_chunk, kKvAlign) : 256;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t R = c->batch, T = c->tokens;
  const int64_t rows_all = T * G * Hkv;               // unit rows over every KV head
  const int64_t units = (int64_t)Hkv * std::min<int64_t>(R, T);
  const int64_t kv_small = std::min<int64_t>(c->pages, INT64_MAX / (64 * 256)) * B * Hkv;
  c->small = std::min<int64_t>(
      units * S, units + std::min<int64_t>((int64_t)kGuideFloor * kPartsPerCu * cus, ceil_div(kv_small, min_chunk)));
  int64_t part_small = std::min<int64_t>((int64_t)kSmallRows * c->small, S * rows_all);
  int64_t merge_small = std::min<int64_t>((int64_t)kSmallRows * units, rows_all);
  if (c->small == 0) part_small = merge_small = 0;
  // requests with more than kSmallRows rows have at least kSmallRows / G + 1 tokens
  // (none when no request may have that many)
  const int64_t Q = std::min<int64_t>(c->qlen > 0 ? c->qlen : T, T);
  const int64_t r_large = Q * G <= kSmallRows ? 0 : std::min<int64_t>(R, T / (kSmallRows / G + 1));
  const int64_t jobs =
      r_large == 0 ? 0
                   : Hkv * std::min<int64_t>(ceil_div(T * G, kLargeRows) + r_large,
                                             r_large * ceil_div(Q * G, kLargeRows));
  const int64_t extra = ceil_div(19 * cus, 16);
  c->large = jobs == 0 ? 0 : jobs + extra;
  const int64_t part_large = jobs == 0 ? 0 : std::min<int64_t>(2 * (int64_t)kLargeRows * extra, S * rows_all);
  const int64_t merge_large = jobs == 0 ? 0 : std::min<int64_t>((int64_t)kLargeRows * extra, rows_all);
  c->partial_rows = part_small + part_large;
  c->merges_small = merge_small;
  c->merges_large = merge_large;
}

}  // namespace ak
