// Internal structures shared by the host planner (plain C++) and the HIP runtime.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/ak.h"

namespace ak {

// Rows of one (request, KV head) unit are numbered rho = j * G + g: query token j
// of the request (position L - n + j), query head hk * G + g.

constexpr int kSmallRows = 16;    // rows of a small (decode-shaped) tile
constexpr int kLargeRows = 256;   // rows of a large (prefill-shaped) tile
constexpr int kKvAlign = 64;      // KV split boundaries are multiples of this
constexpr int kSmallMaxPages = 1024;  // pages a small-tile item may span (its LDS page table)
constexpr int kLargeTile = 32;    // KV tokens per tile of the large-tile cost model
constexpr int kBlockTiles = 4;    // tiles per KV block of the large-tile kernel (split boundary)
constexpr int kSegCost = 3;       // start-up cost of a large-tile segment, in tiles
constexpr int kXcds = 8;          // dies (XCDs) of the chip, each with its own L2
constexpr int kMinPartTiles = 8;  // smallest KV part a large tile job is split into, in tiles
constexpr double kTileBytes = 4.0e6;  // bytes the whole GPU streams in one large-tile time
constexpr int kPartsPerCu = 6;    // decode KV parts per compute unit the split aims at
constexpr int kStreamKPerCu = 4;  // stream-K shares per compute unit: two rounds of its two
                                  // resident decode workgroups (measured: with one round of
                                  // two, every workgroup starts at once and the long fp8
                                  // decode is 18% slower)

struct Item {          // one workgroup's work; 48 bytes
  int32_t r;           // request
  int32_t hk;          // KV head
  int32_t row0;        // first unit row
  int32_t nrows;       // rows in this tile
  int32_t kv_begin;    // first KV position
  int32_t kv_end;      // one past the last KV position
  int32_t pbase;       // partial row of unit row row0 (-1: write out/lse directly)
  int32_t kind;        // 0 small tile, 1 large tile
  int32_t merge0;      // split small tile: its unit's first merge job (also the
                       // index of the unit's arrival counter); -1 otherwise
  int32_t pad[3];
};

struct Req {           // per request; 16 bytes
  int32_t q_off;       // first query row in q/out
  int32_t n;           // query rows
  int32_t L;           // KV length
  int32_t page_off;    // kv_indptr[r]
};

struct MergeJob {      // one (query token, query head) finished from split parts; 32 bytes
  int32_t token;
  int32_t head;
  int32_t pfirst;      // partial row of part 0
  int32_t pstride;     // distance between consecutive parts' partial rows
  int32_t count;       // number of parts
  int32_t pad[3];
};

struct FixedCaps {     // capacities of a fixed plan
  int32_t batch = 0;   // requests
  int64_t tokens = 0;  // query tokens (the row count of q and out)
  int64_t qlen = 0;    // query tokens of one request
  int64_t pages = 0;   // entries of the kv_indices buffer
  int64_t small = 0, large = 0, partial_rows = 0;
  int64_t merges_small = 0, merges_large = 0;   // merge jobs of small units / large jobs
};

}  // namespace ak

struct ak_plan_t {
  int32_t R = 0, Hq = 0, Hkv = 0, D = 0, B = 0, causal = 1, window = -1, G = 1;
  int32_t log2B = 0;
  float sm_scale = 0.f;
  int64_t T = 0;
  int32_t num_cus = 256;
  // dies the large-tile segments are grouped by (1: longest first only); fixed
  // plans keep 1, since the grouping pads the work list beyond their capacity
  int32_t xcds = 1;
  bool host_only = false;
  std::vector<int32_t> kv_lens;
  std::vector<ak::Req> reqs;
  std::vector<ak::Item> small_items, large_items;
  std::vector<ak::MergeJob> merges;   // split small units' jobs first, then large jobs'
  int64_t small_merges = 0;           // jobs of split small units
  bool merge_in_kernel = false;       // small units merged inside the small-tile kernel
  bool shared_pages = false;          // requests share pages: cached (not streaming) K/V reads
  // stream-K decode: small items are grouped by persistent workgroup; workgroup g
  // runs small items wg_first[g] .. wg_first[g+1]-1
  bool stream_k = false;
  std::vector<int32_t> wg_first;
  int64_t partial_rows = 0;
  int64_t split_units = 0;
  // fixed plan: capacities the workspace is sized for (kernels are launched over
  // the whole capacity; entries past the live ones are padding with zero rows)
  bool fixed = false;
  ak::FixedCaps caps;
  int64_t hw_small = 0, hw_large = 0, hw_msmall = 0, hw_mlarge = 0;   // entries uploaded so far
  const int32_t* kv_indices = nullptr;   // device, borrowed
  int64_t num_kv_pages = 0;
  // device workspace (one allocation)
  void* d_buf = nullptr;
  size_t d_bytes = 0;
  ak::Req* d_reqs = nullptr;
  ak::Item* d_small = nullptr;
  ak::Item* d_large = nullptr;
  ak::MergeJob* d_merges = nullptr;
  ak::MergeJob* d_merges_large = nullptr;   // large jobs' merge list
  int32_t* d_counters = nullptr;            // arrival counters of split small units
  int32_t* d_wg_first = nullptr;            // stream-K: first small item of each workgroup
  float* d_part_o = nullptr;
  float* d_part_lse = nullptr;
  int device = 0;
};

namespace ak {

void set_error(const std::string& msg);

// Validates the batch and fills the host side of `p` (everything but the device
// workspace).  Pure host code: reads only the host arrays.
ak_status build_plan_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* last_page_len, int32_t batch_size, int32_t num_qo_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t causal,
                          int32_t window, const ak_plan_opts* opts, int32_t num_cus, ak_plan_t* p);

// Upper bounds on what build_plan_host emits for any batch of at most
// caps->batch requests, caps->tokens query tokens (caps->qlen in one request)
// and caps->pages pages of B tokens (fills small, large, merges_small,
// merges_large, partial_rows).  Guaranteed for page sizes >= 8 and KV lengths up to
// max_splits * (1022 * page_size - 128) with Hkv * sum(L) <= kPartsPerCu * num_cus * 4096.
void fixed_capacities(int32_t Hkv, int32_t G, int32_t B, int32_t num_cus, const ak_plan_opts* opts,
                      FixedCaps* caps);

}  // namespace ak
