// Internal declarations shared by the host runtime (plan, API) and the HIP kernels.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "zl.h"

namespace zl {

// Query-major queue items: a forward item is fwd_rows query rows of one (segment, head); a
// backward dQ item is dq_rows query rows of one (final segment or ring group, head), looping
// over every key range of the segment (all parts of a ring group). Each is 32 rows per wave of
// its workgroup, and a plan uses one size per queue: narrow items (4 waves, two workgroups per
// CU) or wide items (8 waves, one workgroup per CU). Backward dK/dV queue item: 128 key rows
// of one (segment, head), looping over the segment's query rows in blocks of 64.
constexpr int kFwdRowsNarrow = 128;
constexpr int kFwdRowsWide = 256;
constexpr int kDqRowsNarrow = 128;
constexpr int kDqRowsWide = 256;
// Wide items share each K/V block in LDS among 8 waves, which halves the global-to-LDS loads
// per query row. But a compute unit sits idle once its one workgroup runs out of work, so a
// plan takes narrow items for a queue of 1 to kWideRounds rounds of wide items, and for a few
// short items (see zl_plan_build).
constexpr int kWideRounds = 4;
constexpr int kFwdKeys = 64;  // keys per forward step
// Split-KV of forward items (short queues leave compute units idle): a plan whose forward
// queue holds fewer than kSplitWaves waves of items for the device's resident workgroups cuts
// every item that costs more than 1/kSplitTargetWaves of a workgroup's fair share into key
// pieces of about that share (at most kMaxPieces, each at least kMinPieceKeys keys,
// block-aligned). One wave: a
// compute unit running one forward workgroup still reaches about 80% of its two-workgroup
// rate, so longer queues lose little to their tail.
constexpr int kSplitWaves = 1;
constexpr int kSplitTargetWaves = 1;  // about one piece per resident workgroup: each piece
                                      // costs a partial write and its share of a merge
constexpr int kMaxPieces = 16;
constexpr int kMinPieceKeys = 1024;
// Resident workgroups assumed by a host-only plan: 256 CUs x 2 for the narrow forward and dQ
// kernels, x 1 for the wide ones and for the dK/dV kernel.
constexpr int kHostOnlySlots = 512;
constexpr int kHostOnlyWideSlots = 256;
constexpr int kHostOnlyKvSlots = 256;
constexpr int kBwdKeys = 128;
constexpr int kBwdRows = 64;
// Rows (token, head pairs) per item of the backward pre-pass: one pass of its workgroup (16
// groups of 16 lanes, 8 rows each).
constexpr int kPreRows = 128;
// Work queues per launch: one per XCD. Workgroup b starts on queue b % kQueues (the XCD the
// hardware dispatches it to) and steals from the others once its own queue is empty.
constexpr int kQueues = 8;
constexpr int kCounterStride = 16;  // ints between queue counters (64 bytes)

// Workgroups of a grid of `grid` whose home is queue k. The j-th of them takes item j of its
// home queue as its first item without an atomic, so a launch starts queue k's counter at this
// count and the atomics hand out the items after those.
__host__ __device__ constexpr int32_t home_count(int grid, int k) { return (grid - k + kQueues - 1) / kQueues; }

// A segment as the kernels see it. Rows are (token, head) pairs of d contiguous values.
// O, LSE and dO always use the planar query-side layout (q_row0, nh rows per token). Q, K, V
// and their gradients are planar too (Q at q_row0, K and V at kv_row0), or, in the QKV-packed
// layout [tokens][Q, K, V][heads][d] (equal query and key lengths), one buffer in which the
// sequence starts at row 3 q_row0 with 3 nh rows per token and K, V nh and 2 nh rows after Q.
struct alignas(16) SegDev {
  int64_t q_row0;     // query-side row of (token 0, head 0) of the segment's sequence
  int64_t kv_row0;    // key-side row of (token 0, head 0)
  int64_t part_row0;  // slab row of (token q_begin, head head_begin) for a ring part, else -1
  int32_t nh;         // stored heads of the sequence (row stride between tokens = nh rows)
  int32_t q_begin, q_end, kv_begin, kv_end;
  int32_t head_begin, head_end;
  int32_t part;
  int32_t chain_off;  // first (kv_begin, kv_end) pair of this segment's key-range chain
  int32_t chain_len;  // pairs in the chain: 1, or the parts of a ring group (on part 0)
  int32_t lq;         // query tokens of the sequence (head-major row = q_row0 + h * lq + t)
  int32_t pad[3];
};
static_assert(sizeof(SegDev) == 80, "SegDev must stay 80 bytes");

// Q / K / V (and gradient) rows of a segment: token stride, row of (token 0, head 0) of Q and
// of K, and rows from K to V.
struct QkvRows {
  int32_t t_stride;
  int64_t q0, k0;
  int32_t v_off;
};
template <bool kPacked>
__host__ __device__ __forceinline__ QkvRows qkv_rows(const SegDev& sg) {
  if (kPacked) return {3 * sg.nh, 3 * sg.q_row0, 3 * sg.q_row0 + sg.nh, sg.nh};
  return {sg.nh, sg.q_row0, sg.kv_row0, 0};
}

// A KV-split group as the merge kernel sees it: its slab rows (token-major over its head
// subset) and where each lands in O/LSE.
struct alignas(16) GroupDev {
  int64_t part_row;  // slab row of part 0, row 0
  int64_t o_row;     // O/LSE row of (token q_begin, head head_begin)
  int64_t n_rows;    // tokens x n_sub
  int64_t block0;    // first merge block of the group (blocks of merge_rows(d) rows)
  int32_t n_parts;
  int32_t nh;        // stored heads of the sequence: O/LSE rows between consecutive tokens
  int32_t n_sub;     // heads in the group
  int32_t pad;
};
static_assert(sizeof(GroupDev) == 48, "GroupDev must stay 48 bytes");

// Rows one merge workgroup (256 lanes, d/4 lanes per row) handles per pass; merge launches use
// one workgroup per pass up to kMergeMaxGrid workgroups.
constexpr int merge_rows(int d) { return 256 / (d / 4); }
constexpr int64_t kMergeMaxGrid = INT64_C(1) << 20;

// One work item: segment index, head, first row (token) of the block, rows in the block, and
// the range it loops over: for a forward item its keys [kv_begin, kv_end) (the segment's, or a
// piece of them); for a dQ item a run [kv_begin, kv_end) of the 64-key blocks of its segment's
// key-range chain; for a dK/dV item a run of the segment's 64-row query blocks. A piece of a
// split item carries the workspace slot of its piece 0 (split, -1 otherwise) and
// piece = index | (pieces << 16).
struct alignas(16) Tile {
  int32_t seg, head, row0, nrows;
  int32_t kv_begin, kv_end, split, piece;
};
static_assert(sizeof(Tile) == 32, "Tile must stay 32 bytes");

// A set of kQueues work queues: items stored queue by queue, bounds[k]..bounds[k+1] for
// queue k (kernel arguments, so that no item index waits on a load of them), and one counter
// per queue (kCounterStride ints apart) in the caller's workspace.
struct Queues {
  const Tile* items;
  int32_t* counters;
  int32_t bounds[kQueues + 1];
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  float* o_part;
  float* lse_part;
  const SegDev* segs;
  Queues queue;
  float scale_log2;  // softmax scale times log2(e)
  int32_t accumulate;  // ring parts fold into o/lse (running merge) instead of the slab
  int32_t n_split;     // pieces of split items (slots of split_cnt, split_o, split_lse)
  int32_t* split_cnt;  // per split item (at its piece-0 slot): pieces finished
  float* split_o;      // [n_split][fwd_rows][D] normalised piece results
  float* split_lse;    // [n_split][fwd_rows]
  int32_t packed;      // Q, K, V in the QKV-packed layout (selects the kernel instance)
  int32_t* visits;     // per forward item: workgroups that took it (ZL_PLAN_COUNT_VISITS), or null
  int32_t n_visits;    // forward items (counters cleared before the launch)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const float* o;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* dneg;  // per query row: -D = -sum_c dO * O, head-major rows (workspace)
  float* lsec;  // per query row: -LSE / tau, head-major rows (workspace)
  float* sentinel;  // 64 x -inf then 64 x 0 (workspace): row values past a segment's end
  const SegDev* segs;
  Queues kvq;             // dK/dV queues
  Queues dqq;             // dQ queues
  const Tile* pre_tiles;  // (segment, head_begin, first token, tokens) per pre-pass item
  int32_t n_pre;
  const int32_t* kv_ranges;  // (kv_begin, kv_end) pairs of the key-range chains
  float scale;       // softmax scale
  float scale_log2;  // softmax scale times log2(e)
  int32_t packed;    // Q, K, V and their gradients in the QKV-packed layout (kernel instance)
  int32_t n_dq_split;     // pieces of split dQ items (slots of dq_split_cnt, dq_split)
  int32_t* dq_split_cnt;  // per split dQ item (at its piece-0 slot): pieces finished
  float* dq_split;        // [n_dq_split][dq_rows][D] scaled partial dQ of each piece
  int32_t n_kv_split;     // pieces of split dK/dV items (slots of kv_split_cnt, kv_split)
  int32_t* kv_split_cnt;  // per split dK/dV item (at its piece-0 slot): pieces finished
  float* kv_split;        // [n_kv_split][kBwdKeys][2][D] partial tau dK and dV of each piece
  int32_t* kv_visits;     // per dK/dV item, per dQ item: workgroups that took it (ZL_PLAN_COUNT_VISITS),
  int32_t* dq_visits;     // or null; both cleared by the pre-pass
  int32_t n_kv_visits, n_dq_visits;
  int32_t kv_grid, dq_grid;  // workgroups of the dK/dV and dQ launches (the pre-pass sets their
                             // queue counters to the home counts)
};

// Kernel launchers (defined next to their kernels). They return the launch status.
int launch_fwd(int d, int rows, const FwdParams& p, int grid, void* stream);
int launch_bwd(int d, int dq_rows, const BwdParams& p, int grid_pre, int grid, int grid_dq, unsigned stages,
               void* stream);
int launch_plan_merge(int d, const GroupDev* groups, int32_t n_groups, int64_t n_blocks, const float* o_part,
                      const float* lse_part, float* o, float* lse, int grid, void* stream);
int launch_merge(int d, int32_t n_parts, int64_t n_rows, const float* o_part, const float* lse_part,
                 float* o, float* lse, int grid, void* stream);
// Workgroups of each persistent kernel that fit on one compute unit (the forward kernel's for
// items of `rows` query rows).
int fwd_blocks_per_cu(int d, int rows);
int bwd_blocks_per_cu(int d);
int dq_blocks_per_cu(int d, int rows);

void set_error(const std::string& msg);

}  // namespace zl

struct zl_plan;
namespace zl {
void set_table_pointers(zl_plan* plan, void* block);
}  // namespace zl

struct zl_plan {
  int32_t d = 0;
  int32_t n_seq = 0;
  float scale = 0.f;
  uint32_t flags = 0;
  int device = -1;
  int n_cu = 0;
  int64_t q_rows = 0, kv_rows = 0, part_rows = 0;
  int32_t fwd_rows = zl::kFwdRowsNarrow;  // query rows per forward item
  int32_t dq_rows = zl::kDqRowsNarrow;    // query rows per dQ item
  int32_t n_parts_max = 0;
  double fwd_flops = 0.0;
  std::vector<zl::SegDev> segs;
  std::vector<zl::Tile> fwd_tiles, bwd_tiles, pre_tiles, dq_tiles;  // queue by queue
  std::vector<int32_t> fwd_bounds, bwd_bounds, dq_bounds;            // kQueues + 1 each
  std::vector<int32_t> kv_ranges;
  std::vector<zl_group_info_t> groups;
  std::vector<zl::GroupDev> gdev;
  int64_t merge_blocks = 0;  // total blocks of a plan merge launch
  int32_t split_tiles = 0;   // forward items cut into key pieces
  int32_t split_pieces = 0;  // pieces of those items (slots of the split workspace)
  int32_t dq_split_tiles = 0;   // dQ items cut into pieces of their key-block chain
  int32_t dq_split_pieces = 0;  // pieces of those items (slots of the backward split workspace)
  int32_t kv_split_tiles = 0;   // dK/dV items cut into pieces of their query blocks
  int32_t kv_split_pieces = 0;  // pieces of those items
  // device copies: one block carved into the tables at table_off (segments, forward, dK/dV,
  // pre-pass and dQ items, key-range chains, groups); owned (dev_block) unless the
  // plan was built with ZL_PLAN_DEFERRED_UPLOAD, whose tables zl_plan_upload copies into caller
  // memory from `image` (kept until then)
  size_t dev_bytes = 0;
  size_t table_off[7] = {};
  std::vector<char> image;
  void* dev_block = nullptr;
  const zl::SegDev* d_segs = nullptr;
  const zl::Tile* d_fwd = nullptr;
  const zl::Tile* d_bwd = nullptr;
  const zl::Tile* d_pre = nullptr;
  const zl::Tile* d_dq = nullptr;
  const int32_t* d_ranges = nullptr;
  const zl::GroupDev* d_groups = nullptr;
};
