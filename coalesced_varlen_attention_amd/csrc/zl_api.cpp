// C ABI entry points: argument checks, workspace layout and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>

#include "zl_internal.h"

namespace zl {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

}  // namespace zl

namespace {

zl_status fail(zl_status st, const std::string& msg) {
  zl::set_error(msg);
  return st;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Queue counters at the head of each workspace: forward kQueues, backward 2 x kQueues, each
// kCounterStride ints apart.
constexpr size_t kCounterBytes = 2 * zl::kQueues * zl::kCounterStride * sizeof(int32_t);
// Backward workspace after the counters: -D and -LSE / tau per query row, then the sentinel
// rows (64 x -inf, 64 x 0). The key-major kernel addresses the arrays with 32-bit byte
// offsets, so the query rows are limited to 2^29.
constexpr size_t kSentinelBytes = 2 * zl::kBwdRows * sizeof(float);
constexpr int64_t kMaxBwdQueryRows = INT64_C(1) << 29;

// Forward workspace after the queue counters, for split items: one counter per piece slot,
// then each piece's normalised O rows and LSEs.
size_t split_bytes(const zl_plan* plan) {
  const size_t n = (size_t)plan->split_pieces;
  if (n == 0) return 0;
  return align256(n * sizeof(int32_t)) + align256(n * (size_t)plan->fwd_rows * plan->d * sizeof(float)) +
         align256(n * (size_t)plan->fwd_rows * sizeof(float));
}

void set_split(const zl_plan* plan, void* workspace, zl::FwdParams* p) {
  const size_t n = (size_t)plan->split_pieces;
  p->n_split = (int32_t)n;
  if (n == 0) return;
  char* base = (char*)workspace + kCounterBytes;
  p->split_cnt = (int32_t*)base;
  base += align256(n * sizeof(int32_t));
  p->split_o = (float*)base;
  base += align256(n * (size_t)plan->fwd_rows * plan->d * sizeof(float));
  p->split_lse = (float*)base;
}

// Backward workspace after the sentinel rows, for split dQ items: one counter per piece slot,
// then each piece's scaled partial dQ rows.
size_t dq_split_bytes(const zl_plan* plan) {
  const size_t n = (size_t)plan->dq_split_pieces;
  if (n == 0) return 0;
  return align256(n * sizeof(int32_t)) + align256(n * (size_t)plan->dq_rows * plan->d * sizeof(float));
}

// Then, for split dK/dV items: one counter per piece slot, then each piece's partial tau dK and
// dV rows.
size_t kv_split_bytes(const zl_plan* plan) {
  const size_t n = (size_t)plan->kv_split_pieces;
  if (n == 0) return 0;
  return align256(n * sizeof(int32_t)) + align256(n * zl::kBwdKeys * 2 * plan->d * sizeof(float));
}

size_t bwd_fixed_bytes(const zl_plan* plan) {
  return kCounterBytes + 2 * align256((size_t)plan->q_rows * sizeof(float)) + align256(kSentinelBytes);
}

// Scheduler check (ZL_PLAN_COUNT_VISITS): one int32 per work item at the end of each workspace.
bool counts_visits(const zl_plan* plan) { return (plan->flags & ZL_PLAN_COUNT_VISITS) != 0; }
size_t fwd_visit_offset(const zl_plan* plan) { return kCounterBytes + split_bytes(plan); }
size_t bwd_visit_offset(const zl_plan* plan) {
  return bwd_fixed_bytes(plan) + dq_split_bytes(plan) + kv_split_bytes(plan);
}
size_t fwd_visit_bytes(const zl_plan* plan) {
  return counts_visits(plan) ? align256(plan->fwd_tiles.size() * sizeof(int32_t)) : 0;
}
// dK/dV counters, then dQ counters.
size_t bwd_visit_bytes(const zl_plan* plan) {
  return counts_visits(plan) ? align256(plan->bwd_tiles.size() * sizeof(int32_t)) +
                                   align256(plan->dq_tiles.size() * sizeof(int32_t))
                             : 0;
}

void set_fwd_visits(const zl_plan* plan, void* workspace, zl::FwdParams* p) {
  if (!counts_visits(plan)) return;
  p->visits = (int32_t*)((char*)workspace + fwd_visit_offset(plan));
  p->n_visits = (int32_t)plan->fwd_tiles.size();
}

zl_status check_runnable(const zl_plan* plan, const char* who) {
  if (!plan) return fail(ZL_ERR_INVALID, std::string(who) + ": plan is NULL");
  if (!plan->d_segs)
    return fail(ZL_ERR_INVALID, std::string(who) + ((plan->flags & ZL_PLAN_DEFERRED_UPLOAD)
                                                        ? ": the plan's tables were not uploaded (zl_plan_upload)"
                                                        : ": plan was built host-only and cannot run"));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ZL_ERR_HIP, std::string(who) + ": hipGetDevice failed");
  if (dev != plan->device)
    return fail(ZL_ERR_INVALID, std::string(who) + ": current device " + std::to_string(dev) +
                                    " is not the plan's device " + std::to_string(plan->device));
  return ZL_OK;
}

// In the QKV-packed layout the three tensors (and the three gradients) are one buffer.
bool packed_ok(const zl_plan* plan, const void* a, const void* b, const void* c) {
  return !(plan->flags & ZL_PLAN_QKV_PACKED) || (a == b && b == c);
}

bool has_final(const zl_plan* plan) {
  for (const auto& s : plan->segs)
    if (s.part < 0) return true;
  return false;
}

zl_status launch_status(int rc, const char* who) {
  if (rc != 0) {
    hipError_t e = hipGetLastError();
    return fail(ZL_ERR_HIP, std::string(who) + ": kernel launch failed: " + hipGetErrorString(e));
  }
  return ZL_OK;
}

}  // namespace

extern "C" const char* zl_last_error(void) { return zl::g_last_error.c_str(); }

extern "C" zl_status zl_plan_info(const zl_plan* plan, zl_plan_info_t* info) {
  if (!plan || !info) return fail(ZL_ERR_INVALID, "zl_plan_info: NULL argument");
  std::memset(info, 0, sizeof(*info));
  info->ws_fwd = fwd_visit_offset(plan) + fwd_visit_bytes(plan);
  info->ws_bwd = bwd_visit_offset(plan) + bwd_visit_bytes(plan);
  info->q_rows = plan->q_rows;
  info->kv_rows = plan->kv_rows;
  info->qkv_rows = (plan->flags & ZL_PLAN_QKV_PACKED) ? 3 * plan->q_rows : 0;
  info->part_rows = plan->part_rows;
  info->n_groups = (int32_t)plan->groups.size();
  info->n_parts_max = plan->n_parts_max;
  info->fwd_tiles = (int64_t)plan->fwd_tiles.size();
  info->bwd_tiles = (int64_t)plan->bwd_tiles.size();
  info->fwd_flops = plan->fwd_flops;
  info->bwd_flops = 2.5 * plan->fwd_flops;
  info->dq_tiles = (int64_t)plan->dq_tiles.size();
  info->d_head = plan->d;
  info->softmax_scale = plan->scale;
  info->split_tiles = plan->split_tiles;
  info->split_pieces = plan->split_pieces;
  info->dq_split_tiles = plan->dq_split_tiles;
  info->dq_split_pieces = plan->dq_split_pieces;
  info->kv_split_tiles = plan->kv_split_tiles;
  info->kv_split_pieces = plan->kv_split_pieces;
  info->dev_bytes = plan->dev_bytes;
  info->fwd_rows = plan->fwd_rows;
  info->dq_rows = plan->dq_rows;
  info->visits_fwd = info->visits_dkdv = info->visits_dq = -1;
  if (counts_visits(plan)) {
    info->visits_fwd = (int64_t)fwd_visit_offset(plan);
    info->visits_dkdv = (int64_t)bwd_visit_offset(plan);
    info->visits_dq = (int64_t)(bwd_visit_offset(plan) + align256(plan->bwd_tiles.size() * sizeof(int32_t)));
  }
  return ZL_OK;
}

extern "C" zl_status zl_plan_group(const zl_plan* plan, int32_t g, zl_group_info_t* info) {
  if (!plan || !info) return fail(ZL_ERR_INVALID, "zl_plan_group: NULL argument");
  if (g < 0 || g >= (int32_t)plan->groups.size())
    return fail(ZL_ERR_INVALID, "zl_plan_group: group " + std::to_string(g) + " out of range");
  *info = plan->groups[g];
  return ZL_OK;
}

extern "C" zl_status zl_plan_tiles(const zl_plan* plan, int32_t which, int32_t* out, int64_t cap, int64_t* count) {
  if (!plan || !count) return fail(ZL_ERR_INVALID, "zl_plan_tiles: NULL argument");
  if (which < 0 || which > 5) return fail(ZL_ERR_INVALID, "zl_plan_tiles: which must be 0 to 5");
  const auto& v = which == 0 || which == 3 ? plan->fwd_tiles
                  : which == 1 || which == 5 ? plan->bwd_tiles
                                             : plan->dq_tiles;
  const int w = which >= 3 ? 8 : 4;
  *count = (int64_t)v.size();
  if (cap < 0) return fail(ZL_ERR_INVALID, "zl_plan_tiles: negative capacity");
  if (cap > 0 && !out) return fail(ZL_ERR_INVALID, "zl_plan_tiles: out is NULL");
  const int64_t n = std::min<int64_t>(cap, (int64_t)v.size());
  for (int64_t i = 0; i < n; ++i) {
    out[w * i + 0] = v[i].seg;
    out[w * i + 1] = v[i].head;
    out[w * i + 2] = v[i].row0;
    out[w * i + 3] = v[i].nrows;
    if (w == 8) {
      out[w * i + 4] = v[i].kv_begin;
      out[w * i + 5] = v[i].kv_end;
      out[w * i + 6] = v[i].split;
      out[w * i + 7] = v[i].piece;
    }
  }
  return ZL_OK;
}

extern "C" zl_status zl_plan_queues(const zl_plan* plan, int32_t which, int32_t* bounds, int32_t cap,
                                    int32_t* n_queues) {
  if (!plan || !n_queues) return fail(ZL_ERR_INVALID, "zl_plan_queues: NULL argument");
  if (which < 0 || which > 5) return fail(ZL_ERR_INVALID, "zl_plan_queues: which must be 0 to 5");
  const auto& b = which == 0 || which == 3 ? plan->fwd_bounds
                  : which == 1 || which == 5 ? plan->bwd_bounds
                                             : plan->dq_bounds;
  *n_queues = zl::kQueues;
  if (cap < 0 || (cap > 0 && !bounds)) return fail(ZL_ERR_INVALID, "zl_plan_queues: bad output buffer");
  for (int32_t i = 0; i < std::min<int32_t>(cap, (int32_t)b.size()); ++i) bounds[i] = b[i];
  return ZL_OK;
}

// A queue set for a launch: the plan's items on the device, counters in the workspace, and the
// host copy of the bounds as kernel arguments.
zl::Queues make_queues(const zl::Tile* items, int32_t* counters, const std::vector<int32_t>& bounds) {
  zl::Queues q{};
  q.items = items;
  q.counters = counters;
  for (int k = 0; k <= zl::kQueues; ++k) q.bounds[k] = bounds[k];
  return q;
}

extern "C" zl_status zl_attn_fwd(const zl_plan* plan, const void* q, const void* k, const void* v, float* o,
                                 float* lse, float* o_part, float* lse_part, void* workspace, void* stream) {
  zl_status st = check_runnable(plan, "zl_attn_fwd");
  if (st != ZL_OK) return st;
  if (!q || !k || !v) return fail(ZL_ERR_INVALID, "zl_attn_fwd: q, k or v is NULL");
  if (!packed_ok(plan, q, k, v)) return fail(ZL_ERR_INVALID, "zl_attn_fwd: a QKV-packed plan needs q == k == v");
  if (!workspace) return fail(ZL_ERR_INVALID, "zl_attn_fwd: workspace is NULL");
  if (has_final(plan) && (!o || !lse)) return fail(ZL_ERR_INVALID, "zl_attn_fwd: o or lse is NULL");
  if (!plan->groups.empty() && (!o_part || !lse_part))
    return fail(ZL_ERR_INVALID, "zl_attn_fwd: the plan has ring groups but o_part or lse_part is NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(o_part, 16) ||
      !aligned(workspace, 16) || !aligned(lse, 4) || !aligned(lse_part, 4))
    return fail(ZL_ERR_INVALID, "zl_attn_fwd: q/k/v/o/o_part/workspace must be 16-byte aligned, lse 4-byte");
  zl::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.segs = plan->d_segs;
  p.queue = make_queues(plan->d_fwd, (int32_t*)workspace, plan->fwd_bounds);
  p.scale_log2 = plan->scale * 1.4426950408889634f;
  set_split(plan, workspace, &p);
  set_fwd_visits(plan, workspace, &p);
  p.packed = (plan->flags & ZL_PLAN_QKV_PACKED) ? 1 : 0;
  const int per_cu = zl::fwd_blocks_per_cu(plan->d, plan->fwd_rows);
  if (per_cu < 1) return fail(ZL_ERR_HIP, "zl_attn_fwd: forward kernel cannot be resident");
  const int grid = (int)std::min<int64_t>((int64_t)plan->n_cu * per_cu, (int64_t)plan->fwd_tiles.size());
  return launch_status(zl::launch_fwd(plan->d, plan->fwd_rows, p, grid, stream), "zl_attn_fwd");
}

extern "C" zl_status zl_attn_fwd_accumulate(const zl_plan* plan, const void* q, const void* k, const void* v,
                                            float* o, float* lse, void* workspace, void* stream) {
  if (!plan) return fail(ZL_ERR_INVALID, "zl_attn_fwd_accumulate: plan is NULL");
  for (const zl_group_info_t& g : plan->groups)
    if (g.n_parts > 1)
      return fail(ZL_ERR_INVALID,
                  "zl_attn_fwd_accumulate: a group has " + std::to_string(g.n_parts) +
                      " parts in this plan; two parts of one group would fold into the same rows at once");
  zl_status st = check_runnable(plan, "zl_attn_fwd_accumulate");
  if (st != ZL_OK) return st;
  if (!q || !k || !v) return fail(ZL_ERR_INVALID, "zl_attn_fwd_accumulate: q, k or v is NULL");
  if (!packed_ok(plan, q, k, v))
    return fail(ZL_ERR_INVALID, "zl_attn_fwd_accumulate: a QKV-packed plan needs q == k == v");
  if (!workspace) return fail(ZL_ERR_INVALID, "zl_attn_fwd_accumulate: workspace is NULL");
  if (!o || !lse) return fail(ZL_ERR_INVALID, "zl_attn_fwd_accumulate: o or lse is NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(workspace, 16) ||
      !aligned(lse, 4))
    return fail(ZL_ERR_INVALID, "zl_attn_fwd_accumulate: q/k/v/o/workspace must be 16-byte aligned, lse 4-byte");
  zl::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.segs = plan->d_segs;
  p.queue = make_queues(plan->d_fwd, (int32_t*)workspace, plan->fwd_bounds);
  p.scale_log2 = plan->scale * 1.4426950408889634f;
  p.accumulate = 1;
  set_split(plan, workspace, &p);
  set_fwd_visits(plan, workspace, &p);
  p.packed = (plan->flags & ZL_PLAN_QKV_PACKED) ? 1 : 0;
  const int per_cu = zl::fwd_blocks_per_cu(plan->d, plan->fwd_rows);
  if (per_cu < 1) return fail(ZL_ERR_HIP, "zl_attn_fwd_accumulate: forward kernel cannot be resident");
  const int grid = (int)std::min<int64_t>((int64_t)plan->n_cu * per_cu, (int64_t)plan->fwd_tiles.size());
  return launch_status(zl::launch_fwd(plan->d, plan->fwd_rows, p, grid, stream), "zl_attn_fwd_accumulate");
}

extern "C" zl_status zl_lse_merge(int32_t n_parts, int64_t n_rows, int32_t d_head, const float* o_part,
                                  const float* lse_part, float* o, float* lse, void* stream) {
  if (d_head != 64 && d_head != 128)
    return fail(ZL_ERR_UNSUPPORTED, "zl_lse_merge: d_head " + std::to_string(d_head) + " is not 64 or 128");
  if (n_parts < 1) return fail(ZL_ERR_INVALID, "zl_lse_merge: n_parts must be >= 1");
  if (n_rows < 0) return fail(ZL_ERR_INVALID, "zl_lse_merge: n_rows must be >= 0");
  if (n_rows == 0) return ZL_OK;
  if (!o_part || !lse_part || !o || !lse) return fail(ZL_ERR_INVALID, "zl_lse_merge: NULL pointer");
  if (!aligned(o_part, 16) || !aligned(o, 16) || !aligned(lse_part, 4) || !aligned(lse, 4))
    return fail(ZL_ERR_INVALID, "zl_lse_merge: o_part and o must be 16-byte aligned, lse 4-byte");
  const int rows_per_block = zl::merge_rows(d_head);
  const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  const int grid = (int)std::min<int64_t>(blocks, zl::kMergeMaxGrid);
  return launch_status(zl::launch_merge(d_head, n_parts, n_rows, o_part, lse_part, o, lse, grid, stream),
                       "zl_lse_merge");
}

extern "C" zl_status zl_plan_merge(const zl_plan* plan, const float* o_part, const float* lse_part, float* o,
                                   float* lse, void* stream) {
  zl_status st = check_runnable(plan, "zl_plan_merge");
  if (st != ZL_OK) return st;
  if (plan->groups.empty()) return ZL_OK;
  if (!o_part || !lse_part || !o || !lse) return fail(ZL_ERR_INVALID, "zl_plan_merge: NULL pointer");
  if (!aligned(o_part, 16) || !aligned(o, 16) || !aligned(lse_part, 4) || !aligned(lse, 4))
    return fail(ZL_ERR_INVALID, "zl_plan_merge: o_part and o must be 16-byte aligned, lse 4-byte");
  const int grid = (int)std::min<int64_t>(plan->merge_blocks, zl::kMergeMaxGrid);
  return launch_status(zl::launch_plan_merge(plan->d, plan->d_groups, (int32_t)plan->gdev.size(), plan->merge_blocks,
                                             o_part, lse_part, o, lse, grid, stream),
                       "zl_plan_merge");
}

extern "C" zl_status zl_attn_bwd(const zl_plan* plan, const void* q, const void* k, const void* v, const float* o,
                                 const float* lse, const void* d_o, float* dq, float* dk, float* dv, void* workspace,
                                 void* stream) {
  return zl_attn_bwd_stages(plan, q, k, v, o, lse, d_o, dq, dk, dv, workspace, ZL_BWD_ALL, stream);
}

extern "C" zl_status zl_attn_bwd_stages(const zl_plan* plan, const void* q, const void* k, const void* v,
                                        const float* o, const float* lse, const void* d_o, float* dq, float* dk,
                                        float* dv, void* workspace, uint32_t stages, void* stream) {
  if (stages == 0 || (stages & ~ZL_BWD_ALL)) return fail(ZL_ERR_INVALID, "zl_attn_bwd: bad stage mask");
  zl_status st = check_runnable(plan, "zl_attn_bwd");
  if (st != ZL_OK) return st;
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv || !workspace)
    return fail(ZL_ERR_INVALID, "zl_attn_bwd: NULL pointer");
  if (plan->q_rows > kMaxBwdQueryRows)
    return fail(ZL_ERR_UNSUPPORTED, "zl_attn_bwd: more than 2^29 query rows");
  if (!packed_ok(plan, q, k, v) || !packed_ok(plan, dq, dk, dv))
    return fail(ZL_ERR_INVALID, "zl_attn_bwd: a QKV-packed plan needs q == k == v and dq == dk == dv");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(d_o, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16) || !aligned(lse, 4))
    return fail(ZL_ERR_INVALID, "zl_attn_bwd: tensors and workspace must be 16-byte aligned, lse 4-byte");
  zl::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.d_o = d_o;
  p.o = o;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.kvq = make_queues(plan->d_bwd, (int32_t*)workspace, plan->bwd_bounds);
  p.dqq = make_queues(plan->d_dq, (int32_t*)workspace + zl::kQueues * zl::kCounterStride, plan->dq_bounds);
  p.dneg = (float*)((char*)workspace + kCounterBytes);
  p.lsec = (float*)((char*)workspace + kCounterBytes + align256((size_t)plan->q_rows * sizeof(float)));
  p.sentinel = (float*)((char*)workspace + kCounterBytes + 2 * align256((size_t)plan->q_rows * sizeof(float)));
  p.n_dq_split = plan->dq_split_pieces;
  if (p.n_dq_split > 0) {
    char* base = (char*)workspace + bwd_fixed_bytes(plan);
    p.dq_split_cnt = (int32_t*)base;
    p.dq_split = (float*)(base + align256((size_t)p.n_dq_split * sizeof(int32_t)));
  }
  p.n_kv_split = plan->kv_split_pieces;
  if (p.n_kv_split > 0) {
    char* base = (char*)workspace + bwd_fixed_bytes(plan) + dq_split_bytes(plan);
    p.kv_split_cnt = (int32_t*)base;
    p.kv_split = (float*)(base + align256((size_t)p.n_kv_split * sizeof(int32_t)));
  }
  if (counts_visits(plan)) {
    p.kv_visits = (int32_t*)((char*)workspace + bwd_visit_offset(plan));
    p.dq_visits = (int32_t*)((char*)p.kv_visits + align256(plan->bwd_tiles.size() * sizeof(int32_t)));
    p.n_kv_visits = (int32_t)plan->bwd_tiles.size();
    p.n_dq_visits = (int32_t)plan->dq_tiles.size();
  }
  p.segs = plan->d_segs;
  p.pre_tiles = plan->d_pre;
  p.n_pre = (int32_t)plan->pre_tiles.size();
  p.kv_ranges = plan->d_ranges;
  p.scale = plan->scale;
  p.scale_log2 = plan->scale * 1.4426950408889634f;
  p.packed = (plan->flags & ZL_PLAN_QKV_PACKED) ? 1 : 0;
  const int per_cu = zl::bwd_blocks_per_cu(plan->d);
  const int per_cu_dq = zl::dq_blocks_per_cu(plan->d, plan->dq_rows);
  if (per_cu < 1 || per_cu_dq < 1) return fail(ZL_ERR_HIP, "zl_attn_bwd: backward kernels cannot be resident");
  const int grid = (int)std::min<int64_t>((int64_t)plan->n_cu * per_cu, (int64_t)plan->bwd_tiles.size());
  const int grid_dq = (int)std::min<int64_t>((int64_t)plan->n_cu * per_cu_dq, (int64_t)plan->dq_tiles.size());
  const int grid_pre = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)plan->n_cu * 8, p.n_pre));
  p.kv_grid = grid;
  p.dq_grid = grid_dq;
  return launch_status(zl::launch_bwd(plan->d, plan->dq_rows, p, grid_pre, grid, grid_dq, stages, stream), "zl_attn_bwd");
}
