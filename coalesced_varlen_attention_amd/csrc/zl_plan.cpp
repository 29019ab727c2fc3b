// Plan building: validation of the segment list and its lowering into device work queues.
//
// This is the rank-local lowering of the Zellige page (Moldable Sequence Placement for
// Mixed Image-Video DiT Training, §IV-D "Coalesced Attention Engine"): the segments one GPU
// holds (whole sequences, Ulysses head shards, ring KV-split parts; the (q,h,k) axes of
// §IV-A / Table II) become one list of equal-shaped work items for one persistent launch,
// without mixing attention across sequences. The pages order work by decreasing split
// degree and pack fillers by decreasing price (§IV-C, Filler Packing); here the single GPU
// has no collectives to order, so items are ordered by decreasing cost (rows x length of
// the other side, the quadratic attention cost of §II-A) to keep the persistent workgroups
// busy until the end, with ties left in (segment, head, block) order so that items sharing
// K/V run side by side.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <tuple>

#include "zl_internal.h"

namespace zl {

// Point the plan's device table pointers into a block laid out as the plan's image.
void set_table_pointers(zl_plan* plan, void* block) {
  char* b = (char*)block;
  plan->d_segs = (const SegDev*)(b + plan->table_off[0]);
  plan->d_fwd = (const Tile*)(b + plan->table_off[1]);
  plan->d_bwd = (const Tile*)(b + plan->table_off[2]);
  plan->d_pre = (const Tile*)(b + plan->table_off[3]);
  plan->d_dq = (const Tile*)(b + plan->table_off[4]);
  plan->d_ranges = (const int32_t*)(b + plan->table_off[5]);
  plan->d_groups = (const GroupDev*)(b + plan->table_off[6]);
}

}  // namespace zl

namespace {

zl_status fail(zl_status st, const std::string& msg) {
  zl::set_error(msg);
  return st;
}

std::string seg_str(int i, const zl_segment& s) {
  char buf[200];
  snprintf(buf, sizeof(buf), "segment %d {seq %d, heads [%d,%d), q [%d,%d), kv [%d,%d), part %d}", i, s.seq,
           s.head_begin, s.head_end, s.q_begin, s.q_end, s.kv_begin, s.kv_end, s.part);
  return buf;
}

struct Rect {  // a block of rows of one sequence: tokens [t0,t1) x heads [h0,h1)
  int32_t t0, t1, h0, h1;
  int32_t owner;  // segment index (or group id for grouped outputs)
  int32_t group;  // group id, -1 for a final segment
};

bool overlap(const Rect& a, const Rect& b) {
  return a.t0 < b.t1 && b.t0 < a.t1 && a.h0 < b.h1 && b.h0 < a.h1;
}

// Reports the first pair of overlapping rectangles (ignoring pairs in the same group).
bool find_overlap(std::vector<Rect>& rs, bool same_group_ok, int* a, int* b) {
  std::sort(rs.begin(), rs.end(), [](const Rect& x, const Rect& y) { return x.t0 < y.t0; });
  for (size_t i = 0; i < rs.size(); ++i) {
    for (size_t j = i + 1; j < rs.size() && rs[j].t0 < rs[i].t1; ++j) {
      if (same_group_ok && rs[i].group >= 0 && rs[i].group == rs[j].group) continue;
      if (overlap(rs[i], rs[j])) {
        *a = rs[i].owner;
        *b = rs[j].owner;
        return true;
      }
    }
  }
  return false;
}

struct Item {
  zl::Tile t;
  int64_t cost;
};

// Split the items (in (segment, head, block) order) into chunks of consecutive items of one
// unit with bounded total cost, assign the chunks to the kQueues queues by decreasing chunk
// cost to the least-loaded queue, and emit each queue sorted by decreasing item cost (stable).
void distribute(const std::vector<Item>& items, const std::vector<int64_t>& unit, std::vector<zl::Tile>* out,
                std::vector<int32_t>* bounds) {
  int64_t total = 0, biggest = 0;
  for (const Item& it : items) {
    total += it.cost;
    biggest = std::max(biggest, it.cost);
  }
  const int64_t cap = std::max<int64_t>(biggest, total / (zl::kQueues * 16) + 1);
  struct Chunk {
    size_t begin, end;
    int64_t cost;
  };
  std::vector<Chunk> chunks;
  for (size_t i = 0; i < items.size();) {
    Chunk c{i, i, 0};
    while (c.end < items.size() && unit[c.end] == unit[i] && (c.end == i || c.cost + items[c.end].cost <= cap)) {
      c.cost += items[c.end].cost;
      ++c.end;
    }
    chunks.push_back(c);
    i = c.end;
  }
  std::vector<size_t> order(chunks.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return chunks[a].cost > chunks[b].cost; });
  std::vector<int64_t> load(zl::kQueues, 0);
  std::vector<std::vector<size_t>> members(zl::kQueues);
  for (size_t ci : order) {
    const int q = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[q] += chunks[ci].cost;
    members[q].push_back(ci);
  }
  out->clear();
  out->reserve(items.size());
  bounds->assign(1, 0);
  // Per queue: decreasing cost, ties in (segment, head, block) order, as (cost, position) keys.
  struct Key {
    int64_t cost;
    size_t pos;
  };
  std::vector<Key> keys;
  keys.reserve(items.size());
  for (int q = 0; q < zl::kQueues; ++q) {
    std::sort(members[q].begin(), members[q].end());  // back to (segment, head, block) order
    keys.clear();
    for (size_t ci : members[q])
      for (size_t k = chunks[ci].begin; k < chunks[ci].end; ++k) keys.push_back({items[k].cost, k});
    std::sort(keys.begin(), keys.end(),
              [](const Key& a, const Key& b) { return a.cost != b.cost ? a.cost > b.cost : a.pos < b.pos; });
    for (const Key& k : keys) out->push_back(items[k.pos].t);
    bounds->push_back((int32_t)out->size());
  }
}

// Split-KV of the forward queue. With fewer items than resident workgroups, compute units sit
// idle while a few long items run; cutting those items into key pieces, each computed as a
// normalised partial and merged by the last piece to finish (the exact merge of ring
// accumulation), gives every unit work. Applies only when the queue holds fewer than
// kSplitWaves waves; items above the cost target are cut into block-aligned pieces of at
// least kMinPieceKeys keys.
void split_forward(int64_t slots, std::vector<Item>* fwd, std::vector<int64_t>* unit, int32_t* n_tiles,
                   int32_t* n_pieces) {
  *n_tiles = 0;
  *n_pieces = 0;
  if (fwd->empty() || (int64_t)fwd->size() >= (int64_t)zl::kSplitWaves * slots) return;
  double total = 0.0;
  for (const Item& it : *fwd) total += (double)it.cost;
  const double target = total / ((double)zl::kSplitTargetWaves * (double)slots);
  std::vector<Item> out;
  std::vector<int64_t> out_unit;
  int64_t next = 0;
  for (size_t j = 0; j < fwd->size(); ++j) {
    const Item& it = (*fwd)[j];
    const int64_t nk = it.t.kv_end - it.t.kv_begin;
    const int64_t nb = (nk + zl::kFwdKeys - 1) / zl::kFwdKeys;
    int64_t n = (int64_t)std::llround((double)it.cost / target);  // nearest: a ragged queue tail
                                                                  // must not add a piece to every item
    n = std::min<int64_t>(n, std::min<int64_t>(zl::kMaxPieces, nk / zl::kMinPieceKeys));
    if (n < 2 || next + n > INT32_MAX) {
      out.push_back(it);
      out_unit.push_back((*unit)[j]);
      continue;
    }
    for (int64_t pc = 0; pc < n; ++pc) {
      Item x = it;
      x.t.kv_begin = it.t.kv_begin + (int32_t)(nb * pc / n * zl::kFwdKeys);
      x.t.kv_end = pc + 1 == n ? it.t.kv_end : it.t.kv_begin + (int32_t)(nb * (pc + 1) / n * zl::kFwdKeys);
      x.t.split = (int32_t)next;
      x.t.piece = (int32_t)(pc | (n << 16));
      x.cost = (int64_t)x.t.nrows * (x.t.kv_end - x.t.kv_begin);
      out.push_back(x);
      out_unit.push_back((*unit)[j]);
    }
    next += n;
    ++*n_tiles;
  }
  *n_pieces = (int32_t)next;
  fwd->swap(out);
  unit->swap(out_unit);
}

// Split of the backward queues, for the same reason: with fewer items than resident workgroups,
// every item above the fair share is cut into pieces of the 64-row blocks it loops over (at most
// kMaxPieces, each at least kMinPieceKeys rows). A dQ item loops over the key blocks of its
// segment's key-range chain, a dK/dV item over its segment's query blocks; a piece is a run
// [kv_begin, kv_end) of those blocks. Its partial gradient is a plain sum term (every piece uses
// the final LSE and D), and the item's last piece to finish adds the pieces in order.
void split_runs(int64_t slots, std::vector<Item>* dq, std::vector<int64_t>* unit, int32_t* n_tiles,
                int32_t* n_pieces) {
  *n_tiles = 0;
  *n_pieces = 0;
  if (dq->empty() || (int64_t)dq->size() >= (int64_t)zl::kSplitWaves * slots) return;
  double total = 0.0;
  for (const Item& it : *dq) total += (double)it.cost;
  const double target = total / ((double)zl::kSplitTargetWaves * (double)slots);
  std::vector<Item> out;
  std::vector<int64_t> out_unit;
  int64_t next = 0;
  for (size_t j = 0; j < dq->size(); ++j) {
    const Item& it = (*dq)[j];
    const int64_t nb = it.t.kv_end - it.t.kv_begin;
    int64_t n = (int64_t)std::llround((double)it.cost / target);
    n = std::min<int64_t>(n, std::min<int64_t>(zl::kMaxPieces, nb * zl::kBwdRows / zl::kMinPieceKeys));
    if (n < 2 || next + n > INT32_MAX) {
      out.push_back(it);
      out_unit.push_back((*unit)[j]);
      continue;
    }
    for (int64_t pc = 0; pc < n; ++pc) {
      Item x = it;
      x.t.kv_begin = it.t.kv_begin + (int32_t)(nb * pc / n);
      x.t.kv_end = it.t.kv_begin + (int32_t)(nb * (pc + 1) / n);
      x.t.split = (int32_t)next;
      x.t.piece = (int32_t)(pc | (n << 16));
      x.cost = (int64_t)((double)it.cost * (double)(x.t.kv_end - x.t.kv_begin) / (double)nb);
      out.push_back(x);
      out_unit.push_back((*unit)[j]);
    }
    next += n;
    ++*n_tiles;
  }
  *n_pieces = (int32_t)next;
  dq->swap(out);
  unit->swap(out_unit);
}

}  // namespace

extern "C" zl_status zl_plan_build(int32_t n_seq, const int64_t* cu_q, const int64_t* cu_kv,
                                   const int32_t* seq_heads, int32_t n_seg, const zl_segment* segs,
                                   int32_t d_head, float softmax_scale, uint32_t flags, zl_plan** out) {
  if (!out) return fail(ZL_ERR_INVALID, "zl_plan_build: out is NULL");
  *out = nullptr;
  if (d_head != 64 && d_head != 128)
    return fail(ZL_ERR_UNSUPPORTED, "zl_plan_build: d_head " + std::to_string(d_head) + " is not 64 or 128");
  if (flags & ~(ZL_PLAN_HOST_ONLY | ZL_PLAN_NO_SPLIT | ZL_PLAN_QKV_PACKED | ZL_PLAN_COUNT_VISITS |
                ZL_PLAN_DEFERRED_UPLOAD | ZL_PLAN_NARROW_ITEMS | ZL_PLAN_WIDE_ITEMS))
    return fail(ZL_ERR_INVALID, "zl_plan_build: unknown flag bits");
  if ((flags & ZL_PLAN_NARROW_ITEMS) && (flags & ZL_PLAN_WIDE_ITEMS))
    return fail(ZL_ERR_INVALID, "zl_plan_build: ZL_PLAN_NARROW_ITEMS and ZL_PLAN_WIDE_ITEMS exclude each other");
  if (n_seq < 1) return fail(ZL_ERR_INVALID, "zl_plan_build: n_seq must be >= 1");
  if (!cu_q || !cu_kv || !seq_heads) return fail(ZL_ERR_INVALID, "zl_plan_build: NULL sequence array");
  if (n_seg < 1 || !segs) return fail(ZL_ERR_INVALID, "zl_plan_build: need at least one segment");
  if (!std::isfinite(softmax_scale)) return fail(ZL_ERR_INVALID, "zl_plan_build: softmax_scale is not finite");
  if (cu_q[0] != 0 || cu_kv[0] != 0) return fail(ZL_ERR_INVALID, "zl_plan_build: cu_seqlens[0] must be 0");

  auto plan = new (std::nothrow) zl_plan();
  if (!plan) return fail(ZL_ERR_NOMEM, "zl_plan_build: out of host memory");
  std::unique_ptr<zl_plan> guard(plan);
  plan->d = d_head;
  plan->n_seq = n_seq;
  plan->flags = flags;
  plan->scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d_head);

  std::vector<int64_t> lq(n_seq), lkv(n_seq), qoff(n_seq + 1, 0), kvoff(n_seq + 1, 0);
  for (int s = 0; s < n_seq; ++s) {
    lq[s] = cu_q[s + 1] - cu_q[s];
    lkv[s] = cu_kv[s + 1] - cu_kv[s];
    if (lq[s] < 0 || lkv[s] < 0)
      return fail(ZL_ERR_INVALID, "zl_plan_build: cu_seqlens decreases at sequence " + std::to_string(s));
    if (lq[s] > INT32_MAX || lkv[s] > INT32_MAX)
      return fail(ZL_ERR_INVALID, "zl_plan_build: sequence " + std::to_string(s) + " is longer than 2^31-1 tokens");
    if (seq_heads[s] < 1)
      return fail(ZL_ERR_INVALID, "zl_plan_build: seq_heads[" + std::to_string(s) + "] must be >= 1");
    qoff[s + 1] = qoff[s] + lq[s] * seq_heads[s];
    kvoff[s + 1] = kvoff[s] + lkv[s] * seq_heads[s];
    if (qoff[s + 1] > (INT64_C(1) << 48) || kvoff[s + 1] > (INT64_C(1) << 48))
      return fail(ZL_ERR_INVALID, "zl_plan_build: packed row count too large");
  }
  plan->q_rows = qoff[n_seq];
  plan->kv_rows = kvoff[n_seq];
  const bool packed = flags & ZL_PLAN_QKV_PACKED;
  if (packed)
    for (int s = 0; s < n_seq; ++s)
      if (lq[s] != lkv[s])
        return fail(ZL_ERR_INVALID, "zl_plan_build: ZL_PLAN_QKV_PACKED needs equal query and key lengths; sequence " +
                                        std::to_string(s) + " has " + std::to_string(lq[s]) + " and " +
                                        std::to_string(lkv[s]));

  // Segment checks and ring groups (keyed by sequence, query range and head range).
  std::map<std::tuple<int, int, int, int, int>, int> group_of;
  std::vector<std::vector<int>> group_members;
  std::vector<int> seg_group(n_seg, -1);
  for (int i = 0; i < n_seg; ++i) {
    const zl_segment& g = segs[i];
    if (g.seq < 0 || g.seq >= n_seq) return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(i, g) + ": no such sequence");
    const int nh = seq_heads[g.seq];
    if (g.head_begin < 0 || g.head_begin >= g.head_end || g.head_end > nh)
      return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(i, g) + ": head range outside [0," + std::to_string(nh) + ") or empty");
    if (g.q_begin < 0 || g.q_begin >= g.q_end || g.q_end > lq[g.seq])
      return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(i, g) + ": query range outside [0," + std::to_string(lq[g.seq]) + ") or empty");
    if (g.kv_begin < 0 || g.kv_begin >= g.kv_end || g.kv_end > lkv[g.seq])
      return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(i, g) + ": key range outside [0," + std::to_string(lkv[g.seq]) + ") or empty");
    if (g.part < -1) return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(i, g) + ": part must be >= -1");
    if (g.part >= 0) {
      auto key = std::make_tuple(g.seq, g.q_begin, g.q_end, g.head_begin, g.head_end);
      auto it = group_of.find(key);
      int gid;
      if (it == group_of.end()) {
        gid = (int)group_members.size();
        group_of[key] = gid;
        group_members.emplace_back();
      } else {
        gid = it->second;
      }
      group_members[gid].push_back(i);
      seg_group[i] = gid;
    }
  }
  const int n_groups = (int)group_members.size();
  for (int gid = 0; gid < n_groups; ++gid) {
    auto& mem = group_members[gid];
    std::vector<int> seen(mem.size(), -1);
    for (int i : mem) {
      const int p = segs[i].part;
      if (p >= (int)mem.size() || seen[p] >= 0)
        return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(i, segs[i]) + ": ring parts of a group must be numbered 0.." +
                                        std::to_string(mem.size() - 1) + " once each");
      seen[p] = i;
    }
    std::vector<int> by_kv(mem);
    std::sort(by_kv.begin(), by_kv.end(), [&](int a, int b) { return segs[a].kv_begin < segs[b].kv_begin; });
    for (size_t j = 1; j < by_kv.size(); ++j)
      if (segs[by_kv[j]].kv_begin < segs[by_kv[j - 1]].kv_end)
        return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(by_kv[j], segs[by_kv[j]]) + " and " +
                                        seg_str(by_kv[j - 1], segs[by_kv[j - 1]]) + ": ring parts share key rows");
    plan->n_parts_max = std::max<int32_t>(plan->n_parts_max, (int32_t)mem.size());
  }

  // No two writers of the same O rows; no two owners of the same K/V rows (outside a group).
  {
    std::vector<std::vector<Rect>> outs(n_seq), kvs(n_seq);
    std::vector<char> group_done(n_groups, 0);
    for (int i = 0; i < n_seg; ++i) {
      const zl_segment& g = segs[i];
      kvs[g.seq].push_back({g.kv_begin, g.kv_end, g.head_begin, g.head_end, i, seg_group[i]});
      if (seg_group[i] >= 0) {
        if (group_done[seg_group[i]]) continue;
        group_done[seg_group[i]] = 1;
      }
      outs[g.seq].push_back({g.q_begin, g.q_end, g.head_begin, g.head_end, i, seg_group[i]});
    }
    for (int s = 0; s < n_seq; ++s) {
      int a, b;
      if (find_overlap(outs[s], false, &a, &b))
        return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(a, segs[a]) + " and " + seg_str(b, segs[b]) +
                                        " write the same output rows");
      if (find_overlap(kvs[s], true, &a, &b))
        return fail(ZL_ERR_INVALID, "zl_plan_build: " + seg_str(a, segs[a]) + " and " + seg_str(b, segs[b]) +
                                        " own the same K/V rows (their dK/dV would collide)");
    }
  }

  // Group slab layout.
  plan->groups.resize(n_groups);
  int64_t slab = 0;
  for (int gid = 0; gid < n_groups; ++gid) {
    const zl_segment& f = segs[group_members[gid][0]];
    zl_group_info_t& gi = plan->groups[gid];
    gi.n_parts = (int32_t)group_members[gid].size();
    gi.seq = f.seq;
    gi.n_rows = (int64_t)(f.q_end - f.q_begin) * (f.head_end - f.head_begin);
    gi.o_row = qoff[f.seq] + (int64_t)f.q_begin * seq_heads[f.seq] + f.head_begin;
    gi.part_row = slab;
    gi.head_begin = f.head_begin;
    gi.head_end = f.head_end;
    gi.n_heads = seq_heads[f.seq];
    gi.q_begin = f.q_begin;
    gi.q_end = f.q_end;
    slab += gi.n_rows * gi.n_parts;
  }
  plan->part_rows = slab;
  plan->gdev.resize(n_groups);
  for (int gid = 0; gid < n_groups; ++gid) {
    const zl_group_info_t& gi = plan->groups[gid];
    zl::GroupDev& gd = plan->gdev[gid];
    gd.part_row = gi.part_row;
    gd.o_row = gi.o_row;
    gd.n_rows = gi.n_rows;
    gd.block0 = plan->merge_blocks;
    gd.n_parts = gi.n_parts;
    gd.nh = gi.n_heads;
    gd.n_sub = gi.head_end - gi.head_begin;
    gd.pad = 0;
    const int rows = zl::merge_rows(d_head);
    plan->merge_blocks += (gi.n_rows + rows - 1) / rows;
  }

  // Device segment table.
  plan->segs.resize(n_seg);
  for (int i = 0; i < n_seg; ++i) {
    const zl_segment& g = segs[i];
    zl::SegDev& d = plan->segs[i];
    std::memset(&d, 0, sizeof(d));
    d.q_row0 = qoff[g.seq];
    d.kv_row0 = kvoff[g.seq];
    d.nh = seq_heads[g.seq];

    d.lq = (int32_t)lq[g.seq];
    d.q_begin = g.q_begin;
    d.q_end = g.q_end;
    d.kv_begin = g.kv_begin;
    d.kv_end = g.kv_end;
    d.head_begin = g.head_begin;
    d.head_end = g.head_end;
    d.part = g.part;
    d.part_row0 = -1;
    if (g.part >= 0) {
      const zl_group_info_t& gi = plan->groups[seg_group[i]];
      d.part_row0 = gi.part_row + (int64_t)g.part * gi.n_rows;
    }
    plan->fwd_flops += 4.0 * (double)(g.q_end - g.q_begin) * (double)(g.kv_end - g.kv_begin) * (double)d_head *
                       (double)(g.head_end - g.head_begin);
  }

  // Key-range chains for the dQ queue: a final segment's own range, or on part 0 of a ring
  // group every part's range in part order.
  for (int i = 0; i < n_seg; ++i) {
    const zl_segment& g = segs[i];
    zl::SegDev& d = plan->segs[i];
    d.chain_off = (int32_t)(plan->kv_ranges.size() / 2);
    d.chain_len = 0;
    if (g.part > 0) continue;
    std::vector<int> members{i};
    if (g.part == 0) {
      members.assign(group_members[seg_group[i]].begin(), group_members[seg_group[i]].end());
      std::sort(members.begin(), members.end(), [&](int a, int b) { return segs[a].part < segs[b].part; });
    }
    for (int m : members) {
      plan->kv_ranges.push_back(segs[m].kv_begin);
      plan->kv_ranges.push_back(segs[m].kv_end);
    }
    d.chain_len = (int32_t)members.size();
  }

  if (!(flags & ZL_PLAN_HOST_ONLY)) {
    if (hipGetDevice(&plan->device) != hipSuccess) return fail(ZL_ERR_HIP, "zl_plan_build: hipGetDevice failed");
    if (hipDeviceGetAttribute(&plan->n_cu, hipDeviceAttributeMultiprocessorCount, plan->device) != hipSuccess ||
        plan->n_cu < 1)
      return fail(ZL_ERR_HIP, "zl_plan_build: cannot query the compute unit count");
  }

  // Query-major item sizes (forward and dQ queues), unless a flag fixes them. With r rounds of
  // wide items for the resident wide workgroups:
  //   r >= kWideRounds      wide: the tail is short, and each K/V block serves twice the rows;
  //   1 < r < kWideRounds   narrow: a narrow unit's second workgroup keeps it busy through the
  //                         tail, where a wide unit sits idle;
  //   1/2 <= r <= 1         wide: every unit is busy with either size;
  //   r < 1/2               wide if some item is long enough to be cut into key pieces (the
  //                         split below then fills the device), else narrow, which spreads few
  //                         short items over twice the units.
  {
    int64_t wide_fwd = 0, wide_dq = 0, keys_fwd = 0, keys_dq = 0;
    for (int i = 0; i < n_seg; ++i) {
      const int64_t n = (int64_t)(segs[i].head_end - segs[i].head_begin) *
                        ((segs[i].q_end - segs[i].q_begin + zl::kFwdRowsWide - 1) / zl::kFwdRowsWide);
      wide_fwd += n;
      keys_fwd = std::max<int64_t>(keys_fwd, segs[i].kv_end - segs[i].kv_begin);
      if (segs[i].part > 0) continue;  // a ring group's dQ items belong to its part 0
      wide_dq += n;
      int64_t chain = 0;
      for (int c = 0; c < plan->segs[i].chain_len; ++c)
        chain += plan->kv_ranges[2 * (plan->segs[i].chain_off + c) + 1] - plan->kv_ranges[2 * (plan->segs[i].chain_off + c)];
      keys_dq = std::max(keys_dq, chain);
    }
    int64_t fwd_slots = zl::kHostOnlyWideSlots, dq_slots = zl::kHostOnlyWideSlots;
    if (!(flags & ZL_PLAN_HOST_ONLY)) {
      const int per_cu = zl::fwd_blocks_per_cu(d_head, zl::kFwdRowsWide);
      const int per_cu_dq = zl::dq_blocks_per_cu(d_head, zl::kDqRowsWide);
      if (per_cu < 1 || per_cu_dq < 1) return fail(ZL_ERR_HIP, "zl_plan_build: wide kernels cannot be resident");
      fwd_slots = (int64_t)plan->n_cu * per_cu;
      dq_slots = (int64_t)plan->n_cu * per_cu_dq;
    }
    const bool split = !(flags & ZL_PLAN_NO_SPLIT);
    auto wide = [&](int64_t items, int64_t slots, int64_t longest_keys) {
      if (flags & (ZL_PLAN_NARROW_ITEMS | ZL_PLAN_WIDE_ITEMS)) return (flags & ZL_PLAN_WIDE_ITEMS) != 0;
      if (items >= (int64_t)zl::kWideRounds * slots) return true;
      if (items > slots) return false;
      if (2 * items >= slots) return true;
      return split && longest_keys >= 2 * zl::kMinPieceKeys;
    };
    plan->fwd_rows = wide(wide_fwd, fwd_slots, keys_fwd) ? zl::kFwdRowsWide : zl::kFwdRowsNarrow;
    plan->dq_rows = wide(wide_dq, dq_slots, keys_dq) ? zl::kDqRowsWide : zl::kDqRowsNarrow;
  }
  const int fwd_rows = plan->fwd_rows, dq_rows = plan->dq_rows;

  // Work queues. Items of one (segment, head) that share K/V (forward, dQ) or Q/dO (dK/dV)
  // are grouped into chunks of bounded cost; chunks go to the kQueues per-XCD queues by
  // longest-processing-time-first, so that each head's data is mostly read through one XCD's
  // L2; each queue is then sorted by decreasing item cost with a stable tie order.
  std::vector<Item> fwd, bwd, dq;
  std::vector<int64_t> fwd_unit, bwd_unit, dq_unit;  // (segment, head) unit of each item
  {
    size_t n_fwd = 0, n_bwd = 0, n_dq = 0, n_pre = 0;
    for (int i = 0; i < n_seg; ++i) {
      const zl_segment& g = segs[i];
      const size_t nh = (size_t)(g.head_end - g.head_begin);
      const size_t nq = (size_t)(g.q_end - g.q_begin), nk = (size_t)(g.kv_end - g.kv_begin);
      n_fwd += nh * ((nq + fwd_rows - 1) / fwd_rows);
      n_bwd += nh * ((nk + zl::kBwdKeys - 1) / zl::kBwdKeys);
      if (g.part <= 0) {
        n_dq += nh * ((nq + dq_rows - 1) / dq_rows);
        n_pre += nq / (size_t)std::max<size_t>(1, zl::kPreRows / nh) + 1;
      }
    }
    fwd.reserve(n_fwd);
    fwd_unit.reserve(n_fwd);
    bwd.reserve(n_bwd);
    bwd_unit.reserve(n_bwd);
    dq.reserve(n_dq);
    dq_unit.reserve(n_dq);
    plan->pre_tiles.reserve(n_pre);
  }
  for (int i = 0; i < n_seg; ++i) {
    const zl_segment& g = segs[i];
    const int64_t nq = g.q_end - g.q_begin, nk = g.kv_end - g.kv_begin;
    int64_t chain_keys = 0, chain_blocks = 0;
    for (int c = 0; c < plan->segs[i].chain_len; ++c) {
      const int64_t len =
          plan->kv_ranges[2 * (plan->segs[i].chain_off + c) + 1] - plan->kv_ranges[2 * (plan->segs[i].chain_off + c)];
      chain_keys += len;
      chain_blocks += (len + zl::kBwdRows - 1) / zl::kBwdRows;
    }
    for (int h = g.head_begin; h < g.head_end; ++h) {
      const int64_t unit = (int64_t)i * 65536 + h;
      for (int64_t r = g.q_begin; r < g.q_end; r += fwd_rows) {
        const int32_t n = (int32_t)std::min<int64_t>(fwd_rows, g.q_end - r);
        fwd.push_back({{i, h, (int32_t)r, n, g.kv_begin, g.kv_end, -1, 1 << 16}, (int64_t)n * nk});
        fwd_unit.push_back(unit);
      }
      if (g.part <= 0)
        for (int64_t r = g.q_begin; r < g.q_end; r += dq_rows) {
          const int32_t n = (int32_t)std::min<int64_t>(dq_rows, g.q_end - r);
          // A dQ item's key range is its block range [0, chain_blocks) of the segment's chain.
          dq.push_back({{i, h, (int32_t)r, n, 0, (int32_t)chain_blocks, -1, 1 << 16}, (int64_t)n * chain_keys});
          dq_unit.push_back(unit);
        }
      for (int64_t r = g.kv_begin; r < g.kv_end; r += zl::kBwdKeys) {
        const int32_t n = (int32_t)std::min<int64_t>(zl::kBwdKeys, g.kv_end - r);
        // A dK/dV item's range is its run [0, query blocks) of the segment's 64-row query blocks.
        bwd.push_back({{i, h, (int32_t)r, n, 0, (int32_t)((nq + zl::kBwdRows - 1) / zl::kBwdRows), -1, 1 << 16},
                       (int64_t)n * nq});
        bwd_unit.push_back(unit);
      }
    }
    // Backward pre-pass rows: once per output row set (a ring group does it on part 0).
    if (g.part <= 0) {
      const int nhr = g.head_end - g.head_begin;
      const int toks = std::max(1, zl::kPreRows / nhr);
      for (int64_t t = g.q_begin; t < g.q_end; t += toks)
        plan->pre_tiles.push_back(
            {i, g.head_begin, (int32_t)t, (int32_t)std::min<int64_t>(toks, g.q_end - t), 0, 0, -1, 1 << 16});
    }
  }
  if (!(flags & ZL_PLAN_NO_SPLIT)) {
    int64_t slots = fwd_rows == zl::kFwdRowsWide ? zl::kHostOnlyWideSlots : zl::kHostOnlySlots;
    if (!(flags & ZL_PLAN_HOST_ONLY)) {
      const int per_cu = zl::fwd_blocks_per_cu(d_head, fwd_rows);
      if (per_cu < 1) return fail(ZL_ERR_HIP, "zl_plan_build: forward kernel cannot be resident");
      slots = (int64_t)plan->n_cu * per_cu;
    }
    split_forward(slots, &fwd, &fwd_unit, &plan->split_tiles, &plan->split_pieces);
    int64_t dq_slots = dq_rows == zl::kDqRowsWide ? zl::kHostOnlyWideSlots : zl::kHostOnlySlots;
    if (!(flags & ZL_PLAN_HOST_ONLY)) {
      const int per_cu = zl::dq_blocks_per_cu(d_head, dq_rows);
      if (per_cu < 1) return fail(ZL_ERR_HIP, "zl_plan_build: dQ kernel cannot be resident");
      dq_slots = (int64_t)plan->n_cu * per_cu;
    }
    split_runs(dq_slots, &dq, &dq_unit, &plan->dq_split_tiles, &plan->dq_split_pieces);
    int64_t kv_slots = zl::kHostOnlyKvSlots;
    if (!(flags & ZL_PLAN_HOST_ONLY)) {
      const int per_cu = zl::bwd_blocks_per_cu(d_head);
      if (per_cu < 1) return fail(ZL_ERR_HIP, "zl_plan_build: dK/dV kernel cannot be resident");
      kv_slots = (int64_t)plan->n_cu * per_cu;
    }
    split_runs(kv_slots, &bwd, &bwd_unit, &plan->kv_split_tiles, &plan->kv_split_pieces);
  }
  if (fwd.size() > (size_t)INT32_MAX || bwd.size() > (size_t)INT32_MAX || dq.size() > (size_t)INT32_MAX ||
      plan->pre_tiles.size() > (size_t)INT32_MAX)
    return fail(ZL_ERR_INVALID, "zl_plan_build: too many work items");
  distribute(fwd, fwd_unit, &plan->fwd_tiles, &plan->fwd_bounds);
  distribute(bwd, bwd_unit, &plan->bwd_tiles, &plan->bwd_bounds);
  distribute(dq, dq_unit, &plan->dq_tiles, &plan->dq_bounds);

  if (!(flags & ZL_PLAN_HOST_ONLY)) {
    // One image of every device table, carved at 256-byte aligned offsets.
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const struct {
      const void* src;
      size_t bytes;
    } parts[] = {{plan->segs.data(), plan->segs.size() * sizeof(zl::SegDev)},
                 {plan->fwd_tiles.data(), plan->fwd_tiles.size() * sizeof(zl::Tile)},
                 {plan->bwd_tiles.data(), plan->bwd_tiles.size() * sizeof(zl::Tile)},
                 {plan->pre_tiles.data(), plan->pre_tiles.size() * sizeof(zl::Tile)},
                 {plan->dq_tiles.data(), plan->dq_tiles.size() * sizeof(zl::Tile)},
                 {plan->kv_ranges.data(), plan->kv_ranges.size() * sizeof(int32_t)},
                 {plan->gdev.data(), plan->gdev.size() * sizeof(zl::GroupDev)}};
    size_t total = 0;
    constexpr int kTables = sizeof(parts) / sizeof(parts[0]);
    static_assert(kTables == sizeof(plan->table_off) / sizeof(plan->table_off[0]), "one offset per table");
    for (int i = 0; i < kTables; ++i) {
      plan->table_off[i] = total;
      total += align(parts[i].bytes);
    }
    plan->dev_bytes = total;
    plan->image.assign(total, 0);
    for (int i = 0; i < kTables; ++i)
      if (parts[i].bytes) std::memcpy(plan->image.data() + plan->table_off[i], parts[i].src, parts[i].bytes);
    if (!(flags & ZL_PLAN_DEFERRED_UPLOAD)) {
      if (hipMalloc(&plan->dev_block, total) != hipSuccess) {
        plan->dev_block = nullptr;
        (void)hipGetLastError();
        return fail(ZL_ERR_NOMEM, "zl_plan_build: hipMalloc of " + std::to_string(total) + " bytes failed");
      }
      const hipError_t e = hipMemcpy(plan->dev_block, plan->image.data(), total, hipMemcpyHostToDevice);
      if (e != hipSuccess) {
        (void)hipFree(plan->dev_block);
        plan->dev_block = nullptr;
        return fail(ZL_ERR_HIP, std::string("zl_plan_build: upload failed: ") + hipGetErrorString(e));
      }
      plan->image.clear();
      plan->image.shrink_to_fit();
      zl::set_table_pointers(plan, plan->dev_block);
    }
  }
  *out = guard.release();
  return ZL_OK;
}

extern "C" void zl_plan_destroy(zl_plan* plan) {
  if (!plan) return;
  if (plan->dev_block) (void)hipFree(plan->dev_block);  // a deferred plan owns no device memory
  delete plan;
}

namespace {

// Pinned host staging for zl_plan_upload, recycled across plans: an entry is reused once the copy
// that last read it has completed (its event), so neither an upload nor a plan's destruction
// waits for the device. Entries live until the process ends.
struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;  // recorded after the last copy from this entry
  bool recorded = false;
};
std::mutex g_staging_mu;
std::vector<Staging>* g_staging = new std::vector<Staging>();  // never destroyed: see above

}  // namespace

extern "C" zl_status zl_plan_upload(zl_plan* plan, void* dev_tables, size_t bytes, void* stream) {
  if (!plan) return fail(ZL_ERR_INVALID, "zl_plan_upload: plan is NULL");
  if (!(plan->flags & ZL_PLAN_DEFERRED_UPLOAD) || (plan->flags & ZL_PLAN_HOST_ONLY))
    return fail(ZL_ERR_INVALID, "zl_plan_upload: the plan was not built with ZL_PLAN_DEFERRED_UPLOAD");
  if (plan->d_segs) return fail(ZL_ERR_INVALID, "zl_plan_upload: the plan's tables were already uploaded");
  if (!dev_tables || ((uintptr_t)dev_tables & 255))
    return fail(ZL_ERR_INVALID, "zl_plan_upload: dev_tables must be a non-NULL, 256-byte aligned device pointer");
  if (bytes < plan->dev_bytes)
    return fail(ZL_ERR_INVALID, "zl_plan_upload: " + std::to_string(bytes) + " bytes given, the tables need " +
                                    std::to_string(plan->dev_bytes));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return fail(ZL_ERR_INVALID, "zl_plan_upload: the current device is not the plan's device");
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_staging_mu);
  Staging* st = nullptr;
  for (Staging& e : *g_staging)
    if (e.cap >= plan->dev_bytes && (!e.recorded || hipEventQuery(e.done) == hipSuccess)) {
      st = &e;
      break;
    }
  if (!st) {
    Staging e;
    e.cap = std::max<size_t>(plan->dev_bytes, (size_t)1 << 20);
    if (hipHostMalloc(&e.host, e.cap, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      return fail(ZL_ERR_NOMEM, "zl_plan_upload: pinned staging of " + std::to_string(e.cap) + " bytes failed");
    }
    if (hipEventCreateWithFlags(&e.done, hipEventDisableTiming) != hipSuccess) {
      (void)hipHostFree(e.host);
      (void)hipGetLastError();
      return fail(ZL_ERR_HIP, "zl_plan_upload: event creation failed");
    }
    g_staging->push_back(e);
    st = &g_staging->back();
  }
  std::memcpy(st->host, plan->image.data(), plan->dev_bytes);
  hipError_t e = hipMemcpyAsync(dev_tables, st->host, plan->dev_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(st->done, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(ZL_ERR_HIP, std::string("zl_plan_upload: copy failed: ") + hipGetErrorString(e));
  }
  st->recorded = true;
  zl::set_table_pointers(plan, dev_tables);
  plan->image.clear();
  plan->image.shrink_to_fit();
  return ZL_OK;
}
