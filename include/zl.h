/*
 * zl.h -- C ABI of the coalesced varlen attention library (libzl.so) for MI355X / gfx950.
 *
 * The library runs one GPU's share of a mixed image-video DiT batch: non-causal softmax
 * attention, forward and backward, over a packed work list that mixes whole sequences,
 * head subsets of long sequences and KV-split shards. It follows the "Coalesced Attention
 * Engine" of the Zellige page (Moldable Sequence Placement for Mixed Image-Video DiT
 * Training, §IV-D): a rank-local schedule is lowered into one launch that never mixes
 * attention across sequences and writes every output at its input row, so outputs come
 * back in rank-local input order. The q/h/kv ranges of a segment are the three axes of a
 * placement option (§IV-A, Table II: all-gather (q,1,1), Ulysses (1,h,1), ring (1,1,k)).
 *
 * Data layout (all tensors owned by the caller, passed as raw device pointers):
 *   Sequence s has Lq_s = cu_seqlens_q[s+1]-cu_seqlens_q[s] query tokens,
 *   Lkv_s = cu_seqlens_kv[s+1]-cu_seqlens_kv[s] key/value tokens and nh_s = seq_heads[s]
 *   stored heads. Its query-side rows are stored as [Lq_s][nh_s][d] and start at row
 *   sum_{s'<s} Lq_s' * nh_s'; key-side rows likewise with Lkv. A "row" is one
 *   (token, head) pair of d contiguous values. With one head count for every sequence this
 *   is the usual packed varlen [T, H, d] layout.
 *     Q, dO          bf16 [q_rows][d]          K, V       bf16 [kv_rows][d]
 *     O, dQ          fp32 [q_rows][d]          dK, dV     fp32 [kv_rows][d]
 *     LSE            fp32 [q_rows]             (natural-log log-sum-exp per row)
 *
 * Errors: every call returns a zl_status and never throws. A thread-local message for the
 * last failure is available from zl_last_error(). Calls that take a stream enqueue work on
 * it and return without synchronising: a fault on the device shows up at the caller's next
 * synchronisation, not as a status.
 */
#ifndef ZL_H
#define ZL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZL_OK = 0,
  ZL_ERR_INVALID = -1,      /* bad argument: a range, a pointer, an overlap, a plan mismatch */
  ZL_ERR_UNSUPPORTED = -2,  /* d_head other than 64 or 128 */
  ZL_ERR_HIP = -3,          /* a HIP runtime call or kernel launch failed */
  ZL_ERR_NOMEM = -4         /* host or device allocation failed */
} zl_status;

typedef struct zl_plan zl_plan; /* opaque; immutable after zl_plan_build, safe to share */

/*
 * One unit of rank-local work (§IV-D lowering; axes of §IV-A):
 *   queries [q_begin, q_end) of sequence `seq` attend to its keys [kv_begin, kv_end),
 *   for every stored head h in [head_begin, head_end).
 * part == -1: the result is final and is written to O/LSE at the query rows.
 * part >= 0: the segment is ring part `part` of a KV-split group. A group is the set of
 *   segments with equal (seq, q range, head range); its parts must be numbered 0..n-1 and
 *   have disjoint key ranges. The head range may be a subset of the stored heads: a
 *   composed placement, Ulysses over heads and ring over keys (§IV-A, Table II). Each part
 *   writes a normalised partial O and its LSE to the partial slab (see zl_plan_group); the
 *   exact merge is zl_plan_merge (ring attention accumulates the output block by block,
 *   §II-B), or zl_attn_fwd_accumulate folds each part in as it runs.
 * No two segments may write the same O rows, and no two may own the same K/V rows (their
 * dK/dV would collide) unless they are parts of one group, whose key ranges are disjoint.
 */
typedef struct {
  int32_t seq;
  int32_t head_begin, head_end;
  int32_t q_begin, q_end;
  int32_t kv_begin, kv_end;
  int32_t part;
} zl_segment;

typedef struct {
  size_t ws_fwd;          /* workspace bytes zl_attn_fwd needs (device memory, 256-B aligned) */
  size_t ws_bwd;          /* workspace bytes zl_attn_bwd needs */
  int64_t q_rows;         /* packed query-side rows */
  int64_t kv_rows;        /* packed key-side rows */
  int64_t part_rows;      /* rows of the partial slab: o_part holds part_rows*d floats */
  int32_t n_groups;       /* KV-split groups */
  int32_t n_parts_max;    /* most parts in one group */
  int64_t fwd_tiles;      /* work items of the forward queue */
  int64_t bwd_tiles;      /* work items of the backward dK/dV queue */
  double fwd_flops;       /* sum over (segment, head) of 4*Lq*Lkv*d */
  double bwd_flops;       /* 2.5 x fwd_flops */
  int32_t d_head;
  float softmax_scale;
  int64_t dq_tiles;       /* work items of the backward dQ queue */
  int32_t split_tiles;    /* forward items cut into key pieces (split-KV) */
  int32_t split_pieces;   /* pieces of those items */
  int64_t qkv_rows;       /* rows of the packed QKV (and dQKV) buffer: 3 * q_rows, or 0 unless
                             ZL_PLAN_QKV_PACKED */
  int32_t dq_split_tiles;  /* dQ items cut into pieces of their key blocks (split-KV backward) */
  int32_t dq_split_pieces; /* pieces of those items */
  int32_t kv_split_tiles;  /* dK/dV items cut into pieces of their query blocks */
  int32_t kv_split_pieces; /* pieces of those items */
  int64_t visits_fwd;      /* with ZL_PLAN_COUNT_VISITS: byte offset in the forward workspace of one
                              int32 per forward work item (zl_plan_tiles order, which = 0) that
                              counts the workgroups that took the item; -1 without the flag */
  int64_t visits_dkdv;     /* the same in the backward workspace for the dK/dV queue (which = 1) */
  int64_t visits_dq;       /* ... and for the dQ queue (which = 2) */
  size_t dev_bytes;        /* bytes of the plan's device tables (0 for a host-only plan): what
                              zl_plan_upload needs for a ZL_PLAN_DEFERRED_UPLOAD plan */
  int32_t fwd_rows;        /* query rows per forward item: 128 or 256 (see zl_plan_build) */
  int32_t dq_rows;         /* query rows per dQ item: 128 or 256 */
} zl_plan_info_t;

/*
 * A KV-split (ring) group: the segments that share a sequence, query range and head range
 * and carry parts 0..n_parts-1. The group's rows are its (token, head) pairs, token-major:
 * row r is token q_begin + r / n_sub and head head_begin + r % n_sub, with
 * n_sub = head_end - head_begin. In O and LSE that pair lives at row
 * o_row + (r / n_sub) * n_heads + r % n_sub; the rows are contiguous only when the group
 * covers every stored head (n_sub == n_heads). In the partial slab, part b holds the group's
 * rows contiguously from part_row + b * n_rows.
 */
typedef struct {
  int32_t n_parts;        /* parts in the group */
  int32_t seq;            /* its sequence */
  int64_t n_rows;         /* rows of the group: (q_end-q_begin) * (head_end-head_begin) */
  int64_t o_row;          /* O/LSE row of (token q_begin, head head_begin) */
  int64_t part_row;       /* first slab row of part 0; part b starts at part_row + b*n_rows */
  int32_t head_begin, head_end;  /* the group's stored-head range */
  int32_t n_heads;        /* stored heads of the sequence (O/LSE rows between tokens) */
  int32_t q_begin, q_end; /* the group's query range */
} zl_group_info_t;

/* Flags for zl_plan_build. */
#define ZL_PLAN_HOST_ONLY 1u /* build and validate on the host only; no device tables, so the
                                plan can be inspected but not run (used by CPU-only tests) */
#define ZL_PLAN_NO_SPLIT 2u  /* never cut work items into pieces (see zl_plan_build) */
#define ZL_PLAN_QKV_PACKED 4u /* Q, K, V share one buffer, per sequence [tokens][Q, K, V][heads][d]
                                 (the layout of a QKV-packed all-to-all, §IV-D / Table II), and so
                                 do dQ, dK, dV; needs equal query and key lengths. Sequence s starts
                                 at packed row 3 * (its first planar row); O, LSE, dO stay planar.
                                 Pass the packed buffer as q, k and v (and as dq, dk, dv). */
#define ZL_PLAN_DEFERRED_UPLOAD 16u /* build everything but the device tables; zl_plan_upload then
                                       copies them into caller memory on the caller's stream, so a
                                       per-batch plan neither allocates device memory nor waits
                                       for the device (see zl_plan_upload) */
#define ZL_PLAN_COUNT_VISITS 8u /* scheduler check: every kernel also counts, per work item, the
                                   workgroups that took it, in int32 counters the workspace gains at
                                   the offsets zl_plan_info reports (visits_*). The forward launch
                                   clears the forward's, the backward pre-pass the backward's. After
                                   a forward and a backward every counter must read exactly 1. */
#define ZL_PLAN_NARROW_ITEMS 32u /* forward and dQ items of 128 query rows whatever the queues' depth */
#define ZL_PLAN_WIDE_ITEMS 64u   /* forward and dQ items of 256 query rows whatever the queues' depth
                                    (at most one of the two; see zl_plan_build) */

/*
 * Validate the segment list and lower it into device work queues.
 *   n_seq                 number of sequences (>= 1)
 *   cu_seqlens_q/kv       host arrays of n_seq+1 token offsets, [0] == 0, non-decreasing;
 *                         every sequence length must be below 2^31
 *   seq_heads             host array of n_seq stored-head counts (>= 1)
 *   n_seg, segs           host array of segments (see zl_segment), n_seg >= 1
 *   d_head                64 or 128 (else ZL_ERR_UNSUPPORTED)
 *   softmax_scale         tau in softmax(tau * Q K^T); <= 0 selects 1/sqrt(d_head)
 *   flags                 0 or an OR of ZL_PLAN_HOST_ONLY, ZL_PLAN_NO_SPLIT, ZL_PLAN_QKV_PACKED,
 *                         ZL_PLAN_COUNT_VISITS, ZL_PLAN_DEFERRED_UPLOAD and at most one of
 *                         ZL_PLAN_NARROW_ITEMS, ZL_PLAN_WIDE_ITEMS
 *   out                   receives the plan; the caller frees it with zl_plan_destroy
 * The host arrays are copied; the plan owns its device tables (allocated on the current
 * device) and nothing else. The forward queue holds one item per (segment, head, block of
 * info.fwd_rows query rows); the backward has a dK/dV queue with one item per (segment, head,
 * block of 128 key rows) and a dQ queue with one item per (final segment or ring group, head,
 * block of info.dq_rows query rows). Each query-major queue (forward, dQ) takes 256-row items
 * (one 8-wave workgroup per compute unit, each K/V block in LDS shared by twice the rows) or
 * 128-row items (two 4-wave workgroups per compute unit, which keep a unit busy while one of
 * them runs out of work). With r rounds of 256-row items for the resident workgroups: 256 rows
 * for r >= 4; 128 for 1 < r < 4; 256 for 1/2 <= r <= 1; below that 256 if some item has at
 * least 2048 keys and split-KV (below) is on, else 128. ZL_PLAN_WIDE_ITEMS or
 * ZL_PLAN_NARROW_ITEMS fixes both choices. Each is split into one queue per XCD (zl_plan_queues): chunks of
 * consecutive items of one (segment, head) go to the least-loaded queue, largest first, and
 * each queue is sorted by decreasing cost (rows x length of the other side), ties kept in
 * (segment, head, block) order. A workgroup drains its own XCD's queue, then the others.
 * Split-KV: when the forward queue holds fewer items than there are resident forward
 * workgroups (the device's CU count times the kernel's occupancy; for a host-only plan 512
 * for 128-row items, 256 for 256-row items and for the dK/dV kernel),
 * so that compute units would sit idle, every item costing more than a workgroup's fair share
 * (the queue's total cost over the resident workgroups) is cut into block-aligned key pieces
 * of about that share (at most 16, each at least 1024 keys). Each piece is a normalised partial over its keys; the
 * last piece of an item to finish merges them exactly (the ring merge, §II-B) and stores the
 * item's result. The backward queues are split the same way when they hold fewer items than
 * there are resident workgroups of their kernel: a dQ item loops over the 64-key blocks of its
 * segment's key ranges (all parts of a ring group, in part order), a dK/dV item over the
 * segment's 64-row query blocks, and a piece takes a contiguous run of those blocks. A piece's
 * partial gradient is a plain sum term (every piece uses the final LSE and D); the last piece
 * of an item to finish adds the pieces in piece order, so the result does not depend on which
 * piece finishes last. ZL_PLAN_NO_SPLIT turns all of this off. The pieces' partials live in
 * the forward and backward workspaces, whose sizes grow accordingly (info.ws_fwd, info.ws_bwd).
 */
zl_status zl_plan_build(int32_t n_seq, const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                        const int32_t* seq_heads, int32_t n_seg, const zl_segment* segs,
                        int32_t d_head, float softmax_scale, uint32_t flags, zl_plan** out);

/*
 * Copy the device tables of a plan built with ZL_PLAN_DEFERRED_UPLOAD into caller memory, on
 * `stream` (the lowering of §IV-D done per rank per step without stalling the device):
 *   dev_tables   device memory of at least info.dev_bytes bytes, 256-B aligned, owned by the
 *                caller; it must stay allocated, and unmodified, while any launch that uses the
 *                plan may still run
 *   bytes        its size
 *   stream       hipStream_t (NULL = default): the copy is ordered on it; launches with the plan on
 *                another stream must be ordered after it (an event)
 * The tables go through pinned host staging that the library recycles once the copy that read it
 * has completed, so the call returns without waiting for the device, and zl_plan_destroy of such
 * a plan frees no device memory and does not synchronise. Once per plan; ZL_ERR_INVALID for a
 * plan built otherwise or already uploaded, or for a short or misaligned buffer. Not for use while
 * the stream is being captured into a graph (the staging would be reused under the graph).
 */
zl_status zl_plan_upload(zl_plan* plan, void* dev_tables, size_t bytes, void* stream);

/* Sizes and counts of a plan. */
zl_status zl_plan_info(const zl_plan* plan, zl_plan_info_t* info);

/* Layout of KV-split group g (0 <= g < n_groups), in the order of first appearance. */
zl_status zl_plan_group(const zl_plan* plan, int32_t g, zl_group_info_t* info);

/*
 * Copy a work queue to the host for inspection: which = 0 forward, 1 backward dK/dV,
 * 2 backward dQ (items of a ring group name its part-0 segment).
 * Each item is 4 int32: segment index, head, first row of the block, rows in the block.
 * which = 3 is the forward queue again with 8 int32 per item: the same 4, then the item's
 * key range [kv_begin, kv_end), the workspace slot of its piece 0 (-1 unless the item is a
 * piece of a split item) and its piece index | (pieces << 16). which = 4 is the dQ queue with
 * 8 int32 per item in the same form, the key range given as a range of 64-key blocks of the
 * segment's key-range chain; which = 5 is the dK/dV queue in the same form, the range given as
 * a range of the segment's 64-row query blocks.
 * Writes min(cap, count) items to out (may be NULL when cap == 0); *count gets the total.
 */
zl_status zl_plan_tiles(const zl_plan* plan, int32_t which, int32_t* out, int64_t cap, int64_t* count);

/*
 * Queue boundaries of a work list (which as for zl_plan_tiles): items bounds[k]..bounds[k+1]
 * of zl_plan_tiles' order form queue k. Writes min(cap, n_queues + 1) ints; *n_queues gets
 * the queue count.
 */
zl_status zl_plan_queues(const zl_plan* plan, int32_t which, int32_t* bounds, int32_t cap, int32_t* n_queues);

/*
 * Free a plan and its device tables. NULL is ignored. The tables of a plan built without
 * ZL_PLAN_DEFERRED_UPLOAD are released with hipFree, which first waits for all work queued on the
 * device (an implicit device synchronisation): such a plan may be destroyed while launches that
 * use it are still queued, but not while a stream of its device is being captured into a graph.
 * A deferred plan owns no device memory; destroying it neither frees nor waits.
 */
void zl_plan_destroy(zl_plan* plan);

/*
 * Forward (§IV-D coalesced call; §II-A attention). One persistent launch processes every
 * segment of the plan:
 *   q, k, v     bf16 device tensors in the packed layout
 *   o, lse      fp32 outputs for part == -1 segments, written at their query rows
 *   o_part,     fp32 partial slab, [part_rows][d] and [part_rows]; may be NULL only if the
 *   lse_part    plan has no KV-split group
 *   workspace   device memory of info.ws_fwd bytes, 256-B aligned, not shared with a
 *               concurrent call (it holds the queue counters)
 *   stream      hipStream_t, NULL for the default stream
 * Rows that no segment covers are left untouched. Pointers must be 16-B aligned.
 */
zl_status zl_attn_fwd(const zl_plan* plan, const void* q, const void* k, const void* v,
                      float* o, float* lse, float* o_part, float* lse_part,
                      void* workspace, void* stream);

/*
 * Forward with a running merge (ring accumulation, §II-B: the output is accumulated block by
 * block as key/value blocks arrive). Like zl_attn_fwd, except that every ring part folds its
 * normalised partial result O_b, LSE_b into the running result held in o and lse at the
 * group's rows (o_row of zl_plan_group), with no partial slab:
 *   LSE' = M + ln(exp(LSE - M) + exp(LSE_b - M)),  M = max(LSE, LSE_b)
 *   O'   = exp(LSE - LSE') * O + exp(LSE_b - LSE') * O_b
 * Before a group's first block the caller sets its rows of lse to -inf; such rows take the
 * part as it is and their o is not read. Folding the parts of a group one call at a time, in
 * any order, gives the exact merge of zl_lse_merge (up to rounding).
 *   q, k, v     bf16 device tensors in the packed layout
 *   o, lse      fp32 running results (in/out for ring parts; output for part == -1 segments)
 *   workspace   device memory of info.ws_fwd bytes, 256-B aligned, not shared with a
 *               concurrent call
 *   stream      hipStream_t, NULL for the default stream
 * A plan used here may hold at most one part of each group (ZL_ERR_INVALID otherwise): two
 * parts of a group would fold into the same rows at once. Calls that fold into the same rows
 * must be ordered (one stream, or events). Pointers must be 16-B aligned.
 */
zl_status zl_attn_fwd_accumulate(const zl_plan* plan, const void* q, const void* k, const void* v,
                                 float* o, float* lse, void* workspace, void* stream);

/*
 * Exact merge of n_parts normalised partial results over disjoint key blocks (ring
 * accumulation, §II-B): for every row r,
 *   LSE[r] = M + ln sum_b exp(lse_part[b][r] - M),  M = max_b lse_part[b][r]
 *   O[r]   = sum_b exp(lse_part[b][r] - LSE[r]) * o_part[b][r]
 * A part with lse = -inf has weight 0; a row whose parts are all -inf gets O = 0 and
 * LSE = -inf.
 *   o_part  fp32 [n_parts][n_rows][d_head]     lse_part  fp32 [n_parts][n_rows]
 *   o       fp32 [n_rows][d_head] (output)     lse       fp32 [n_rows] (output)
 * For a plan's group g that covers every stored head (its O rows are then contiguous), pass
 * o_part + part_row*d, lse_part + part_row, o + o_row*d and lse + o_row from zl_plan_group;
 * zl_plan_merge does every group of a plan, head subsets included, in one launch.
 * d_head is 64 or 128; pointers 16-B aligned.
 */
zl_status zl_lse_merge(int32_t n_parts, int64_t n_rows, int32_t d_head,
                       const float* o_part, const float* lse_part, float* o, float* lse, void* stream);

/*
 * The merge of zl_lse_merge for every KV-split group of a plan, in one launch (§II-B ring
 * accumulation): each group's slab rows are merged over its parts and written to its rows of
 * o and lse, following the row map of zl_plan_group (head subsets land at their strided O
 * rows). Rows outside the groups are left untouched.
 *   o_part, lse_part   the slab zl_attn_fwd wrote (part_rows rows)
 *   o, lse             fp32 [q_rows][d] and [q_rows]
 * A plan with no group makes this a no-op. Pointers 16-B aligned (lse 4-B).
 */
zl_status zl_plan_merge(const zl_plan* plan, const float* o_part, const float* lse_part, float* o, float* lse,
                        void* stream);

/*
 * Backward (the exact backward of §V-A): gradients of f = sum over covered rows of
 * dO . O with respect to Q, K and V, given the final (merged) O and LSE.
 *   q, k, v, d_o   bf16 device tensors; o, lse the forward's final fp32 outputs
 *   dq             fp32 [q_rows][d]: overwritten for every covered row; a KV-split group
 *                  gets the sum over its parts
 *   dk, dv         fp32 [kv_rows][d]: overwritten for every covered row
 *   workspace      device memory of info.ws_bwd bytes (queue counters, per-row -D and
 *                  -LSE / tau, sentinel rows, split dQ and dK/dV partials), not shared
 *                  with a concurrent call
 * Rows that no segment covers are left untouched. Pointers must be 16-B aligned. Plans with
 * more than 2^29 query rows are rejected (ZL_ERR_UNSUPPORTED).
 */
zl_status zl_attn_bwd(const zl_plan* plan, const void* q, const void* k, const void* v,
                      const float* o, const float* lse, const void* d_o,
                      float* dq, float* dk, float* dv, void* workspace, void* stream);

/* Stages of the backward, for zl_attn_bwd_stages. */
#define ZL_BWD_PRE 1u   /* D_i = dO_i . O_i for every covered query row; resets both queues */
#define ZL_BWD_DKDV 2u  /* key-major kernel: dK and dV */
#define ZL_BWD_DQ 4u    /* query-major kernel: dQ */
#define ZL_BWD_ALL 7u

/*
 * The backward split into its three launches, for callers that time or schedule them
 * separately: `stages` is a non-zero mask of ZL_BWD_* bits, launched in the order PRE, DKDV,
 * DQ. DKDV and DQ read what PRE left in `workspace`, and each consumes its queue: run PRE
 * (on the same workspace and inputs) before every DKDV and every DQ. zl_attn_bwd is
 * zl_attn_bwd_stages(..., ZL_BWD_ALL). Arguments as for zl_attn_bwd.
 */
zl_status zl_attn_bwd_stages(const zl_plan* plan, const void* q, const void* k, const void* v,
                             const float* o, const float* lse, const void* d_o,
                             float* dq, float* dk, float* dv, void* workspace, uint32_t stages, void* stream);

/*
 * The backward of zl_attn_bwd with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The scratch zl_attn_bwd keeps in its workspace (queue counters, -D and -LSE / tau
 * per query row, sentinel rows, split partials) lives instead in a fixed device array of
 * ZL_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on until the process
 * ends; its address is looked up on the first call on each device. Nothing is allocated or
 * freed. Plans whose info.ws_bwd exceeds ZL_NOALLOC_SCRATCH_BYTES are rejected with
 * ZL_ERR_UNSUPPORTED. Every call on a device shares that device's array: calls that overlap
 * on one device (two streams, or two threads) race and must be ordered by the caller. Each
 * call rewrites what it reads of the array, so no clearing is needed between calls. Arguments
 * and results as for zl_attn_bwd; the same kernels run.
 */
#define ZL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
zl_status zl_attn_bwd_noalloc(const zl_plan* plan, const void* q, const void* k, const void* v,
                              const float* o, const float* lse, const void* d_o,
                              float* dq, float* dk, float* dv, void* stream);

/* Thread-local message describing the last failure on this thread ("" if none). */
const char* zl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZL_H */
