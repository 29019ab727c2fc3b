"""Host-side plan tests (no GPU): validation, work queues, cost order, ring-group layout."""
import ctypes

import pytest

import coalesced_varlen_attention_amd as z
import workloads as W

ZL_ERR_INVALID, ZL_ERR_UNSUPPORTED = -1, -2


def host_plan(pack):
    return z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, pack.scale, host_only=True)


def expect_error(status, seq_q, seq_kv, heads, segs, d=128, scale=None, match=None, **kw):
    with pytest.raises(z.ZlError) as e:
        z.Plan(seq_q, seq_kv, heads, segs, d, scale, host_only=True, **kw)
    assert e.value.status == status
    if match:
        assert match in str(e.value), str(e.value)


@pytest.mark.parametrize("name,rows,fwd,bwd,dq_rows,dq", [
    ("tiny", 128, 44, 44, 128, 44), ("image", 256, 5376, 10752, 256, 5376),
    ("mixed", 256, 16840, 33675, 256, 16840), ("ring", 256, 11840, 23680, 256, 1480),
    ("long", 256, 14845, 29685, 256, 14845), ("shard", 128, 1280, 1280, 128, 1280)])
def test_tile_counts(name, rows, fwd, bwd, dq_rows, dq):
    """Item counts, with the query-major item sizes the plan picks: 256 rows when the queue holds
    at least 4 rounds of 256-row items for the 256 resident wide workgroups of a host-only plan
    (image: 5,376 items, 21 rounds; the ring shard's dQ queue, one item list per group rather
    than per part: 1,480 items, 5.8 rounds), else 128 rows (the 5-head shard: 640 wide items,
    2.5 rounds; the tiny pack's 24, too short to split)."""
    p = host_plan(W.config(name))
    assert p.info["fwd_rows"] == rows and p.info["dq_rows"] == dq_rows
    assert p.info["fwd_tiles"] == fwd and p.info["bwd_tiles"] == bwd and p.info["dq_tiles"] == dq
    assert all(t[3] <= rows for t in p.tiles(0)) and max(t[3] for t in p.tiles(0)) == rows
    assert max(t[3] for t in p.tiles(2)) == dq_rows


def test_item_rows_rule_and_flags():
    """The size rule for r rounds of wide items (256 host-only wide workgroups), for the forward
    and the dQ queue alike: wide from 4 rounds (1,024 items); narrow above one round and below 4;
    wide from half a round to one; below half a round wide only if split pieces will fill the
    device (an item of at least 2,048 keys, split on). The flags fix both sizes either way and
    exclude each other."""
    def plan(n_heads, keys=2048, **kw):  # n_heads x 8 wide items of one 2,048-query sequence
        return z.Plan((2048,), (keys,), (n_heads,), ((0, 0, n_heads, 0, 2048, 0, keys, -1),), 64,
                      host_only=True, **kw).info
    def rows(info):
        return info["fwd_rows"], info["dq_rows"]
    assert rows(plan(128)) == (256, 256) and plan(128)["fwd_tiles"] == plan(128)["dq_tiles"] == 1024
    assert rows(plan(127)) == (128, 128) and plan(127)["fwd_tiles"] == 127 * 16
    assert rows(plan(33)) == (128, 128)                               # 264 items: just over one round
    assert rows(plan(32)) == rows(plan(16)) == (256, 256)             # 256 and 128 items
    assert rows(plan(16, keys=100, split=False)) == (256, 256)
    assert rows(plan(15)) == (256, 256) and plan(15)["split_tiles"] > 0 and plan(15)["dq_split_tiles"] > 0
    assert rows(plan(15, keys=2047)) == (128, 128)                    # too short to cut into two pieces
    assert rows(plan(15, split=False)) == (128, 128)
    assert rows(plan(127, item_rows=256)) == (256, 256)
    assert rows(plan(128, item_rows=128)) == (128, 128)
    with pytest.raises(ValueError):
        plan(4, item_rows=192)
    lib = z.lib()
    out = ctypes.c_void_p()
    seg = z._Segment(0, 0, 1, 0, 4, 0, 4, -1)
    cu = (ctypes.c_int64 * 2)(0, 4)
    heads = (ctypes.c_int32 * 1)(1)
    st = lib.zl_plan_build(1, ctypes.addressof(cu), ctypes.addressof(cu), ctypes.addressof(heads), 1,
                           ctypes.addressof(seg), 64, 0.0, 1 | z.ZL_PLAN_NARROW_ITEMS | z.ZL_PLAN_WIDE_ITEMS,
                           ctypes.byref(out))
    assert st == ZL_ERR_INVALID and b"exclude" in lib.zl_last_error()


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_flops_and_rows(name):
    pack = W.config(name)
    p = host_plan(pack)
    assert p.info["fwd_flops"] == pack.flops_fwd()
    assert p.info["bwd_flops"] == 2.5 * pack.flops_fwd()
    assert p.info["q_rows"] == pack.q_rows() and p.info["kv_rows"] == pack.kv_rows()
    assert abs(p.info["softmax_scale"] - pack.d ** -0.5) < 1e-7


def test_mixed_pack_metric_flops():
    # 60.31 TFLOP forward, 211.08 TFLOP forward+backward on the mixed image-video pack
    p = host_plan(W.mixed())
    assert abs(p.info["fwd_flops"] - 60.308e12) < 0.01e12
    assert abs(3.5 * p.info["fwd_flops"] - 211.08e12) < 0.01e12
    # fp32 O of this pack exceeds 2^31 bytes: offsets must be 64-bit
    assert p.info["q_rows"] * 128 * 4 > 2 ** 31


def _per_queue_cost_order(tiles, costs, bounds):
    """Within each queue: decreasing cost, equal costs in (segment, head, block) order."""
    for q in range(len(bounds) - 1):
        lo, hi = bounds[q], bounds[q + 1]
        for i in range(lo, hi - 1):
            assert costs[i] >= costs[i + 1], f"queue {q} not in decreasing cost order"
            if costs[i] == costs[i + 1]:
                assert tiles[i][:3] < tiles[i + 1][:3], "equal-cost items not in (segment, head, block) order"


def _balanced(costs, bounds, tol=0.15):
    loads = [sum(costs[bounds[q]:bounds[q + 1]]) for q in range(len(bounds) - 1)]
    mean = sum(loads) / len(loads)
    biggest = max(costs) if costs else 0
    assert max(loads) <= mean * (1 + tol) + biggest, f"queue loads {loads}"


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("name", ["tiny", "mixed", "ring", "long"])
def test_queue_covers_every_block_once_in_cost_order(name, which):
    pack = W.config(name)
    p = host_plan(pack)
    tiles = p.tiles(which)
    bounds = p.queues(which)
    assert len(bounds) == 9 and bounds[0] == 0 and bounds[-1] == len(tiles)
    assert all(a <= b for a, b in zip(bounds, bounds[1:]))
    block = p.info["fwd_rows"] if which == 0 else 128
    seen = set()
    for (seg, h, r0, n) in tiles:
        s, h0, h1, q0, q1, k0, k1, part = pack.segments[seg]
        lo, hi = (q0, q1) if which == 0 else (k0, k1)
        assert h0 <= h < h1 and lo <= r0 and r0 + n <= hi and 1 <= n <= block
        assert (r0 - lo) % block == 0 and (n == block or r0 + n == hi)
        assert (seg, h, r0) not in seen
        seen.add((seg, h, r0))
    expected = sum((s[2] - s[1]) * -(-((s[4] - s[3]) if which == 0 else (s[6] - s[5])) // block) for s in pack.segments)
    assert len(seen) == expected
    other = lambda t: (pack.segments[t[0]][6] - pack.segments[t[0]][5]) if which == 0 else (pack.segments[t[0]][4] - pack.segments[t[0]][3])
    costs = [t[3] * other(t) for t in tiles]
    _per_queue_cost_order(tiles, costs, bounds)
    _balanced(costs, bounds)


def test_queue_keeps_heads_together():
    """Chunks of one (segment, head) stay together: the mixed pack's forward items of a head
    land in few queues, so a head's K/V is read through few L2s."""
    pack = W.mixed()
    p = host_plan(pack)
    tiles, bounds = p.tiles(0), p.queues(0)
    where = {}
    for q in range(8):
        for (seg, h, r0, n) in tiles[bounds[q]:bounds[q + 1]]:
            where.setdefault((seg, h), set()).add(q)
    spread = sum(len(v) for v in where.values()) / len(where)
    assert spread < 1.5, spread


@pytest.mark.parametrize("name", ["tiny", "mixed", "ring"])
def test_dq_queue(name):
    """One dQ item per (final segment or ring group, head, block of query rows), in decreasing
    cost (rows x keys of the whole group) order; a ring group's items name its part-0 segment.
    Every pack here has a segment longer than a block, so the largest item is one block."""
    pack = W.config(name)
    p = host_plan(pack)
    tiles = p.tiles(2)
    assert p.info["dq_tiles"] == len(tiles)
    block = max(t[3] for t in tiles)
    assert block in (128, 256)
    owners = [i for i, s in enumerate(pack.segments) if s[7] <= 0]
    keys_of = {}
    for i in owners:
        s = pack.segments[i]
        if s[7] < 0:
            keys_of[i] = s[6] - s[5]
        else:
            keys_of[i] = sum(t[6] - t[5] for t in pack.segments if t[7] >= 0 and t[:5] == s[:5])
    seen = set()
    for (seg, h, r0, n) in tiles:
        assert seg in keys_of
        s = pack.segments[seg]
        assert s[1] <= h < s[2] and s[3] <= r0 and r0 + n <= s[4] and (r0 - s[3]) % block == 0
        seen.add((seg, h, r0))
    assert len(seen) == len(tiles) == sum((pack.segments[i][2] - pack.segments[i][1]) *
                                          -(-(pack.segments[i][4] - pack.segments[i][3]) // block) for i in owners)
    costs = [t[3] * keys_of[t[0]] for t in tiles]
    bounds = p.queues(2)
    assert bounds[-1] == len(tiles)
    _per_queue_cost_order(tiles, costs, bounds)
    _balanced(costs, bounds)


def test_ring_group_layout():
    pack = W.ring()
    p = host_plan(pack)
    assert p.info["n_groups"] == 1 and p.info["n_parts_max"] == 8
    g = p.groups[0]
    assert g == {"n_parts": 8, "seq": 0, "n_rows": 9450 * 40, "o_row": 0, "part_row": 0, "head_begin": 0,
                 "head_end": 40, "n_heads": 40, "q_begin": 0, "q_end": 9450}
    assert p.info["part_rows"] == 8 * 9450 * 40


def test_two_groups_stack_in_the_slab():
    seg = ((0, 0, 2, 0, 10, 0, 5, 0), (0, 0, 2, 0, 10, 5, 9, 1), (1, 0, 3, 4, 8, 0, 3, 1), (1, 0, 3, 4, 8, 3, 6, 0))
    p = z.Plan((10, 12), (9, 6), (2, 3), seg, 64, host_only=True)
    g0, g1 = p.groups
    assert g0["n_rows"] == 20 and g0["part_row"] == 0 and g0["o_row"] == 0
    assert g1["n_rows"] == 12 and g1["part_row"] == 40 and g1["o_row"] == 20 + 4 * 3
    assert p.info["part_rows"] == 40 + 24


def test_validation_errors():
    ok = (0, 0, 2, 0, 8, 0, 8, -1)
    expect_error(ZL_ERR_UNSUPPORTED, [8], [8], [2], [ok], d=96, match="d_head")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(1, 0, 2, 0, 8, 0, 8, -1)], match="no such sequence")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 3, 0, 8, 0, 8, -1)], match="head range")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 1, 1, 0, 8, 0, 8, -1)], match="head range")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 3, 3, 0, 8, -1)], match="query range")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 9, 0, 8, -1)], match="query range")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 8, -1, 8, -1)], match="key range")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 8, 0, 8, -2)], match="part")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [], match="at least one segment")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [ok], scale=float("inf"), match="scale")
    # overlapping outputs / aliased keys
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [ok, (0, 1, 2, 4, 8, 0, 8, -1)], match="same output rows")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 4, 0, 8, -1), (0, 0, 2, 4, 8, 2, 5, -1)],
                 match="same K/V rows")
    # ring groups
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 8, 0, 4, 0), (0, 1, 2, 0, 8, 4, 8, 0)],
                 match="same output rows")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 8, 0, 4, 0), (0, 0, 2, 0, 8, 4, 8, 0)],
                 match="numbered")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 8, 0, 4, 0), (0, 0, 2, 0, 8, 4, 8, 2)],
                 match="numbered")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 8, 0, 5, 0), (0, 0, 2, 0, 8, 4, 8, 1)],
                 match="share key rows")
    expect_error(ZL_ERR_INVALID, [8], [8], [2], [(0, 0, 2, 0, 8, 0, 4, 0), (0, 0, 2, 0, 8, 4, 8, 1), ok],
                 match="same output rows")


def test_bad_sequence_arrays():
    lib = z.lib()
    out = ctypes.c_void_p()
    seg = z._Segment(0, 0, 1, 0, 4, 0, 4, -1)
    cu_bad0 = (ctypes.c_int64 * 2)(1, 5)
    cu = (ctypes.c_int64 * 2)(0, 4)
    dec = (ctypes.c_int64 * 3)(0, 4, 3)
    heads = (ctypes.c_int32 * 2)(1, 1)
    zero_heads = (ctypes.c_int32 * 1)(0)
    st = lib.zl_plan_build(1, ctypes.addressof(cu_bad0), ctypes.addressof(cu), ctypes.addressof(heads), 1,
                           ctypes.addressof(seg), 64, 0.0, 1, ctypes.byref(out))
    assert st == ZL_ERR_INVALID and b"cu_seqlens[0]" in lib.zl_last_error()
    st = lib.zl_plan_build(2, ctypes.addressof(dec), ctypes.addressof(dec), ctypes.addressof(heads), 1,
                           ctypes.addressof(seg), 64, 0.0, 1, ctypes.byref(out))
    assert st == ZL_ERR_INVALID and b"decreases" in lib.zl_last_error()
    st = lib.zl_plan_build(1, ctypes.addressof(cu), ctypes.addressof(cu), ctypes.addressof(zero_heads), 1,
                           ctypes.addressof(seg), 64, 0.0, 1, ctypes.byref(out))
    assert st == ZL_ERR_INVALID and b"seq_heads" in lib.zl_last_error()
    st = lib.zl_plan_build(1, ctypes.addressof(cu), ctypes.addressof(cu), ctypes.addressof(heads), 1,
                           ctypes.addressof(seg), 64, 0.0, 128, ctypes.byref(out))
    assert st == ZL_ERR_INVALID and b"flag" in lib.zl_last_error()
    assert lib.zl_plan_build(1, None, None, None, 1, None, 64, 0.0, 1, ctypes.byref(out)) == ZL_ERR_INVALID


def test_host_only_plan_cannot_run_and_merge_checks():
    p = host_plan(W.tiny())
    lib = z.lib()
    assert lib.zl_attn_fwd(p.handle, 16, 16, 16, 16, 16, None, None, 16, None) == ZL_ERR_INVALID
    assert b"host-only" in lib.zl_last_error()
    assert lib.zl_attn_bwd(p.handle, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, None) == ZL_ERR_INVALID
    assert lib.zl_attn_fwd(None, 16, 16, 16, 16, 16, None, None, 16, None) == ZL_ERR_INVALID
    assert lib.zl_lse_merge(2, 10, 96, 16, 16, 16, 16, None) == ZL_ERR_UNSUPPORTED
    assert lib.zl_lse_merge(0, 10, 128, 16, 16, 16, 16, None) == ZL_ERR_INVALID
    assert lib.zl_lse_merge(2, -1, 128, 16, 16, 16, 16, None) == ZL_ERR_INVALID
    assert lib.zl_lse_merge(2, 0, 128, None, None, None, None, None) == 0
    assert lib.zl_lse_merge(2, 10, 128, 24, 16, 16, 16, None) == ZL_ERR_INVALID  # misaligned o_part


def test_scale_override():
    pack = W.tiny()
    p = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, 0.3, host_only=True)
    assert abs(p.info["softmax_scale"] - 0.3) < 1e-7


def test_accumulate_rejects_two_parts_of_one_group():
    lib = z.lib()
    seg = ((0, 0, 2, 0, 40, 0, 30, 0), (0, 0, 2, 0, 40, 30, 70, 1))
    p = z.Plan((40,), (70,), (2,), seg, 64, host_only=True)
    assert lib.zl_attn_fwd_accumulate(p.handle, 16, 16, 16, 16, 16, 16, None) == ZL_ERR_INVALID
    assert b"parts" in lib.zl_last_error()
    one = z.Plan((40,), (70,), (2,), ((0, 0, 2, 0, 40, 30, 70, 0),), 64, host_only=True)
    assert lib.zl_attn_fwd_accumulate(one.handle, 16, 16, 16, 16, 16, 16, None) == ZL_ERR_INVALID
    assert b"host-only" in lib.zl_last_error()
    assert lib.zl_attn_fwd_accumulate(None, 16, 16, 16, 16, 16, 16, None) == ZL_ERR_INVALID


def test_head_subset_groups():
    """Composed placements: ring groups over head subsets of one sequence (Ulysses x ring)."""
    seg = ((0, 0, 2, 0, 10, 0, 5, 0), (0, 0, 2, 0, 10, 5, 9, 1),   # heads [0,2): 2 parts
           (0, 2, 5, 3, 7, 0, 3, 1), (0, 2, 5, 3, 7, 3, 9, 0),     # heads [2,5), queries [3,7)
           (1, 0, 5, 0, 6, 0, 6, -1))                              # a final segment beside them
    p = z.Plan((10, 6), (9, 6), (5, 5), seg, 128, host_only=True)
    g0, g1 = p.groups
    assert g0["n_rows"] == 10 * 2 and g0["o_row"] == 0 and g0["part_row"] == 0 and g0["n_heads"] == 5
    assert (g0["head_begin"], g0["head_end"]) == (0, 2)
    assert g1["n_rows"] == 4 * 3 and g1["o_row"] == 3 * 5 + 2 and g1["part_row"] == 2 * 20
    assert (g1["head_begin"], g1["head_end"], g1["q_begin"], g1["q_end"]) == (2, 5, 3, 7)
    assert p.info["part_rows"] == 2 * 20 + 2 * 12


def _pieces_by_item(p):
    items = {}
    for (seg, head, row0, nrows, k0, k1, split, piece) in p.tiles(3):
        items.setdefault((seg, head, row0, nrows), []).append((k0, k1, split, piece & 0xFFFF, piece >> 16))
    return items


def test_split_kv_cuts_long_items_of_a_short_queue():
    """One head of 8192 tokens in 128-row forward items: 64 items, far below one per resident
    workgroup (512 assumed for a host-only plan), so every item is cut into 8 key pieces of 1024
    keys. (Left to choose, the plan takes 256-row items here, whose pieces fill its 256 slots.)"""
    p = z.Plan((8192,), (8192,), (1,), ((0, 0, 1, 0, 8192, 0, 8192, -1),), 128, host_only=True, item_rows=128)
    assert p.info["split_tiles"] == 64 and p.info["split_pieces"] == 64 * 8
    assert p.info["fwd_tiles"] == 64 * 8
    slots = set()
    for key, pieces in _pieces_by_item(p).items():
        pieces.sort()
        assert len(pieces) == 8
        assert pieces[0][0] == 0 and pieces[-1][1] == 8192
        for a, b in zip(pieces[:-1], pieces[1:]):
            assert a[1] == b[0]                                  # contiguous, disjoint
        for (k0, k1, split, idx, n) in pieces:
            assert n == 8 and k0 % 64 == 0 and k1 - k0 >= 1024
        assert sorted(x[3] for x in pieces) == list(range(8))
        assert len({x[2] for x in pieces}) == 1                  # one slot per item
        slots.add(pieces[0][2])
    assert sorted(slots) == list(range(0, 512, 8))
    # the workspace holds a counter, 128 O rows and 128 LSEs per piece
    nosplit = z.Plan((8192,), (8192,), (1,), ((0, 0, 1, 0, 8192, 0, 8192, -1),), 128, host_only=True, split=False,
                     item_rows=128)
    assert nosplit.info["split_tiles"] == 0 and nosplit.info["fwd_tiles"] == 64
    extra = p.info["ws_fwd"] - nosplit.info["ws_fwd"]
    assert extra >= 512 * (4 + 128 * 128 * 4 + 128 * 4)
    # with 256-row items each piece holds 256 O rows and LSEs
    wide = z.Plan((8192,), (8192,), (1,), ((0, 0, 1, 0, 8192, 0, 8192, -1),), 128, host_only=True, item_rows=256)
    assert wide.info["fwd_rows"] == 256 and wide.info["split_tiles"] == 32
    n = wide.info["split_pieces"]
    assert wide.info["ws_fwd"] - nosplit.info["ws_fwd"] >= n * (4 + 256 * 128 * 4 + 256 * 4)


def test_split_kv_ragged_and_short_items():
    """Pieces are block-aligned with the ragged tail in the last one; items with fewer than
    2048 keys stay whole; unsplit items carry slot -1 and one piece."""
    seg = ((0, 0, 2, 0, 300, 0, 4100, -1), (1, 0, 2, 0, 200, 0, 2000, -1))
    p = z.Plan((300, 200), (4100, 2000), (2, 2), seg, 64, host_only=True)
    for key, pieces in _pieces_by_item(p).items():
        if key[0] == 1:
            assert pieces == [(0, 2000, -1, 0, 1)]
            continue
        pieces.sort()
        n = len(pieces)
        assert 2 <= n <= 4 and pieces[0][0] == 0 and pieces[-1][1] == 4100
        assert all(k0 % 64 == 0 for (k0, *_r) in pieces)


def test_split_kv_leaves_large_packs_alone():
    for name in ("image", "mixed", "ring", "long", "shard"):
        assert host_plan(W.config(name)).info["split_tiles"] == 0, name
    p = host_plan(W.config("head1"))  # 128 wide items < 256 resident wide workgroups: 2 pieces each
    assert p.info["fwd_rows"] == 256 and p.info["split_tiles"] == 128 and p.info["split_pieces"] == 128 * 2


def test_qkv_packed_plan():
    seg = ((0, 0, 2, 0, 10, 0, 10, -1), (1, 0, 3, 0, 6, 0, 6, -1))
    p = z.Plan((10, 6), (10, 6), (2, 3), seg, 64, host_only=True, qkv_packed=True)
    assert p.info["qkv_rows"] == 3 * (10 * 2 + 6 * 3) and p.info["q_rows"] == 38
    assert z.Plan((10, 6), (10, 6), (2, 3), seg, 64, host_only=True).info["qkv_rows"] == 0
    expect_error(ZL_ERR_INVALID, [10], [12], [2], [(0, 0, 2, 0, 10, 0, 12, -1)], match="equal query and key",
                 qkv_packed=True)


def _dq_pieces(p):
    """dQ queue (which = 4) grouped by item: (first block, end block, slot, piece, pieces)."""
    items = {}
    for (seg, h, r0, n, b0, b1, split, piece) in p.tiles(4):
        items.setdefault((seg, h, r0, n), []).append((b0, b1, split, piece & 0xffff, piece >> 16))
    return items


def test_dq_split_cuts_items_of_a_short_queue():
    """One head of 8192 tokens: 32 dQ items of 256 query rows over a chain of 128 key blocks, far
    fewer than the resident wide dQ workgroups a host-only plan assumes (one per CU x 256 CUs):
    each item becomes 8 pieces of 16 blocks (1024 keys), contiguous, with one workspace slot per
    item."""
    seg = ((0, 0, 1, 0, 8192, 0, 8192, -1),)
    p = z.Plan((8192,), (8192,), (1,), seg, 128, host_only=True, item_rows=256)
    nosplit = z.Plan((8192,), (8192,), (1,), seg, 128, host_only=True, split=False, item_rows=256)
    rows = max(t[3] for t in nosplit.tiles(2))
    assert rows == 256 and p.info["dq_rows"] == 256
    n_items = 8192 // rows
    assert p.info["dq_split_tiles"] == n_items and p.info["dq_split_pieces"] == 8 * n_items
    assert p.info["dq_tiles"] == 8 * n_items and nosplit.info["dq_split_tiles"] == 0
    assert nosplit.info["dq_tiles"] == n_items
    assert all(t[4:] == (0, 128, -1, 1 << 16) for t in nosplit.tiles(4))
    items = _dq_pieces(p)
    assert len(items) == n_items
    slots = set()
    for key, pieces in items.items():
        pieces.sort()
        assert [x[3] for x in pieces] == list(range(8)) and all(x[4] == 8 for x in pieces)
        assert pieces[0][0] == 0 and pieces[-1][1] == 128
        assert all(a[1] == b[0] for a, b in zip(pieces[:-1], pieces[1:]))
        assert all(x[1] - x[0] == 16 for x in pieces)
        assert len({x[2] for x in pieces}) == 1
        slots.add(pieces[0][2])
    assert sorted(slots) == list(range(0, 8 * n_items, 8))
    # the workspace holds a counter and `rows` rows of partial dQ per piece
    assert p.info["ws_bwd"] - nosplit.info["ws_bwd"] >= 8 * n_items * (4 + rows * 128 * 4)
    # costs stay proportional to the keys: the queue still sorts by decreasing cost
    t4 = p.tiles(4)
    _per_queue_cost_order([(t[0], t[1], (t[2], t[4])) for t in t4], [t[3] * 64 * (t[5] - t[4]) for t in t4],
                          p.queues(4))


def test_dq_split_over_a_ring_chain():
    """A ring group of 3 parts of 2000 keys: its dQ items walk a chain of 3 x 32 blocks, and the
    pieces cut that chain into runs that may cross part boundaries; the ragged tail item too."""
    seg = tuple((0, 0, 1, 0, 300, 2000 * b, 2000 * (b + 1), b) for b in range(3))
    p = z.Plan((300,), (6000,), (1,), seg, 64, host_only=True)
    items = _dq_pieces(p)
    assert p.info["dq_split_tiles"] == len(items)
    rows = max(k[3] for k in items)
    assert sorted(k[2:] for k in items) == [(r, min(rows, 300 - r)) for r in range(0, 300, rows)]
    for key, pieces in items.items():
        pieces.sort()
        n = pieces[0][4]
        assert 2 <= n <= 96 * 64 // 1024 and len(pieces) == n
        assert pieces[0][0] == 0 and pieces[-1][1] == 96
        assert all(a[1] == b[0] for a, b in zip(pieces[:-1], pieces[1:]))
        assert all(x[1] - x[0] >= 16 for x in pieces)


def test_random_packs_build_valid_plans():
    """Every seeded random pack of the GPU parity test is a valid segment list, and its queues
    cover each (segment, head) block exactly once (host-only plans)."""
    from tests import random_packs as R
    for seed in R.SEEDS:
        pack = R.random_pack(seed)
        p = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, host_only=True)
        assert p.info["q_rows"] == pack.q_rows() and p.info["kv_rows"] == pack.kv_rows()
        rows = p.info["fwd_rows"]
        n_fwd = sum((s[2] - s[1]) * -(-(s[4] - s[3]) // rows) for s in pack.segments)
        assert len({t[:3] for t in p.tiles(0)}) == n_fwd
        n_bwd = sum((s[2] - s[1]) * -(-(s[6] - s[5]) // 128) for s in pack.segments)
        assert len({t[:3] for t in p.tiles(1)}) == n_bwd


def test_dkdv_split_cuts_items_of_a_short_queue():
    """One head of 8192 tokens: 64 dK/dV items of 128 keys over 128 query blocks of 64 rows, fewer
    than the 256 resident dK/dV workgroups assumed for a host-only plan (one per CU): each item
    becomes 4 pieces of 32 query blocks with one workspace slot per item; the unsplit plan's
    items span all 128 blocks."""
    seg = ((0, 0, 1, 0, 8192, 0, 8192, -1),)
    p = z.Plan((8192,), (8192,), (1,), seg, 128, host_only=True)
    nosplit = z.Plan((8192,), (8192,), (1,), seg, 128, host_only=True, split=False)
    assert p.info["kv_split_tiles"] == 64 and p.info["kv_split_pieces"] == 256 and p.info["bwd_tiles"] == 256
    assert nosplit.info["kv_split_tiles"] == 0 and nosplit.info["bwd_tiles"] == 64
    assert all(t[4:] == (0, 128, -1, 1 << 16) for t in nosplit.tiles(5))
    items = {}
    for (seg_, h, r0, n, b0, b1, split, piece) in p.tiles(5):
        items.setdefault((seg_, h, r0, n), []).append((b0, b1, split, piece & 0xffff, piece >> 16))
    assert len(items) == 64
    slots = set()
    for key, pieces in items.items():
        pieces.sort()
        assert [x[3] for x in pieces] == list(range(4)) and all(x[4] == 4 for x in pieces)
        assert pieces[0][0] == 0 and pieces[-1][1] == 128
        assert all(a[1] == b[0] for a, b in zip(pieces[:-1], pieces[1:]))
        assert len({x[2] for x in pieces}) == 1
        slots.add(pieces[0][2])
    assert sorted(slots) == list(range(0, 256, 4))
    # a counter and 128 keys x (dK, dV) rows of partials per piece
    assert p.info["ws_bwd"] - nosplit.info["ws_bwd"] >= 256 * (4 + 128 * 2 * 128 * 4)
    assert sorted(t[:4] for t in nosplit.tiles(1)) == sorted(set(t[:4] for t in p.tiles(1)))


def test_visit_counters_layout():
    """ZL_PLAN_COUNT_VISITS adds one int32 per work item of each queue at the end of the
    workspaces, at the offsets the plan reports; without the flag the offsets are -1 and the
    workspaces keep their size."""
    pack = W.config("mixed")
    plain = host_plan(pack)
    p = z.Plan(pack.seq_q, pack.seq_kv, pack.heads, pack.segments, pack.d, pack.scale, host_only=True,
               count_visits=True)
    a, b = plain.info, p.info
    assert a["visits_fwd"] == a["visits_dkdv"] == a["visits_dq"] == -1
    assert b["visits_fwd"] == a["ws_fwd"] and b["visits_dkdv"] == a["ws_bwd"]
    assert b["ws_fwd"] >= b["visits_fwd"] + 4 * b["fwd_tiles"]
    assert b["visits_dq"] >= b["visits_dkdv"] + 4 * b["bwd_tiles"]
    assert b["ws_bwd"] >= b["visits_dq"] + 4 * b["dq_tiles"]
    assert all(x % 256 == 0 for x in (b["visits_fwd"], b["visits_dkdv"], b["visits_dq"]))
    assert p.tiles(0) == plain.tiles(0) and p.tiles(1) == plain.tiles(1) and p.tiles(2) == plain.tiles(2)


def test_deferred_upload_needs_a_device_plan():
    """zl_plan_upload refuses a plan built without ZL_PLAN_DEFERRED_UPLOAD (here a host-only one)
    before touching the device."""
    p = host_plan(W.config("tiny"))
    assert p.info["dev_bytes"] == 0
    st = z.lib().zl_plan_upload(p.handle, None, 0, None)
    assert st == ZL_ERR_INVALID and b"DEFERRED" in z.lib().zl_last_error()
