"""Host checks of the lane and address arithmetic the HIP kernels rely on,
restated from the formulas in their sources and checked for the properties
the kernels need (exact cover, bank-conflict freedom, reduction results).
Nothing here runs on the GPU.

* MLA head staging (mla_kv_head.hip): rows of 128 bytes, eight 16-byte
  pieces, piece c of row r in slot c ^ (r % 8); a direct global -> LDS load
  of 1 KiB writes byte 16 l from lane l (row l / 8 of the block, slot l % 8)
  and fetches piece (l % 8) ^ (l / 8); a fragment read (MFMA step s) takes
  row fr = l % 16 of a 16-row tile and piece 4 s + l / 16.
* QSAPrepare rows (qsa_prepare.hip, Di = 128): load k of a block brings
  rows 4 k .. 4 k + 3, lane l fetching 16-byte piece l % 16 of row
  4 k + l / 16 and writing it at LDS byte 1024 k + 16 l; lane p then reads
  the 4-byte word 64 i + p for the dimension pair (2 p, 2 p + 1) of row i.
  At most W row loads are in flight: W issued first, load K + W issued after
  group K is added; the wait before group K allows min(NK - K, W) - 1
  outstanding loads.
* Block selection (qsa_select.hip): the DPP lane permutations used by the
  reductions (quad permutes, row_ror:8, half-row and row mirrors), and the
  transposing reduction of the Q head sum and the eight-lane partial combine.
"""

import numpy as np
import pytest

# ---------------------------------------------------------------------------
# MLA staging

def mla_dma(lane, block):
    """(row in the stage, slot) written and (row, piece) fetched by `lane` of
    the 1 KiB load of `block`."""
    row = 8 * block + lane // 8
    slot = lane % 8
    piece = (lane % 8) ^ (lane // 8)
    return (row, slot), (row, piece)

def mla_read(lane, tile_row0, step):
    """(row, piece) wanted by a fragment read and the byte offset it reads."""
    fr, fc = lane % 16, lane // 16
    row = tile_row0 + fr
    piece = 4 * step + fc
    slot = piece ^ (fr % 8)                  # swz of the row: tile_row0 % 16 == 0
    return (row, piece), row * 128 + 16 * slot

def test_mla_dma_covers_every_piece_once():
    for block in range(36):                  # the W stage: 288 rows
        written = {}
        for lane in range(64):
            (row, slot), (frow, piece) = mla_dma(lane, block)
            assert frow == row
            # the slot holds the piece its own permutation says it holds
            assert slot == piece ^ (row % 8)
            written[(row, piece)] = slot
        assert sorted(written) == [(r, p) for r in range(8 * block, 8 * block + 8) for p in range(8)]

def test_mla_fragment_reads_find_what_the_loads_wrote():
    slot_of = {}
    for block in range(32):                  # the x stage: 256 rows
        for lane in range(64):
            (row, slot), (_, piece) = mla_dma(lane, block)
            slot_of[(row, piece)] = slot
    for tile_row0 in range(0, 256, 16):
        for step in (0, 1):
            for lane in range(64):
                (row, piece), off = mla_read(lane, tile_row0, step)
                assert off == row * 128 + 16 * slot_of[(row, piece)]

def test_mla_fragment_reads_are_bank_conflict_free_per_eight_lanes():
    # the LDS serves a 16-byte read eight lanes (128 bytes) at a time: the
    # eight lanes of a group must hit eight different 16-byte bank groups
    for tile_row0 in range(0, 256, 16):
        for step in (0, 1):
            offs = [mla_read(lane, tile_row0, step)[1] for lane in range(64)]
            for g in range(8):
                groups = {(o % 128) // 16 for o in offs[8 * g:8 * g + 8]}
                assert len(groups) == 8

def test_mla_former_permutation_conflicted_for_eight_lanes():
    # the permutation it replaced, (r / 4) mod 4 over four 16-byte pieces of
    # 64-byte rows, serves 16 lanes at a time but not 8 (what the counters
    # showed): a pin that the check above can fail
    def off(lane):
        fr, fc = lane % 16, lane // 16
        return fr * 64 + 16 * (fc ^ ((fr >> 2) & 3))
    offs = [off(lane) for lane in range(64)]
    assert any(len({(o % 128) // 16 for o in offs[8 * g:8 * g + 8]}) < 8 for g in range(8))
    assert all(len({(o % 256) // 16 for o in offs[16 * g:16 * g + 16]}) == 16 for g in range(4))

# ---------------------------------------------------------------------------
# QSAPrepare direct row loads

def test_qsa_row_loads_land_where_the_column_reads_look():
    dims_at_byte = {}
    for k in range(16):
        for lane in range(64):
            row, piece = 4 * k + lane // 16, lane % 16
            byte = 1024 * k + 16 * lane
            for e in range(8):                   # the piece's eight bf16 dims
                dims_at_byte[byte + 2 * e] = (row, 8 * piece + e)
    assert len(dims_at_byte) == 64 * 128         # every (row, dim) staged once
    for i in range(64):
        for p in range(64):
            word = 64 * i + p
            assert dims_at_byte[4 * word] == (i, 2 * p)          # low half
            assert dims_at_byte[4 * word + 2] == (i, 2 * p + 1)  # high half

def window_schedule(nk, w, extra_older=0):
    """The wave's vector-memory program: ('load', k) and ('wait', n) in issue
    order, extra_older loads (the cos/sin and weight values) first."""
    prog = [("load", -1 - i) for i in range(extra_older)]
    prog += [("load", k) for k in range(min(w, nk))]
    for k in range(nk):
        prog.append(("wait", min(nk - k, w) - 1))
        prog.append(("use", k))
        if k + w < nk:
            prog.append(("load", k + w))
    return prog

def loads_done_at_each_use(prog):
    """With in-order completion, a wait for at most n outstanding guarantees
    every load but the n youngest issued so far: the set guaranteed at each use."""
    issued, guaranteed, out = [], set(), {}
    for op, v in prog:
        if op == "load":
            issued.append(v)
        elif op == "wait":
            guaranteed |= set(issued[:len(issued) - v] if v else issued)
        else:
            out[v] = set(guaranteed)
    return out

@pytest.mark.parametrize("w", range(1, 17))
@pytest.mark.parametrize("extra", [0, 3])
def test_qsa_row_window_waits_cover_each_group(w, extra):
    prog = window_schedule(16, w, extra)
    assert sorted(v for op, v in prog if op == "load" and v >= 0) == list(range(16))
    done = loads_done_at_each_use(prog)
    for k in range(16):
        assert k in done[k]                       # the group's load has landed
    # never more than w row loads in flight
    inflight = 0
    for op, v in prog:
        if op == "load" and v >= 0:
            inflight += 1
            assert inflight <= w
        elif op == "use":
            inflight -= 1

def test_qsa_row_window_pin_fails_with_a_wait_one_too_weak():
    # waiting for min(NK - K, W) outstanding instead of that minus one lets a
    # group be read before its load lands: the check above must catch it
    prog = [(op, v + 1) if op == "wait" else (op, v) for op, v in window_schedule(16, 10)]
    done = loads_done_at_each_use(prog)
    assert any(k not in done[k] for k in range(16))

# ---------------------------------------------------------------------------
# DPP lane permutations inside a 16-lane row (the source lane of each lane)

def quad_perm(sel):
    return [4 * (i // 4) + sel[i % 4] for i in range(16)]

XOR1 = quad_perm([1, 0, 3, 2])
XOR2 = quad_perm([2, 3, 0, 1])
HALF_MIRROR = [8 * (i // 8) + 7 - i % 8 for i in range(16)]
MIRROR = [15 - i for i in range(16)]
ROR8 = [(i + 8) % 16 for i in range(16)]

def dpp(vals, perm):
    return [vals[perm[i]] for i in range(16)]

def test_dpp_permutations_are_the_xor_partners_claimed():
    assert XOR1 == [i ^ 1 for i in range(16)]
    assert XOR2 == [i ^ 2 for i in range(16)]
    assert ROR8 == [i ^ 8 for i in range(16)]
    assert HALF_MIRROR == [i ^ 7 for i in range(16)]
    assert MIRROR == [i ^ 15 for i in range(16)]

def test_eight_lane_combine_gives_every_lane_the_total():
    # xor 1, xor 2, then the half-row mirror (xor 7): the per-head combine of
    # eight lanes of partials in the selection kernel
    rng = np.random.default_rng(1)
    v = [int(x) for x in rng.integers(0, 1000, 16)]
    s = list(v)
    for perm in (XOR1, XOR2, HALF_MIRROR):
        t = dpp(s, perm)
        s = [s[i] + t[i] for i in range(16)]
    for i in range(16):
        assert s[i] == sum(v[8 * (i // 8):8 * (i // 8) + 8])

def transposing_reduce(vals):
    """The selection kernel's head-lane reduction: 16 lanes with 4 block
    values each; lane fr keeps / sends by bits 3 and 2 of fr."""
    b3 = [bool(fr & 8) for fr in range(16)]
    b2 = [bool(fr & 4) for fr in range(16)]
    k0 = [vals[f][2] if b3[f] else vals[f][0] for f in range(16)]
    s0 = [vals[f][0] if b3[f] else vals[f][2] for f in range(16)]
    k1 = [vals[f][3] if b3[f] else vals[f][1] for f in range(16)]
    s1 = [vals[f][1] if b3[f] else vals[f][3] for f in range(16)]
    r0, r1 = dpp(s0, ROR8), dpp(s1, ROR8)
    x0 = [k0[f] + r0[f] for f in range(16)]
    x1 = [k1[f] + r1[f] for f in range(16)]
    k = [x1[f] if b2[f] else x0[f] for f in range(16)]
    s = [x0[f] if b2[f] else x1[f] for f in range(16)]
    rs = dpp(s, HALF_MIRROR)
    y = [k[f] + rs[f] for f in range(16)]
    t = dpp(y, XOR2)
    y = [y[f] + t[f] for f in range(16)]
    t = dpp(y, XOR1)
    return [y[f] + t[f] for f in range(16)]

@pytest.mark.parametrize("seed", range(4))
def test_transposing_reduction_gives_block_fr_over_4(seed):
    rng = np.random.default_rng(seed)
    vals = [[int(x) for x in rng.integers(-1000, 1000, 4)] for _ in range(16)]
    out = transposing_reduce(vals)
    for fr in range(16):
        assert out[fr] == sum(vals[f][fr >> 2] for f in range(16)), fr

def test_transposing_reduction_pin_fails_with_a_wrong_partner():
    # replacing the half-row mirror (xor 7) by xor 2 pairs lanes that hold
    # different blocks: the check above must catch it
    global HALF_MIRROR
    saved = HALF_MIRROR
    try:
        HALF_MIRROR = XOR2
        rng = np.random.default_rng(7)
        vals = [[int(x) for x in rng.integers(-1000, 1000, 4)] for _ in range(16)]
        out = transposing_reduce(vals)
        assert any(out[fr] != sum(vals[f][fr >> 2] for f in range(16)) for fr in range(16))
    finally:
        HALF_MIRROR = saved

def test_quad_rank_lanes_cover_every_key_pair_once():
    # up to 128 candidates: lane r of a quad reads key pairs 4 t + r, t < 16
    for J4 in range(4, 129, 4):
        seen = []
        for r in range(4):
            for t in range(16):
                p = r + 4 * t
                if 2 * p < J4:
                    seen.append(p)
        assert sorted(seen) == list(range(J4 // 2))
