"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test checks the oracle against brute force, a closed form, an invariant
or a value printed on the pages, chosen so that a plausible slip in the oracle
(a dropped scale, a wrong slice bound, exp vs exp2, a transposed operand, a
window off by one block) fails at least one of them.  The mutation tests at
the end plant such slips in a copy of the oracle and check they are caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import varlen_oracle as vo
from packed_variable_length_varlen_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.float().numpy()


# ---------------------------------------------------------------- integers


def _validator_pins(validate):
    """What the flat branch's boundary contract fixes (PR #6711, "Reference /
    Acknowledgement": q/kv cu_seqlens with max lengths and padded_tokens = 0):
    a well-formed array is accepted unchanged, and each way of breaking the
    contract is refused."""
    assert list(validate([0, 17, 81, 210], total=210, max_len=129)) == [0, 17, 81, 210]
    assert list(validate([0, 0, 5, 5], total=5, max_len=5)) == [0, 0, 5, 5]  # empty requests
    assert list(validate([0])) == [0]                                        # no request at all
    with pytest.raises(ValueError):
        validate([1, 17, 81, 210])                  # does not start at 0
    with pytest.raises(ValueError):
        validate([0, 17, 16, 210])                  # decreasing
    with pytest.raises(ValueError):
        validate([0, 17, 81, 211], total=210)       # rows past the last request (padding)
    with pytest.raises(ValueError):
        validate([0, 17, 81, 209], total=210)       # fewer rows than the tensor holds
    with pytest.raises(ValueError):
        validate([0, 17, 81, 210], max_len=128)     # a request over the declared max
    with pytest.raises(ValueError):
        validate([])                                # not num_reqs + 1 entries
    with pytest.raises(ValueError):
        validate([[0, 1], [1, 2]])                  # not 1-D


def test_validate_cu_seqlens_accepts_the_contract_and_refuses_the_rest():
    _validator_pins(vo.validate_cu_seqlens)


def test_varlen_attention_refuses_malformed_boundaries():
    q, k, v = (_np(t) for t in wl.random_varlen_case(5, [3, 4], 1, 4, torch.float32))
    good = [0, 3, 7]
    oracle.varlen_attention(q, k, v, good, good, 0.5)
    for bad in ([0, 8, 7], [1, 3, 7], [0, 3, 6], [0, 3, 8]):
        with pytest.raises(ValueError):
            oracle.varlen_attention(q, k, v, bad, good, 0.5)
        with pytest.raises(ValueError):
            oracle.varlen_attention(q, k, v, good, bad, 0.5)


def _planted_validator(old: str, new: str):
    """validate_cu_seqlens with one line of its source replaced (a planted slip)."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(vo.validate_cu_seqlens))
    assert old in src
    ns = dict(vo.__dict__)
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    return ns["validate_cu_seqlens"]


@pytest.mark.parametrize("old,new", [
    ("np.any(lengths < 0)", "False"),                     # monotonicity check skipped
    ("cu[0] != 0", "False"),                              # start not checked
    ("cu[-1] != total", "cu[-1] > total"),                # padding rows let through
    ("lengths.max() > max_len", "lengths.max() > max_len + 1"),  # max off by one
])
def test_planted_validator_slips_are_caught(monkeypatch, old, new):
    bad = _planted_validator(old, new)
    with pytest.raises(pytest.fail.Exception):
        _validator_pins(bad)
    # the attention oracle looks the validator up at call time, so the slip
    # reaches it too and the refusal test catches it there as well
    if old == "np.any(lengths < 0)":
        monkeypatch.setattr(vo, "validate_cu_seqlens", bad)
        with pytest.raises(pytest.fail.Exception):
            test_varlen_attention_refuses_malformed_boundaries()


def test_text_mask_lengths_count_true_entries():
    rng = np.random.default_rng(0)
    lengths = rng.integers(0, 257, size=9)
    mask = np.zeros((9, 256), dtype=bool)
    for r, t in enumerate(lengths):
        mask[r, :t] = True
    assert list(oracle.lengths_from_text_mask(mask)) == list(lengths)
    # a non-prefix mask counts its True entries wherever they sit
    m2 = np.zeros((2, 8), dtype=bool)
    m2[0, [1, 3, 7]] = True
    assert list(oracle.lengths_from_text_mask(m2)) == [3, 0]


def test_cu_seqlens_by_token_enumeration():
    lengths = [5, 0, 3, 0, 0, 7]
    cu = oracle.cu_seqlens_from_lengths(lengths)
    owner = []  # brute force: list each token's request, boundaries are first positions
    for r, n in enumerate(lengths):
        owner += [r] * n
    for r in range(len(lengths)):
        first = next((i for i, o in enumerate(owner) if o >= r), len(owner))
        assert cu[r] == first
    assert cu[-1] == len(owner)


def test_token_counts_printed_on_pages():
    g = json.load(open(os.path.join(GOLDEN, "token_counts.json")))
    for case in g["cases"]:
        assert oracle.image_tokens([case["grid"]])[0] == case["tokens"], case["what"]
    for case in g["sp_pad"]:
        assert oracle.sp_auto_pad(case["seq_len"], case["world_size"]) == (case["padded"], case["pad"])


def test_joint_cu_matches_concatenated_lengths():
    mask = np.zeros((3, 256), dtype=bool)
    mask[0, :10] = True
    mask[1, :1] = True
    mask[2, :256] = True
    hw = [(2, 3), (0, 0), (4, 4)]
    cu_joint, cu_text, cu_img, img_dst = oracle.joint_cu_seqlens(mask, hw)
    assert list(cu_joint) == [0, 16, 17, 17 + 256 + 16]
    assert list(cu_text) == [0, 10, 11, 267]
    assert list(cu_img) == [0, 6, 6, 22]
    assert list(img_dst) == [10, 17, 17 + 256]


def test_pack_unpack_roundtrip_and_row_origin():
    rng = np.random.default_rng(1)
    lengths = [3, 0, 5, 1]
    S = 6
    src = rng.standard_normal((4, S, 2, 3))
    cu = oracle.cu_seqlens_from_lengths(lengths)
    flat = oracle.pack_by_cu_seqlens(src, cu)
    assert flat.shape == (9, 2, 3)
    # every packed row comes from the request whose [cu[r], cu[r+1]) holds it
    for i in range(flat.shape[0]):
        r = int(np.searchsorted(cu, i, side="right") - 1)
        assert np.array_equal(flat[i], src[r, i - cu[r]])
    back = oracle.unpack_by_cu_seqlens(flat, cu, S, zero_fill=True)
    for r, n in enumerate(lengths):
        assert np.array_equal(back[r, :n], src[r, :n])
        assert not back[r, n:].any()
    keep = np.full_like(src, 7.0)
    back2 = oracle.unpack_by_cu_seqlens(flat, cu, S, zero_fill=False, dst=keep.copy())
    for r, n in enumerate(lengths):
        assert np.all(back2[r, n:] == 7.0)


def test_joint_pack_with_offsets_equals_packing_concatenation():
    rng = np.random.default_rng(2)
    tl = [4, 0, 2]
    nl = [3, 5, 0]
    text = rng.standard_normal((3, 4, 5))
    img = rng.standard_normal((3, 5, 5))
    mask = np.zeros((3, 4), dtype=bool)
    for r, t in enumerate(tl):
        mask[r, :t] = True
    cu_joint, cu_text, cu_img, img_dst = oracle.joint_cu_seqlens(mask, [(1, n) for n in nl])
    out = np.zeros((int(cu_joint[-1]), 5))
    oracle.pack_by_cu_seqlens(text, cu_text, dst_row_offsets=cu_joint[:-1], dst=out)
    oracle.pack_by_cu_seqlens(img, cu_img, dst_row_offsets=img_dst, dst=out)
    # other construction: concatenate each request's pieces, then pack plainly
    joined = np.zeros((3, 9, 5))
    for r in range(3):
        joined[r, :tl[r] + nl[r]] = np.concatenate([text[r, :tl[r]], img[r, :nl[r]]])
    ref = oracle.pack_by_cu_seqlens(joined, cu_joint)
    assert np.array_equal(out, ref)


def test_tile_order_counts_uniqueness_and_order():
    q_cu = oracle.cu_seqlens_from_lengths([100, 0, 300, 129, 1])
    kv_cu = oracle.cu_seqlens_from_lengths([100, 7, 300, 129, 1])
    H, BM = 3, 64
    tiles = oracle.tile_order(q_cu, kv_cu, H, BM)
    assert len(tiles) == H * sum(math.ceil(n / BM) for n in [100, 0, 300, 129, 1])
    assert len(set(tiles)) == len(tiles)
    # longest key length first: request 2 (300), 3 (129), 0 (100), 4 (1); request 1 has no q rows
    reqs = [t[0] for t in tiles]
    firsts = [r for i, r in enumerate(reqs) if i == 0 or reqs[i - 1] != r]
    assert firsts == [2, 3, 0, 4]
    # index order beyond the longest-first limit
    tiles2 = oracle.tile_order(q_cu, kv_cu, H, BM, lpt_max_reqs=2)
    firsts2 = [r for i, r in enumerate([t[0] for t in tiles2]) if i == 0 or tiles2[i - 1][0] != r]
    assert firsts2 == [0, 2, 3, 4]
    # ties by index
    cu_eq = oracle.cu_seqlens_from_lengths([50, 50, 50])
    t3 = oracle.tile_order(cu_eq, cu_eq, 1, 64)
    assert [t[0] for t in t3] == [0, 1, 2]


def test_split_plan_worked_values():
    """Hand-computed plans: one joint 16,640-token request with 24 heads has
    130 * 24 = 3120 tiles; on 512 slots six rounds run whole and the 48 left
    are cut into min(16, 512 // 48, 16640 // 256) = 10 key ranges."""
    assert oracle.split_plan(3120, 512, 16640) == (3072, 48, 10)
    # a whole number of rounds: nothing to cut
    assert oracle.split_plan(3072, 512, 16640) == (3072, 0, 1)
    # the tail fills more than half of the slots: nothing to cut
    assert oracle.split_plan(512 + 300, 512, 16640) == (812, 0, 1)
    # one round only: every tile is cut, capped at MAX_SPLIT
    assert oracle.split_plan(20, 512, 1 << 20) == (0, 20, 16)
    # short keys cap the ranges: 700 keys -> 2 ranges; 511 keys -> none
    assert oracle.split_plan(20, 512, 700) == (0, 20, 2)
    assert oracle.split_plan(20, 512, 511) == (20, 0, 1)
    # no slots (split off) or no tiles
    assert oracle.split_plan(20, 0, 1 << 20) == (20, 0, 1)
    assert oracle.split_plan(0, 512, 1 << 20) == (0, 0, 1)


def test_split_ranges_tile_the_keys():
    for nkt in (0, 1, 2, 5, 16, 17, 260):
        for parts in (2, 3, 10, 16):
            spans = [oracle.split_range(nkt, p, parts) for p in range(parts)]
            assert spans[0][0] == 0 and spans[-1][1] == nkt
            assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
            assert all(lo <= hi for lo, hi in spans)
            sizes = [hi - lo for lo, hi in spans]
            assert max(sizes) - min(sizes) <= 1


def test_block_schedule_with_split_covers_every_tile_once():
    q_cu = oracle.cu_seqlens_from_lengths([17, 64, 129, 300, 2000])
    kv_cu = oracle.cu_seqlens_from_lengths([17, 640, 129, 3000, 2000])
    H, bm, chunk = 2, 128, 4
    tiles = oracle.tile_order(q_cu, kv_cu, H, bm)
    for slots in (8, 12, 40, 512):
        full, tail, parts = oracle.split_plan(len(tiles), slots, 3000)
        sched = oracle.block_schedule(q_cu, kv_cu, H, bm, 2000, chunk, slots=slots, max_kv=3000)
        G = oracle.grid_blocks(5, 2000, H, bm, chunk, slots=slots)
        assert sched.shape == (G, 5)
        used = [tuple(x) for x in sched if x[0] >= 0]
        assert len(used) == full + tail * parts <= len(tiles) + slots
        # every tile: whole exactly once, or each of its parts exactly once
        seen = {}
        for r, h, qt, p, n in used:
            seen.setdefault((r, h, qt), []).append((p, n))
        assert sorted(seen) == sorted(tiles)
        for t, ps in seen.items():
            n = ps[0][1]
            assert sorted(ps) == [(p, n) for p in range(n)]
        split_tiles = [t for t, ps in seen.items() if ps[0][1] > 1]
        assert len(split_tiles) == tail
        assert set(split_tiles) == set(tiles[full:])


def test_chiplet_queues_partition_the_items_in_block_order():
    """Every logical item sits in exactly one chiplet queue, and entry k of
    queue x is the item block_to_logical deals to the k-th block of chiplet x
    (block 8k + x); queue lengths differ by at most one chunk."""
    for n_items, chunk in [(0, 32), (1, 32), (255, 32), (256, 32), (1560, 32), (3048, 32), (12480, 32), (77, 5)]:
        qs = oracle.chiplet_queues(n_items, chunk)
        assert len(qs) == oracle.XCDS
        assert sorted(t for q in qs for t in q) == list(range(n_items))
        for x, q in enumerate(qs):
            assert q == [oracle.block_to_logical(8 * k + x, chunk) for k in range(len(q))]
        lens = [len(q) for q in qs]
        assert max(lens) - min(lens) <= chunk


def test_grid_spare_blocks_of_the_queue_launch():
    """The workspace launch adds an eighth of the item bound in spare blocks,
    still whole (chiplets x chunk) groups; the static launch does not."""
    for R, max_q, H, slots in [(1, 16640, 24, 256), (4, 16640, 24, 256), (4, 33024, 24, 256), (3, 210, 2, 0)]:
        upper = R * H * -(-max_q // 256) + slots
        g0 = oracle.grid_blocks(R, max_q, H, 256, 32, slots=slots)
        g1 = oracle.grid_blocks(R, max_q, H, 256, 32, slots=slots, queues=True)
        assert g0 >= upper and g1 >= upper + -(-upper // 8)
        assert g0 % 256 == 0 and g1 % 256 == 0 and g1 - 256 < upper + -(-upper // 8) <= g1


def test_block_schedule_is_a_bijection_onto_tiles():
    q_cu = oracle.cu_seqlens_from_lengths([17, 64, 129, 300])
    for chunk in (1, 4, 16):
        sched = oracle.block_schedule(q_cu, q_cu, 2, 32, 300, chunk)
        tiles = oracle.tile_order(q_cu, q_cu, 2, 32)
        G = oracle.grid_blocks(4, 300, 2, 32, chunk)
        assert sched.shape == (G, 5) and G % (8 * chunk) == 0
        assert (sched[sched[:, 0] >= 0][:, 3:] == (0, 1)).all()
        used = [tuple(x[:3]) for x in sched if x[0] >= 0]
        assert sorted(used) == sorted(tiles)
        assert len(used) == len(tiles)
        # the logical map itself is a permutation of [0, G)
        assert sorted(oracle.block_to_logical(b, chunk) for b in range(G)) == list(range(G))


def test_mixfusion_plan_printed_example():
    g = json.load(open(os.path.join(GOLDEN, "mixfusion_plan_caseB.json")))
    p = g["pixels_per_token_side"]
    counts = oracle.image_tokens([(h // p, w // p) for h, w in g["image_sizes"]])
    assert list(counts) == g["token_counts"]
    ok, size, count = oracle.mixfusion_chunk_plan(counts, g["min_chunk_tokens"], g["max_chunks"])
    e = g["expected"]
    assert (ok, size, count) == (e["accepted"], e["chunk_size"], e["chunk_count"])
    # rejections named by the knobs: gcd below the minimum, too many chunks
    assert oracle.mixfusion_chunk_plan([4096, 4096 + 128])[0] is False
    assert oracle.mixfusion_chunk_plan([256] * 129)[0] is False
    assert oracle.mixfusion_chunk_plan([256] * 128) == (True, 256, 128)


# ---------------------------------------------------------------- varlen attention


def _brute_varlen(q, k, v, q_cu, kv_cu, scale):
    return oracle.dense_masked_attention(q, k, v, oracle.block_diagonal_mask(q_cu, kv_cu), scale)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_varlen_matches_block_diagonal_brute_force_on_tiny_workload(dtype):
    inp = wl.make_varlen_inputs(wl.WORKLOADS["tiny-3req"], dtype)
    mask = inp.text_mask
    cu, cu_text, _, _ = oracle.joint_cu_seqlens(mask, inp.img_hw)
    q = oracle.pack_by_cu_seqlens(_np(inp.q_text), cu_text)
    k = oracle.pack_by_cu_seqlens(_np(inp.k_text), cu_text)
    v = oracle.pack_by_cu_seqlens(_np(inp.v_text), cu_text)
    assert list(cu) == [0, 17, 81, 210]
    o, lse = oracle.varlen_attention(q, k, v, cu, cu, inp.scale)
    ob, lseb = _brute_varlen(q, k, v, cu, cu, inp.scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("qlens,kvlens", [
    ([5, 0, 33, 1], [5, 0, 33, 1]),
    ([7, 3, 20], [1, 40, 9]),           # q != kv lengths
    ([4, 6], [0, 6]),                   # a request with queries but no keys
    ([0, 0, 3], [0, 2, 3]),
])
def test_varlen_matches_brute_force_edge_cases(qlens, kvlens):
    q, k, v = wl.random_varlen_case(11, qlens, 2, 16, torch.float32, kvlens)
    q_cu = oracle.cu_seqlens_from_lengths(qlens)
    kv_cu = oracle.cu_seqlens_from_lengths(kvlens)
    o, lse = oracle.varlen_attention(_np(q), _np(k), _np(v), q_cu, kv_cu, 0.25)
    ob, lseb = _brute_varlen(_np(q), _np(k), _np(v), q_cu, kv_cu, 0.25)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lseb))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=0, atol=1e-12)
    # no keys: output exactly zero and lse = -inf
    for r, (a, b) in enumerate(zip(qlens, kvlens)):
        if a and not b:
            assert not o[q_cu[r]:q_cu[r + 1]].any()
            assert np.all(np.isneginf(lse[q_cu[r]:q_cu[r + 1]]))


def test_varlen_closed_forms():
    rng = np.random.default_rng(3)
    D = 8
    scale = 0.5
    # one key: out = v, lse = scale * q.k
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    v = rng.standard_normal((1, 1, D))
    o, lse = oracle.varlen_attention(q, k, v, [0, 1], [0, 1], scale)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], scale * float(q[0, 0] @ k[0, 0]), atol=1e-14)
    # zero queries: uniform weights -> mean of V, lse = ln(L)
    L = 13
    q0 = np.zeros((L, 1, D))
    k0 = rng.standard_normal((L, 1, D))
    v0 = rng.standard_normal((L, 1, D))
    o, lse = oracle.varlen_attention(q0, k0, v0, [0, L], [0, L], scale)
    np.testing.assert_allclose(o, np.broadcast_to(v0.mean(axis=0), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(L), atol=1e-14)
    # constant V -> constant output
    vc = np.full((L, 1, D), -1.75)
    o, _ = oracle.varlen_attention(rng.standard_normal((L, 1, D)), k0, vc, [0, L], [0, L], scale)
    np.testing.assert_allclose(o, -1.75, atol=1e-14)
    # two keys with score gap ln 3: weights 3/4 and 1/4, lse = ln 4
    qa = np.zeros((1, 1, D))
    qa[0, 0, 0] = math.log(3.0) / scale
    kb = np.zeros((2, 1, D))
    kb[0, 0, 0] = 1.0
    vb = rng.standard_normal((2, 1, D))
    o, lse = oracle.varlen_attention(qa, kb, vb, [0, 1], [0, 2], scale)
    np.testing.assert_allclose(o[0, 0], 0.75 * vb[0, 0] + 0.25 * vb[1, 0], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(4.0), atol=1e-14)


def test_varlen_invariants_alone_permutation_duplicates_normalisation():
    lens = [9, 30, 4]
    q, k, v = (_np(t).astype(np.float64) for t in wl.random_varlen_case(5, lens, 3, 16, torch.float32))
    cu = oracle.cu_seqlens_from_lengths(lens)
    o, lse = oracle.varlen_attention(q, k, v, cu, cu, 0.3)
    # a request alone equals the same request inside the packed batch
    for r in range(3):
        sl = slice(cu[r], cu[r + 1])
        oa, la = oracle.varlen_attention(q[sl], k[sl], v[sl], [0, lens[r]], [0, lens[r]], 0.3)
        assert np.array_equal(oa, o[sl]) and np.array_equal(la, lse[sl])
    # permuting request order permutes outputs
    perm = [2, 0, 1]
    qp = np.concatenate([q[cu[r]:cu[r + 1]] for r in perm])
    kp = np.concatenate([k[cu[r]:cu[r + 1]] for r in perm])
    vp = np.concatenate([v[cu[r]:cu[r + 1]] for r in perm])
    cup = oracle.cu_seqlens_from_lengths([lens[r] for r in perm])
    op, _ = oracle.varlen_attention(qp, kp, vp, cup, cup, 0.3)
    for i, r in enumerate(perm):
        assert np.array_equal(op[cup[i]:cup[i + 1]], o[cu[r]:cu[r + 1]])
    # two identical requests give identical outputs
    q2 = np.concatenate([q[:9], q[:9]])
    k2 = np.concatenate([k[:9], k[:9]])
    v2 = np.concatenate([v[:9], v[:9]])
    o2, _ = oracle.varlen_attention(q2, k2, v2, [0, 9, 18], [0, 9, 18], 0.3)
    assert np.array_equal(o2[:9], o2[9:])
    # softmax rows sum to one: sum_j exp(scale q.k_j - lse) = 1, by explicit loops
    for i in (0, 10, 38):
        r = int(np.searchsorted(cu, i, side="right") - 1)
        for h in range(3):
            tot = sum(math.exp(0.3 * float(q[i, h] @ k[j, h]) - lse[i, h]) for j in range(cu[r], cu[r + 1]))
            assert abs(tot - 1.0) < 1e-12


def test_varlen_row_subset_equals_full():
    lens = [40, 70]
    q, k, v = (_np(t) for t in wl.random_varlen_case(8, lens, 2, 8, torch.float32))
    cu = oracle.cu_seqlens_from_lengths(lens)
    o, lse = oracle.varlen_attention(q, k, v, cu, cu, 0.4)
    rows = [109, 0, 39, 40, 55]
    os_, ls = oracle.varlen_attention(q, k, v, cu, cu, 0.4, rows=rows, row_chunk=2)
    # rows are independent; only BLAS blocking of the dot products may differ
    np.testing.assert_allclose(os_, o[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ls, lse[rows], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- block-local


@pytest.mark.parametrize("n", [10, 96, 101])
@pytest.mark.parametrize("win", [(0, 0), (1, 0), (0, 1), (1, 1), (2, 1)])
def test_block_local_matches_block_difference_mask(n, win):
    lb, la = win
    rng = np.random.default_rng(n * 10 + lb * 3 + la)
    q, k, v = (rng.standard_normal((1, n, 2, 8)) for _ in range(3))
    o, lse = oracle.block_local_attention(q, k, v, 24, lb, la, 0.35)
    mask = oracle.block_difference_mask(n, 24, lb, la)
    ob, lseb = oracle.dense_masked_attention(q[0], k[0], v[0], mask, 0.35)
    np.testing.assert_allclose(o[0], ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], lseb, rtol=0, atol=1e-12)


def test_block_local_special_cases():
    rng = np.random.default_rng(9)
    # own-block only with n a multiple of the block = varlen with 24-token requests
    n = 96
    q, k, v = (rng.standard_normal((1, n, 2, 8)) for _ in range(3))
    o, lse = oracle.block_local_attention(q, k, v, 24, 0, 0, 0.35)
    cu = list(range(0, n + 1, 24))
    ov, lv = oracle.varlen_attention(q[0], k[0], v[0], cu, cu, 0.35)
    np.testing.assert_allclose(o[0], ov, atol=1e-13)
    np.testing.assert_allclose(lse[0], lv, atol=1e-13)
    # windows at least as wide as the sequence = full dense attention
    n = 50
    q, k, v = (rng.standard_normal((2, n, 2, 8)) for _ in range(3))
    o, _ = oracle.block_local_attention(q, k, v, 24, 3, 3, 0.35)
    for b in range(2):
        od, _ = oracle.dense_masked_attention(q[b], k[b], v[b], np.ones((n, n), bool), 0.35)
        np.testing.assert_allclose(o[b], od, atol=1e-13)
    # a sequence shorter than one block = plain dense attention whatever the window
    n = 10
    q, k, v = (rng.standard_normal((1, n, 1, 8)) for _ in range(3))
    for lb, la in [(0, 0), (1, 1)]:
        o, _ = oracle.block_local_attention(q, k, v, 24, lb, la, 0.35)
        od, _ = oracle.dense_masked_attention(q[0], k[0], v[0], np.ones((n, n), bool), 0.35)
        np.testing.assert_allclose(o[0], od, atol=1e-13)


def test_block_local_key_ranges_by_enumeration():
    n, blk = 101, 24
    for lb, la in [(0, 0), (1, 0), (0, 1), (1, 1), (2, 3)]:
        mask = oracle.block_difference_mask(n, blk, lb, la)
        for i in range(n):
            lo, hi = oracle.block_local_key_range(i, n, blk, lb, la)
            allowed = [j for j in range(n) if mask[i, j]]
            assert allowed == list(range(lo, hi))


def test_block_local_vocoder_sampled_rows_against_mask():
    inp = wl.make_block_local_inputs(wl.BLOCK_LOCAL_WORKLOADS["vocoder-dit"], torch.bfloat16)
    q, k, v = (_np(t)[0].astype(np.float64) for t in (inp.q, inp.k, inp.v))
    n = q.shape[0]
    for lb, la in wl.BLOCK_LOCAL_WORKLOADS["vocoder-dit"].windows:
        o, _ = oracle.block_local_attention(_np(inp.q), _np(inp.k), _np(inp.v), 24, lb, la, inp.scale)
        for i in (0, 23, 24, 1000, 1991, 1992, 2002):
            keys = [j for j in range(n) if -lb <= j // 24 - i // 24 <= la]
            s = inp.scale * np.einsum("jhd,hd->hj", k[keys], q[i])   # [H, keys]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            ref = np.einsum("hj,jhd->hd", p / p.sum(axis=1, keepdims=True), v[keys])
            np.testing.assert_allclose(o[0, i], ref, atol=1e-12)


# ---------------------------------------------------------------- CFG combine


def test_cfg_combine_endpoints_and_linearity():
    rng = np.random.default_rng(4)
    p, n = rng.standard_normal(6), rng.standard_normal(6)
    assert np.array_equal(oracle.cfg_combine(p, n, 0.0), n)
    np.testing.assert_allclose(oracle.cfg_combine(p, n, 1.0), p, atol=1e-15)
    np.testing.assert_allclose(oracle.cfg_combine(p, n, 4.0) - oracle.cfg_combine(p, n, 3.0), p - n, atol=1e-14)
    # by hand, with scale 2.5: 1 + 2.5*(2 - 1) = 3.5 and 3 + 2.5*(-1 - 3) = -7
    assert np.array_equal(oracle.cfg_combine(np.array([2.0, -1.0]), np.array([1.0, 3.0]), 2.5), [3.5, -7.0])


# ---------------------------------------------------------------- planted mistakes


def _planted(monkeypatch, fn):
    monkeypatch.setattr(vo, "_softmax_attend", fn)


@pytest.mark.parametrize("mistake", ["no_scale", "exp2", "drop_last_key", "transpose_v"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    good = vo._softmax_attend

    def bad(q, k, v, scale):
        if mistake == "no_scale":
            return good(q, k, v, 1.0)
        if mistake == "drop_last_key":
            return good(q, k[:-1], v[:-1], scale) if k.shape[0] > 1 else good(q, k, v, scale)
        if mistake == "transpose_v":
            o, l = good(q, k, v, scale)
            return o[:, ::-1], l
        # exp2 in place of exp
        s = scale * (q @ k.T)
        p = np.exp2(s - s.max(axis=1, keepdims=True))
        return (p @ v) / p.sum(axis=1, keepdims=True), s.max(axis=1) + np.log2(p.sum(axis=1))

    lens = [9, 30]
    q, k, v = (_np(t) for t in wl.random_varlen_case(6, lens, 2, 8, torch.float32))
    cu = oracle.cu_seqlens_from_lengths(lens)
    ob, lb = _brute_varlen(q, k, v, cu, cu, 0.3)
    _planted(monkeypatch, bad)
    o, l = oracle.varlen_attention(q, k, v, cu, cu, 0.3)
    assert not (np.allclose(o, ob, atol=1e-6) and np.allclose(l, lb, atol=1e-6))


def test_planted_window_off_by_one_is_caught(monkeypatch):
    real = vo.block_local_key_range

    def bad(i, n, block, lb, la):
        lo, hi = real(i, n, block, lb, la)
        return lo, min(n, hi + block)  # one block too many after the window

    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 101, 1, 8)) for _ in range(3))
    ob, _ = oracle.dense_masked_attention(q[0], k[0], v[0], oracle.block_difference_mask(101, 24, 1, 0), 0.35)
    monkeypatch.setattr(vo, "block_local_key_range", bad)
    o, _ = vo.block_local_attention(q, k, v, 24, 1, 0, 0.35)
    assert not np.allclose(o[0], ob, atol=1e-6)
