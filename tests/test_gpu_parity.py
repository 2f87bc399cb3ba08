"""GPU path vs the CPU oracle, through the C ABI (via the Python binding).

Integer work (boundaries, pack/unpack, the tile schedule) must be bit-exact.
Attention must be within the stated tolerances of the fp64 oracle: bf16
max-abs 2e-2 and mean-abs 2e-3, fp32 max-abs 1e-5.  Output buffers are
surrounded by canary rows that must survive every call.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import packed_variable_length_varlen_amd as vl
from packed_variable_length_varlen_amd import workloads as wl
from tests.helpers import check_close, check_lse, sample_rows, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def canary_out(shape, dtype, pad=3):
    """An output view with `pad` NaN-filled canary rows on either side."""
    full = torch.full((shape[0] + 2 * pad,) + tuple(shape[1:]), float("nan"), dtype=dtype, device=DEV)
    return full, full[pad:pad + shape[0]]


def assert_canary(full, pad=3):
    head = full[:pad].float()
    tail = full[full.shape[0] - pad:].float()
    assert torch.isnan(head).all() and torch.isnan(tail).all(), "a kernel wrote outside its output"


# ------------------------------------------------------------------ boundaries


@pytest.mark.parametrize("cfg", ["tiny-3req", "joint-16k", "mixres-4req", "edit-cfg-4seq"])
def test_joint_cu_seqlens_bitexact(cfg):
    log(f"[joint_cu] {cfg}")
    spec = wl.WORKLOADS[cfg]
    rng = np.random.default_rng(spec.seed)
    R = len(spec.img_grids)
    mask = np.zeros((R, wl.TEXT_CAP), dtype=bool)
    for r, (lo, hi) in enumerate(spec.text_ranges):
        mask[r, :int(rng.integers(lo, hi + 1))] = True
    hw = np.array(spec.img_grids, dtype=np.int32).reshape(R, 2)
    outs = vl.joint_cu_seqlens(torch.from_numpy(mask.astype(np.uint8)).to(DEV), torch.from_numpy(hw).to(DEV))
    ref = oracle.joint_cu_seqlens(mask, hw)
    for got, exp in zip(outs, ref):
        assert np.array_equal(got.cpu().numpy(), exp.astype(np.int32))


@pytest.mark.parametrize("R", [0, 1, 5, 255, 256, 257, 1000, 3000])
def test_cu_seqlens_and_joint_random_bitexact(R):
    log(f"[cu] R={R}")
    rng = np.random.default_rng(R)
    lengths = rng.integers(0, 5000, size=R).astype(np.int32)
    cu = vl.cu_seqlens_from_lengths(torch.from_numpy(lengths).to(DEV))
    assert np.array_equal(cu.cpu().numpy(), oracle.cu_seqlens_from_lengths(lengths).astype(np.int32))
    # scattered (non-prefix) masks and empty grids
    mask = rng.random((R, 77)) < 0.3
    hw = rng.integers(0, 40, size=(R, 2)).astype(np.int32)
    outs = vl.joint_cu_seqlens(torch.from_numpy(mask.astype(np.uint8)).to(DEV), torch.from_numpy(hw).to(DEV))
    for got, exp in zip(outs, oracle.joint_cu_seqlens(mask, hw)):
        assert np.array_equal(got.cpu().numpy(), exp.astype(np.int32))


# ------------------------------------------------------------------ pack / unpack


@pytest.mark.parametrize("row_shape,dtype", [((24, 128), torch.bfloat16), ((3,), torch.float32),
                                             ((3,), torch.bfloat16), ((5,), torch.uint8),
                                             ((2, 64), torch.float32)])
def test_pack_unpack_bitexact_vector_widths(row_shape, dtype):
    log(f"[pack] row {row_shape} {dtype}")
    lengths = [0, 17, 1, 300, 0, 129, 64]
    S = 320
    rng = np.random.default_rng(7)
    src = torch.from_numpy(rng.standard_normal((len(lengths), S) + row_shape).astype(np.float32)).to(dtype)
    cu = oracle.cu_seqlens_from_lengths(lengths)
    T = int(cu[-1])
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    full, dst = canary_out((T,) + row_shape, dtype) if dtype != torch.uint8 else (None, torch.empty((T,) + row_shape, dtype=dtype, device=DEV))
    vl.pack_by_cu_seqlens(src.to(DEV), cu_d, dst)
    ref = oracle.pack_by_cu_seqlens(src.numpy() if dtype != torch.bfloat16 else src.view(torch.int16).numpy(), cu)
    got = dst.cpu().numpy() if dtype != torch.bfloat16 else dst.cpu().view(torch.int16).numpy()
    assert np.array_equal(got, ref)
    if full is not None:
        assert_canary(full)
    # unpack back, with and without zero fill
    for zero_fill in (True, False):
        back = torch.full((len(lengths), S) + row_shape, 7, dtype=dtype, device=DEV)
        vl.unpack_by_cu_seqlens(dst, cu_d, back, zero_fill=zero_fill)
        init = np.full((len(lengths), S) + row_shape, 7, dtype=ref.dtype)
        if dtype == torch.bfloat16:
            init = torch.full((1,), 7, dtype=dtype).view(torch.int16).numpy()[0] * np.ones_like(init)
        exp = oracle.unpack_by_cu_seqlens(ref, cu, S, zero_fill=zero_fill, dst=init)
        gotb = back.cpu().numpy() if dtype != torch.bfloat16 else back.cpu().view(torch.int16).numpy()
        assert np.array_equal(gotb, exp)


def test_joint_pack_with_offsets_bitexact():
    log("[pack] joint text+image with offsets")
    inp = wl.make_varlen_inputs(wl.WORKLOADS["mixres-4req"], torch.bfloat16)
    mask_d = torch.from_numpy(inp.text_mask.astype(np.uint8)).to(DEV)
    hw_d = torch.tensor(inp.img_hw, dtype=torch.int32, device=DEV)
    cu_j, cu_t, cu_i, img_dst = vl.joint_cu_seqlens(mask_d, hw_d)
    T = inp.total_tokens
    H, D = inp.spec.H, inp.spec.D
    full, q = canary_out((T, H, D), torch.bfloat16)
    vl.pack_by_cu_seqlens(inp.q_text.to(DEV), cu_t, q, dst_row_offsets=cu_j[:-1])
    vl.pack_by_cu_seqlens(inp.q_img.to(DEV), cu_i, q, dst_row_offsets=img_dst)
    assert_canary(full)
    cj, ct, ci, idst = oracle.joint_cu_seqlens(inp.text_mask, inp.img_hw)
    ref = np.zeros((T, H, D), dtype=np.int16)
    oracle.pack_by_cu_seqlens(inp.q_text.view(torch.int16).numpy(), ct, dst_row_offsets=cj[:-1], dst=ref)
    oracle.pack_by_cu_seqlens(inp.q_img.view(torch.int16).numpy(), ci, dst_row_offsets=idst, dst=ref)
    assert np.array_equal(q.cpu().view(torch.int16).numpy(), ref)


@pytest.mark.parametrize("cfg", ["joint-16k", "mixres-4req"])
def test_joint_pack_unpack_batched_bitexact(cfg):
    """The six joint pack copies of Q, K, V (text and image pieces) in one
    launch, and the two unpacks of the output in another, against the oracle."""
    log(f"[pack] batched joint {cfg}")
    inp = wl.make_varlen_inputs(wl.WORKLOADS[cfg], torch.bfloat16)
    mask_d = torch.from_numpy(inp.text_mask.astype(np.uint8)).to(DEV)
    hw_d = torch.tensor(inp.img_hw, dtype=torch.int32, device=DEV).reshape(-1, 2)
    cu_j, cu_t, cu_i, img_dst = vl.joint_cu_seqlens(mask_d, hw_d)
    T = inp.total_tokens
    H, D = inp.spec.H, inp.spec.D
    cj, ct, ci, idst = oracle.joint_cu_seqlens(inp.text_mask, inp.img_hw)
    outs, items, refs = [], [], []
    for txt, img in ((inp.q_text, inp.q_img), (inp.k_text, inp.k_img), (inp.v_text, inp.v_img)):
        full, dst = canary_out((T, H, D), torch.bfloat16)
        outs.append(full)
        items += [(txt.to(DEV), cu_t, dst, cu_j[:-1]), (img.to(DEV), cu_i, dst, img_dst)]
        ref = np.zeros((T, H, D), dtype=np.int16)
        oracle.pack_by_cu_seqlens(txt.view(torch.int16).numpy(), ct, dst_row_offsets=cj[:-1], dst=ref)
        oracle.pack_by_cu_seqlens(img.view(torch.int16).numpy(), ci, dst_row_offsets=idst, dst=ref)
        refs.append(ref)
    vl.pack_by_cu_seqlens_batched(items)
    torch.cuda.synchronize()
    for full, ref in zip(outs, refs):
        assert_canary(full)
        assert np.array_equal(full[3:3 + T].cpu().view(torch.int16).numpy(), ref)
    flat = outs[0][3:3 + T]
    for zero_fill in (True, False):
        o_txt = torch.full_like(inp.q_text, 3.0, device=DEV)
        o_img = torch.full_like(inp.q_img, 3.0, device=DEV)
        vl.unpack_by_cu_seqlens_batched([(flat, cu_t, o_txt, cu_j[:-1]), (flat, cu_i, o_img, img_dst)],
                                        zero_fill=zero_fill)
        torch.cuda.synchronize()
        three = torch.full((1,), 3.0, dtype=torch.bfloat16).view(torch.int16).numpy()[0]
        for got, cu_ref, offs, slab in ((o_txt, ct, cj[:-1], inp.q_text), (o_img, ci, idst, inp.q_img)):
            init = np.full(tuple(slab.shape), three, dtype=np.int16)
            exp = oracle.unpack_by_cu_seqlens(refs[0], cu_ref, slab.shape[1], src_row_offsets=offs,
                                              zero_fill=zero_fill, dst=init)
            assert np.array_equal(got.cpu().view(torch.int16).numpy(), exp)


def test_pack_batched_mixed_widths_and_empty():
    """Copies whose rows are not whole 16-byte vectors take one launch each;
    empty copies and requests are no-ops; the result equals single calls."""
    log("[pack] batched mixed widths")
    rng = np.random.default_rng(11)
    specs = [([0, 17, 1, 300], (3,), torch.bfloat16), ([5, 0, 9], (8,), torch.bfloat16),
             ([], (8,), torch.bfloat16), ([2, 2], (5,), torch.float32)]
    items, singles, refs = [], [], []
    for lengths, row, dtype in specs:
        S = max(lengths + [1]) + 3
        src = torch.from_numpy(rng.standard_normal((len(lengths), S) + row).astype(np.float32)).to(dtype).to(DEV)
        cu = oracle.cu_seqlens_from_lengths(lengths)
        cu_d = torch.from_numpy(cu.astype(np.int32)).to(DEV)
        T = int(cu[-1])
        a = torch.zeros((T,) + row, dtype=dtype, device=DEV)
        b = torch.zeros_like(a)
        items.append((src, cu_d, a, None))
        vl.pack_by_cu_seqlens(src, cu_d, b)
        singles.append((a, b))
    vl.pack_by_cu_seqlens_batched(items)
    torch.cuda.synchronize()
    for a, b in singles:
        assert torch.equal(a, b)
    with pytest.raises(vl.VarlenError):
        vl.pack_by_cu_seqlens_batched(items * 3)


def test_batched_copies_many_pairs():
    """More (copy, request) pairs than the compact path takes (3 x 1000
    requests), including empty requests, pack and unpack with zero fill."""
    log("[pack] batched, 3000 pairs")
    rng = np.random.default_rng(12)
    items, ref_dsts = [], []
    for c in range(3):
        lengths = [int(x) for x in rng.integers(0, 6, size=1000)]
        S = 6
        src = torch.from_numpy(rng.standard_normal((1000, S, 8)).astype(np.float32)).to(torch.bfloat16).to(DEV)
        cu = oracle.cu_seqlens_from_lengths(lengths)
        cu_d = torch.from_numpy(cu.astype(np.int32)).to(DEV)
        dst = torch.zeros((int(cu[-1]), 8), dtype=torch.bfloat16, device=DEV)
        items.append((src, cu_d, dst, None))
        ref = oracle.pack_by_cu_seqlens(src.cpu().view(torch.int16).numpy(), cu)
        ref_dsts.append((dst, ref, cu, src))
    vl.pack_by_cu_seqlens_batched(items)
    torch.cuda.synchronize()
    for dst, ref, cu, src in ref_dsts:
        assert np.array_equal(dst.cpu().view(torch.int16).numpy(), ref)
    backs = []
    for dst, ref, cu, src in ref_dsts:
        backs.append(torch.full_like(src, 9.0))
    vl.unpack_by_cu_seqlens_batched([(d, it[1], b, None) for (d, _, _, _), it, b in zip(ref_dsts, items, backs)])
    torch.cuda.synchronize()
    for (dst, ref, cu, src), b in zip(ref_dsts, backs):
        exp = oracle.unpack_by_cu_seqlens(ref, cu, src.shape[1], zero_fill=True)
        assert np.array_equal(b.cpu().view(torch.int16).numpy(), exp)


# ------------------------------------------------------------------ tile schedule


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("case", ["lpt", "ties", "index_order", "empty", "qkv_differ"])
def test_tile_map_bitexact(case, split):
    log(f"[tile_map] {case} split={split}")
    rng = np.random.default_rng(3)
    if case == "lpt":
        ql = [17, 64, 129, 4096, 300, 1]
        kl = ql
    elif case == "ties":
        ql = [128] * 5 + [256, 256]
        kl = ql
    elif case == "index_order":
        ql = list(rng.integers(0, 700, size=150))
        kl = ql
    elif case == "empty":
        ql = [0, 0, 5, 0]
        kl = [0, 3, 5, 0]
    else:
        ql = [100, 1, 200, 33]
        kl = [5, 400, 1, 33]
    H, D = 3, 128
    q_cu = oracle.cu_seqlens_from_lengths(ql)
    kv_cu = oracle.cu_seqlens_from_lengths(kl)
    max_q = max(max(ql), 1)
    max_kv = int(max(kl))
    bm, chunk, G, slots = vl.varlen_launch_shape(max_q, len(ql), H, D, max_kv=max_kv, split=split)
    if split and max_kv // oracle.MIN_SPLIT_KEYS >= 2:
        assert slots >= 256, "a split launch sizes itself by the device's resident work-groups"
    else:
        assert slots == 0, "no split without the flag or with keys too short to cut"
    got = vl.varlen_tile_map(torch.from_numpy(q_cu.astype(np.int32)).to(DEV),
                             torch.from_numpy(kv_cu.astype(np.int32)).to(DEV), max_q, H, D,
                             max_kv=max_kv, split=split).cpu().numpy()
    ref = oracle.block_schedule(q_cu, kv_cu, H, bm, max_q, chunk, slots=slots, max_kv=max_kv, queues=split)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref.astype(np.int32))
    if split and case == "lpt":
        assert (got[:, 4] > 1).any(), "this case has a tail to split"


# ------------------------------------------------------------------ varlen attention


def _run_varlen(q, k, v, q_cu, kv_cu, scale, f32, max_q=None, max_kv=None, split=False):
    ql = np.diff(q_cu)
    kl = np.diff(kv_cu)
    max_q = int(ql.max()) if max_q is None and ql.size else (max_q or 0)
    max_kv = int(kl.max()) if max_kv is None and kl.size else (max_kv or 0)
    dtype = torch.float32 if f32 else torch.bfloat16
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    full, out = canary_out(tuple(q.shape), dtype)
    lse_full, lse = canary_out((q.shape[0], q.shape[1]), torch.float32)
    fn = vl.varlen_attn_fwd_f32 if f32 else (vl.varlen_attn_fwd_split if split else vl.varlen_attn_fwd)
    fn(qd, kd, vd, torch.from_numpy(np.asarray(q_cu, dtype=np.int32)).to(DEV),
       torch.from_numpy(np.asarray(kv_cu, dtype=np.int32)).to(DEV), max_q, max_kv, scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert_canary(full)
    assert_canary(lse_full)
    return out, lse


@pytest.mark.parametrize("f32", [False, True])
def test_varlen_tiny_workload_full(f32):
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[varlen] tiny-3req {dtype}")
    inp = wl.make_varlen_inputs(wl.WORKLOADS["tiny-3req"], dtype)
    cu, cu_t, _, _ = oracle.joint_cu_seqlens(inp.text_mask, inp.img_hw)
    q = torch.from_numpy(oracle.pack_by_cu_seqlens(inp.q_text.float().numpy(), cu_t)).to(dtype)
    k = torch.from_numpy(oracle.pack_by_cu_seqlens(inp.k_text.float().numpy(), cu_t)).to(dtype)
    v = torch.from_numpy(oracle.pack_by_cu_seqlens(inp.v_text.float().numpy(), cu_t)).to(dtype)
    out, lse = _run_varlen(q, k, v, cu, cu, inp.scale, f32)
    ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v), cu, cu, inp.scale)
    mx, mean = check_close(to64(out), ro, f32, "tiny-3req")
    check_lse(to64(lse), rl, f32, "tiny-3req")
    log(f"   max-abs {mx:.3g} mean-abs {mean:.3g}")


EDGE_CASES = [
    ("ragged", [1, 31, 32, 33, 127, 128, 129, 200], None, 2),
    ("empty_and_zero_kv", [0, 5, 40, 0, 3], [0, 0, 40, 7, 3], 3),
    ("q_ne_kv", [7, 140, 20], [300, 9, 129], 2),
    ("single_key", [65], [1], 1),
    ("many_requests_index_order", [int(x) for x in np.random.default_rng(5).integers(0, 90, size=100)], None, 1),
]


@pytest.mark.parametrize("name,ql,kl,H", EDGE_CASES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("f32", [False, True])
def test_varlen_edge_cases(name, ql, kl, H, D, f32):
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[varlen] {name} D={D} {dtype}")
    kl = ql if kl is None else kl
    q, k, v = wl.random_varlen_case(17, ql, H, D, dtype, kl)
    q_cu = oracle.cu_seqlens_from_lengths(ql)
    kv_cu = oracle.cu_seqlens_from_lengths(kl)
    scale = wl.softmax_scale(D)
    out, lse = _run_varlen(q, k, v, q_cu, kv_cu, scale, f32)
    ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v), q_cu, kv_cu, scale)
    check_close(to64(out), ro, f32, name)
    check_lse(to64(lse), rl, f32, name)


def test_varlen_loose_max_bounds_and_large_values():
    """max_q/max_kv only size the launch: larger bounds give the same bits;
    scaled inputs (|s| up to ~60) stay finite and within tolerance."""
    log("[varlen] loose bounds / large scores")
    ql = [100, 300, 7]
    q, k, v = wl.random_varlen_case(23, ql, 2, 128, torch.bfloat16)
    cu = oracle.cu_seqlens_from_lengths(ql)
    o1, l1 = _run_varlen(q, k, v, cu, cu, 0.088388, False)
    o2, l2 = _run_varlen(q, k, v, cu, cu, 0.088388, False, max_q=1000, max_kv=5000)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    q4 = (q.float() * 4).to(torch.bfloat16)
    o3, l3 = _run_varlen(q4, k, v, cu, cu, 0.088388, False)
    ro, rl = oracle.varlen_attention(to64(q4), to64(k), to64(v), cu, cu, 0.088388)
    check_close(to64(o3), ro, False, "scaled q")


@pytest.mark.parametrize("f32", [False, True])
def test_varlen_growing_scores_rescale(f32):
    """Key norms ramp from 1x to 60x along each request, so the row maxima
    climb by far more than 2^8 (in exp2 units, up to ~400) many times over
    the key tiles: every lazy rescale (and, on the bf16 path, the fold of the
    matrix-core row sums into the running sum at a rescale) is exercised,
    and the weights of a fixed offset would overflow.  Unsplit and split
    launches against the oracle."""
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[varlen] growing scores {dtype}")
    ql = [700, 1500, 129]
    H, D = 2, 128
    q, k, v = wl.random_varlen_case(43, ql, H, D, torch.float32)
    cu = oracle.cu_seqlens_from_lengths(ql)
    ramp = torch.cat([torch.linspace(1.0, 60.0, n) for n in ql]).reshape(-1, 1, 1)
    q, k, v = q.to(dtype), (k * ramp).to(dtype), v.to(dtype)
    scale = wl.softmax_scale(D)
    ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v), cu, cu, scale)
    assert rl.max() > 200.0, "the case must drive the scores far past one rescale step"
    for split in ([False] if f32 else [False, True]):
        out, lse = _run_varlen(q, k, v, cu, cu, scale, f32, split=split)
        assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
        if f32:
            # the fp32 bound (1e-5) holds for unit-scale inputs; the fp32
            # rounding of a dot product grows with its magnitude, here up to
            # 60x (lse ~ 280 alone has an fp32 ulp of 3e-5), so the bound
            # scales by the ramp's top factor
            tol = 60 * 1e-5
            eo = np.abs(to64(out) - ro).max()
            el = np.abs(to64(lse) - rl).max()
            log(f"   fp32 out max-abs {eo:.3g}, lse max-abs {el:.3g} (bound {tol:.3g})")
            assert eo <= tol and el <= tol
        else:
            check_close(to64(out), ro, f32, f"growing scores split={split}")
            check_lse(to64(lse), rl, f32, f"growing scores split={split}")


def test_varlen_check_cu_seqlens_option():
    """check_cu_seqlens=True validates on the host before the launch: a valid
    array gives the same bits as the unchecked call, malformed ones raise and
    never reach the kernels."""
    log("[varlen] check_cu_seqlens")
    ql = [17, 64, 129]
    q, k, v = (t.to(DEV) for t in wl.random_varlen_case(47, ql, 2, 64, torch.bfloat16))
    cu = torch.tensor([0, 17, 81, 210], dtype=torch.int32, device=DEV)
    for fn in (vl.varlen_attn_fwd, vl.varlen_attn_fwd_split):
        o1 = fn(q, k, v, cu, cu, 129, 129)
        o2 = fn(q, k, v, cu, cu, 129, 129, check_cu_seqlens=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        for bad in ([0, 17, 16, 210], [0, 17, 81, 211], [1, 17, 81, 210]):
            bcu = torch.tensor(bad, dtype=torch.int32, device=DEV)
            with pytest.raises(vl.VarlenError):
                fn(q, k, v, bcu, bcu, 129, 129, check_cu_seqlens=True)
        with pytest.raises(vl.VarlenError):  # a length past the launch bound
            fn(q, k, v, cu, cu, 100, 100, check_cu_seqlens=True)


def test_varlen_invariants_bitwise():
    """Alone == inside the packed batch, permutation permutes outputs, two
    identical requests give identical outputs, and two runs give the same
    bits (the tiles never mix requests)."""
    log("[varlen] invariants")
    ql = [300, 77, 1000, 129]
    H, D = 3, 128
    q, k, v = wl.random_varlen_case(31, ql, H, D, torch.bfloat16)
    cu = oracle.cu_seqlens_from_lengths(ql)
    out, lse = _run_varlen(q, k, v, cu, cu, 0.1, False)
    out2, lse2 = _run_varlen(q, k, v, cu, cu, 0.1, False)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for r in range(len(ql)):
        sl = slice(int(cu[r]), int(cu[r + 1]))
        oa, la = _run_varlen(q[sl], k[sl], v[sl], [0, ql[r]], [0, ql[r]], 0.1, False)
        assert torch.equal(oa, out[sl]) and torch.equal(la, lse[sl])
    perm = [2, 0, 3, 1]
    qp = torch.cat([q[int(cu[r]):int(cu[r + 1])] for r in perm])
    kp = torch.cat([k[int(cu[r]):int(cu[r + 1])] for r in perm])
    vp = torch.cat([v[int(cu[r]):int(cu[r + 1])] for r in perm])
    cup = oracle.cu_seqlens_from_lengths([ql[r] for r in perm])
    op, _ = _run_varlen(qp, kp, vp, cup, cup, 0.1, False)
    for i, r in enumerate(perm):
        assert torch.equal(op[int(cup[i]):int(cup[i + 1])], out[int(cu[r]):int(cu[r + 1])])
    # two identical requests in one batch give identical outputs
    sl = slice(int(cu[0]), int(cu[1]))
    qd, kd, vd = (torch.cat([t[sl], t[sl]]) for t in (q, k, v))
    cud = [0, ql[0], 2 * ql[0]]
    od, ld = _run_varlen(qd, kd, vd, cud, cud, 0.1, False)
    assert torch.equal(od[:ql[0]], od[ql[0]:]) and torch.equal(ld[:ql[0]], ld[ql[0]:])


# ------------------------------------------------------------------ key split of the last round


def _split_parts(ql, kl, H, D):
    """parts of the split plan the device would use for this batch."""
    bm, _, _, slots = vl.varlen_launch_shape(max(ql), len(ql), H, D, max_kv=max(kl), split=True)
    T = len(oracle.tile_order(oracle.cu_seqlens_from_lengths(ql), oracle.cu_seqlens_from_lengths(kl), H, bm))
    return oracle.split_plan(T, slots, max(kl)), slots


def _varlen_random_cases(seed: int, count: int):
    """Seeded random packed batches: 1-6 requests of 0-1200 query rows (some
    empty), keys equal to the queries or drawn apart (0-1500, some empty),
    1-4 heads, D of 64 or 128."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        R = int(rng.integers(1, 7))
        ql = [0 if rng.random() < 0.15 else int(rng.integers(1, 1201)) for _ in range(R)]
        if rng.random() < 0.6:
            kl = list(ql)
        else:
            kl = [0 if rng.random() < 0.1 else int(rng.integers(1, 1501)) for _ in range(R)]
        cases.append((ql, kl, int(rng.integers(1, 5)), int(rng.choice([64, 128]))))
    return cases


VL_RANDOM = _varlen_random_cases(91, 10)


@pytest.mark.parametrize("case", VL_RANDOM, ids=[f"R{len(c[0])}-H{c[2]}-D{c[3]}-{i}" for i, c in enumerate(VL_RANDOM)])
def test_varlen_random_batches(case):
    """Each random batch through the three launches (bf16, bf16 with the
    workspace: staged V^T and the key split of the last round, fp32), every
    output row and lse against the oracle, canaries around both; the
    workspace launch once more on V packed straight into V^T from a padded
    per-request buffer, bit for bit."""
    ql, kl, H, D = case
    log(f"[varlen] random ql={ql} kl={kl} H={H} D={D}")
    q_cu = oracle.cu_seqlens_from_lengths(ql)
    kv_cu = oracle.cu_seqlens_from_lengths(kl)
    scale = wl.softmax_scale(D)
    for f32, split in ((False, False), (False, True), (True, False)):
        dtype = torch.float32 if f32 else torch.bfloat16
        q, k, v = wl.random_varlen_case(sum(ql) + 7 * sum(kl) + D, ql, H, D, dtype, kl)
        out, lse = _run_varlen(q, k, v, q_cu, kv_cu, scale, f32, split=split)
        ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v), q_cu, kv_cu, scale)
        what = f"random {case} {'f32' if f32 else 'bf16'}{' split' if split else ''}"
        check_close(to64(out), ro, f32, what)
        check_lse(to64(lse), rl, f32, what)
        if split:
            R = len(kl)
            slab = torch.zeros((R, max(max(kl), 1), H, D), dtype=dtype)
            for r in range(R):
                slab[r, :kl[r]] = v[kv_cu[r]:kv_cu[r + 1]]
            i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)
            ws = torch.empty(vl.varlen_split_workspace_bytes(sum(kl), R, H, D), dtype=torch.uint8, device=DEV)
            vl.pack_v_transposed([(slab.to(DEV), i32(kv_cu), i32(kv_cu[:-1]))], i32(kv_cu), sum(kl), ws)
            o2 = torch.empty_like(out)
            l2 = torch.empty_like(lse)
            vl.varlen_attn_fwd_vt(q.to(DEV), k.to(DEV), i32(q_cu), i32(kv_cu), int(max(ql)), int(max(kl)), ws, scale,
                                  out=o2, lse=l2)
            torch.cuda.synchronize()
            assert torch.equal(o2.view(torch.int16), out.view(torch.int16)), f"{what}: packed V^T out differs"
            assert torch.equal(l2, lse), f"{what}: packed V^T lse differs"


# Request lengths of the three full-size workloads' shapes (text + image rows).
QUEUE_LENS = [[16600], [4196, 7089, 16434, 4182], [32868, 32773, 32968, 32771]]


@pytest.mark.parametrize("lens", QUEUE_LENS, ids=["joint", "mixres", "edit"])
def test_queue_launch_writes_every_row_full_size(lens):
    """The workspace launch takes its items through the chiplet work queues,
    so which work-group runs an item changes from call to call.  At full size,
    three calls into NaN-filled out / lse: every element is written, and
    equals, bit for bit, the allocation-free launch (static block map, same
    split plan, V read row-major)."""
    H, D = 24, 128
    T = sum(lens)
    log(f"[queues] lens={lens} T={T}")
    g = torch.Generator(device=DEV)
    g.manual_seed(T)
    q, k, v = (torch.randn((T, H, D), generator=g, device=DEV).to(torch.bfloat16) for _ in range(3))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=DEV)
    m = max(lens)
    scale = wl.softmax_scale(D)
    ref_out, ref_lse = vl.varlen_attn_fwd_noalloc(q, k, v, cu, cu, m, m, scale, return_lse=True)
    ws = torch.empty(vl.varlen_split_workspace_bytes(T, len(lens), H, D), dtype=torch.uint8, device=DEV)
    for rep in range(3):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((T, H), float("nan"), device=DEV)
        vl.varlen_attn_fwd_split(q, k, v, cu, cu, m, m, scale, out=out, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item(), f"call {rep}: rows left unwritten"
        assert not torch.isnan(lse).any().item(), f"call {rep}: lse left unwritten"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"call {rep}: out differs"
        assert torch.equal(lse, ref_lse), f"call {rep}: lse differs"
    del q, k, v, ws, out, lse, ref_out, ref_lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D", [64, 128])
def test_packed_vt_pieces_and_gaps_vs_oracle(D):
    """V packed from two padded pieces straight into V^T (pack_v_transposed)
    and attended through it (varlen_attn_fwd_vt), q != kv: keys no piece
    covers read as zero V (a gap inside request 0, a trailing gap in request
    2), a piece of no rows covers nothing, a request without keys gives
    0 / -inf.  Against the oracle on the V
    those pieces pack, and bit for bit against varlen_attn_fwd_split on the
    same V packed flat."""
    H = 2
    kl = [70, 1, 700, 0]
    ql = [33, 5, 130, 7]
    a_len = [30, 0, 600, 0]     # piece A: the first rows of each request
    gap = [10, 0, 100, 0]       # then rows no piece covers
    b_len = [kl[r] - a_len[r] - gap[r] for r in range(4)]  # piece B: the rest
    R = len(kl)
    kv_cu = oracle.cu_seqlens_from_lengths(kl)
    q_cu = oracle.cu_seqlens_from_lengths(ql)
    rng = np.random.default_rng(D + 5)
    bf = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    q, k = bf(int(q_cu[-1]), H, D), bf(int(kv_cu[-1]), H, D)
    slab_a, slab_b = bf(R, max(a_len), H, D), bf(R, max(b_len), H, D)
    v_flat = torch.zeros((int(kv_cu[-1]), H, D), dtype=torch.bfloat16)
    for r in range(R):
        v_flat[kv_cu[r]:kv_cu[r] + a_len[r]] = slab_a[r, :a_len[r]]
        o = kv_cu[r] + a_len[r] + gap[r]
        v_flat[o:o + b_len[r]] = slab_b[r, :b_len[r]]
    scale = wl.softmax_scale(D)
    ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v_flat), q_cu, kv_cu, scale)
    ref_out, ref_lse = _run_varlen(q, k, v_flat, q_cu, kv_cu, scale, False, split=True)
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)
    T = int(kv_cu[-1])
    ws = torch.full((vl.varlen_split_workspace_bytes(T, R, H, D),), 0xFF, dtype=torch.uint8, device=DEV)
    # plus a piece of no rows (an all-text batch's image buffer): it covers nothing
    empty = torch.empty((R, 0, H, D), dtype=torch.bfloat16, device=DEV)
    vl.pack_v_transposed([(slab_a.to(DEV), i32(oracle.cu_seqlens_from_lengths(a_len)), i32(kv_cu[:-1])),
                          (empty, i32([0] * (R + 1)), i32(kv_cu[:-1])),
                          (slab_b.to(DEV), i32(oracle.cu_seqlens_from_lengths(b_len)),
                           i32(np.asarray(kv_cu[:-1]) + np.asarray(a_len) + np.asarray(gap)))],
                         i32(kv_cu), T, ws)
    for rep in range(2):
        out = torch.full((int(q_cu[-1]), H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((int(q_cu[-1]), H), float("nan"), device=DEV)
        vl.varlen_attn_fwd_vt(q.to(DEV), k.to(DEV), i32(q_cu), i32(kv_cu), max(ql), max(kl), ws, scale,
                              out=out, lse=lse)
        torch.cuda.synchronize()
        check_close(to64(out), ro, False, f"packed V^T D={D} call {rep}")
        check_lse(to64(lse), rl, False, f"packed V^T D={D} call {rep}")
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"call {rep}: out differs from split"
        assert torch.equal(lse, ref_lse), f"call {rep}: lse differs from split"


def test_packed_vt_overlapping_pieces_first_wins():
    """Where two pieces cover the same key, the first one given supplies it:
    piece A covers every key, piece B (listed second) the middle of each
    request with other values, and the result equals the split launch on
    piece A's V alone, bit for bit; listed the other way round, the middle
    keys come from B."""
    H, D = 2, 64
    kl = [100, 37]
    R = len(kl)
    kv_cu = oracle.cu_seqlens_from_lengths(kl)
    rng = np.random.default_rng(77)
    bf = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    q, k = bf(int(kv_cu[-1]), H, D), bf(int(kv_cu[-1]), H, D)
    slab_a, slab_b = bf(R, max(kl), H, D), bf(R, 20, H, D)
    b_len, b_at = [20, 10], [30, 5]                 # piece B: keys b_at .. b_at + b_len of each request
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)
    piece_a = (slab_a.to(DEV), i32(kv_cu), i32(kv_cu[:-1]))
    piece_b = (slab_b.to(DEV), i32(oracle.cu_seqlens_from_lengths(b_len)), i32(np.asarray(kv_cu[:-1]) + b_at))
    T = int(kv_cu[-1])
    scale = wl.softmax_scale(D)
    for order in ("ab", "ba"):
        v_flat = torch.zeros((T, H, D), dtype=torch.bfloat16)
        for r in range(R):
            v_flat[kv_cu[r]:kv_cu[r + 1]] = slab_a[r, :kl[r]]
            if order == "ba":
                v_flat[kv_cu[r] + b_at[r]:kv_cu[r] + b_at[r] + b_len[r]] = slab_b[r, :b_len[r]]
        ref_out, ref_lse = _run_varlen(q, k, v_flat, kv_cu, kv_cu, scale, False, split=True)
        ws = torch.empty(vl.varlen_split_workspace_bytes(T, R, H, D), dtype=torch.uint8, device=DEV)
        vl.pack_v_transposed([piece_a, piece_b] if order == "ab" else [piece_b, piece_a], i32(kv_cu), T, ws)
        out, lse = vl.varlen_attn_fwd_vt(q.to(DEV), k.to(DEV), i32(kv_cu), i32(kv_cu), max(kl), max(kl), ws, scale,
                                         return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"order {order}: out differs"
        assert torch.equal(lse, ref_lse), f"order {order}: lse differs"


@pytest.mark.parametrize("cfg", ["joint-16k", "mixres-4req", "edit-cfg-4seq"])
def test_packed_vt_equals_split_full_size(cfg):
    """The step's fused path at full size: V packed from its text and image
    pieces straight into V^T in a workspace filled with 0xFF bytes (NaN V,
    counters at -1), then the attention that reads it, twice: out and lse
    equal, bit for bit, the flat pack + varlen_attn_fwd_split."""
    log(f"[packed vt] {cfg}: generating inputs")
    inp = wl.make_varlen_inputs(wl.WORKLOADS[cfg], torch.bfloat16)
    res = _pipeline(inp)
    H, D, T, R = inp.spec.H, inp.spec.D, inp.total_tokens, inp.R
    mask_d = torch.from_numpy(inp.text_mask.astype(np.uint8)).to(DEV)
    hw_d = torch.tensor(inp.img_hw, dtype=torch.int32, device=DEV).reshape(-1, 2)
    cu_j, cu_t, cu_i, img_dst = vl.joint_cu_seqlens(mask_d, hw_d)
    ws = torch.full((vl.varlen_split_workspace_bytes(T, R, H, D),), 0xFF, dtype=torch.uint8, device=DEV)
    vl.pack_v_transposed([(inp.v_text.to(DEV), cu_t, cu_j[:-1]), (inp.v_img.to(DEV), cu_i, img_dst)], cu_j, T, ws)
    for rep in range(2):
        out = torch.full_like(res["out"], float("nan"))
        lse = torch.full_like(res["lse"], float("nan"))
        vl.varlen_attn_fwd_vt(res["q"], res["k"], cu_j, cu_j, inp.max_len, inp.max_len, ws, inp.scale,
                              out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), res["out"].view(torch.int16)), f"call {rep}: out differs"
        assert torch.equal(lse, res["lse"]), f"call {rep}: lse differs"
    del res, ws, out, lse
    torch.cuda.empty_cache()


def test_queue_launches_on_two_streams_do_not_interfere():
    """Two workspace launches in flight at once on two streams, each with its
    own workspace (its own queue counters) and its own batch: each result
    equals, bit for bit, the same launch run alone."""
    H, D = 8, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    batches = []
    for lens in ([3000, 1200, 5000], [700, 4100, 2600, 90]):
        T = sum(lens)
        q, k, v = (torch.randn((T, H, D), generator=g, device=DEV).to(torch.bfloat16) for _ in range(3))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=DEV)
        ws = torch.empty(vl.varlen_split_workspace_bytes(T, len(lens), H, D), dtype=torch.uint8, device=DEV)
        batches.append((q, k, v, cu, max(lens), ws))
    scale = wl.softmax_scale(D)
    alone = []
    for q, k, v, cu, m, ws in batches:
        alone.append(vl.varlen_attn_fwd_split(q, k, v, cu, cu, m, m, scale, workspace=ws, return_lse=True))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        outs = []
        for (q, k, v, cu, m, ws), st in zip(batches, streams):
            with torch.cuda.stream(st):
                outs.append(vl.varlen_attn_fwd_split(q, k, v, cu, cu, m, m, scale, workspace=ws, return_lse=True))
        torch.cuda.synchronize()
        for (o, l), (o0, l0) in zip(outs, alone):
            assert torch.equal(o.view(torch.int16), o0.view(torch.int16)), f"round {rep}: out differs"
            assert torch.equal(l, l0), f"round {rep}: lse differs"


SPLIT_CASES = [
    # one round only: every tile is cut
    ("one_request", [3000], None, 2, 128),
    # ragged q tiles, a kv length with empty key ranges, a request with no keys
    ("ragged_empty_parts", [300, 130, 1, 2000], [5000, 70, 0, 2000], 3, 128),
    ("d64_q_ne_kv", [77, 640, 129], [1500, 9, 1300], 2, 64),
    # more than 64 requests: index order, through the chiplet queues
    ("many_requests", [int(x) for x in np.random.default_rng(8).integers(0, 700, size=150)], None, 3, 64),
    # 64 requests, the most whose bounds the queue launch decodes from
    # registers (one per lane), and 65, decoded through memory
    ("64_requests", [int(x) for x in np.random.default_rng(9).integers(0, 700, size=64)], None, 2, 64),
    ("65_requests", [int(x) for x in np.random.default_rng(9).integers(0, 700, size=65)], None, 2, 64),
]


@pytest.mark.parametrize("name,ql,kl,H,D", SPLIT_CASES)
def test_varlen_split_vs_oracle(name, ql, kl, H, D):
    kl = ql if kl is None else kl
    (full, tail, parts), slots = _split_parts(ql, kl, H, D)
    log(f"[split] {name}: slots {slots} full {full} tail {tail} parts {parts}")
    assert parts >= 2, "the case must exercise the split"
    q, k, v = wl.random_varlen_case(41, ql, H, D, torch.bfloat16, kl)
    q_cu = oracle.cu_seqlens_from_lengths(ql)
    kv_cu = oracle.cu_seqlens_from_lengths(kl)
    scale = wl.softmax_scale(D)
    out, lse = _run_varlen(q, k, v, q_cu, kv_cu, scale, False, split=True)
    ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v), q_cu, kv_cu, scale)
    check_close(to64(out), ro, False, name)
    check_lse(to64(lse), rl, False, name)
    # the same launch on V packed straight into V^T from a padded buffer: the same bits
    R = len(kl)
    slab = torch.zeros((R, max(max(kl), 1), H, D), dtype=torch.bfloat16)
    for r in range(R):
        slab[r, :kl[r]] = v[kv_cu[r]:kv_cu[r + 1]]
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)
    ws = torch.empty(vl.varlen_split_workspace_bytes(int(kv_cu[-1]), R, H, D), dtype=torch.uint8, device=DEV)
    vl.pack_v_transposed([(slab.to(DEV), i32(kv_cu), None)], i32(kv_cu), int(kv_cu[-1]), ws)
    ov, lv = vl.varlen_attn_fwd_vt(q.to(DEV), k.to(DEV), i32(q_cu), i32(kv_cu), max(ql), max(kl), ws, scale,
                                   return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(ov.view(torch.int16), out.view(torch.int16)) and torch.equal(lv, lse), f"{name}: packed V^T"
    # against the unsplit launch: the same math up to fp32 summation order
    o1, l1 = _run_varlen(q, k, v, q_cu, kv_cu, scale, False)
    assert (o1.float() - out.float()).abs().max().item() <= 2 ** -7
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(lse))
    assert (l1[fin] - lse[fin]).abs().max().item() <= 1e-4


def test_varlen_split_after_full_rounds():
    """More tiles than slots: the whole rounds run unsplit, the tail is cut.
    Compared with the oracle on every row of the tail tiles and a sample of
    the rest."""
    H, D = 1, 64
    _, _, _, slots = vl.varlen_launch_shape(128, 1, H, D, max_kv=1024, split=True)
    R = slots + 5
    ql = [128] * R
    kl = [1024] * R
    (full, tail, parts), _ = _split_parts(ql, kl, H, D)
    log(f"[split] {R} requests: slots {slots} full {full} tail {tail} parts {parts}")
    assert (full, tail, parts) == (slots, 5, 4)
    q, k, v = wl.random_varlen_case(43, ql, H, D, torch.bfloat16, kl)
    q_cu = oracle.cu_seqlens_from_lengths(ql)
    kv_cu = oracle.cu_seqlens_from_lengths(kl)
    scale = wl.softmax_scale(D)
    out, lse = _run_varlen(q, k, v, q_cu, kv_cu, scale, False, split=True)
    # tiles are visited in request order here (more than 64 requests): the
    # tail tiles are the last five requests
    tail_rows = np.arange(int(q_cu[R - 5]), int(q_cu[R]))
    rows = np.union1d(tail_rows, np.random.default_rng(1).choice(int(q_cu[R - 5]), 300, replace=False))
    ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v), q_cu, kv_cu, scale, rows=rows)
    check_close(to64(out)[rows], ro, False, "split tail")
    check_lse(to64(lse)[rows], rl, False, "split tail")


def test_varlen_split_workspace_checked():
    """A split launch refuses a missing or short workspace before launching."""
    ql = [3000]
    q, k, v = wl.random_varlen_case(47, ql, 1, 128, torch.bfloat16)
    cu = torch.tensor([0, 3000], dtype=torch.int32, device=DEV)
    need = vl.varlen_split_workspace_bytes(3000, 1, 1, 128)
    assert need > 0
    short = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(vl.VarlenError):
        vl.varlen_attn_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), cu, cu, 3000, 3000, workspace=short)
    exact = torch.empty(need, dtype=torch.uint8, device=DEV)
    o_split = vl.varlen_attn_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), cu, cu, 3000, 3000, workspace=exact)
    ro, _ = oracle.varlen_attention(to64(q), to64(k), to64(v), [0, 3000], [0, 3000], wl.softmax_scale(128),
                                    rows=np.arange(0, 3000, 7))
    check_close(to64(o_split)[::7], ro, False, "exact workspace")


# (lengths, kv lengths or None, heads, head size): no key split (max_kv < 512),
# ragged tails, empty requests, many requests (gaps between their V^T columns)
VT_CASES = [
    ([300], None, 2, 128),
    ([17, 64, 129, 1, 0, 255], None, 3, 128),
    ([40, 90, 7], [130, 0, 511], 2, 64),
    ([5] * 100, [33] * 100, 1, 128),
]


@pytest.mark.parametrize("ql,kl,H,D", VT_CASES)
def test_varlen_staged_vt_equals_direct_v(ql, kl, H, D):
    """The workspace launch reads V through the staged V^T; without a key
    split it feeds the MFMAs exactly the operands the direct launch reads, so
    out and lse are the same bits."""
    kl = kl or ql
    log(f"[varlen] staged V^T vs direct V: R={len(ql)} H={H} D={D}")
    q, k, v = wl.random_varlen_case(51, ql, H, D, torch.bfloat16, kv_lengths=kl)
    q_cu, kv_cu = oracle.cu_seqlens_from_lengths(ql), oracle.cu_seqlens_from_lengths(kl)
    o1, l1 = _run_varlen(q, k, v, q_cu, kv_cu, wl.softmax_scale(D), False, split=True)
    o2, l2 = _run_varlen(q, k, v, q_cu, kv_cu, wl.softmax_scale(D), False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _pipeline(inp):
    """The hot path on the GPU: boundaries from the text mask and grids, joint
    pack of q/k/v, varlen attention, unpack of the outputs."""
    H, D = inp.spec.H, inp.spec.D
    T = inp.total_tokens
    mask_d = torch.from_numpy(inp.text_mask.astype(np.uint8)).to(DEV)
    hw_d = torch.tensor(inp.img_hw, dtype=torch.int32, device=DEV).reshape(-1, 2)
    cu_j, cu_t, cu_i, img_dst = vl.joint_cu_seqlens(mask_d, hw_d)
    # the launches the benchmark times: one batched pack of the six pieces
    packed, items = [], []
    for txt, img in ((inp.q_text, inp.q_img), (inp.k_text, inp.k_img), (inp.v_text, inp.v_img)):
        dst = torch.empty((T, H, D), dtype=inp.dtype, device=DEV)
        items += [(txt.to(DEV), cu_t, dst, cu_j[:-1]), (img.to(DEV), cu_i, dst, img_dst)]
        packed.append(dst)
    vl.pack_by_cu_seqlens_batched(items)
    q, k, v = packed
    max_len = inp.max_len
    # bf16 runs the workspace launch (V^T staging, key split of the last round,
    # chiplet queues); test_packed_vt_equals_split_full_size checks that the
    # benchmarked form, on V packed straight into V^T, gives the same bits
    fn = vl.varlen_attn_fwd_f32 if inp.dtype == torch.float32 else vl.varlen_attn_fwd_split
    out, lse = fn(q, k, v, cu_j, cu_j, max_len, max_len, inp.scale, return_lse=True)
    out_txt = torch.empty_like(inp.q_text, device=DEV)
    out_img = torch.empty_like(inp.q_img, device=DEV)
    vl.unpack_by_cu_seqlens_batched([(out, cu_t, out_txt, cu_j[:-1]), (out, cu_i, out_img, img_dst)])
    torch.cuda.synchronize()
    return dict(cu=cu_j, q=q, k=k, v=v, out=out, lse=lse, out_txt=out_txt, out_img=out_img)


@pytest.mark.parametrize("cfg", ["joint-16k", "mixres-4req", "edit-cfg-4seq"])
def test_full_size_workloads_sampled(cfg):
    log(f"[pipeline] {cfg}: generating inputs")
    inp = wl.make_varlen_inputs(wl.WORKLOADS[cfg], torch.bfloat16)
    log(f"[pipeline] {cfg}: T={inp.total_tokens} running GPU path")
    res = _pipeline(inp)
    cj, ct, ci, idst = oracle.joint_cu_seqlens(inp.text_mask, inp.img_hw)
    assert np.array_equal(res["cu"].cpu().numpy(), cj.astype(np.int32))
    T, H, D = inp.total_tokens, inp.spec.H, inp.spec.D
    qn = np.zeros((T, H, D), dtype=np.float32)
    kn = np.zeros((T, H, D), dtype=np.float32)
    vn = np.zeros((T, H, D), dtype=np.float32)
    for dst, txt, img in ((qn, inp.q_text, inp.q_img), (kn, inp.k_text, inp.k_img), (vn, inp.v_text, inp.v_img)):
        oracle.pack_by_cu_seqlens(txt.float().numpy(), ct, dst_row_offsets=cj[:-1], dst=dst)
        oracle.pack_by_cu_seqlens(img.float().numpy(), ci, dst_row_offsets=idst, dst=dst)
    # pack is bit-exact on the full tensors
    assert np.array_equal(res["q"].float().cpu().numpy(), qn)
    assert np.array_equal(res["k"].float().cpu().numpy(), kn)
    assert np.array_equal(res["v"].float().cpu().numpy(), vn)
    rows = sample_rows(cj)
    log(f"[pipeline] {cfg}: oracle on {rows.size} sampled rows")
    ro, rl = oracle.varlen_attention(qn, kn, vn, cj, cj, inp.scale, rows=rows)
    out = res["out"].float().cpu().numpy()[rows].astype(np.float64)
    mx, mean = check_close(out, ro, False, f"{cfg}")
    check_lse(res["lse"].cpu().numpy()[rows].astype(np.float64), rl, False, f"{cfg}")
    log(f"   max-abs {mx:.3g} mean-abs {mean:.3g}")
    # the workspace-free entry point at the same full size, same sampled rows
    o_nw, l_nw = vl.varlen_attn_fwd(res["q"], res["k"], res["v"], res["cu"], res["cu"], inp.max_len, inp.max_len,
                                    inp.scale, return_lse=True)
    torch.cuda.synchronize()
    mx2, mean2 = check_close(o_nw.float().cpu().numpy()[rows].astype(np.float64), ro, False, f"{cfg} no workspace")
    check_lse(l_nw.cpu().numpy()[rows].astype(np.float64), rl, False, f"{cfg} no workspace")
    log(f"   no workspace: max-abs {mx2:.3g} mean-abs {mean2:.3g}")
    del o_nw, l_nw
    # unpack is the exact inverse on the real rows and zero on the padding
    out_full = res["out"].cpu()
    ref_txt = oracle.unpack_by_cu_seqlens(out_full.view(torch.int16).numpy(), ct, wl.TEXT_CAP,
                                          src_row_offsets=cj[:-1])
    assert np.array_equal(res["out_txt"].cpu().view(torch.int16).numpy(), ref_txt)
    ref_img = oracle.unpack_by_cu_seqlens(out_full.view(torch.int16).numpy(), ci, inp.img_cap,
                                          src_row_offsets=idst)
    assert np.array_equal(res["out_img"].cpu().view(torch.int16).numpy(), ref_img)


# ------------------------------------------------------------------ block-local attention


@pytest.mark.parametrize("n", [10, 96, 101, 2003])
@pytest.mark.parametrize("win", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("f32", [False, True])
def test_block_local_vs_oracle(n, win, f32):
    dtype = torch.float32 if f32 else torch.bfloat16
    lb, la = win
    log(f"[block_local] n={n} win={win} {dtype}")
    spec = wl.BLOCK_LOCAL_WORKLOADS["vocoder-dit"]
    inp = wl.make_block_local_inputs(spec, dtype, n=n, seed=1000 + n)
    full, out = canary_out(tuple(inp.q.shape), dtype, pad=1)
    fn = vl.block_local_attn_fwd_f32 if f32 else vl.block_local_attn_fwd
    _, lse = fn(inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV), spec.block, lb, la, inp.scale, out=out,
                return_lse=True)
    torch.cuda.synchronize()
    assert_canary(full, pad=1)
    ro, rl = oracle.block_local_attention(to64(inp.q), to64(inp.k), to64(inp.v), spec.block, lb, la, inp.scale)
    check_close(to64(out), ro, f32, f"block-local n={n} {win}")
    check_lse(to64(lse), rl, f32, f"block-local n={n} {win}", rounded_weights=False)


# (the fp32 entry takes one wave per query block when D = 64 and block <= 32:
# blocks of 1, 17, 24 and 32 frames, a sequence shorter than one block, and
# windows wider than the sequence -- up to the largest int -- on both paths)
@pytest.mark.parametrize("case", [(2, 300, 7, 2, 1, 128), (1, 33, 40, 0, 0, 64), (3, 61, 5, 3, 0, 128),
                                  (1, 500, 24, 30, 30, 64), (2, 301, 17, 2, 3, 64), (1, 5, 24, 0, 0, 64),
                                  (1, 96, 32, 1, 1, 64), (1, 70, 1, 3, 2, 64),
                                  (1, 100, 24, 0, 2147483647, 64), (1, 100, 24, 2147483647, 1, 128)])
@pytest.mark.parametrize("f32", [False, True])
def test_block_local_other_shapes(case, f32):
    B, n, block, lb, la, D = case
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[block_local] B={B} n={n} block={block} lb={lb} la={la} D={D} {dtype}")
    rng = np.random.default_rng(n)
    q, k, v = (torch.from_numpy(rng.standard_normal((B, n, 2, D)).astype(np.float32)).to(dtype)
               for _ in range(3))
    fn = vl.block_local_attn_fwd_f32 if f32 else vl.block_local_attn_fwd
    full, out = canary_out(tuple(q.shape), dtype, pad=1)
    _, lse = fn(q.to(DEV), k.to(DEV), v.to(DEV), block, lb, la, wl.softmax_scale(D), out=out, return_lse=True)
    torch.cuda.synchronize()
    assert_canary(full, pad=1)
    ro, rl = oracle.block_local_attention(to64(q), to64(k), to64(v), block, lb, la, wl.softmax_scale(D))
    check_close(to64(out), ro, f32, f"block-local {case}")
    check_lse(to64(lse), rl, f32, f"block-local {case}", rounded_weights=False)


# Random small shapes through the block-aligned kernels (D = 64, blocks of
# 1..32 frames: one wave per query block, buffer loads bounded to the valid
# rows, V through LDS) and the tiled fallbacks (blocks above 32, wider bf16
# windows): batch rows, head counts, ragged last blocks and windows that
# reach past either end, each with canary rows around out and lse.
_BL_RNG = np.random.default_rng(77)
BL_RANDOM = [tuple(int(_BL_RNG.integers(lo, hi)) for lo, hi in ((1, 4), (1, 260), (1, 5), (1, 41), (0, 4), (0, 4)))
             for _ in range(12)]


@pytest.mark.parametrize("case", BL_RANDOM)
@pytest.mark.parametrize("f32", [False, True])
def test_block_local_random_shapes(case, f32):
    B, n, H, block, lb, la = case
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[block_local] random B={B} n={n} H={H} block={block} lb={lb} la={la} {dtype}")
    rng = np.random.default_rng(n * 131 + block)
    q, k, v = (torch.from_numpy(rng.standard_normal((B, n, H, 64)).astype(np.float32)).to(dtype) for _ in range(3))
    fn = vl.block_local_attn_fwd_f32 if f32 else vl.block_local_attn_fwd
    full, out = canary_out(tuple(q.shape), dtype, pad=1)
    lse_full, lse = canary_out((B, n, H), torch.float32, pad=1)
    fn(q.to(DEV), k.to(DEV), v.to(DEV), block, lb, la, 0.125, out=out, lse=lse)
    torch.cuda.synchronize()
    assert_canary(full, pad=1)
    assert_canary(lse_full, pad=1)
    ro, rl = oracle.block_local_attention(to64(q), to64(k), to64(v), block, lb, la, 0.125)
    check_close(to64(out), ro, f32, f"block-local random {case}")
    check_lse(to64(lse), rl, f32, f"block-local random {case}", rounded_weights=False)


# Windows at the edges of the kernel choice: D = 64 blocks of <= 32 frames
# take the one-wave-per-block kernels (bf16 up to 96 keys: one, two or three
# 32-key chunks; fp32 at any width), the rest the tiled kernels.  (block,
# look_back, look_ahead): 96 keys in three whole chunks, 93 and 95 keys with
# a ragged last chunk, 97 and 128 keys on the tiled side, 32 keys in one
# chunk and 33 in two; n leaves a ragged last block and clips the windows at
# both ends.
BL_EDGES = [(32, 1, 1), (31, 1, 1), (19, 2, 2), (97, 0, 0), (32, 2, 1), (32, 0, 0), (33, 0, 0), (11, 1, 1)]


@pytest.mark.parametrize("edge", BL_EDGES)
@pytest.mark.parametrize("f32", [False, True])
def test_block_local_window_edges(edge, f32):
    block, lb, la = edge
    B, n, H = 2, 7 * block + block // 2 + 1, 3
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[block_local] window edge block={block} lb={lb} la={la} ({(1 + lb + la) * block} keys) n={n} {dtype}")
    rng = np.random.default_rng(block * 7 + lb * 3 + la)
    q, k, v = (torch.from_numpy(rng.standard_normal((B, n, H, 64)).astype(np.float32)).to(dtype) for _ in range(3))
    fn = vl.block_local_attn_fwd_f32 if f32 else vl.block_local_attn_fwd
    full, out = canary_out(tuple(q.shape), dtype, pad=1)
    lse_full, lse = canary_out((B, n, H), torch.float32, pad=1)
    fn(q.to(DEV), k.to(DEV), v.to(DEV), block, lb, la, 0.125, out=out, lse=lse)
    torch.cuda.synchronize()
    assert_canary(full, pad=1)
    assert_canary(lse_full, pad=1)
    ro, rl = oracle.block_local_attention(to64(q), to64(k), to64(v), block, lb, la, 0.125)
    check_close(to64(out), ro, f32, f"block-local edge {edge}")
    check_lse(to64(lse), rl, f32, f"block-local edge {edge}", rounded_weights=False)


@pytest.mark.parametrize("f32", [False, True])
def test_block_local_own_block_agrees_with_varlen_on_block_requests(f32):
    """Own-block windows with n a multiple of the block are varlen attention
    over equal 24-token requests (a cross-entry-point identity the oracle pins
    on the CPU).  The two entry points run different kernels (fp32 vs bf16-
    rounded row sums, 32- vs 64-key chunks), so they are not bit-identical:
    each is checked against the oracle, and against the other to the output
    tolerance."""
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[block_local] own-block vs varlen {dtype}")
    rng = np.random.default_rng(44)
    n, H, D = 24 * 40, 2, 64
    q, k, v = (torch.from_numpy(rng.standard_normal((1, n, H, D)).astype(np.float32)).to(dtype)
               for _ in range(3))
    bl_fn = vl.block_local_attn_fwd_f32 if f32 else vl.block_local_attn_fwd
    vl_fn = vl.varlen_attn_fwd_f32 if f32 else vl.varlen_attn_fwd
    ob = bl_fn(q.to(DEV), k.to(DEV), v.to(DEV), 24, 0, 0, 0.125)
    cu = torch.arange(0, n + 1, 24, dtype=torch.int32, device=DEV)
    ov = vl_fn(q[0].to(DEV), k[0].to(DEV), v[0].to(DEV), cu, cu, 24, 24, 0.125)
    torch.cuda.synchronize()
    ro, _ = oracle.varlen_attention(to64(q[0]), to64(k[0]), to64(v[0]), cu.cpu().numpy(), cu.cpu().numpy(), 0.125)
    check_close(to64(ob[0]), ro, f32, "own-block block-local")
    check_close(to64(ov), ro, f32, "own-block varlen")
    check_close(to64(ob[0]), to64(ov), f32, "block-local vs varlen")


# ------------------------------------------------------------------ errors


def test_error_paths_return_codes():
    log("[errors]")
    q = torch.zeros((10, 2, 96), dtype=torch.bfloat16, device=DEV)
    cu = torch.tensor([0, 10], dtype=torch.int32, device=DEV)
    with pytest.raises(vl.VarlenError, match="unsupported"):
        vl.varlen_attn_fwd(q, q, q, cu, cu, 10, 10)
    q2 = torch.zeros((10, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(vl.VarlenError):
        vl.varlen_attn_fwd(q2, q2, q2, cu, cu, 10, 10, padded_tokens=4)
    with pytest.raises(vl.VarlenError):
        vl.varlen_attn_fwd(q2, q2, q2, cu, cu, 10, 10, attn_mask=torch.ones(1))
    with pytest.raises(vl.VarlenError, match="invalid"):
        vl.block_local_attn_fwd(q2[None], q2[None], q2[None], 0, 0, 0)
    with pytest.raises(vl.VarlenError):
        vl.varlen_attn_fwd(q2.cpu(), q2.cpu(), q2.cpu(), cu.cpu(), cu.cpu(), 10, 10)
    # wrong-shaped out / lse raise in the binding, before any launch (the C ABI
    # cannot check buffer sizes): the buffers keep their canary contents
    b4 = q2[None]
    for fn in (vl.block_local_attn_fwd, vl.varlen_attn_fwd):
        args = (b4, b4, b4, 24, 0, 0) if fn is vl.block_local_attn_fwd else (q2, q2, q2, cu, cu, 10, 10)
        full = b4 if fn is vl.block_local_attn_fwd else q2
        short = torch.full((full.numel() - 64,), 7.0, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(vl.VarlenError, match="out must"):
            fn(*args, out=short.view(-1, 2, 32) if fn is vl.varlen_attn_fwd else short.view(1, -1, 2, 32))
        lse_shape = (1, 10, 3) if fn is vl.block_local_attn_fwd else (10, 3)
        lse_bad = torch.full(lse_shape, 7.0, dtype=torch.float32, device=DEV)
        with pytest.raises(vl.VarlenError, match="lse must"):
            fn(*args, lse=lse_bad)
        torch.cuda.synchronize()
        assert bool((short == 7.0).all()) and bool((lse_bad == 7.0).all())
    # a cu_seqlens that leaves rows outside every request is refused by the host check
    cu_short = torch.tensor([0, 8], dtype=torch.int32, device=DEV)
    with pytest.raises(vl.VarlenError, match="padded_tokens"):
        vl.varlen_attn_fwd(q2, q2, q2, cu_short, cu_short, 10, 10, check_cu_seqlens=True)


# ------------------------------------------------------------------ CFG combine fused into unpack


def _bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


@pytest.mark.parametrize("row_elems", [3072, 8])
def test_unpack_cfg_combine_vs_oracle(row_elems):
    log(f"[cfg] row {row_elems}")
    rng = np.random.default_rng(row_elems)
    # sequences [r1+, r1-, r2+, r2-, r3+, r3-]: text of differing length, then an image
    # segment whose length the positive and negative pass of a request share.
    img = [300, 77, 1]
    txt = [[20, 3], [9, 1], [0, 5]]
    seqs = []
    for r in range(3):
        for sgn in range(2):
            seqs.append((txt[r][sgn], img[r]))
    lengths = [t + n for t, n in seqs]
    cu = oracle.cu_seqlens_from_lengths(lengths)
    T = int(cu[-1])
    flat = torch.from_numpy(rng.standard_normal((T, row_elems)).astype(np.float32)).to(torch.bfloat16)
    pos_rows = np.array([cu[2 * r] + txt[r][0] for r in range(3)], dtype=np.int32)
    neg_rows = np.array([cu[2 * r + 1] + txt[r][1] for r in range(3)], dtype=np.int32)
    seg_cu = oracle.cu_seqlens_from_lengths(img).astype(np.int32)
    scale = np.array([4.0, 2.5, 7.0], dtype=np.float32)
    max_len = 310
    dst = torch.full((3, max_len, row_elems), 5.0, dtype=torch.bfloat16, device=DEV)
    vl.unpack_cfg_combine(flat.to(DEV), torch.from_numpy(seg_cu).to(DEV), torch.from_numpy(pos_rows).to(DEV),
                          torch.from_numpy(neg_rows).to(DEV), torch.from_numpy(scale).to(DEV), dst)
    torch.cuda.synchronize()
    got = dst.float().cpu().numpy().astype(np.float64)
    f64 = flat.float().numpy().astype(np.float64)
    for r in range(3):
        n = img[r]
        ref = oracle.cfg_combine(f64[pos_rows[r]:pos_rows[r] + n], f64[neg_rows[r]:neg_rows[r] + n], float(scale[r]))
        err = np.abs(got[r, :n] - ref)
        assert np.all(err <= _bf16_ulp(ref)), f"request {r}: max err {err.max()}"
        assert not got[r, n:].any(), "padding rows must be zero"
    # scale 0 gives the negative rows and scale 1 the positive rows, bit for bit
    for s, rows in ((0.0, neg_rows), (1.0, pos_rows)):
        sc = torch.full((3,), s, dtype=torch.float32, device=DEV)
        vl.unpack_cfg_combine(flat.to(DEV), torch.from_numpy(seg_cu).to(DEV), torch.from_numpy(pos_rows).to(DEV),
                              torch.from_numpy(neg_rows).to(DEV), sc, dst)
        torch.cuda.synchronize()
        for r in range(3):
            a = dst[r, :img[r]].cpu()
            b = flat[rows[r]:rows[r] + img[r]]
            if not torch.equal(a, b):
                bad = (a != b).nonzero()
                log(f"scale {s} request {r}: {bad.shape[0]} mismatches, first {bad[:4].tolist()}, "
                    f"got {a[tuple(bad[0])].item()} want {b[tuple(bad[0])].item()}")
            assert torch.equal(a, b)


# ------------------------------------------------------------------ SP pad tails and production block-local


@pytest.mark.parametrize("f32", [False, True])
def test_sp_padded_queries_attend_real_keys_only(f32):
    """Sequence-parallel auto-pad (PR #4293): the query side covers the padded
    length, the key side only the real tokens, so the pad never changes a real
    row's output and needs no attention mask."""
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[sp-pad] {dtype}")
    real = [6889, 1000, 4095]
    padded = [oracle.sp_auto_pad(n, 8)[0] for n in real]
    assert padded[0] == 6896
    q, k, v = wl.random_varlen_case(91, padded, 2, 128, dtype, real)
    q_cu = oracle.cu_seqlens_from_lengths(padded)
    kv_cu = oracle.cu_seqlens_from_lengths(real)
    out, lse = _run_varlen(q, k, v, q_cu, kv_cu, wl.softmax_scale(128), f32)
    rows = sample_rows(q_cu, n_random=128)
    ro, rl = oracle.varlen_attention(to64(q), to64(k), to64(v), q_cu, kv_cu, wl.softmax_scale(128), rows=rows)
    check_close(to64(out)[rows], ro, f32, "sp pad")
    check_lse(to64(lse)[rows], rl, f32, "sp pad")
    # the real rows equal an unpadded run over the same real tokens
    keep = np.concatenate([np.arange(q_cu[r], q_cu[r] + real[r]) for r in range(3)])
    o2, _ = _run_varlen(q[torch.from_numpy(keep)], k, v, kv_cu, kv_cu, wl.softmax_scale(128), f32)
    assert torch.equal(out[torch.from_numpy(keep).to(out.device)].cpu(), o2.cpu())


@pytest.mark.parametrize("f32", [True, False])
def test_block_local_production_shape(f32):
    """Token2Wav DiT shape of PR #7975: fp32, CFG as batch 2, 4000 mel frames
    (167 blocks of 24, last block 16 frames), own-block and one-neighbour layers."""
    dtype = torch.float32 if f32 else torch.bfloat16
    log(f"[block_local] production shape {dtype}")
    spec = wl.BLOCK_LOCAL_WORKLOADS["vocoder-dit"]
    inp = wl.make_block_local_inputs(spec, dtype, n=4000, B=2, seed=4000)
    fn = vl.block_local_attn_fwd_f32 if f32 else vl.block_local_attn_fwd
    for lb, la in [(0, 0), (1, 0), (0, 1)]:
        out, lse = fn(inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV), 24, lb, la, inp.scale, return_lse=True)
        torch.cuda.synchronize()
        ro, rl = oracle.block_local_attention(to64(inp.q), to64(inp.k), to64(inp.v), 24, lb, la, inp.scale)
        check_close(to64(out), ro, f32, f"production block-local ({lb},{la})")
        check_lse(to64(lse), rl, f32, f"production block-local ({lb},{la})", rounded_weights=False)
