"""The C-ABI library on a host without a GPU: it loads, exports every symbol
the header declares, and rejects bad host scalars with the documented status
codes before launching anything."""

import ctypes
import os
import re

import pytest

import oracle
import packed_variable_length_varlen_amd as vl
from packed_variable_length_varlen_amd import build as vl_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "varlen.h")

VL_OK, VL_EINVAL, VL_EUNSUPPORTED = 0, -1, -2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vl.lib_path()):
        vl_build.build()
    return vl.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("varlen_attn_fwd", "varlen_attn_fwd_f32", "block_local_attn_fwd",
                 "block_local_attn_fwd_f32", "pack_by_cu_seqlens", "unpack_by_cu_seqlens",
                 "cu_seqlens_from_lengths", "joint_cu_seqlens", "varlen_tile_map"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    assert lib.vl_version() >= 100
    assert lib.vl_status_string(VL_EUNSUPPORTED) == b"unsupported size"


def test_bad_scalars_rejected_before_launch(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    # head_dim other than 64 / 128
    assert lib.varlen_attn_fwd(p, p, p, p, p, 8, 8, 1, 2, 96, 0.1, p, None, None) == VL_EUNSUPPORTED
    assert lib.varlen_attn_fwd_f32(p, p, p, p, p, 8, 8, 1, 2, 80, 0.1, p, None, None) == VL_EUNSUPPORTED
    # negative / zero sizes
    assert lib.varlen_attn_fwd(p, p, p, p, p, -1, 8, 1, 2, 64, 0.1, p, None, None) == VL_EINVAL
    assert lib.varlen_attn_fwd(p, p, p, p, p, 8, 8, 1, 0, 64, 0.1, p, None, None) == VL_EINVAL
    # null tensors
    assert lib.varlen_attn_fwd(None, p, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, None) == VL_EINVAL
    # misaligned tensors
    odd = ctypes.c_void_p(18)
    assert lib.varlen_attn_fwd(odd, p, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, None) == VL_EINVAL
    # NaN scale
    assert lib.varlen_attn_fwd(p, p, p, p, p, 8, 8, 1, 2, 64, float("nan"), p, None, None) == VL_EINVAL
    # zero, negative or infinite scale (the running maximum is taken over raw scores)
    for bad in (0.0, -0.125, float("inf"), float("-inf")):
        assert lib.varlen_attn_fwd(p, p, p, p, p, 8, 8, 1, 2, 64, bad, p, None, None) == VL_EINVAL
        assert lib.varlen_attn_fwd_f32(p, p, p, p, p, 8, 8, 1, 2, 64, bad, p, None, None) == VL_EINVAL
        assert lib.block_local_attn_fwd(p, p, p, 1, 10, 2, 64, 24, 0, 0, bad, p, None, None) == VL_EINVAL
        assert lib.varlen_attn_fwd_split(p, p, p, p, p, 8, 8, 1, 2, 64, bad, p, None, 8, p, 1 << 30,
                                         None) == VL_EINVAL
    # nothing to do is success without a launch
    assert lib.varlen_attn_fwd(None, None, None, None, None, 0, 0, 0, 2, 64, 0.1, None, None, None) == VL_OK
    # block-local: block < 1, negative look counts, bad D
    assert lib.block_local_attn_fwd(p, p, p, 1, 10, 2, 64, 0, 0, 0, 0.1, p, None, None) == VL_EINVAL
    assert lib.block_local_attn_fwd(p, p, p, 1, 10, 2, 64, 24, -1, 0, 0.1, p, None, None) == VL_EINVAL
    assert lib.block_local_attn_fwd_f32(p, p, p, 1, 10, 2, 32, 24, 0, 0, 0.1, p, None, None) == VL_EUNSUPPORTED
    assert lib.block_local_attn_fwd(p, p, p, 0, 10, 2, 64, 24, 0, 0, 0.1, p, None, None) == VL_OK
    # pack / unpack
    assert lib.pack_by_cu_seqlens(p, 4, p, 2, 0, p, None, None) == VL_EINVAL
    assert lib.pack_by_cu_seqlens(p, 4, p, 70000, 16, p, None, None) == VL_EINVAL
    assert lib.unpack_by_cu_seqlens(p, None, p, -1, 16, p, 4, 1, None) == VL_EINVAL
    assert lib.pack_by_cu_seqlens(None, 4, None, 0, 16, None, None, None) == VL_OK
    # batched pack / unpack: count bounds, bad descriptors, empty work
    descs = (vl._CopyDesc * 9)()
    assert lib.pack_by_cu_seqlens_batched(ctypes.cast(descs, ctypes.c_void_p), 9, None) == VL_EINVAL
    assert lib.pack_by_cu_seqlens_batched(ctypes.cast(descs, ctypes.c_void_p), -1, None) == VL_EINVAL
    assert lib.pack_by_cu_seqlens_batched(None, 2, None) == VL_EINVAL
    assert lib.pack_by_cu_seqlens_batched(None, 0, None) == VL_OK
    descs[0] = vl._CopyDesc(16, 16, 16, None, -4, 16, 1, 0)      # negative max_len
    assert lib.unpack_by_cu_seqlens_batched(ctypes.cast(descs, ctypes.c_void_p), 1, None) == VL_EINVAL
    descs[0] = vl._CopyDesc(None, 16, 16, None, 4, 16, 1, 0)     # null source with work to do
    assert lib.pack_by_cu_seqlens_batched(ctypes.cast(descs, ctypes.c_void_p), 1, None) == VL_EINVAL
    descs[0] = vl._CopyDesc(None, None, None, None, 4, 16, 0, 0)  # no requests: nothing to launch
    assert lib.pack_by_cu_seqlens_batched(ctypes.cast(descs, ctypes.c_void_p), 1, None) == VL_OK
    # cu helpers
    assert lib.cu_seqlens_from_lengths(p, -1, p, None) == VL_EINVAL
    assert lib.joint_cu_seqlens(p, -1, p, 2, p, p, p, p, None) == VL_EINVAL
    # tile map: output too small
    assert lib.varlen_tile_map(p, p, 300, 300, 4, 2, 128, 0, 0, p, 1, None) == VL_EINVAL
    # split entry point: same scalar checks as the plain one, plus its
    # workspace (short -> EINVAL) and the 32-bit V^T row limit, all before any launch
    assert lib.varlen_attn_fwd_split(p, p, p, p, p, 8, 8, 1, 2, 96, 0.1, p, None, 8, p, 1 << 20, None) \
        == VL_EUNSUPPORTED
    assert lib.varlen_attn_fwd_split(p, p, p, p, p, -1, 8, 1, 2, 64, 0.1, p, None, 8, p, 1 << 20, None) == VL_EINVAL
    assert lib.varlen_attn_fwd_split(p, p, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, -1, p, 1 << 20, None) == VL_EINVAL
    assert lib.varlen_attn_fwd_split(p, p, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, 8, p, 16, None) == VL_EINVAL
    assert lib.varlen_attn_fwd_split(p, p, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, 8, None, 1 << 20, None) \
        == VL_EINVAL
    assert lib.varlen_attn_fwd_split(p, p, p, p, p, 8, 8, 1, 2, 128, 0.1, p, None, 9_000_000, p, 1 << 40, None) \
        == VL_EUNSUPPORTED
    # V packed straight into V^T, and the attention that reads it: piece
    # count, descriptor rows and requests, head_dim, workspace
    vd = (vl._CopyDesc * 9)()
    for i in range(9):
        vd[i] = vl._CopyDesc(16, None, 16, None, 4, 2 * 64 * 2, 1, 0)  # H = 2, D = 64 rows, one request
    vp = ctypes.cast(vd, ctypes.c_void_p)
    assert lib.pack_v_transposed(vp, 0, p, 1, 2, 64, 8, p, 1 << 20, None) == VL_EINVAL
    assert lib.pack_v_transposed(vp, 9, p, 1, 2, 64, 8, p, 1 << 20, None) == VL_EINVAL
    assert lib.pack_v_transposed(None, 1, p, 1, 2, 64, 8, p, 1 << 20, None) == VL_EINVAL
    assert lib.pack_v_transposed(vp, 1, p, 1, 2, 96, 8, p, 1 << 20, None) == VL_EUNSUPPORTED
    assert lib.pack_v_transposed(vp, 1, p, 1, 4, 64, 8, p, 1 << 20, None) == VL_EINVAL   # rows of H = 2, not 4
    assert lib.pack_v_transposed(vp, 1, p, 2, 2, 64, 8, p, 1 << 20, None) == VL_EINVAL   # descriptor has 1 request
    assert lib.pack_v_transposed(vp, 1, p, 1, 2, 64, -1, p, 1 << 20, None) == VL_EINVAL
    assert lib.pack_v_transposed(vp, 1, p, 1, 2, 64, 8, p, 16, None) == VL_EINVAL         # short workspace
    assert lib.pack_v_transposed(vp, 1, p, 1, 2, 64, 8, None, 1 << 20, None) == VL_EINVAL
    vd[0] = vl._CopyDesc(24, None, 16, None, 4, 2 * 64 * 2, 1, 0)                        # misaligned source
    assert lib.pack_v_transposed(vp, 1, p, 1, 2, 64, 8, p, 1 << 20, None) == VL_EINVAL
    vd[0] = vl._CopyDesc(None, None, 16, None, 4, 2 * 64 * 2, 1, 0)                      # null source with rows
    assert lib.pack_v_transposed(vp, 1, p, 1, 2, 64, 8, p, 1 << 20, None) == VL_EINVAL
    vd[0] = vl._CopyDesc(16, None, 16, None, 4, 2 * 64 * 2, 0, 0)                        # no requests: nothing to do
    assert lib.pack_v_transposed(vp, 1, p, 0, 2, 64, 0, p, 0, None) == VL_OK
    assert lib.varlen_attn_fwd_vt(p, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, 8, p, 16, None) == VL_EINVAL
    assert lib.varlen_attn_fwd_vt(p, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, 8, None, 1 << 20, None) == VL_EINVAL
    assert lib.varlen_attn_fwd_vt(p, p, p, p, 8, 8, 1, 2, 96, 0.1, p, None, 8, p, 1 << 20, None) == VL_EUNSUPPORTED
    assert lib.varlen_attn_fwd_vt(None, p, p, p, 8, 8, 1, 2, 64, 0.1, p, None, 8, p, 1 << 20, None) == VL_EINVAL
    assert lib.varlen_split_workspace_bytes(8, 1, 2, 96, p) == VL_EUNSUPPORTED
    assert lib.varlen_split_workspace_bytes(8, 1, 2, 64, None) == VL_EINVAL
    assert lib.varlen_split_workspace_bytes(-1, 1, 2, 64, p) == VL_EINVAL


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("max_q,R,H,D", [(210, 3, 2, 64), (16640, 1, 24, 128), (16640, 4, 24, 128),
                                         (33024, 4, 24, 128), (1, 100, 1, 64), (0, 3, 2, 64)])
def test_launch_shape_matches_schedule_spec(lib, max_q, R, H, D, split):
    bm, chunk, G, slots = vl.varlen_launch_shape(max_q, R, H, D, max_kv=max_q, split=split)
    if not split:
        assert slots == 0
    expect = oracle.grid_blocks(R, max_q, H, bm, chunk, slots=slots, queues=bool(split)) if max_q > 0 and R > 0 else 0
    assert G == expect
    assert G % (8 * chunk) == 0


@pytest.mark.parametrize("kv_rows,R,H,D", [(0, 1, 1, 64), (100, 3, 2, 64), (16640, 1, 24, 128),
                                           (131592, 4, 24, 128), (64, 1000, 2, 128)])
def test_split_workspace_size_is_the_documented_layout(lib, kv_rows, R, H, D):
    """Partial results of the key split (slots x 256 rows x (D floats + 2
    floats), rounded up to 256 bytes), then V^T: H x D rows of
    roundup(kv_rows, 64) + 64 R bf16 columns, rounded up to 256 bytes, then
    256 bytes for the counters of the chiplet work queues."""
    _, _, _, slots = vl.varlen_launch_shape(4096, 1, 1, D, max_kv=4096, split=True)
    partial = -(-(slots * 256 * (D * 4 + 8)) // 256) * 256
    vt_ld = -(-kv_rows // 64) * 64 + 64 * R
    vt = -(-(H * D * vt_ld * 2) // 256) * 256
    assert vl.varlen_split_workspace_bytes(kv_rows, R, H, D) == partial + vt + 256


def test_mixfusion_plan_native_matches_oracle_and_pages(lib):
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "mixfusion_plan_caseB.json")))
    e = g["expected"]
    got = vl.mixfusion_chunk_plan(g["token_counts"], g["min_chunk_tokens"], g["max_chunks"])
    assert got == (e["accepted"], e["chunk_size"], e["chunk_count"])
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        counts = [int(256 * rng.integers(1, 40) * rng.choice([1, 2, 3])) if rng.random() < 0.7
                  else int(rng.integers(1, 5000)) for _ in range(n)]
        assert vl.mixfusion_chunk_plan(counts) == oracle.mixfusion_chunk_plan(counts)
    with pytest.raises(vl.VarlenError):
        vl.mixfusion_chunk_plan([5, 0])


def test_workload_lengths_match_the_generated_inputs():
    """varlen_lengths (used by bench.py to lay out the other workloads) takes
    the same text-length draws as make_varlen_inputs."""
    import torch
    from packed_variable_length_varlen_amd import workloads as wl
    for name in ("tiny-3req",):
        spec = wl.WORKLOADS[name]
        inp = wl.make_varlen_inputs(spec, torch.float32)
        assert wl.varlen_lengths(spec) == [t + i for t, i in zip(inp.text_len, inp.img_tokens)]
    # the full-size layouts: text drawn in the configured ranges, image grids as configured
    for name in ("joint-16k", "mixres-4req", "edit-cfg-4seq"):
        spec = wl.WORKLOADS[name]
        lens = wl.varlen_lengths(spec)
        assert len(lens) == len(spec.img_grids)
        for n, (lo, hi), (h, w) in zip(lens, spec.text_ranges, spec.img_grids):
            assert lo <= n - h * w <= hi


def test_bench_pair_counts_match_the_oracle():
    """The FLOP counts bench.py reports (4 D H per in-request or in-window
    pair) rest on its pair counts: block-local pairs equal the oracle's key
    ranges summed over frames and the True entries of the dense
    block-difference mask; the vocoder shape gives the counts 47,929 / 95,425
    / 142,921 (own block / one neighbour / both); varlen pairs equal the
    entries of the block-diagonal mask."""
    import numpy as np
    import bench
    for n, block in ((10, 24), (96, 24), (101, 24), (2003, 24), (70, 1), (33, 40)):
        for lb, la in ((0, 0), (1, 0), (0, 1), (1, 1), (3, 2)):
            by_range = sum(hi - lo for lo, hi in (oracle.block_local_key_range(i, n, block, lb, la) for i in range(n)))
            dense = int(np.count_nonzero(oracle.block_difference_mask(n, block, lb, la)))
            assert bench.block_local_pairs(n, block, lb, la) == by_range == dense, (n, block, lb, la)
    assert [bench.block_local_pairs(2003, 24, lb, la) for lb, la in ((0, 0), (1, 0), (0, 1), (1, 1))] == \
        [47929, 95425, 95425, 142921]
    cu = oracle.cu_seqlens_from_lengths([17, 0, 64, 129, 1])
    assert bench.varlen_pairs(cu) == int(np.count_nonzero(oracle.block_diagonal_mask(cu, cu)))


def test_validate_cu_seqlens_host_check():
    """The binding's opt-in host check of cu_seqlens (the kernels take them on
    trust): accepts well-formed arrays, rejects the malformed ones."""
    vl.validate_cu_seqlens([0, 17, 81, 210], rows=210, max_len=129)
    vl.validate_cu_seqlens([0, 0, 5, 5], rows=5, max_len=5)          # empty requests
    for bad, rows, max_len in (([], 10, 10), ([1, 5], 10, 10),        # empty / not starting at 0
                               ([0, 5, 4], 10, 10),                     # decreasing
                               ([0, 5, 11], 10, 10),                    # past the packed rows
                               ([0, 0, 5, 5], 8, 5),                    # rows no request covers
                               ([0, 5, 10], 10, 4)):                    # longer than the launch bound
        with pytest.raises(vl.VarlenError):
            vl.validate_cu_seqlens(bad, rows=rows, max_len=max_len)
