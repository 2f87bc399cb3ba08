"""The allocation-free varlen entry point (varlen_attn_fwd_noalloc) against
the workspace entry point it mirrors (varlen_attn_fwd_split): same split plan,
partials in the library's static device array instead of the workspace, V read
row-major instead of staged transposed -- the same bits.  Two calls in a row,
the second smaller, so stale partials of the first call would show."""

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


# (lengths, H, D): the first needs a key split after one full round of
# work-groups (16 q-tiles x 24 heads on 256 slots), the second, smaller, a
# split of every tile (80 tiles), the third no split at all (keys < 512)
CASES = [([4000], 24, 128), ([600, 130, 1500], 8, 64), ([300, 77, 129], 2, 128)]


def test_noalloc_equals_workspace_launch_on_consecutive_calls():
    for seed, (lens, H, D) in enumerate(CASES):
        log(f"[noalloc] call {seed}: lengths={lens} H={H} D={D}")
        q, k, v = (t.to(DEV) for t in wl.random_varlen_case(700 + seed, lens, H, D, torch.bfloat16))
        cu_np = oracle.cu_seqlens_from_lengths(lens)
        cu = torch.tensor(cu_np, dtype=torch.int32, device=DEV)
        m = max(lens)
        scale = wl.softmax_scale(D)
        o_ref, l_ref = vl.varlen_attn_fwd_split(q, k, v, cu, cu, m, m, scale, return_lse=True)
        o_na, l_na = vl.varlen_attn_fwd_noalloc(q, k, v, cu, cu, m, m, scale, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref), f"call {seed}: out differs from the workspace launch"
        assert torch.equal(l_na, l_ref), f"call {seed}: lse differs from the workspace launch"
        rows = sample_rows(cu_np, n_random=64)
        ro, rl = oracle.varlen_attention(to64(q.cpu()), to64(k.cpu()), to64(v.cpu()), cu_np, cu_np, scale, rows=rows)
        check_close(to64(o_na)[rows], ro, False, f"noalloc call {seed}")
        check_lse(to64(l_na)[rows], rl, False, f"noalloc call {seed}")
        _, _, _, slots = vl.varlen_launch_shape(m, len(lens), H, D, max_kv=m, split=True)
        log(f"   bitwise equal (split slots {slots})")
