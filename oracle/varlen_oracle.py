"""CPU oracle for packed variable-length attention -- TEST INFRASTRUCTURE ONLY.

This module is the plain, slow, obviously-correct statement of what the GPU
library computes.  Only the tests, the package smoke check and the CPU-baseline
leg of the benchmark may import it; the product path never does, and this file
imports nothing from the product package (the two share no code).

Everything floating-point is computed in float64 from the exact values of the
inputs (bf16 and fp32 widen to fp64 without rounding).  Integer work is plain
Python / NumPy integer arithmetic.

Sources (vLLM-Omni pull-request pages):
  * "Replace per-bucket varlen loop with flat varlen attention for mixfusion"
    (PR #6711), sections "Key changes", "Reference / Acknowledgement" and
    "How to enable MixFusion";
  * "Support dynamic batching for heterogeneous diffusion requests"
    (PR #4024), sections "How batching works", "Correctness model" and
    "CFG behavior";
  * "Use block-sparse attention in Qwen2.5-Omni Token2Wav DiT" (PR #7975),
    the review comments on the window/validity-mask code, the two commit
    messages, and the "Purpose" / "Change" sections.

Readings of points the pages leave open are stated where they are used; each
is also listed with its justification in the design notes.  Every function
here is pinned by CPU tests against something other than itself (brute force,
closed forms, invariants, or values printed on the pages).
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")

# --------------------------------------------------------------------------
# cu_seqlens: validation and construction
# --------------------------------------------------------------------------


def validate_cu_seqlens(cu, total: Optional[int] = None, max_len: Optional[int] = None) -> np.ndarray:
    """Check the varlen boundary contract and return cu as int64.

    PR #6711 "Reference / Acknowledgement": the flat branch takes
    q_cu_seqlens / kv_cu_seqlens with max_q_len / max_kv_len and requires
    padded_tokens = 0.  Reading: cu[0] = 0, non-decreasing, cu[R] = total
    rows, and every length <= the declared max.
    """
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be a 1-D array of length num_reqs + 1")
    if cu[0] != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    lengths = np.diff(cu)
    if np.any(lengths < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    if total is not None and cu[-1] != total:
        raise ValueError(f"cu_seqlens[-1]={cu[-1]} != total rows {total}")
    if max_len is not None and lengths.size and lengths.max() > max_len:
        raise ValueError("a request is longer than the declared max length")
    return cu


def lengths_from_text_mask(text_mask) -> np.ndarray:
    """Real text length of each request = number of True entries in its row.

    PR #6711 "Key changes": cu_seqlens are built from the real text lengths
    via mask.sum; PR #4024 "How batching works": text lengths come from the
    real prompt mask.
    """
    m = np.asarray(text_mask)
    out = np.zeros(m.shape[0], dtype=np.int64)
    for r in range(m.shape[0]):
        out[r] = int(sum(1 for x in m[r] if x))
    return out


def image_tokens(img_hw) -> np.ndarray:
    """Image tokens of each request = grid height x grid width.

    PR #4024 "How batching works": the image grid shapes stay in img_shapes;
    a request's image token count is the product of its grid.
    """
    hw = np.asarray(img_hw, dtype=np.int64).reshape(-1, 2)
    return np.array([int(h) * int(w) for h, w in hw], dtype=np.int64)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """cu[0] = 0, cu[r+1] = cu[r] + lengths[r] (plain running sum)."""
    cu = [0]
    for n in lengths:
        n = int(n)
        if n < 0:
            raise ValueError("negative length")
        cu.append(cu[-1] + n)
    return np.array(cu, dtype=np.int64)


def joint_cu_seqlens(text_mask, img_hw):
    """Boundaries of a joint [text ; image] packed batch.

    Each request is its real text tokens followed by its image tokens (the
    joint text+image sequence of PR #4024 "How batching works"; text first is
    the reading taken for the order inside a request).  Returns
      cu_joint[R+1]  boundaries of the packed joint sequences,
      cu_text[R+1]   running sum of text lengths,
      cu_img[R+1]    running sum of image token counts,
      img_dst[R]     packed row where request r's image tokens start
                     (= cu_joint[r] + text_len[r]).
    """
    t = lengths_from_text_mask(text_mask)
    n = image_tokens(img_hw)
    if t.shape[0] != n.shape[0]:
        raise ValueError("text_mask and img_hw disagree on the number of requests")
    cu_joint = cu_seqlens_from_lengths([a + b for a, b in zip(t, n)])
    cu_text = cu_seqlens_from_lengths(t)
    cu_img = cu_seqlens_from_lengths(n)
    img_dst = np.array([cu_joint[r] + t[r] for r in range(t.shape[0])], dtype=np.int64)
    return cu_joint, cu_text, cu_img, img_dst


# --------------------------------------------------------------------------
# pack / unpack
# --------------------------------------------------------------------------


def pack_by_cu_seqlens(src_padded, cu_seqlens, dst_rows: Optional[int] = None,
                       dst_row_offsets=None, dst=None) -> np.ndarray:
    """Gather only the real rows of a padded per-request buffer into a flat one.

    PR #4024 "How batching works": a batch is formed from each request's
    real tokens alone, with no padding to a common length, so pad rows never
    reach attention.  src_padded has shape [R, S, ...]; request r has
    len_r = cu[r+1] - cu[r] real rows at src[r, 0:len_r].  They go to
    dst[off_r + i] with off_r = dst_row_offsets[r] if given, else cu[r].
    Rows of dst that no request writes keep their previous content (dst given)
    or are zero (dst allocated here).
    """
    src = np.asarray(src_padded)
    cu = validate_cu_seqlens(cu_seqlens)
    R = cu.size - 1
    if src.shape[0] != R:
        raise ValueError("src_padded must have one slab per request")
    offs = cu[:-1] if dst_row_offsets is None else np.asarray(dst_row_offsets, dtype=np.int64)
    if dst is None:
        rows = int(cu[-1]) if dst_rows is None else int(dst_rows)
        dst = np.zeros((rows,) + src.shape[2:], dtype=src.dtype)
    for r in range(R):
        n = int(cu[r + 1] - cu[r])
        if n > src.shape[1]:
            raise ValueError("request longer than the padded slab")
        for i in range(n):
            dst[int(offs[r]) + i] = src[r, i]
    return dst


def unpack_by_cu_seqlens(src_flat, cu_seqlens, max_len: int, src_row_offsets=None,
                         zero_fill: bool = True, dst=None) -> np.ndarray:
    """Scatter a flat packed buffer back to a padded per-request buffer.

    PR #6711 "Key changes": output unpacked by cu_seqlens; PR #4024
    "Correctness model": outputs are scattered back to the request-local
    state.  dst[r, i] = src[off_r + i] for i < len_r, off_r = src_row_offsets[r]
    or cu[r].  Rows i >= len_r are zero when zero_fill, else left untouched.
    """
    src = np.asarray(src_flat)
    cu = validate_cu_seqlens(cu_seqlens)
    R = cu.size - 1
    offs = cu[:-1] if src_row_offsets is None else np.asarray(src_row_offsets, dtype=np.int64)
    if dst is None:
        dst = np.zeros((R, int(max_len)) + src.shape[1:], dtype=src.dtype)
    for r in range(R):
        n = int(cu[r + 1] - cu[r])
        if n > max_len:
            raise ValueError("request longer than max_len")
        for i in range(int(max_len)):
            if i < n:
                dst[r, i] = src[int(offs[r]) + i]
            elif zero_fill:
                dst[r, i] = 0
    return dst


# --------------------------------------------------------------------------
# Tile schedule (a design choice of this library, not of the pages)
# --------------------------------------------------------------------------

LPT_MAX_REQS = 64   # requests are visited longest-first only up to this count
XCDS = 8            # chiplets a launch is dealt across, round-robin by block id
MAX_SPLIT = 16      # key ranges a tile of the last round is cut into, at most
MIN_SPLIT_KEYS = 256  # ... and at most max_kv // MIN_SPLIT_KEYS of them


def tile_order(q_cu, kv_cu, H: int, block_m: int, lpt_max_reqs: int = LPT_MAX_REQS
               ) -> List[Tuple[int, int, int]]:
    """Logical list of (request, head, q-tile) work items of the varlen kernel.

    Spec: when R <= lpt_max_reqs, requests are visited by key length
    descending, ties by request index ascending; otherwise in index order.
    Within a request: heads ascending, then q-tiles ascending.  A request with
    q_len = 0 has no tiles; nt_r = ceil(q_len_r / block_m).
    No token of one request shares a tile with another request, which is the
    "tokens from one request cannot attend to another" contract of PR #4024
    "Correctness model".
    """
    qc = validate_cu_seqlens(q_cu)
    kc = validate_cu_seqlens(kv_cu)
    R = qc.size - 1
    if kc.size - 1 != R:
        raise ValueError("q and kv cu_seqlens disagree on the number of requests")
    qlen = [int(qc[r + 1] - qc[r]) for r in range(R)]
    kvlen = [int(kc[r + 1] - kc[r]) for r in range(R)]
    if R <= lpt_max_reqs:
        order = sorted(range(R), key=lambda r: (-kvlen[r], r))
    else:
        order = list(range(R))
    tiles = []
    for r in order:
        nt = (qlen[r] + block_m - 1) // block_m
        for h in range(H):
            for qt in range(nt):
                tiles.append((r, h, qt))
    return tiles


def split_plan(T: int, slots: int, max_kv: int) -> Tuple[int, int, int]:
    """(full, tail, parts) of the key split of the last, partial round.

    With `slots` work-groups resident at once and T tiles, tiles [0, full)
    run whole, full = T - T mod slots (0 when T < slots).  The tail = T - full
    remaining tiles are cut into parts = min(MAX_SPLIT, slots // tail,
    max_kv // MIN_SPLIT_KEYS) key ranges each when that is at least 2, i.e.
    when the tail would leave at least half of the slots idle; otherwise
    nothing is split: (T, 0, 1).  slots <= 0 turns the split off.
    """
    if slots <= 0 or T <= 0:
        return T, 0, 1
    full = (T // slots) * slots if T >= slots else 0
    tail = T - full
    if tail == 0:
        return T, 0, 1
    parts = min(MAX_SPLIT, slots // tail, max_kv // MIN_SPLIT_KEYS)
    if parts < 2:
        return T, 0, 1
    return full, tail, parts


def split_range(nkt: int, part: int, parts: int) -> Tuple[int, int]:
    """Key tiles [lo, hi) of range `part` of `parts` over nkt key tiles."""
    return part * nkt // parts, (part + 1) * nkt // parts


def grid_blocks(num_reqs: int, max_q: int, H: int, block_m: int, chunk: int, xcds: int = XCDS,
                slots: int = 0, queues: bool = False) -> int:
    """Launch size the host derives from scalars only: an upper bound on the
    tile count plus one round of slots when the key split is on, plus (with
    the chiplet work queues of the workspace launch) an eighth of that bound
    in spare blocks, rounded up to a whole number of (xcds x chunk) groups."""
    upper = num_reqs * H * ((max_q + block_m - 1) // block_m) + max(slots, 0)
    if queues:
        upper += (upper + 7) // 8
    group = xcds * chunk
    return ((upper + group - 1) // group) * group


def block_to_logical(b: int, chunk: int, xcds: int = XCDS) -> int:
    """Launched block id -> logical work item.

    Block ids are dealt to chiplets round-robin (x = b mod xcds); the i-th
    block a chiplet receives takes logical item ((i div chunk) * xcds + x) *
    chunk + (i mod chunk), so runs of `chunk` consecutive logical tiles (same
    request and head, hence the same K/V) stay on one chiplet's L2.
    """
    x = b % xcds
    i = b // xcds
    return ((i // chunk) * xcds + x) * chunk + (i % chunk)


def chiplet_queues(n_items: int, chunk: int, xcds: int = XCDS) -> List[List[int]]:
    """The chiplet work queues of the workspace launch: queue x lists, in
    order, the logical items [0, n_items) that block_to_logical deals to the
    blocks of chiplet x (its k-th block's item is the queue's k-th entry).  A
    block takes the next entry of its own chiplet's queue, or of another queue
    once its own is empty; which block runs an item decides nothing about the
    item's result."""
    queues: List[List[int]] = [[] for _ in range(xcds)]
    for t in range(n_items):
        queues[(t // chunk) % xcds].append(t)
    return queues


def work_items(q_cu, kv_cu, H: int, block_m: int, slots: int = 0, max_kv: int = 0,
               lpt_max_reqs: int = LPT_MAX_REQS) -> List[Tuple[int, int, int, int, int]]:
    """Logical list of (request, head, q-tile, part, parts) work items: the
    tiles of tile_order, with those of the last partial round replaced by
    their key ranges (split_plan), tile by tile."""
    tiles = tile_order(q_cu, kv_cu, H, block_m, lpt_max_reqs)
    full, tail, parts = split_plan(len(tiles), slots, max_kv)
    items = [(r, h, qt, 0, 1) for r, h, qt in tiles[:full]]
    for r, h, qt in tiles[full:full + tail]:
        items.extend((r, h, qt, p, parts) for p in range(parts))
    return items


def block_schedule(q_cu, kv_cu, H: int, block_m: int, max_q: int, chunk: int,
                   lpt_max_reqs: int = LPT_MAX_REQS, xcds: int = XCDS, slots: int = 0,
                   max_kv: int = 0, queues: bool = False) -> np.ndarray:
    """(request, head, q-tile, part, parts) of every launched block, all -1 if
    idle: the static map (with the chiplet queues, the item each block takes
    while every chiplet keeps to its own queue in block order)."""
    items = work_items(q_cu, kv_cu, H, block_m, slots, max_kv, lpt_max_reqs)
    R = len(validate_cu_seqlens(q_cu)) - 1
    G = grid_blocks(R, max_q, H, block_m, chunk, xcds, slots, queues)
    out = np.full((G, 5), -1, dtype=np.int64)
    for b in range(G):
        t = block_to_logical(b, chunk, xcds)
        if t < len(items):
            out[b] = items[t]
    return out


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _softmax_attend(q, k, v, scale: float):
    """softmax(scale * q k^T) v for one head: q [m, D], k [n, D], v [n, D].

    Returns (out [m, D], lse [m]); lse is the natural-log sum of
    exp(scale * q.k) over the keys.  With no keys: out = 0, lse = -inf.
    """
    m = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((m, v.shape[1])), np.full(m, NEG_INF)
    s = scale * (q @ k.T)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ v) / l
    lse = (mx + np.log(l))[:, 0]
    return out, lse


def varlen_attention(q, k, v, q_cu, kv_cu, scale: float, rows: Optional[Sequence[int]] = None,
                     row_chunk: int = 2048):
    """Flat varlen non-causal attention over packed [T, H, D] tensors.

    PR #6711 "Key changes" / "Reference": one attention pass over flat packed
    [total_tokens, heads, head_dim] Q/K/V whose request boundaries are
    q_cu_seqlens / kv_cu_seqlens.  PR #4024 "Correctness model": tokens from
    one request cannot attend to tokens of another.  So for request r and
    head h:  O = softmax(scale * Q_r K_r^T) V_r over the keys of r only.

    rows: optional subset of global query rows; results are returned for
    those rows only, in the given order (rows are independent, so computing a
    subset is exact).  Returns (out [Tq or len(rows), H, D], lse [.., H]).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    qc = validate_cu_seqlens(q_cu, total=q.shape[0])
    kc = validate_cu_seqlens(kv_cu, total=k.shape[0])
    R = qc.size - 1
    if kc.size - 1 != R:
        raise ValueError("q and kv cu_seqlens disagree on the number of requests")
    H = q.shape[1]
    scale = float(scale)
    if rows is None:
        sel = np.arange(q.shape[0])
    else:
        sel = np.asarray(rows, dtype=np.int64)
    out = np.zeros((sel.size, H, v.shape[2]))
    lse = np.full((sel.size, H), NEG_INF)
    # Request of each selected row: the r with qc[r] <= row < qc[r+1].
    req_of = np.searchsorted(qc, sel, side="right") - 1
    for r in range(R):
        idx = np.nonzero(req_of == r)[0]
        if idx.size == 0:
            continue
        qrows = sel[idx]
        k_r = k[kc[r]:kc[r + 1]]
        v_r = v[kc[r]:kc[r + 1]]
        for c0 in range(0, idx.size, row_chunk):
            ci = idx[c0:c0 + row_chunk]
            qr = q[qrows[c0:c0 + row_chunk]]
            for h in range(H):
                o, ls = _softmax_attend(qr[:, h, :], k_r[:, h, :], v_r[:, h, :], scale)
                out[ci, h, :] = o
                lse[ci, h] = ls
    return out, lse


def block_local_key_range(i: int, n: int, block: int, look_back: int, look_ahead: int) -> Tuple[int, int]:
    """Keys [lo, hi) that frame i attends to under block-local attention.

    PR #7975 (review of the window code and the first commit message): frames
    are grouped in blocks of `block`; query block b = i div block attends to
    its own block, `look_back` blocks before it and `look_ahead` blocks after
    it; blocks past either end do not exist and the padded tail of a partial
    last block is masked, so the key set is every frame j < n whose block lies
    in [b - look_back, b + look_ahead].
    """
    b = i // block
    nb = (n + block - 1) // block
    lo_b = max(0, b - look_back)
    hi_b = min(nb - 1, b + look_ahead)
    return lo_b * block, min(n, (hi_b + 1) * block)


def block_local_attention(q, k, v, block: int, look_back: int, look_ahead: int, scale: float):
    """Block-local attention over [B, n, H, D] tensors (see block_local_key_range).

    Each query block is computed with the plain softmax definition over its
    window of keys.  Returns (out [B, n, H, D], lse [B, n, H]).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    if block < 1 or look_back < 0 or look_ahead < 0:
        raise ValueError("block must be >= 1 and look counts >= 0")
    B, n, H, D = q.shape
    out = np.zeros((B, n, H, v.shape[3]))
    lse = np.full((B, n, H), NEG_INF)
    for b in range(B):
        for i0 in range(0, n, block):
            i1 = min(n, i0 + block)
            lo, hi = block_local_key_range(i0, n, block, look_back, look_ahead)
            for h in range(H):
                o, ls = _softmax_attend(q[b, i0:i1, h], k[b, lo:hi, h], v[b, lo:hi, h], float(scale))
                out[b, i0:i1, h] = o
                lse[b, i0:i1, h] = ls
    return out, lse


# --------------------------------------------------------------------------
# Brute force (tiny inputs only): dense attention under an explicit mask
# --------------------------------------------------------------------------


def dense_masked_attention(q, k, v, mask, scale: float):
    """Dense [Tq, Tk] attention with a boolean mask (True = may attend).

    q [Tq, H, D], k/v [Tk, H, D].  Masked scores are -inf before the softmax;
    a row with no allowed key gives out = 0 and lse = -inf.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    mask = np.asarray(mask, dtype=bool)
    Tq, H, _ = q.shape
    out = np.zeros((Tq, H, v.shape[2]))
    lse = np.full((Tq, H), NEG_INF)
    for h in range(H):
        s = float(scale) * np.einsum("id,jd->ij", q[:, h], k[:, h])
        s = np.where(mask, s, NEG_INF)
        for i in range(Tq):
            if not mask[i].any():
                continue
            mx = s[i].max()
            p = np.exp(s[i] - mx)
            l = p.sum()
            out[i, h] = (p @ v[:, h]) / l
            lse[i, h] = mx + math.log(l)
    return out, lse


def block_diagonal_mask(q_cu, kv_cu) -> np.ndarray:
    """mask[i, j] = query row i and key row j belong to the same request."""
    qc = validate_cu_seqlens(q_cu)
    kc = validate_cu_seqlens(kv_cu)
    Tq, Tk = int(qc[-1]), int(kc[-1])
    rq = np.empty(Tq, dtype=np.int64)
    rk = np.empty(Tk, dtype=np.int64)
    for r in range(qc.size - 1):
        rq[qc[r]:qc[r + 1]] = r
        rk[kc[r]:kc[r + 1]] = r
    return rq[:, None] == rk[None, :]


def block_difference_mask(n: int, block: int, look_back: int, look_ahead: int) -> np.ndarray:
    """The dense mask the block-local path replaces (PR #7975 "Purpose"):
    diff[i, j] = block(j) - block(i); allowed iff -look_back <= diff <= look_ahead."""
    blk = np.arange(n) // block
    diff = blk[None, :] - blk[:, None]
    return (diff >= -look_back) & (diff <= look_ahead)


# --------------------------------------------------------------------------
# Around the path (next rows): per-request CFG combine, MixFusion chunk plan
# --------------------------------------------------------------------------


def cfg_combine(positive, negative, true_cfg_scale):
    """negative + s * (positive - negative), applied per request after the
    split (PR #4024 "CFG behavior"); s may differ per request."""
    p = _f64(positive)
    n = _f64(negative)
    return n + float(true_cfg_scale) * (p - n)


def mixfusion_chunk_plan(token_counts: Iterable[int], min_chunk_tokens: int = 256, max_chunks: int = 128):
    """Accept or reject a flat-varlen MixFusion layout.

    PR #6711 "How to enable MixFusion": the layout is rejected when the gcd
    of the token counts is below mixfusion_min_chunk_tokens (default 256) or
    when the resulting chunk count exceeds mixfusion_max_chunks (default 128).
    Reading: chunk_size = gcd, chunk_count = total tokens / chunk_size.
    Returns (accepted, chunk_size, chunk_count).
    """
    counts = [int(c) for c in token_counts]
    if not counts or any(c <= 0 for c in counts):
        return False, 0, 0
    g = 0
    for c in counts:
        a, b = g, c
        while b:
            a, b = b, a % b
        g = a
    count = sum(counts) // g
    ok = g >= min_chunk_tokens and count <= max_chunks
    return ok, g, count


def sp_auto_pad(seq_len: int, world_size: int):
    """Sequence-parallel auto-pad: the smallest multiple of world_size that is
    >= seq_len, and the pad (PR #4293 debug lines: 20596 -> 20600 with
    pad_size=4 and 6889 -> 6896 with pad_size=7 at world_size=8).
    Returns (padded_len, pad)."""
    if world_size < 1 or seq_len < 0:
        raise ValueError("world_size must be >= 1 and seq_len >= 0")
    padded = -(-int(seq_len) // int(world_size)) * int(world_size)
    return padded, padded - int(seq_len)
