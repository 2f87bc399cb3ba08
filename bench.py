"""Benchmark of the packed varlen attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. boundaries (cu_seqlens) from the real text mask and the image grids,
  2. joint text+image pack of Q, K and V into flat [T, H, D] (one launch),
  3. flat varlen attention (bf16 MFMA, fp32 accumulation; the last, partial
     round of work-groups cut along the keys and merged),
  4. unpack of the output back to the per-request text / image layout (one
     launch),
  5. block-local attention of the vocoder-DiT shape (n=2003, 24-frame blocks,
     H=16, D=64) for each of the four window types (own block, one back,
     one ahead, both).
The default workload is the single joint request of a 2048x2048 image
(16,384 image tokens + 8..256 text tokens, H=24, D=128, bf16).

value = algorithmic FLOP of one step / step time, where the FLOP count is
4*D*H per in-request (query, key) pair (the varlen pairs plus the in-window
block-local pairs); work the kernels avoid is never counted.

Prints ONE JSON line on stdout; details go to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("attn.hip", "vl_device.h"):
        with open(os.path.join(HERE, "packed_variable_length_varlen_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch of the attention kernel from committed rocprofv3
    --pmc counters (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel factor);
    None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, "varlen_attn_bf16_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("workloads", {}).get(workload, {}).get("hbm_bytes_per_launch")


def varlen_pairs(cu) -> int:
    cu = [int(x) for x in cu]
    return sum((cu[i + 1] - cu[i]) ** 2 for i in range(len(cu) - 1))


def block_local_pairs(n: int, block: int, lb: int, la: int) -> int:
    nb = (n + block - 1) // block
    tot = 0
    for b in range(nb):
        rows = min(n, (b + 1) * block) - b * block
        lo = max(0, b - lb) * block
        hi = min(n, (min(nb - 1, b + la) + 1) * block)
        tot += rows * (hi - lo)
    return tot


def cpu_baseline(inp, cu_host, budget_s: float = 15.0):
    """Time the CPU oracle on a bounded sample of the same workload: query rows
    of the varlen attention, taken in blocks of 128 until ~budget_s has passed.
    Returns the oracle's throughput in TFLOP/s (same 4*D*H per pair count)."""
    import oracle  # the reported CPU baseline only
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    H, D = inp.spec.H, inp.spec.D
    cj, ct, ci, idst = oracle.joint_cu_seqlens(inp.text_mask, inp.img_hw)
    T = int(cj[-1])
    packed = []
    for txt, img in ((inp.q_text, inp.q_img), (inp.k_text, inp.k_img), (inp.v_text, inp.v_img)):
        dst = np.zeros((T, H, D), dtype=np.float32)
        oracle.pack_by_cu_seqlens(txt.float().numpy(), ct, dst_row_offsets=cj[:-1], dst=dst)
        oracle.pack_by_cu_seqlens(img.float().numpy(), ci, dst_row_offsets=idst, dst=dst)
        packed.append(dst)
    q, k, v = packed
    rng = np.random.default_rng(0)
    order = rng.permutation(T)
    flops = 0.0
    rows_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and rows_done < T:
        rows = np.sort(order[rows_done:rows_done + 128])
        oracle.varlen_attention(q, k, v, cj, cj, inp.scale, rows=rows)
        req = np.searchsorted(cj, rows, side="right") - 1
        flops += float(sum(4 * D * H * int(cj[r + 1] - cj[r]) for r in req))
        rows_done += rows.size
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows_done} of {T} query rows x {H} heads of the varlen attention "
                      f"(fp64 NumPy oracle, {dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="joint-16k", choices=["joint-16k", "mixres-4req", "edit-cfg-4seq"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the attention timings at the other full-size workloads (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": args.warmup + args.steps}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import packed_variable_length_varlen_amd as vl
    from packed_variable_length_varlen_amd import workloads as wl

    vl.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    spec = wl.WORKLOADS[args.workload]
    err(f"[bench] generating {args.workload} ({spec.name})")
    inp = wl.make_varlen_inputs(spec, torch.bfloat16)
    H, D = spec.H, spec.D
    R = inp.R
    T = inp.total_tokens
    max_len = inp.max_len

    # inputs resident in HBM before timing
    mask_d = torch.from_numpy(inp.text_mask.astype(np.uint8)).to(dev)
    hw_d = torch.tensor(inp.img_hw, dtype=torch.int32, device=dev).reshape(R, 2)
    slabs = [(t.to(dev), i.to(dev)) for t, i in ((inp.q_text, inp.q_img), (inp.k_text, inp.k_img),
                                                  (inp.v_text, inp.v_img))]
    cu_j = torch.empty(R + 1, dtype=torch.int32, device=dev)
    cu_t = torch.empty(R + 1, dtype=torch.int32, device=dev)
    cu_i = torch.empty(R + 1, dtype=torch.int32, device=dev)
    img_dst = torch.empty(R, dtype=torch.int32, device=dev)
    packed = [torch.empty((T, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    out_txt = torch.empty_like(slabs[0][0])
    out_img = torch.empty_like(slabs[0][1])

    # workspace of the attention call (allocated once): staged V^T and the
    # partial results of the key split of the last round
    workspace = torch.empty(vl.varlen_split_workspace_bytes(T, R, H, D), dtype=torch.uint8, device=dev)

    bl_spec = wl.BLOCK_LOCAL_WORKLOADS["vocoder-dit"]
    bl = wl.make_block_local_inputs(bl_spec, torch.bfloat16)
    bq, bk, bv = bl.q.to(dev), bl.k.to(dev), bl.v.to(dev)
    bouts = [torch.empty_like(bq) for _ in bl_spec.windows]

    # the joint pack of Q, K, V (text and image pieces: six copies) and the
    # unpack of the output (two copies), one launch each
    pack_items = []
    for (txt, img), dst in zip(slabs, packed):
        pack_items += [(txt, cu_t, dst, cu_j[:-1]), (img, cu_i, dst, img_dst)]
    unpack_items = [(out, cu_t, out_txt, cu_j[:-1]), (out, cu_i, out_img, img_dst)]

    stream = torch.cuda.current_stream()
    ev = {"attn": [], "pack": [], "unpack": [], "blocal": []}

    def mark(record):
        if not record:
            return None
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(record: bool):
        vl.joint_cu_seqlens(mask_d, hw_d, outs=(cu_j, cu_t, cu_i, img_dst))
        e0 = mark(record)
        vl.pack_by_cu_seqlens_batched(pack_items)
        e1 = mark(record)
        vl.varlen_attn_fwd_split(packed[0], packed[1], packed[2], cu_j, cu_j, max_len, max_len, inp.scale,
                                 out=out, workspace=workspace)
        e2 = mark(record)
        vl.unpack_by_cu_seqlens_batched(unpack_items)
        e3 = mark(record)
        for (lb, la), o in zip(bl_spec.windows, bouts):
            vl.block_local_attn_fwd(bq, bk, bv, bl_spec.block, lb, la, bl.scale, out=o)
        e4 = mark(record)
        if record:
            ev["pack"].append((e0, e1))
            ev["attn"].append((e1, e2))
            ev["unpack"].append((e2, e3))
            ev["blocal"].append((e3, e4))

    err(f"[bench] T={T} R={R} H={H} D={D}: warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    err(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    attn_ms = ms["attn"]
    row_bytes = H * D * 2
    real_rows = sum(inp.text_len) + sum(inp.img_tokens)
    pack_bytes = 3 * 2 * real_rows * row_bytes
    unpack_bytes = real_rows * row_bytes + R * (wl.TEXT_CAP + inp.img_cap) * row_bytes
    err(f"[bench] pack q/k/v: {ms['pack']*1e3:.1f} us, {pack_bytes/ms['pack']/1e6:.0f} GB/s "
        f"({100*pack_bytes/ms['pack']/1e6/HBM_PEAK_GBS:.1f}% of HBM); unpack out: {ms['unpack']*1e3:.1f} us, "
        f"{unpack_bytes/ms['unpack']/1e6:.0f} GB/s ({100*unpack_bytes/ms['unpack']/1e6/HBM_PEAK_GBS:.1f}% of HBM); "
        f"block-local x4: {ms['blocal']*1e3:.1f} us")

    cu_host = cu_j.cpu().numpy()  # after timing: only for the FLOP count
    pairs = varlen_pairs(cu_host)
    bl_pairs = [block_local_pairs(bl_spec.n, bl_spec.block, lb, la) for lb, la in bl_spec.windows]
    flop_varlen = 4.0 * D * H * pairs
    flop_bl = 4.0 * bl_spec.D * bl_spec.H * sum(bl_pairs)
    step_flop = flop_varlen + flop_bl
    ms_per_step = dt * 1e3 / args.steps
    value = step_flop / (dt / args.steps) / 1e12
    achieved = flop_varlen / (attn_ms * 1e-3) / 1e12
    workload = f"{spec.name}+{bl_spec.name}-4windows"
    traffic = load_traffic(args.workload)

    err(f"[bench] step {ms_per_step:.3f} ms, attention {attn_ms:.3f} ms = {achieved:.1f} TFLOP/s "
        f"({100 * achieved / BF16_PEAK_TFLOPS:.1f}% of bf16 peak); pairs {pairs}")

    # Bandwidth-bound pieces in isolation: median / p10 / p90 of per-call event
    # times, warm (calls back to back) and with the 256 MB last-level cache
    # flushed before each call by reading a 512 MB buffer (a read leaves no
    # dirty lines to be written back during the measured call).  All calls
    # are enqueued before the one synchronisation, so no launch gap is timed.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def call_stats(fn, flushed: bool, reps: int = 30, warm: int = 5):
        for _ in range(warm):
            fn()
        pairs_ev = []
        for _ in range(reps):
            if flushed:
                torch.sum(flush)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            pairs_ev.append((a, b))
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) * 1e3 for a, b in pairs_ev]  # us
        return [float(np.percentile(times, q)) for q in (50, 10, 90)]

    def bw(nbytes, us):
        return round(nbytes / us / 1e3, 1)  # GB/s

    detail = {}
    for name, fn, nbytes in (("pack", lambda: vl.pack_by_cu_seqlens_batched(pack_items), pack_bytes),
                             ("unpack", lambda: vl.unpack_by_cu_seqlens_batched(unpack_items), unpack_bytes)):
        rec = {"bytes": int(nbytes)}
        for tag, fl in (("warm", False), ("flushed", True)):
            med, p10, p90 = call_stats(fn, fl)
            rec[tag] = {"us_median": round(med, 2), "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                        "GB/s": bw(nbytes, med), "pct_of_hbm": round(100 * nbytes / med / 1e3 / HBM_PEAK_GBS, 1)}
        detail[name] = rec
        err(f"[bench] {name}: warm {rec['warm']['pct_of_hbm']}% / flushed {rec['flushed']['pct_of_hbm']}% of HBM")
    # block-local, one call per window type: % of MFMA peak as the metric asks,
    # and % of HBM over its unique bytes (q, k, v read, out written) as the roofline
    bl_bytes = 4 * bl_spec.B * bl_spec.n * bl_spec.H * bl_spec.D * 2
    detail["block_local"] = []
    for (lb, la), o, npairs in zip(bl_spec.windows, bouts, bl_pairs):
        med, p10, p90 = call_stats(lambda: vl.block_local_attn_fwd(bq, bk, bv, bl_spec.block, lb, la, bl.scale, out=o),
                                   True)
        fl = 4.0 * bl_spec.D * bl_spec.H * npairs
        detail["block_local"].append({"look_back": lb, "look_ahead": la, "us_median": round(med, 2),
                                      "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                                      "TFLOP/s": round(fl / med / 1e6, 2),
                                      "pct_of_bf16_peak": round(100 * fl / med / 1e6 / BF16_PEAK_TFLOPS, 3),
                                      "pct_of_hbm_unique_bytes": round(100 * bl_bytes / med / 1e3 / HBM_PEAK_GBS, 1)})
    err(f"[bench] block-local (flushed) us: {[d['us_median'] for d in detail['block_local']]}")
    # block-local at the DiT vocoder's production shape: CFG as batch 2, 4000
    # frames (167 blocks, the last of 16), own-block and one-neighbour windows,
    # in the pages' fp32 and in bf16
    prod_n, prod_b = 4000, 2
    detail["block_local_production"] = []
    for pdt in (torch.float32, torch.bfloat16):
        pin = wl.make_block_local_inputs(bl_spec, pdt, n=prod_n, B=prod_b, seed=prod_n)
        pq, pk, pv = pin.q.to(dev), pin.k.to(dev), pin.v.to(dev)
        po = torch.empty_like(pq)
        fn = vl.block_local_attn_fwd_f32 if pdt == torch.float32 else vl.block_local_attn_fwd
        pbytes = 4 * prod_b * prod_n * bl_spec.H * bl_spec.D * pq.element_size()
        for lb, la in ((0, 0), (1, 0), (0, 1)):
            med, p10, p90 = call_stats(lambda: fn(pq, pk, pv, bl_spec.block, lb, la, pin.scale, out=po), True)
            fl = 4.0 * bl_spec.D * bl_spec.H * prod_b * block_local_pairs(prod_n, bl_spec.block, lb, la)
            detail["block_local_production"].append({
                "dtype": "f32" if pdt == torch.float32 else "bf16", "B": prod_b, "n": prod_n,
                "look_back": lb, "look_ahead": la, "us_median": round(med, 2), "us_p10": round(p10, 2),
                "us_p90": round(p90, 2), "TFLOP/s": round(fl / med / 1e6, 2),
                "pct_of_hbm_unique_bytes": round(100 * pbytes / med / 1e3 / HBM_PEAK_GBS, 1)})
        del pq, pk, pv, po, pin
    err(f"[bench] block-local production (flushed) us: "
        f"{[(d['dtype'], d['look_back'], d['look_ahead'], d['us_median']) for d in detail['block_local_production']]}")

    # The attention call alone at the other full-size workloads (same launch,
    # per-call HIP events, median of 10): their token layout from the recipe's
    # text-length draws, Q/K/V N(0,1) drawn on the device (seeded).
    detail["attention_other_workloads"] = []
    for other in ("joint-16k", "mixres-4req", "edit-cfg-4seq"):
        if other == args.workload or args.no_other_workloads:
            continue
        ospec = wl.WORKLOADS[other]
        lens = wl.varlen_lengths(ospec)
        oT = sum(lens)
        ocu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(ospec.seed)
        oq, ok_, ov = (torch.randn((oT, ospec.H, ospec.D), generator=gen, device=dev).to(torch.bfloat16)
                       for _ in range(3))
        oout = torch.empty_like(oq)
        ows = torch.empty(vl.varlen_split_workspace_bytes(oT, len(lens), ospec.H, ospec.D), dtype=torch.uint8,
                          device=dev)
        ofn = lambda: vl.varlen_attn_fwd_split(oq, ok_, ov, ocu, ocu, max(lens), max(lens), wl.softmax_scale(ospec.D),
                                               out=oout, workspace=ows)
        for _ in range(3):
            ofn()
        oev = []
        for _ in range(10):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            ofn()
            b.record(stream)
            oev.append((a, b))
        torch.cuda.synchronize()
        oms = float(np.median([a.elapsed_time(b) for a, b in oev]))
        oflop = 4.0 * ospec.D * ospec.H * sum(x * x for x in lens)
        otf = oflop / (oms * 1e-3) / 1e12
        detail["attention_other_workloads"].append({
            "workload": ospec.name, "total_tokens": oT, "requests": len(lens), "ms_median": round(oms, 4),
            "TFLOP/s": round(otf, 2), "pct_of_bf16_peak": round(100 * otf / BF16_PEAK_TFLOPS, 2)})
        err(f"[bench] attention at {other}: {oms:.3f} ms = {otf:.1f} TFLOP/s ({100 * otf / BF16_PEAK_TFLOPS:.1f}%)")
        if other == "edit-cfg-4seq":
            # the per-request CFG combine fused into the unpack of this output:
            # sequences [r1+, r1-, r2+, r2-], image rows after each text piece,
            # true CFG scale 4.0; reads two rows and writes one per output row
            img = [int(h) * int(w) for h, w in ospec.img_grids]
            ocu_h = np.concatenate([[0], np.cumsum(lens)])
            nreq = len(lens) // 2
            pos = torch.tensor([ocu_h[2 * r] + lens[2 * r] - img[2 * r] for r in range(nreq)], dtype=torch.int32,
                               device=dev)
            neg = torch.tensor([ocu_h[2 * r + 1] + lens[2 * r + 1] - img[2 * r + 1] for r in range(nreq)],
                               dtype=torch.int32, device=dev)
            seg = torch.tensor(np.concatenate([[0], np.cumsum(img[0::2])]), dtype=torch.int32, device=dev)
            cfg_s = torch.full((nreq,), 4.0, dtype=torch.float32, device=dev)
            cdst = torch.empty((nreq, max(img[0::2]), ospec.H, ospec.D), dtype=torch.bfloat16, device=dev)
            cfn = lambda: vl.unpack_cfg_combine(oout, seg, pos, neg, cfg_s, cdst)
            for _ in range(3):
                cfn()
            cev = []
            for _ in range(10):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                cfn()
                b.record(stream)
                cev.append((a, b))
            torch.cuda.synchronize()
            cus = float(np.median([a.elapsed_time(b) for a, b in cev])) * 1e3
            cbytes = 3 * sum(img[0::2]) * ospec.H * ospec.D * 2
            detail["cfg_combine_unpack"] = {"workload": ospec.name, "bytes": int(cbytes), "us_median": round(cus, 2),
                                            "GB/s": round(cbytes / cus / 1e3, 1),
                                            "pct_of_hbm": round(100 * cbytes / cus / 1e3 / HBM_PEAK_GBS, 1)}
            err(f"[bench] CFG combine + unpack at {other}: {cus:.1f} us, "
                f"{100 * cbytes / cus / 1e3 / HBM_PEAK_GBS:.1f}% of HBM")
            del cdst
        del oq, ok_, ov, oout, ows

    cpu = None
    if not args.no_cpu_baseline:
        err("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(inp, cu_host)
        err(f"[bench] oracle {cpu['value']} TFLOP/s on {cpu['cores']} threads")

    line = {
        "metric": "varlen attention fwd TFLOP/s (in-request pairs) and % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "total_tokens": T,
            "requests": R,
            "heads": H,
            "head_dim": D,
            "in_request_pairs": pairs,
            "block_local_pairs": bl_pairs,
            "pct_of_bf16_peak_step": round(100 * value / BF16_PEAK_TFLOPS, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "vt_transpose_kernel<128> + attn_bf16_pp_kernel<128, 64, true> + "
                      "split_merge_kernel<128, 256> (varlen_attn_fwd_split)",
            "kernel_ms": round(attn_ms, 4),
        },
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
