"""Benchmark of the packed varlen attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. boundaries (cu_seqlens) from the real text mask and the image grids,
  2. joint text+image pack of Q and K into flat [T, H, D] (one launch) and of
     V straight into the transposed layout the attention kernel reads (V^T in
     the attention call's workspace; the pack and the V^T staging in one pass),
  3. flat varlen attention on that V^T (bf16 MFMA, fp32 accumulation; the
     last, partial round of work-groups cut along the keys and merged),
  4. unpack of the output back to the per-request text / image layout (one
     launch),
  5. block-local attention of the vocoder-DiT shape (n=2003, 24-frame blocks,
     H=16, D=64) for each of the four window types (own block, one back,
     one ahead, both).
The default workload is the largest single-GPU one: the edit-style batch of
four CFG sequences [r1+, r1-, r2+, r2-], each 32,768 image tokens (noise +
source latents) after its text (about 131.5k packed tokens, H=24, D=128,
bf16).  Every input is drawn by the seeded NumPy recipe of workloads.py (the
same bits the parity tests check) and is resident in HBM before timing.

value = algorithmic FLOP of one step / step time, where the FLOP count is
4*D*H per in-request (query, key) pair (the varlen pairs plus the in-window
block-local pairs); work the kernels avoid is never counted.

The `detail` object holds the same step at the two other full-size workloads,
the bandwidth-bound pieces alone (the flat pack of all six Q/K/V pieces and the
unpack; warm and with the last-level cache flushed),
each beside the runtime's own device-to-device memcpy of the same bytes timed
the same way (the practical ceiling at that size), the block-local calls per window and weighted by the DiT's layer mix, the
production block-local shape, the fused CFG combine, and the launch floor.
The CPU baseline is the fp64 oracle run by a process pool (one BLAS thread per
worker) on a bounded sample of the headline workload's (request, head, query
rows) units; its rate is extrapolated to the whole workload.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import re
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BOX_CPU_SHARE = 16          # worker processes at most (the CPU share of one GPU)


def err(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the attention sources (attn.hip, vl_device.h) with comments and
    blank lines removed: a change of code changes it, a change of comments
    does not."""
    h = hashlib.sha256()
    for name in ("attn.hip", "vl_device.h"):
        with open(os.path.join(HERE, "packed_variable_length_varlen_amd", "csrc", name)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = re.sub(r"//.*$", "", line).rstrip()
            if code.strip():
                h.update((code + "\n").encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per attention call from committed rocprofv3 --pmc counters
    (FETCH_SIZE + WRITE_SIZE of its kernels, scaled by a copy-kernel factor);
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


# ------------------------------------------------------------------ CPU baseline (oracle, process pool)

# Packed fp64 q/k/v and boundaries of the workload the pool samples.  Set in
# the parent before the pool is forked (before any GPU use), so the workers
# share them copy-on-write and receive only indices.
_ORACLE = {}


def _oracle_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_task(task):
    """One unit of the sample: query rows [a, b) of request r, head h, against
    the request's keys (rows are independent, so a subset is exact)."""
    import oracle
    r, h, a, b = task
    d = _ORACLE
    cu = d["cu"]
    k0, k1 = int(cu[r]), int(cu[r + 1])
    q = d["q"][int(cu[r]) + a:int(cu[r]) + b, h:h + 1]
    k = d["k"][k0:k1, h:h + 1]
    v = d["v"][k0:k1, h:h + 1]
    oracle.varlen_attention(q, k, v, [0, b - a], [0, k1 - k0], d["scale"])
    return 4.0 * q.shape[2] * (b - a) * (k1 - k0)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def prepare_oracle_pool(inp):
    """Pack the workload for the oracle (fp64) and fork the worker pool."""
    import oracle
    H, D = inp.spec.H, inp.spec.D
    cj, ct, ci, idst = oracle.joint_cu_seqlens(inp.text_mask, inp.img_hw)
    T = int(cj[-1])
    packed = []
    for txt, img in ((inp.q_text, inp.q_img), (inp.k_text, inp.k_img), (inp.v_text, inp.v_img)):
        dst = np.zeros((T, H, D), dtype=np.float32)
        oracle.pack_by_cu_seqlens(txt.float().numpy(), ct, dst_row_offsets=cj[:-1], dst=dst)
        oracle.pack_by_cu_seqlens(img.float().numpy(), ci, dst_row_offsets=idst, dst=dst)
        packed.append(dst.astype(np.float64))
        del dst
    _ORACLE.update(q=packed[0], k=packed[1], v=packed[2], cu=cj, scale=inp.scale, H=H, D=D)
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    workers = max(1, min(BOX_CPU_SHARE, share))
    pool = mp.get_context("fork").Pool(workers, initializer=_oracle_worker_init)
    return pool, workers, share


def run_cpu_baseline(pool, workers: int, share: int, budget_s: float):
    """Time the oracle on a bounded sample: (request, head, 256 query rows)
    units dealt round-robin over requests and heads, submitted until about
    budget_s of wall time has passed; rate = their FLOP / wall time."""
    d = _ORACLE
    cu = [int(x) for x in d["cu"]]
    R, H, D = len(cu) - 1, d["H"], d["D"]
    rng = np.random.default_rng(0)
    units = []
    for i in range(R * H * 64):
        r, h = (i // H) % R, i % H
        L = cu[r + 1] - cu[r]
        if L == 0:
            continue
        a = int(rng.integers(0, max(1, L - 256) + 1))
        units.append((r, h, a, min(L, a + 256)))
    t0 = time.perf_counter()
    pending, flops, done, it = [], 0.0, 0, iter(units)
    for _ in range(2 * workers):
        pending.append(pool.apply_async(_oracle_task, (next(it),)))
    while pending:
        res = pending.pop(0)
        flops += res.get()
        done += 1
        if time.perf_counter() - t0 < budget_s:
            nxt = next(it, None)
            if nxt is not None:
                pending.append(pool.apply_async(_oracle_task, (nxt,)))
    dt = time.perf_counter() - t0
    pool.close()
    pool.join()
    total_flops = 4.0 * D * H * varlen_pairs(cu)
    rate = flops / dt
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": f"{done} units of (request, head, <=256 query rows) of the varlen attention, "
                      f"{flops / 1e12:.3f} TFLOP in {dt:.1f} s on {workers} worker processes "
                      f"(fp64 NumPy oracle, one BLAS thread each)",
            "nproc": os.cpu_count(), "cpu_share": share, "cpu_model": cpu_model(),
            "full_workload_oracle_s_extrapolated": round(total_flops / rate, 1)}


# ------------------------------------------------------------------ GPU timing


class VarlenStep:
    """The varlen part of the step for one workload, inputs resident in HBM."""

    def __init__(self, vl, wl, inp, dev):
        self.vl, self.inp = vl, inp
        H, D = inp.spec.H, inp.spec.D
        R, T = inp.R, inp.total_tokens
        self.H, self.D, self.R, self.T = H, D, R, T
        self.max_len = inp.max_len
        self.mask_d = torch.from_numpy(inp.text_mask.astype(np.uint8)).to(dev)
        self.hw_d = torch.tensor(inp.img_hw, dtype=torch.int32, device=dev).reshape(R, 2)
        self.slabs = [(t.to(dev), i.to(dev)) for t, i in ((inp.q_text, inp.q_img), (inp.k_text, inp.k_img),
                                                          (inp.v_text, inp.v_img))]
        self.cu_j = torch.empty(R + 1, dtype=torch.int32, device=dev)
        self.cu_t = torch.empty(R + 1, dtype=torch.int32, device=dev)
        self.cu_i = torch.empty(R + 1, dtype=torch.int32, device=dev)
        self.img_dst = torch.empty(R, dtype=torch.int32, device=dev)
        self.packed = [torch.empty((T, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        self.out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        self.out_txt = torch.empty_like(self.slabs[0][0])
        self.out_img = torch.empty_like(self.slabs[0][1])
        # workspace of the attention call (allocated once): V^T (packed there
        # straight from the V pieces), the partial results of the key split of
        # the last round and the counters of the chiplet work queues
        self.workspace = torch.empty(vl.varlen_split_workspace_bytes(T, R, H, D), dtype=torch.uint8, device=dev)
        # the flat pack of all six pieces (the pack primitive, timed alone) ...
        self.pack_items = []
        for (txt, img), dst in zip(self.slabs, self.packed):
            self.pack_items += [(txt, self.cu_t, dst, self.cu_j[:-1]), (img, self.cu_i, dst, self.img_dst)]
        # ... and the step's: Q and K flat, V straight into V^T
        self.pack_qk_items = self.pack_items[:4]
        self.pack_v_items = [(self.slabs[2][0], self.cu_t, self.cu_j[:-1]), (self.slabs[2][1], self.cu_i, self.img_dst)]
        self.unpack_items = [(self.out, self.cu_t, self.out_txt, self.cu_j[:-1]),
                             (self.out, self.cu_i, self.out_img, self.img_dst)]
        row_bytes = H * D * 2
        real_rows = sum(inp.text_len) + sum(inp.img_tokens)
        self.pack_bytes = 3 * 2 * real_rows * row_bytes
        self.unpack_bytes = real_rows * row_bytes + R * (wl.TEXT_CAP + inp.img_cap) * row_bytes

    def cu(self):
        self.vl.joint_cu_seqlens(self.mask_d, self.hw_d, outs=(self.cu_j, self.cu_t, self.cu_i, self.img_dst))

    def pack_flat(self):
        self.vl.pack_by_cu_seqlens_batched(self.pack_items)

    def pack(self):
        self.vl.pack_by_cu_seqlens_batched(self.pack_qk_items)
        self.vl.pack_v_transposed(self.pack_v_items, self.cu_j, self.T, self.workspace)

    def attention_split(self):
        q, k, v = self.packed
        self.vl.varlen_attn_fwd_split(q, k, v, self.cu_j, self.cu_j, self.max_len, self.max_len, self.inp.scale,
                                      out=self.out, workspace=self.workspace)

    def attention(self):
        q, k, _ = self.packed
        self.vl.varlen_attn_fwd_vt(q, k, self.cu_j, self.cu_j, self.max_len, self.max_len, self.workspace,
                                   self.inp.scale, out=self.out)

    def unpack(self):
        self.vl.unpack_by_cu_seqlens_batched(self.unpack_items)

    def pairs(self) -> int:
        return varlen_pairs(self.cu_j.cpu().numpy())


def new_event(stream):
    e = torch.cuda.Event(enable_timing=True)
    e.record(stream)
    return e


def time_steps(stream, parts, steps: int, warmup: int):
    """Runs `steps` steps of the callables in `parts` (name, fn or None =
    untimed) after `warmup` untimed steps.  Returns (wall seconds of the timed
    steps, {name: mean ms per step from the HIP events around it})."""
    def step(record):
        evs = []
        for name, fn in parts:
            e0 = new_event(stream) if record and name else None
            fn()
            if e0 is not None:
                evs.append((name, e0, new_event(stream)))
        return evs

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = [step(True) for _ in range(steps)]
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = {}
    for evs in recs:
        for name, a, b in evs:
            ms.setdefault(name, []).append(a.elapsed_time(b))
    return dt, {k: float(np.mean(v)) for k, v in ms.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="edit-cfg-4seq", choices=["joint-16k", "mixres-4req", "edit-cfg-4seq"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle sampling")
    ap.add_argument("--no-detail", action="store_true",
                    help="only the timed steps (profiling runs: one workload's launches per trace)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the steps at the other full-size workloads")
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

    # ---- inputs, drawn on the host by the seeded recipe (before any GPU use)
    spec = wl.WORKLOADS[args.workload]
    err(f"[bench] generating {args.workload} ({spec.name})")
    inp = wl.make_varlen_inputs(spec, torch.bfloat16)
    others = []
    if not (args.no_detail or args.no_other_workloads):
        for name in ("joint-16k", "mixres-4req", "edit-cfg-4seq"):
            if name != args.workload:
                err(f"[bench] generating {name}")
                others.append((name, wl.make_varlen_inputs(wl.WORKLOADS[name], torch.bfloat16)))
    bl_spec = wl.BLOCK_LOCAL_WORKLOADS["vocoder-dit"]
    bl = wl.make_block_local_inputs(bl_spec, torch.bfloat16)
    pool = None
    if not args.no_cpu_baseline:
        err("[bench] packing the workload for the CPU oracle and forking its worker pool")
        pool, workers, share = prepare_oracle_pool(inp)

    # ---- GPU
    vl.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    main_step = VarlenStep(vl, wl, inp, dev)
    H, D, R, T = main_step.H, main_step.D, main_step.R, main_step.T
    bq, bk, bv = bl.q.to(dev), bl.k.to(dev), bl.v.to(dev)
    bouts = [torch.empty_like(bq) for _ in bl_spec.windows]

    def block_local_all():
        for (lb, la), o in zip(bl_spec.windows, bouts):
            vl.block_local_attn_fwd(bq, bk, bv, bl_spec.block, lb, la, bl.scale, out=o)

    parts = [(None, main_step.cu), ("pack", main_step.pack), ("attn", main_step.attention),
             ("unpack", main_step.unpack), ("blocal", block_local_all)]
    err(f"[bench] T={T} R={R} H={H} D={D}: warmup {args.warmup}, timing {args.steps} steps")
    dt, ms = time_steps(stream, parts, args.steps, args.warmup)
    pairs = main_step.pairs()
    bl_pairs = [block_local_pairs(bl_spec.n, bl_spec.block, lb, la) for lb, la in bl_spec.windows]
    flop_varlen = 4.0 * D * H * pairs
    flop_bl = 4.0 * bl_spec.D * bl_spec.H * sum(bl_pairs)
    ms_per_step = dt * 1e3 / args.steps
    value = (flop_varlen + flop_bl) / (dt / args.steps) / 1e12
    attn_ms = ms["attn"]
    achieved = flop_varlen / (attn_ms * 1e-3) / 1e12
    err(f"[bench] step {ms_per_step:.3f} ms = {value:.1f} TFLOP/s; attention {attn_ms:.3f} ms = "
        f"{achieved:.1f} TFLOP/s ({100 * achieved / BF16_PEAK_TFLOPS:.1f}% of bf16 peak); "
        f"pack {ms['pack'] * 1e3:.1f} us ({100 * main_step.pack_bytes / ms['pack'] / 1e6 / HBM_PEAK_GBS:.1f}% of HBM), "
        f"unpack {ms['unpack'] * 1e3:.1f} us "
        f"({100 * main_step.unpack_bytes / ms['unpack'] / 1e6 / HBM_PEAK_GBS:.1f}% of HBM), "
        f"block-local x4 {ms['blocal'] * 1e3:.1f} us")

    def step_record(s: VarlenStep, ms_, step_ms, pairs_):
        fl = 4.0 * s.D * s.H * pairs_
        return {"workload": s.inp.spec.name, "total_tokens": s.T, "requests": s.R, "in_request_pairs": pairs_,
                "step_ms": round(step_ms, 4),
                "attention_ms": round(ms_["attn"], 4), "attention_TFLOP/s": round(fl / ms_["attn"] / 1e9, 2),
                "attention_pct_of_bf16_peak": round(100 * fl / ms_["attn"] / 1e9 / BF16_PEAK_TFLOPS, 2),
                "pack_us": round(ms_["pack"] * 1e3, 2),
                "pack_pct_of_hbm": round(100 * s.pack_bytes / ms_["pack"] / 1e6 / HBM_PEAK_GBS, 1),
                "unpack_us": round(ms_["unpack"] * 1e3, 2),
                "unpack_pct_of_hbm": round(100 * s.unpack_bytes / ms_["unpack"] / 1e6 / HBM_PEAK_GBS, 1)}

    detail = {"steps": [step_record(main_step, ms, ms_per_step, pairs)]}
    traffic = load_traffic(args.workload)

    if not args.no_detail:
        # the same step with the flat pack of all six pieces and the V^T
        # staging inside the attention call (varlen_attn_fwd_split): what
        # packing V straight into V^T saves, on this machine, the two forms
        # timed in alternating rounds so that clock drift hits both alike
        unfused = [(None, main_step.cu), ("pack", main_step.pack_flat), ("attn", main_step.attention_split),
                   ("unpack", main_step.unpack), ("blocal", block_local_all)]
        per = max(2, args.steps // 4)
        acc = {"fused": [], "unfused": []}
        for _ in range(4):
            for tag, pp_ in (("fused", parts), ("unfused", unfused)):
                rdt, rms = time_steps(stream, pp_, per, 1)
                acc[tag].append((rdt * 1e3 / per, rms["pack"] * 1e3, rms["attn"]))
        fused_ms = float(np.median([x[0] for x in acc["fused"]]))
        unf = [float(np.median([x[i] for x in acc["unfused"]])) for i in range(3)]
        detail["step_flat_pack_and_staging_call"] = {
            "rounds": 4, "steps_per_round": per, "step_ms": round(unf[0], 4), "pack_us": round(unf[1], 2),
            "attention_ms": round(unf[2], 4),
            "attention_pct_of_bf16_peak": round(100 * flop_varlen / (unf[2] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
            "fused_step_ms_same_rounds": round(fused_ms, 4),
            "step_ms_saved_by_the_fused_pack": round(unf[0] - fused_ms, 4)}
        err(f"[bench] same step with the flat pack and the staging call: "
            f"{detail['step_flat_pack_and_staging_call']['step_ms']} ms "
            f"(fused V^T pack saves {detail['step_flat_pack_and_staging_call']['step_ms_saved_by_the_fused_pack']} ms)")
        flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)

        def call_stats(fn, flushed: bool, reps: int = 50, warm: int = 10):
            """median / p10 / p90 of per-call HIP event times (us); all calls are
            enqueued before one synchronisation, so no launch gap is timed;
            flushed: a 512 MB buffer is read before each call, so the 256 MB
            last-level cache holds none of the call's data and no dirty lines."""
            for _ in range(warm):
                fn()
            evs = []
            for _ in range(reps):
                if flushed:
                    torch.sum(flush)
                a = new_event(stream)
                fn()
                evs.append((a, new_event(stream)))
            torch.cuda.synchronize()
            t = [a.elapsed_time(b) * 1e3 for a, b in evs]
            return [float(np.percentile(t, q)) for q in (50, 10, 90)]

        def bw_record(nbytes, fn):
            rec = {"bytes": int(nbytes)}
            for tag, fl in (("warm", False), ("flushed", True)):
                med, p10, p90 = call_stats(fn, fl)
                rec[tag] = {"us_median": round(med, 2), "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                            "GB/s": round(nbytes / med / 1e3, 1),
                            "pct_of_hbm": round(100 * nbytes / med / 1e3 / HBM_PEAK_GBS, 1)}
            return rec

        # the other full-size workloads: the same step (without the block-local
        # calls), then their pack / unpack alone
        steps_all = [main_step]
        for name, oinp in others:
            err(f"[bench] step at {name}")
            s = VarlenStep(vl, wl, oinp, dev)
            odt, oms = time_steps(stream, [(None, s.cu), ("pack", s.pack), ("attn", s.attention),
                                           ("unpack", s.unpack)], max(10, args.steps // 2), 3)
            detail["steps"].append(step_record(s, oms, odt * 1e3 / max(10, args.steps // 2), s.pairs()))
            err(f"[bench]   attention {oms['attn']:.3f} ms = {detail['steps'][-1]['attention_TFLOP/s']} TFLOP/s "
                f"({detail['steps'][-1]['attention_pct_of_bf16_peak']}%)")
            steps_all.append(s)

        def pipelined_flushed(fns, reps: int = 10):
            """Per-call time of len(fns) calls on distinct buffers, queued back
            to back after one flush (each call's data is cold: the others'
            exceed the last-level cache); the launch gaps overlap the previous
            call as in a pipeline.  Median over reps (us)."""
            for f in fns:
                f()
            evs = []
            for _ in range(reps):
                torch.sum(flush)
                a = new_event(stream)
                for f in fns:
                    f()
                evs.append((a, new_event(stream)))
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b) * 1e3 / len(fns) for a, b in evs]))

        def memcpy_reference(nbytes, pipelined: bool = True):
            """The runtime's own device-to-device copy (hipMemcpyAsync through
            torch's copy_) moving the same bytes (half read, half written),
            timed the same ways: the practical ceiling for a copy of this size."""
            n = int(nbytes) // 4 * 2
            bufs = [(torch.empty(n, dtype=torch.uint8, device=dev).fill_(1), torch.empty(n, dtype=torch.uint8,
                                                                                        device=dev))
                    for _ in range(3 if pipelined else 1)]
            fns = [(lambda a=a, b=b: b.copy_(a)) for a, b in bufs]
            rec = {}
            for tag, fl in (("warm", False), ("flushed", True)):
                med = call_stats(fns[0], fl)[0]
                rec[tag] = {"us_median": round(med, 2), "pct_of_hbm": round(100 * 2 * n / med / 1e3 / HBM_PEAK_GBS, 1)}
            if pipelined:
                us = pipelined_flushed(fns)
                rec["pipelined_flushed"] = {"us_per_call": round(us, 2),
                                            "pct_of_hbm": round(100 * 2 * n / us / 1e3 / HBM_PEAK_GBS, 1)}
            del bufs, fns
            return rec

        detail["copies_alone"] = []
        for s in steps_all:
            # two more buffer sets of the same copies for the pipelined figure
            extra = []
            for _ in range(2):
                slabs = [(t.clone(), i.clone()) for t, i in s.slabs]
                packed = [torch.empty_like(t) for t in s.packed]
                pitems = []
                for (txt, img), dst in zip(slabs, packed):
                    pitems += [(txt, s.cu_t, dst, s.cu_j[:-1]), (img, s.cu_i, dst, s.img_dst)]
                out = s.out.clone()
                uitems = [(out, s.cu_t, torch.empty_like(s.out_txt), s.cu_j[:-1]),
                          (out, s.cu_i, torch.empty_like(s.out_img), s.img_dst)]
                extra.append((pitems, uitems))
            for what, fn, nbytes in (("pack", s.pack_flat, s.pack_bytes), ("unpack", s.unpack, s.unpack_bytes)):
                rec = {"workload": s.inp.spec.name, "copy": what, **bw_record(nbytes, fn)}
                k = 0 if what == "pack" else 1
                call = vl.pack_by_cu_seqlens_batched if what == "pack" else vl.unpack_by_cu_seqlens_batched
                fns = [fn] + [(lambda it=e[k], c=call: c(it)) for e in extra]
                us = pipelined_flushed(fns)
                rec["pipelined_flushed"] = {"calls": len(fns), "us_per_call": round(us, 2),
                                            "GB/s": round(nbytes / us / 1e3, 1),
                                            "pct_of_hbm": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1)}
                rec["memcpy_same_bytes"] = memcpy_reference(nbytes)
                detail["copies_alone"].append(rec)
                m = rec["memcpy_same_bytes"]
                err(f"[bench] {what} at {s.inp.spec.name}: warm {rec['warm']['pct_of_hbm']}% / "
                    f"flushed {rec['flushed']['pct_of_hbm']}% / pipelined flushed "
                    f"{rec['pipelined_flushed']['pct_of_hbm']}% of HBM (memcpy of the same bytes: "
                    f"{m['warm']['pct_of_hbm']} / {m['flushed']['pct_of_hbm']} / "
                    f"{m['pipelined_flushed']['pct_of_hbm']}%)")
            del extra
            torch.cuda.empty_cache()

        # the per-request CFG combine fused into the unpack at the edit shape:
        # sequences [r1+, r1-, r2+, r2-], image rows after each text piece,
        # true CFG scale 4.0; reads two rows and writes one per output row
        edit = next((s for s in steps_all if s.inp.spec.name == wl.WORKLOADS["edit-cfg-4seq"].name), None)
        if edit is not None:
            ei = edit.inp
            cu_h = edit.cu_j.cpu().numpy()
            nreq = ei.R // 2
            img = ei.img_tokens
            pos = torch.tensor([cu_h[2 * r] + ei.text_len[2 * r] for r in range(nreq)], dtype=torch.int32, device=dev)
            neg = torch.tensor([cu_h[2 * r + 1] + ei.text_len[2 * r + 1] for r in range(nreq)], dtype=torch.int32,
                               device=dev)
            seg = torch.tensor(np.concatenate([[0], np.cumsum(img[0::2])]), dtype=torch.int32, device=dev)
            cfg_s = torch.full((nreq,), 4.0, dtype=torch.float32, device=dev)
            cdst = torch.empty((nreq, max(img[0::2]), H, D), dtype=torch.bfloat16, device=dev)
            cbytes = 3 * sum(img[0::2]) * ei.spec.H * ei.spec.D * 2
            detail["cfg_combine_unpack"] = {"workload": ei.spec.name, **bw_record(
                cbytes, lambda: vl.unpack_cfg_combine(edit.out, seg, pos, neg, cfg_s, cdst)),
                "memcpy_same_bytes": memcpy_reference(cbytes, pipelined=False)}
            err(f"[bench] CFG combine + unpack: warm {detail['cfg_combine_unpack']['warm']['pct_of_hbm']}% / "
                f"flushed {detail['cfg_combine_unpack']['flushed']['pct_of_hbm']}% of HBM")
            del cdst
        for s in steps_all[1:]:
            del s.packed, s.slabs, s.out, s.out_img, s.workspace
        torch.cuda.empty_cache()

        # block-local, one call per window type (cache flushed): % of MFMA
        # peak as the metric asks, and % of HBM over its unique bytes (q, k, v
        # read, out written) as the roofline
        bl_bytes = 4 * bl_spec.B * bl_spec.n * bl_spec.H * bl_spec.D * 2
        detail["block_local"] = []
        win_us = {}
        for (lb, la), o, npairs in zip(bl_spec.windows, bouts, bl_pairs):
            med, p10, p90 = call_stats(
                lambda: vl.block_local_attn_fwd(bq, bk, bv, bl_spec.block, lb, la, bl.scale, out=o), True)
            fl = 4.0 * bl_spec.D * bl_spec.H * npairs
            win_us[(lb, la)] = (med, fl)
            detail["block_local"].append({"look_back": lb, "look_ahead": la, "us_median": round(med, 2),
                                          "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                                          "TFLOP/s": round(fl / med / 1e6, 2),
                                          "pct_of_bf16_peak": round(100 * fl / med / 1e6 / BF16_PEAK_TFLOPS, 3),
                                          "pct_of_hbm_unique_bytes": round(100 * bl_bytes / med / 1e3 / HBM_PEAK_GBS,
                                                                           1)})
        detail["block_local_memcpy_same_bytes"] = memcpy_reference(bl_bytes, pipelined=False)
        err(f"[bench] block-local (flushed) us: {[d['us_median'] for d in detail['block_local']]} "
            f"(memcpy of the same bytes, flushed: {detail['block_local_memcpy_same_bytes']['flushed']['us_median']})")
        # the DiT's layer mix per forward: the configuration's 22 own-block
        # layers + 3 layers with a block back and ahead, and the pages' 19
        # own-block + 3 one-neighbour layers (one back / one ahead averaged)
        own = win_us[(0, 0)]
        one = ((win_us[(1, 0)][0] + win_us[(0, 1)][0]) / 2, (win_us[(1, 0)][1] + win_us[(0, 1)][1]) / 2)
        both = win_us[(1, 1)]
        detail["block_local_layer_mix"] = []
        for name, mix in (("config 22 own-block + 3 both-neighbour layers", [(22, own), (3, both)]),
                          ("pages 19 own-block + 3 one-neighbour layers", [(19, own), (3, one)])):
            us = sum(c * t for c, (t, _) in mix)
            fl = sum(c * f for c, (_, f) in mix)
            detail["block_local_layer_mix"].append({"mix": name, "layers": sum(c for c, _ in mix),
                                                    "us_per_forward": round(us, 2),
                                                    "TFLOP/s": round(fl / us / 1e6, 2)})
        # the same mixes as a forward issues them: every layer's call queued
        # back to back on its own q/k/v/out (each layer has its own
        # activations) after one flush, so launch gaps overlap the previous
        # call; the windowed layers spread evenly over the stack.  The pages'
        # one-neighbour layers: all one back, then all one ahead, averaged.
        n_layers = 25
        lay = [tuple(t.clone() for t in (bq, bk, bv)) + (torch.empty_like(bq),) for _ in range(n_layers)]

        def forward_us(windows, reps: int = 10):
            calls = [(lambda x=lay[i], w=windows[i]: vl.block_local_attn_fwd(
                x[0], x[1], x[2], bl_spec.block, w[0], w[1], bl.scale, out=x[3])) for i in range(len(windows))]
            return pipelined_flushed(calls, reps) * len(calls)

        def spread(n, special, w_special):
            pos = {round((j + 1) * n / (len(special) + 1)) - 1 for j in range(len(special))}
            it = iter(w_special)
            return [next(it) if i in pos else (0, 0) for i in range(n)]

        fl_of = {w: f for w, (_, f) in win_us.items()}
        detail["block_local_layer_mix_pipelined"] = []
        for name, variants in (
                ("config 22 own-block + 3 both-neighbour layers", [spread(25, [0] * 3, [(1, 1)] * 3)]),
                ("pages 19 own-block + 3 one-neighbour layers", [spread(22, [0] * 3, [(1, 0)] * 3),
                                                                 spread(22, [0] * 3, [(0, 1)] * 3)])):
            us = float(np.mean([forward_us(v) for v in variants]))
            fl = float(np.mean([sum(fl_of[w] for w in v) for v in variants]))
            detail["block_local_layer_mix_pipelined"].append({
                "mix": name, "layers": len(variants[0]), "us_per_forward": round(us, 2),
                "us_per_layer": round(us / len(variants[0]), 2), "TFLOP/s": round(fl / us / 1e6, 2)})
        err(f"[bench] block-local layer mix, queued as a forward: "
            f"{[(d['layers'], d['us_per_forward'], d['us_per_layer']) for d in detail['block_local_layer_mix_pipelined']]}")
        del lay
        # block-local at the DiT vocoder's production shape: CFG as batch 2,
        # 4000 frames (167 blocks, the last of 16), own-block and one-neighbour
        # windows, in the pages' fp32 and in bf16
        prod_n, prod_b = 4000, 2
        detail["block_local_production"] = []
        detail["block_local_production_memcpy_same_bytes"] = {}
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
            detail["block_local_production_memcpy_same_bytes"]["f32" if pdt == torch.float32 else "bf16"] = \
                memcpy_reference(pbytes, pipelined=False)
        err(f"[bench] block-local production (flushed) us: "
            f"{[(d['dtype'], d['look_back'], d['look_ahead'], d['us_median']) for d in detail['block_local_production']]}"
            f" (memcpy of the same bytes, flushed: "
            f"{[(k, m['flushed']['us_median']) for k, m in detail['block_local_production_memcpy_same_bytes'].items()]})")
        # launch floor on this stream: an event pair with nothing between, and
        # one around a one-element kernel
        one_el = torch.zeros(1, device=dev)
        detail["launch_floor_us"] = {"empty_event_pair": round(call_stats(lambda: None, False)[0], 2),
                                     "one_element_kernel": round(call_stats(lambda: one_el.add_(1.0), False)[0], 2)}
        err(f"[bench] launch floor: {detail['launch_floor_us']}")

    cpu = None
    if pool is not None:
        err(f"[bench] timing the CPU oracle on a bounded sample ({workers} worker processes)")
        cpu = run_cpu_baseline(pool, workers, share, args.cpu_budget)
        err(f"[bench] oracle {cpu['value']} TFLOP/s; whole workload ~{cpu['full_workload_oracle_s_extrapolated']} s")

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
        "data": "synthetic (seeded NumPy N(0,1) recipe at the pages' token shapes)",
        "config": {
            "workload": f"{spec.name}+{bl_spec.name}-4windows",
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
            "kernel": "zero_counters_kernel + attn_bf16_pp_kernel<128, 64, true> + "
                      "split_merge_kernel<128, 256> (varlen_attn_fwd_vt)",
            "kernel_ms": round(attn_ms, 4),
            "algorithmic_flop_per_launch": flop_varlen,
        },
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
