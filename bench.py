"""Benchmark of the MSA layer on one MI355X.

One step = one pass of the whole hot path over one batch of seeded synthetic input already
resident in HBM: index branch (msa_index_topk) -> inverted index (msa_plan) -> KV-outer
attention (msa_attn_main) -> LSE combine (msa_combine); Q-outer workloads run
msa_sparse_attn_fwd in place of the two middle calls. Prints one JSON line.

value = useful FLOPs (4*D per unmasked selected (query, head, key) triple: QK^T and PV only,
"Sparse Attention", Chapter 3) / whole-step time. Each kernel is also timed with HIP events
recorded on the stream the library launches on.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_gqa_amd import msa  # noqa: E402
from synth import msa_inputs as mi    # noqa: E402

PEAK_HBM = 8.0e12            # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15           # dense bf16 MFMA FLOP/s
PEAK_FP8 = 5.0e15            # dense fp8 MFMA FLOP/s
PEAK_FP4 = 10.1e15           # dense fp4 MFMA FLOP/s
CSRC = "block_sparse_gqa_amd/csrc"
# sources each call's kernels are built from (a traffic figure is kept only while they are
# unchanged)
COMMON = (f"{CSRC}/msa_device.h", f"{CSRC}/msa_internal.h")
CALL_SOURCES = {
    "index": (f"{CSRC}/index_topk.hip",) + COMMON,
    "select": (f"{CSRC}/select_tiles.hip",) + COMMON,
    "plan": (f"{CSRC}/plan.hip",) + COMMON,
    "attn_main": (f"{CSRC}/attn_kv.hip", f"{CSRC}/attn_tile.h") + COMMON,
    "attn_q": (f"{CSRC}/attn_q.hip", f"{CSRC}/attn_tile.h") + COMMON,
    "combine": (f"{CSRC}/combine.hip",) + COMMON,
}

WORKLOADS = {
    # name -> (config key, description)
    "m3": ("m3", "M3-shape MSA prefill: B=1, N=32768 causal, Hq=64, Hkv=4, D=128, block 128, "
                 "top-16, proxy dim 64, rank-8 block-reuse bias, bf16"),
    "tiny": ("tiny", "tiny MSA prefill: B=1, N=2048 causal, Hq=16, Hkv=1, top-4, proxy dim 32, bf16"),
    "qtile": ("qtile", "per-Q-tile block-sparse fwd: N=8192 non-causal, Hq=Hkv=16, 16 of 64 blocks "
                       "per Q128 tile, bf16"),
    "m3_fp8_long": ("m3_fp8_long", "long-context fp8 MSA prefill: N=131072 causal, Hq=64, Hkv=4, "
                                   "top-16, fp8 e4m3 Q/K/V, bf16 proxies and partials"),
    "decode": ("decode", "MSA decode: 64 requests x 1 query, Nk uniform over multiples of 128 in "
                         "[16384, 131072], Hq=64, Hkv=4, top-16, bf16"),
    # R1 / R4 selector -> per-tile attention ("Sparse Attention", Chapter 4 benchmark shape)
    "sel_r1": ("sel_r1", "R1 selector + per-tile block-sparse fwd: B=2, 4096 queries, 16384 keys, "
                         "non-causal, Hq=16, Hkv=1, 16 blocks per Q128 tile, bf16"),
    "sel_r4": ("sel_r4", "R4 selector + per-tile block-sparse fwd: B=2, 4096 queries, 16384 keys, "
                         "non-causal, Hq=16, Hkv=1, 16 blocks per Q128 tile, bf16"),
    # the same workloads with e4m3 proxies (low-precision index scoring)
    "m3_fp8_long_i8": ("m3_fp8_long_i8", "long-context fp8 MSA prefill as m3_fp8_long, proxies "
                                         "fp8 e4m3 with per-tensor scales"),
    "decode_i8": ("decode_i8", "MSA decode as decode, proxies fp8 e4m3 with per-tensor scales"),
    # and with 4-bit MXFP4 proxies (E2M1 codes, one E8M0 scale per 32 elements)
    "m3_fp8_long_i4": ("m3_fp8_long_i4", "long-context fp8 MSA prefill as m3_fp8_long, proxies "
                                         "MXFP4 (4-bit, one scale per 32 elements)"),
    "decode_i4": ("decode_i4", "MSA decode as decode, proxies MXFP4 (4-bit, one scale per 32 "
                               "elements)"),
}


def kernel_sha(paths=None) -> str:
    """Hash of the given sources (default: every source of the library and its header)."""
    if paths is None:
        d = os.path.join(ROOT, CSRC)
        paths = [os.path.join(CSRC, f) for f in sorted(os.listdir(d))
                 if f.endswith((".hip", ".h"))] + ["include/msa.h"]
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def useful_pairs(cfg, cu_q, cu_k, lists_np: np.ndarray, list_q: int) -> tuple[int, int]:
    """(useful (query, head, key) triples, distinct selected (seq, group, block) buckets)."""
    g = cfg.hq // cfg.hkv
    total, buckets = 0, 0
    tiles_max = -(-int(np.max(np.diff(cu_q))) // list_q) if list_q > 1 else 0
    for s in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[s]), int(cu_q[s + 1])
        nk = int(cu_k[s + 1] - cu_k[s])
        nq = q1 - q0
        if nq == 0:
            continue
        nb = -(-nk // 128)
        pos = nk - nq + np.arange(nq)
        lst = lists_np[s * tiles_max + np.arange(nq) // list_q] if list_q > 1 else lists_np[q0:q1]
        for h in range(cfg.hkv):
            l = lst[:, h, :].astype(np.int64)
            srt = np.sort(np.where((l >= 0) & (l < nb), l, -1), axis=1)
            dup = np.zeros_like(srt, dtype=bool)
            dup[:, 1:] = (srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] >= 0)
            b = np.where(dup, -1, srt)
            start = b * 128
            end = np.minimum(start + 128, nk)
            if cfg.causal:
                end = np.minimum(end, pos[:, None] + 1)
                b = np.where(start <= pos[:, None], b, -1)
            ok = b >= 0
            total += int(np.where(ok, np.maximum(end - start, 0), 0).sum()) * g
            buckets += int(np.unique(b[ok]).size)
    return total, buckets


def index_work(cfg, cu_q, cu_k) -> tuple[float, float]:
    """(proxy FLOPs, proxy bytes) the index branch must do: 2*dp per (query, group, key) over
    the keys of every visible block other than the local one; q_idx and those k_idx rows once
    (eb bytes per element), plus the lists written."""
    eb = {"fp8": 1.0, "mxfp4": 0.5 + 1.0 / 32}.get(cfg.idx_dtype, 2.0)
    flops, kbytes = 0.0, 0.0
    for s in range(len(cu_q) - 1):
        nq = int(cu_q[s + 1] - cu_q[s])
        nk = int(cu_k[s + 1] - cu_k[s])
        if nq == 0:
            continue
        pos = nk - nq + np.arange(nq)
        nb = -(-nk // 128)
        if cfg.causal:
            keys = 128.0 * np.maximum(pos // 128, 0)            # blocks 0 .. c-1, all full
            kread = min(nk, 128 * (int(pos[-1]) // 128))
        else:
            keys = np.full(nq, float(nk - min(128, nk)))         # all but the local block
            kread = nk
        flops += 2.0 * cfg.dp * cfg.hkv * float(np.sum(keys))
        kbytes += eb * cfg.dp * cfg.hkv * kread
    tq = int(cu_q[-1])
    return flops, kbytes + eb * cfg.dp * cfg.hkv * tq + 4.0 * cfg.hkv * cfg.topk * tq


def roof(ms, bound, amount, peak_mfma=PEAK_BF16):
    """Roofline entry of one kernel: amount = bytes (hbm) or FLOPs (mfma, against the peak of
    the contraction's own dtype) per call."""
    t = ms * 1e-3
    if bound == "hbm":
        return {"ms": ms, "bound": "hbm", "achieved": amount / t / 1e9, "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": amount / t / PEAK_HBM, "algorithmic": amount}
    return {"ms": ms, "bound": "mfma", "achieved": amount / t / 1e12, "peak": peak_mfma / 1e12,
            "unit": "TFLOP/s", "frac": amount / t / peak_mfma, "algorithmic": amount}


class Timer:
    """HIP events on the current stream around each call of a step."""

    def __init__(self, names):
        self.names = names
        self.ev = []

    def step(self):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]
        self.ev.append(evs)
        return evs

    def ms(self):
        out = {n: 0.0 for n in self.names}
        for evs in self.ev:
            for i, n in enumerate(self.names):
                out[n] += evs[i].elapsed_time(evs[i + 1])
        return {n: v / max(1, len(self.ev)) for n, v in out.items()}


def cpu_baseline(case, budget_s: float) -> dict:
    """The oracle, untuned, on a bounded sample of the same workload (whole 128-query blocks,
    index branch + sparse attention for their rows), scaled to useful TFLOP/s."""
    from oracle import msa_case
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    nqb = -(-case.max_q // 128)
    rows_done, flops, t_used = [], 0, 0.0
    rng = np.random.default_rng(0)
    blocks = rng.permutation(max(1, nqb))
    t0 = time.perf_counter()
    what = "index branch"
    if case.cfg.selector:
        # the selector oracle over every tile (its time counted), then the lists it chose
        from oracle import selectors
        from synth.msa_inputs import widen
        c = case.cfg
        q, k = widen(case.q), widen(case.k)
        case.lists = np.full(((len(case.cu_q) - 1) * nqb, c.hkv, c.topk), -1, dtype=np.int32)
        for s in range(len(case.cu_q) - 1):
            q0, q1, k0, k1 = case.cu_q[s], case.cu_q[s + 1], case.cu_k[s], case.cu_k[s + 1]
            lst, _ = selectors.select_tiles(q[q0:q1], k[k0:k1], c.selector, 128,
                                            c.hq // c.hkv, c.topk, c.causal)
            case.lists[s * nqb:s * nqb + lst.shape[0]] = lst
        del q, k
        what = f"R{case.cfg.selector} selector over every tile"
    for b in blocks:
        rows = np.arange(b * 128, min(case.total_q, (b + 1) * 128))
        if case.cfg.length_seed_draw is not None:      # decode: one query per request
            rows = np.arange(min(case.total_q, 8)) + 8 * (len(rows_done))
            rows = rows[rows < case.total_q]
        if rows.size == 0:
            break
        out = msa_case.run(case, rows=rows)
        lists = np.full((case.total_q, case.cfg.hkv, case.cfg.topk), -1, dtype=np.int32)
        lists[out.rows] = out.topk_idx
        p, _ = useful_pairs(case.cfg, case.cu_q, case.cu_k, lists, 1)
        flops += 4 * 128 * p
        rows_done.append(rows.size)
        t_used = time.perf_counter() - t0
        if t_used >= budget_s:
            break
    n_rows = int(sum(rows_done))
    return {"value": flops / max(t_used, 1e-9) / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_rows} query rows ({len(rows_done)} groups of whole 128-query blocks, "
                      f"all heads) of the same workload, {what} + sparse attention, "
                      f"fp64 NumPy, {t_used:.1f} s wall on {platform.processor() or 'host'}"}


def load_traffic(workload: str) -> dict:
    """HBM bytes per launch of each call (FETCH_SIZE and WRITE_SIZE, scaled by what the same
    counters read for a device copy of known size), from profiles/traffic_<workload>.json;
    a call whose sources changed since the counters were taken gets None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    out = {}
    for call, e in t.get("calls", {}).items():
        ok = call in CALL_SOURCES and e.get("sha") == kernel_sha(CALL_SOURCES[call])
        out[call] = e.get("traffic_bytes") if ok else None
    return out


def measure_ceilings(dev, mib: int = 2048) -> dict:
    """Memory ceilings measured on this GPU over a buffer of `mib` MiB, best of five after
    warm-up, in GB/s: torch's fill (write) and copy (read + write), the library's read probe
    (read; torch's sum, a slower reader, beside it)."""
    n = (mib << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)

    def best(fn, nbytes):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return nbytes / min(ts) / 1e9
    nb = n * 4
    sink = torch.empty(1024 * 256, dtype=torch.float32, device=dev)
    out = {"write_gbps": best(lambda: a.fill_(2.0), nb),
           "copy_gbps": best(lambda: b.copy_(a), 2 * nb),
           "read_gbps": best(lambda: msa.msa_probe_read(a, nb, 4 * nb, sink), 4 * nb),
           "torch_sum_gbps": best(lambda: a.sum(), nb),
           "buffer_mib": mib,
           "how": "torch fill_ (write) and copy_ (read + write) on one buffer; read: the "
                  "library's read probe over the same buffer (far beyond the 256 MiB "
                  "last-level cache), 4 passes; best of 5 each"}
    del a, b, sink
    torch.cuda.empty_cache()
    return out


def _amdgpu_files() -> dict | None:
    """sysfs files of the one AMD GPU: hwmon power reading and cap (microwatts), current
    graphics clock level. None when there is not exactly one such device."""
    devs = [d for d in glob.glob("/sys/class/drm/card*/device")
            if os.path.exists(os.path.join(d, "vendor"))
            and open(os.path.join(d, "vendor")).read().strip() == "0x1002"
            and glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_input"))]
    if len(devs) != 1:
        return None
    hw = glob.glob(os.path.join(devs[0], "hwmon", "hwmon*"))[0]
    return {"power": os.path.join(hw, "power1_input"), "cap": os.path.join(hw, "power1_cap"),
            "sclk": os.path.join(devs[0], "pp_dpm_sclk")}


def _read_sclk(path: str):
    """Current graphics clock (MHz): the level marked '*' in pp_dpm_sclk."""
    try:
        for line in open(path):
            if "*" in line:
                num = "".join(ch if ch.isdigit() else " " for ch in line.split(":", 1)[-1]).split()
                return float(num[0]) if num else None
    except OSError:
        return None
    return None


def power_sample(fn, secs: float = 6.0, settle: float = 2.5) -> dict | None:
    """Socket power and graphics clock while `fn` (one call, launched asynchronously) runs
    back to back for `secs` seconds: amdgpu's hwmon reading is taken between batches of calls
    after `settle` seconds (the power manager's steady state), the median reported. Files
    are read, no tool is run. None when the GPU's sysfs files are not there."""
    f = _amdgpu_files()
    if f is None:
        return None
    fn()
    torch.cuda.synchronize()
    watts, mhz = [], []
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        n += 8
        el = time.perf_counter() - t0
        if el > settle:
            try:
                watts.append(int(open(f["power"]).read()) / 1e6)
            except (OSError, ValueError):
                pass
            c = _read_sclk(f["sclk"])
            if c:
                mhz.append(c)
        torch.cuda.synchronize()
        if el > secs:
            break
    el = time.perf_counter() - t0
    try:
        cap = int(open(f["cap"]).read()) / 1e6
    except (OSError, ValueError):
        cap = None
    if not watts:
        return None
    w = float(np.median(watts))
    ms = el * 1e3 / n
    return {"socket_w": w, "cap_w": cap, "gfx_mhz": float(np.median(mhz)) if mhz else None,
            "ms_per_call": ms, "joule_per_call": w * ms * 1e-3, "samples": len(watts),
            "how": "calls back to back; amdgpu hwmon power1_input and pp_dpm_sclk, median"}


def gemm_ceiling(dev, n: int = 8192, secs: float = 5.0) -> dict:
    """bf16 MFMA ceiling measured on this GPU under its power manager: torch.matmul (the
    vendor BLAS) on n x n x n bf16 back to back for `secs` seconds, the rate taken from the
    host clock over all the calls; the power and clock seen meanwhile."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    t0 = time.perf_counter()
    k = 0
    pw = power_sample(lambda: torch.matmul(a, b, out=c), secs=secs, settle=secs / 2)
    if pw is None:            # no power reading: time the loop alone
        while time.perf_counter() - t0 < secs:
            for _ in range(8):
                torch.matmul(a, b, out=c)
            torch.cuda.synchronize()
            k += 8
        ms = (time.perf_counter() - t0) * 1e3 / k
    else:
        ms = pw["ms_per_call"]
    del a, b, c
    torch.cuda.empty_cache()
    return {"gemm_bf16_tflops": 2.0 * n ** 3 / (ms * 1e-3) / 1e12, "n": n, "power": pw,
            "how": "torch.matmul bf16 %d^3 back to back for %.0f s, host clock" % (n, secs)}


def mix_ceiling(ceil: dict, read_bytes: float, write_bytes: float) -> float:
    """Measured ceiling (GB/s) for a kernel that reads and writes these amounts: the time the
    measured read and write rates need for them, as one rate."""
    t = read_bytes / ceil["read_gbps"] + write_bytes / ceil["write_gbps"]
    return (read_bytes + write_bytes) / t if t > 0 else 0.0


def bench_backward(args, case, shape, desc, t) -> None:
    """Main-branch backward: one step = msa_sparse_attn_bwd (inverted index, D = rowsum(dO O),
    the KV-stationary dK / dV / dQ-partial kernel, the dQ sum) on the forward's lists, O and
    LSE. value = useful FLOPs (10 D per unmasked selected (query, head, key) triple: S, dP, dV,
    dK, dQ) / time."""
    q, k, v, o, lse, topk, cu_q, cu_k, q_idx, k_idx = t
    cfg = case.cfg
    if cfg.dtype != "bf16":
        print("the backward runs on bf16 workloads only", file=sys.stderr)
        sys.exit(2)
    dout = mi.grad_output(case).to("cuda")
    bws = torch.empty(msa.msa_bwd_workspace_size(shape), dtype=torch.uint8, device="cuda")
    dq = torch.empty((case.total_q, cfg.hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.empty((case.total_k, cfg.hkv, 128), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)

    def bwd():
        msa.msa_sparse_attn_bwd(shape, q, k, v, o, lse, dout, case.softmax_scale, topk, cu_q,
                                cu_k, bws, dq, dk, dv)
    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        bwd()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = sum(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)) / args.steps
    pairs, nsb = useful_pairs(cfg, case.cu_q, case.cu_k, topk.cpu().numpy(), cfg.list_q)
    flops = 10.0 * 128 * pairs
    res = {
        "metric": "main-branch backward TFLOP/s (useful pairs); ms per backward call",
        "value": flops / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded NumPy draws, see DESIGN.md input recipe)",
        "config": {"workload": args.workload + "_backward", "description": desc,
                   "global_batch": len(case.cu_q) - 1, "seq_len": case.max_q, "hq": cfg.hq,
                   "hkv": cfg.hkv, "d": 128, "block": 128, "topk": cfg.topk,
                   "causal": cfg.causal, "parallelism": "single GPU"},
        "call_ms_events": ev_ms,
        "useful_gflop": flops / 1e9, "nsb": nsb,
        "roofline": {"bound": "mfma", "kernel": "msa_sparse_attn_bwd (all its kernels)",
                     "achieved": flops / (ev_ms * 1e-3) / 1e12, "peak": PEAK_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": flops / (ev_ms * 1e-3) / PEAK_BF16,
                     "traffic": None},
    }
    if q_idx is not None and cfg.idx_dtype == "bf16":
        # the proxy backward of the same step (gradients of the proxies toward the main weights)
        pws = torch.empty(msa.msa_proxy_bwd_workspace_size(shape), dtype=torch.uint8,
                          device="cuda")
        dqi = torch.empty((case.total_q, cfg.hkv, cfg.dp), dtype=torch.float32, device="cuda")
        dki = torch.empty((case.total_k, cfg.hkv, cfg.dp), dtype=torch.float32, device="cuda")

        def pbwd():
            msa.msa_proxy_attn_bwd(shape, q, k, q_idx, k_idx, lse, case.softmax_scale,
                                   1.0 / math.sqrt(cfg.dp), topk, cu_q, cu_k, pws, dqi, dki)
        for _ in range(args.warmup):
            pbwd()
        torch.cuda.synchronize()
        pev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        pev[0].record()
        for i in range(args.steps):
            pbwd()
            pev[i + 1].record()
        torch.cuda.synchronize()
        res["proxy_backward_ms"] = sum(pev[i].elapsed_time(pev[i + 1])
                                       for i in range(args.steps)) / args.steps
        if not args.no_ceilings:
            res["power"] = {"backward": power_sample(bwd), "proxy_backward": power_sample(pbwd)}
        del pws
        # both backward passes in one call (msa_train_bwd)
        tws = torch.empty(msa.msa_train_bwd_workspace_size(shape), dtype=torch.uint8,
                          device="cuda")

        def tbwd():
            msa.msa_train_bwd(shape, q, k, v, o, lse, dout, case.softmax_scale, q_idx, k_idx,
                              1.0 / math.sqrt(cfg.dp), topk, cu_q, cu_k, tws, dq, dk, dv, dqi,
                              dki)
        for _ in range(args.warmup):
            tbwd()
        torch.cuda.synchronize()
        tev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        tev[0].record()
        for i in range(args.steps):
            tbwd()
            tev[i + 1].record()
        torch.cuda.synchronize()
        res["train_backward_ms"] = sum(tev[i].elapsed_time(tev[i + 1])
                                       for i in range(args.steps)) / args.steps
        del tws
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_backward(case, topk.cpu().numpy(), dout,
                                                    args.cpu_budget)
    print(json.dumps(res), flush=True)


def cpu_baseline_backward(case, lists: np.ndarray, dout, budget_s: float) -> dict:
    """The backward oracle, untuned, on growing suffixes of the first sequence (a suffix keeps
    the queries' positions), scaled to useful TFLOP/s."""
    from oracle.msa_backward import sparse_attention_backward
    from synth.msa_inputs import widen
    cfg = case.cfg
    q0, q1 = int(case.cu_q[0]), int(case.cu_q[1])
    k0, k1 = int(case.cu_k[0]), int(case.cu_k[1])
    k, v = widen(case.k[k0:k1]), widen(case.v[k0:k1])
    n, t_used, flops = 0, 0.0, 0.0
    t0 = time.perf_counter()
    while n < q1 - q0 and t_used < budget_s:
        m = min(128, q1 - q0 - n)
        a, b = q1 - n - m, q1 - n
        part = lists[a:q1].copy()
        part[m:] = -1                          # rows already done take no keys
        sparse_attention_backward(widen(case.q[a:q1]), k, v, part, widen(dout[a:q1].cpu()),
                                  case.softmax_scale, cfg.block, cfg.causal)
        sub = np.full_like(lists, -1)
        sub[a:b] = lists[a:b]
        p, _ = useful_pairs(cfg, case.cu_q, case.cu_k, sub, 1)
        flops += 10.0 * 128 * p
        n += m
        t_used = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    return {"value": flops / max(t_used, 1e-9) / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the last {n} queries of sequence 0 (all heads), backward oracle, fp64 "
                      f"NumPy, {t_used:.1f} s wall"}


def prepare(workload: str, seed: int, mode_name: str, dev: str) -> dict:
    """Seeded inputs of a workload, uploaded to HBM, with the buffers of one layer call."""
    cfg_key, desc = WORKLOADS[workload]
    t_gen = time.perf_counter()
    case = mi.make_case(cfg_key, seed=seed)
    t_gen = time.perf_counter() - t_gen
    cfg = case.cfg
    dtype = msa.MSA_FP8_E4M3 if cfg.dtype == "fp8" else msa.MSA_BF16
    shape = msa.make_shape(batch=len(case.cu_q) - 1, total_q=case.total_q, total_k=case.total_k,
                           max_q=case.max_q, max_k=case.max_k, hq=cfg.hq, hkv=cfg.hkv,
                           topk=cfg.topk, dp=cfg.dp, causal=cfg.causal, dtype=dtype,
                           list_q=cfg.list_q)
    mode = {"auto": msa.MSA_AUTO, "kv": msa.MSA_KV_OUTER, "q": msa.MSA_Q_OUTER}[mode_name]
    chosen = msa.msa_resolve_mode(shape, mode)
    up = lambda t: None if t is None else t.contiguous().to(dev)
    c = dict(workload=workload, desc=desc, case=case, cfg=cfg, dtype=dtype, shape=shape,
             chosen=chosen, t_gen=t_gen)
    c["q"], c["k"], c["v"] = up(case.q), up(case.k), up(case.v)
    c["q_idx"], c["k_idx"] = up(case.q_idx), up(case.k_idx)
    c["idx8"] = cfg.idx_dtype == "fp8"
    c["idx4"] = cfg.idx_dtype == "mxfp4"
    c["q_isc"], c["k_isc"] = up(case.q_idx_scale), up(case.k_idx_scale)
    c["idx_descale"] = (torch.tensor(case.idx_descale, dtype=torch.float32, device=dev)
                        if c["idx8"] else None)
    c["cu_q"] = torch.from_numpy(case.cu_q).to(dev)
    c["cu_k"] = torch.from_numpy(case.cu_k).to(dev)
    c["descale"] = torch.tensor(case.descale, dtype=torch.float32, device=dev) if dtype else None
    c["given"] = torch.from_numpy(case.lists).to(dev) if case.lists is not None else None
    sel = c["sel"] = cfg.selector              # per-tile lists from the R1 / R4 selector
    c["n_lists"] = (case.total_q if cfg.list_q == 1
                    else (len(case.cu_q) - 1) * -(-case.max_q // 128))
    c["topk"] = c["given"] if c["given"] is not None else torch.empty(
        (c["n_lists"], cfg.hkv, cfg.topk), dtype=torch.int32, device=dev)
    c["iws"] = torch.empty(max(msa.msa_index_workspace_size(shape)
                               if c["given"] is None and not sel else 0, 256),
                           dtype=torch.uint8, device=dev)
    c["sws"] = torch.empty(msa.msa_select_workspace_size(shape, sel) if sel else 256,
                           dtype=torch.uint8, device=dev)
    c["ws"] = torch.empty(msa.msa_workspace_size(shape, chosen), dtype=torch.uint8, device=dev)
    c["o"] = torch.empty((case.total_q, cfg.hq, 128), dtype=torch.bfloat16, device=dev)
    c["lse"] = torch.empty((case.total_q, cfg.hq), dtype=torch.float32, device=dev)
    return c


def make_step(c: dict):
    """One layer call on the workload's buffers, HIP events recorded between its calls (on
    torch's current stream, the one the library launches on)."""
    shape, chosen, scale = c["shape"], c["chosen"], c["case"].softmax_scale
    given, sel, idx8 = c["given"], c["sel"], c["idx8"]
    q, k, v, topk, ws, o, lse = c["q"], c["k"], c["v"], c["topk"], c["ws"], c["o"], c["lse"]
    cu_q, cu_k = c["cu_q"], c["cu_k"]
    kv = chosen == msa.MSA_KV_OUTER
    first = (["select"] if sel else ["index"]) if given is None else []
    names = first + (["plan", "attn_main"] if kv else ["attn_q"]) + ["combine"]

    def step(evs=None):
        i = 0
        if evs:
            evs[0].record()
        if given is None and sel:
            msa.msa_select_tiles(shape, sel, q, k, cu_q, cu_k, topk, None, c["sws"])
        elif given is None and idx8:
            msa.msa_index_topk_fp8(shape, c["q_idx"], c["k_idx"], c["idx_descale"], cu_q, cu_k,
                                   topk, None, c["iws"])
        elif given is None and c["idx4"]:
            msa.msa_index_topk_mxfp4(shape, c["q_idx"], c["q_isc"], c["k_idx"], c["k_isc"], cu_q,
                                     cu_k, topk, None, c["iws"])
        elif given is None:
            msa.msa_index_topk(shape, c["q_idx"], c["k_idx"], cu_q, cu_k, topk, None, c["iws"])
        if given is None and evs:
            i += 1
            evs[i].record()
        if kv:
            msa.msa_plan(shape, topk, cu_q, cu_k, ws)
            if evs:
                i += 1
                evs[i].record()
            msa.msa_attn_main(shape, q, k, v, c["descale"], scale, cu_q, cu_k, ws)
        else:
            msa.msa_sparse_attn_fwd(shape, q, k, v, c["descale"], scale, topk, cu_q, cu_k, chosen,
                                    ws, o, lse)
        if evs:
            i += 1
            evs[i].record()
        msa.msa_combine(shape, chosen, ws, o, lse)
        if evs:
            i += 1
            evs[i].record()
    return step, names


def call_fns(c: dict) -> dict:
    """Each call of a step as a function of no arguments, on the workload's buffers (the
    workspace must hold a plan for attn_main and partials for combine: run a step first)."""
    shape, chosen, scale = c["shape"], c["chosen"], c["case"].softmax_scale
    q, k, v, topk, ws, o, lse = c["q"], c["k"], c["v"], c["topk"], c["ws"], c["o"], c["lse"]
    cu_q, cu_k = c["cu_q"], c["cu_k"]
    fns = {}
    if c["given"] is None and c["sel"]:
        fns["select"] = lambda: msa.msa_select_tiles(shape, c["sel"], q, k, cu_q, cu_k, topk,
                                                     None, c["sws"])
    elif c["given"] is None and c["idx8"]:
        fns["index"] = lambda: msa.msa_index_topk_fp8(shape, c["q_idx"], c["k_idx"],
                                                      c["idx_descale"], cu_q, cu_k, topk, None,
                                                      c["iws"])
    elif c["given"] is None and c["idx4"]:
        fns["index"] = lambda: msa.msa_index_topk_mxfp4(shape, c["q_idx"], c["q_isc"],
                                                        c["k_idx"], c["k_isc"], cu_q, cu_k,
                                                        topk, None, c["iws"])
    elif c["given"] is None:
        fns["index"] = lambda: msa.msa_index_topk(shape, c["q_idx"], c["k_idx"], cu_q, cu_k,
                                                  topk, None, c["iws"])
    if chosen == msa.MSA_KV_OUTER:
        fns["plan"] = lambda: msa.msa_plan(shape, topk, cu_q, cu_k, ws)
        fns["attn_main"] = lambda: msa.msa_attn_main(shape, q, k, v, c["descale"], scale, cu_q,
                                                     cu_k, ws)
    else:
        fns["attn_q"] = lambda: msa.msa_sparse_attn_fwd(shape, q, k, v, c["descale"], scale,
                                                        topk, cu_q, cu_k, chosen, ws, o, lse)
    fns["combine"] = lambda: msa.msa_combine(shape, chosen, ws, o, lse)
    return fns


def power_table(c: dict, dev, secs: float = 6.0) -> dict:
    """Power and clock of each call of the step run back to back, of the whole step, of the
    vendor bf16 GEMM and of a 2 GiB device copy; the idle reading first."""
    f = _amdgpu_files()
    out = {"metric": "socket power and graphics clock per call", "workload": c["workload"],
           "description": c["desc"]}
    if f is None:
        out["error"] = "no amdgpu hwmon power reading"
        return out
    torch.cuda.synchronize()
    time.sleep(3.0)
    out["idle_w"] = int(open(f["power"]).read()) / 1e6
    step, _ = make_step(c)
    step()
    torch.cuda.synchronize()
    calls = {name: power_sample(fn, secs) for name, fn in call_fns(c).items()}
    calls["step"] = power_sample(step, secs)
    out["calls"] = calls
    out["gemm"] = gemm_ceiling(dev)
    x = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    pw = power_sample(lambda: y.copy_(x), secs)
    if pw:
        pw["gbps"] = 2 * x.numel() / (pw["ms_per_call"] * 1e-3) / 1e9
    out["copy_2gib"] = pw
    del x, y
    torch.cuda.empty_cache()
    return out


def run_forward(c: dict, steps: int, warmup: int, ceil: dict | None) -> dict:
    """Time `steps` layer calls after `warmup`; the result line of the workload."""
    case, cfg, dtype, chosen = c["case"], c["cfg"], c["dtype"], c["chosen"]
    step, names = make_step(c)
    timer = Timer(names)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: every kernel bracketed by HIP events on the stream the library launches on
    # (torch's current stream), the whole region by the host clock
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer.step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    kms = timer.ms()

    kv = chosen == msa.MSA_KV_OUTER
    given, sel = c["given"], c["sel"]
    lists_np = c["topk"].cpu().numpy()
    pairs, nsb = useful_pairs(cfg, case.cu_q, case.cu_k, lists_np, cfg.list_q)
    flops = 4.0 * 128 * pairs
    g = cfg.hq // cfg.hkv
    eb = 1 if dtype else 2
    peak_mma = PEAK_FP8 if dtype else PEAK_BF16
    n_ent = int(c["ws"][:4].view(torch.int32)[0].item()) if kv else 0
    traffic = load_traffic(c["workload"])
    res = {
        "metric": "main-attn TFLOP/s (useful pairs) + % MFMA/HBM roofline; ms per layer call",
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8" if dtype else "bf16",
        "data": "synthetic (seeded NumPy draws, see DESIGN.md input recipe)",
        "config": {"workload": c["workload"], "description": c["desc"],
                   "mode": {1: "kv_outer", 2: "q_outer"}[chosen],
                   "global_batch": len(case.cu_q) - 1, "seq_len": case.max_q,
                   "hq": cfg.hq, "hkv": cfg.hkv, "d": 128, "block": 128, "topk": cfg.topk,
                   "dp": cfg.dp, "causal": cfg.causal, "parallelism": "single GPU"},
        "kernel_ms": kms,
        "useful_gflop": flops / 1e9,
        "nsb": nsb, "nsb_over_n": nsb / max(1, case.total_q), "entries": n_ent,
    }
    main_name = "attn_main" if kv else "attn_q"
    t_main = kms[main_name] * 1e-3
    res["main_attn_tflops"] = flops / t_main / 1e12
    res["main_attn_mfma_frac"] = flops / t_main / peak_mma
    kr = {}
    if given is None and sel:
        # representatives read Q and K once; the lists are written
        kr["select"] = roof(kms["select"], "hbm", (case.total_q * cfg.hq + case.total_k * cfg.hkv)
                            * 128 * 2 + c["n_lists"] * cfg.hkv * cfg.topk * 4)
    elif given is None:
        ifl, ib = index_work(cfg, case.cu_q, case.cu_k)
        pk = {"fp8": PEAK_FP8, "mxfp4": PEAK_FP4}.get(cfg.idx_dtype, PEAK_BF16)
        kr["index"] = roof(kms["index"], "mfma", ifl, pk) if ifl / ib > pk / PEAK_HBM else \
            roof(kms["index"], "hbm", ib)
    if kv:
        q_bytes = case.total_q * cfg.hq * 128 * eb          # Q, each query once
        kv_bytes = nsb * 2 * 128 * 128 * eb                 # selected K and V blocks once
        part_bytes = n_ent * g * 128 * 2 + n_ent * g * 4    # bf16 partial O, fp32 LSE written
        alg = q_bytes + kv_bytes + part_bytes
        kname = "attn_kv_f8_kernel" if dtype else "attn_kv_tiled_kernel"
        res["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": alg / t_main / 1e9,
                           "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": alg / t_main / PEAK_HBM,
                           "traffic": traffic.get("attn_main"), "algorithmic_bytes": alg}
        if ceil:
            pm = mix_ceiling(ceil, q_bytes + kv_bytes, part_bytes)
            res["roofline"]["peak_measured"] = pm
            res["roofline"]["frac_measured"] = alg / t_main / 1e9 / pm
        comb_read = n_ent * g * (128 * 2 + 4) + case.total_q * cfg.hkv * cfg.topk * 4
        comb_write = case.total_q * cfg.hq * (128 * 2 + 4)
        comb_alg = comb_read + comb_write
        res["combine_gbps"] = comb_alg / (kms["combine"] * 1e-3) / 1e9
        e_max = case.total_q * cfg.hkv * cfg.topk
        kr["plan"] = roof(kms["plan"], "hbm", e_max * 4 + n_ent * 8 + e_max * 4)
        kr["attn_main"] = roof(kms["attn_main"], "hbm", alg)
        kr["combine"] = roof(kms["combine"], "hbm", comb_alg)
        if ceil:
            kr["attn_main"]["peak_measured"] = res["roofline"]["peak_measured"]
            kr["combine"]["peak_measured"] = mix_ceiling(ceil, comb_read, comb_write)
            kr["combine"]["frac_measured"] = (comb_alg / (kms["combine"] * 1e-3) / 1e9
                                              / kr["combine"]["peak_measured"])
    else:
        qbytes = nsb * 2 * 128 * 128 * eb + case.total_q * cfg.hq * 128 * (eb + 2)
        # the Q-outer kernel that runs: bf16 per-tile lists, bf16 per-query lists, fp8 lists
        qname = ("attn_q_kernel" if dtype else
                 "attn_qt_kernel" if cfg.list_q > 1 else "attn_qd_kernel")
        if flops / qbytes > peak_mma / PEAK_HBM:
            res["roofline"] = {"bound": "mfma", "kernel": qname,
                               "achieved": flops / t_main / 1e12, "peak": peak_mma / 1e12,
                               "unit": "TFLOP/s", "frac": flops / t_main / peak_mma,
                               "traffic": traffic.get("attn_q")}
            kr["attn_q"] = roof(kms["attn_q"], "mfma", flops, peak_mma)
        else:
            res["roofline"] = {"bound": "hbm", "kernel": qname,
                               "achieved": qbytes / t_main / 1e9, "peak": PEAK_HBM / 1e9,
                               "unit": "GB/s", "frac": qbytes / t_main / PEAK_HBM,
                               "traffic": traffic.get("attn_q"), "algorithmic_bytes": qbytes}
            kr["attn_q"] = roof(kms["attn_q"], "hbm", qbytes)
        kr["combine"] = {"ms": kms["combine"]}
    for call, e in kr.items():
        if call in traffic:
            e["traffic"] = traffic[call]
    res["kernels"] = kr
    if ceil is not None:
        # the main call back to back after the timed region: power and clock it runs at
        shape, scale = c["shape"], case.softmax_scale
        if kv:
            fn = lambda: msa.msa_attn_main(shape, c["q"], c["k"], c["v"], c["descale"], scale,
                                           c["cu_q"], c["cu_k"], c["ws"])
        else:
            fn = lambda: msa.msa_sparse_attn_fwd(shape, c["q"], c["k"], c["v"], c["descale"],
                                                 scale, c["topk"], c["cu_q"], c["cu_k"], chosen,
                                                 c["ws"], c["o"], c["lse"])
        res["roofline"]["power"] = power_sample(fn)
        gem = ceil.get("gemm")
        if gem and not dtype:
            res["roofline"]["mfma_ceiling_measured_tflops"] = gem["gemm_bf16_tflops"]
            res["roofline"]["mfma_frac_measured"] = flops / t_main / 1e12 / gem["gemm_bf16_tflops"]
    res["kernel_sha"] = kernel_sha()
    res["gen_seconds"] = round(c["t_gen"], 1)
    return res


def calibrate(dev) -> dict:
    """Read bandwidth of HBM (a 4 GiB working set) and of the caches (working sets of 16 MiB,
    which fits the 4 MiB L2 of each of the 8 XCDs, and 64 to 192 MiB, within the 256 MiB
    last-level cache), each the best of five probe launches reading 16 GiB."""
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(1024 * 256, dtype=torch.float32, device=dev)
    total = 16 << 30
    out = {}
    for name, ws in (("hbm_4096mib", 4 << 30), ("mall_192mib", 192 << 20),
                     ("mall_128mib", 128 << 20), ("mall_64mib", 64 << 20),
                     ("l2_16mib", 16 << 20)):
        for _ in range(2):
            msa.msa_probe_read(buf, ws, total, sink)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            msa.msa_probe_read(buf, ws, total, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        out[name + "_gbps"] = total / min(ts) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    out["beta_mall"] = out["mall_128mib_gbps"] / out["hbm_4096mib_gbps"]
    return out


def crossover_sweep(args, dev) -> dict:
    """KV-outer against Q-outer across block reuse: 2048 queries in requests of n_q queries
    that share one list of 16 blocks per group (each request its own 2048-key cache, every
    block listed: nsb / N = 64 / n_q), Hq = 64, Hkv = 4, D = 128, bf16, non-causal. Each point
    times the main branch and the combine of both schedules on the same inputs."""
    n_total, nk, hq, hkv, topk = 2048, 2048, 64, 4, 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    q = torch.randn((n_total, hq, 128), generator=gen, device=dev).to(torch.bfloat16)
    k = torch.randn((n_total * nk, hkv, 128), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((n_total * nk, hkv, 128), generator=gen, device=dev).to(torch.bfloat16)
    o = torch.empty((n_total, hq, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((n_total, hq), dtype=torch.float32, device=dev)
    points = []
    n_q = 1
    while n_q <= n_total:
        n_req = n_total // n_q
        cu_q = torch.arange(0, n_total + 1, n_q, dtype=torch.int32, device=dev)
        cu_k = torch.arange(0, n_req * nk + 1, nk, dtype=torch.int32, device=dev)
        lists = torch.from_numpy(mi.shared_lists(n_q, n_req, nk // 128, hkv, topk,
                                                 args.seed)).to(dev)
        shape = msa.make_shape(batch=n_req, total_q=n_total, total_k=n_req * nk, max_q=n_q,
                               max_k=nk, hq=hq, hkv=hkv, topk=topk, dp=64, causal=False)
        row = {"n_q": n_q, "requests": n_req, "nsb_over_n": hkv * topk / n_q}
        for mode, name in ((msa.MSA_KV_OUTER, "kv_outer_ms"), (msa.MSA_Q_OUTER, "q_outer_ms")):
            ws = torch.empty(msa.msa_workspace_size(shape, mode), dtype=torch.uint8, device=dev)

            def call():
                msa.msa_sparse_attn_fwd(shape, q, k, v, None, 1.0 / math.sqrt(128), lists, cu_q,
                                        cu_k, mode, ws, o, lse)
                msa.msa_combine(shape, mode, ws, o, lse)
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                call()
            e1.record()
            torch.cuda.synchronize()
            row[name] = e0.elapsed_time(e1) / 10
            del ws
        row["auto"] = {1: "kv_outer", 2: "q_outer"}[msa.msa_resolve_mode(shape, msa.MSA_AUTO)]
        row["model_x"] = msa.msa_crossover(shape, 1.0, 0.0)
        points.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        n_q *= 2
    # measured crossover: where log(kv / q) changes sign, interpolated in log(nsb / N)
    cross = None
    for a, b in zip(points, points[1:]):
        ra = math.log(a["kv_outer_ms"] / a["q_outer_ms"])
        rb = math.log(b["kv_outer_ms"] / b["q_outer_ms"])
        if (ra > 0) != (rb > 0):
            xa, xb = math.log(a["nsb_over_n"]), math.log(b["nsb_over_n"])
            cross = math.exp(xa + (xb - xa) * ra / (ra - rb))
    return {"points": points, "measured_crossover_nsb_over_n": cross}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="m3", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="auto", choices=["auto", "kv", "q"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--secondary", default="m3_fp8_long",
                    help="a second workload timed in the same run and reported under "
                         "'secondary' (only with the default workload; 'none' to skip)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured memory and GEMM ceilings and the power samples")
    ap.add_argument("--backward", action="store_true",
                    help="time the main-branch backward (msa_sparse_attn_bwd) instead")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also time a plain device copy of this many MiB (counter scaling)")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure HBM and cache read bandwidth with the library's probe")
    ap.add_argument("--crossover", action="store_true",
                    help="time KV-outer against Q-outer across block reuse levels")
    ap.add_argument("--power", action="store_true",
                    help="power and clock of each call run back to back (amdgpu hwmon), "
                         "with the GEMM and copy references, instead of the timed run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how the layer would shard).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    if args.calibrate or args.crossover:
        res = {"metric": "memory bandwidth and schedule crossover", "n_gpus": 1}
        if args.calibrate:
            res["bandwidth"] = calibrate(dev)
        if args.crossover:
            res["crossover"] = crossover_sweep(args, dev)
        print(json.dumps(res), flush=True)
        return
    c = prepare(args.workload, args.seed, args.mode, dev)
    if args.power:
        print(json.dumps(power_table(c, dev)), flush=True)
        return
    if args.backward:
        step, _ = make_step(c)
        step()                                 # lists, O and LSE of the forward
        bench_backward(args, c["case"], c["shape"], c["desc"],
                       (c["q"], c["k"], c["v"], c["o"], c["lse"], c["topk"], c["cu_q"],
                        c["cu_k"], c["q_idx"], c["k_idx"]))
        return
    ceil = None
    if not args.no_ceilings:
        ceil = measure_ceilings(dev)
        ceil["gemm"] = gemm_ceiling(dev)
    res = run_forward(c, args.steps, args.warmup, ceil)
    if ceil:
        res["ceilings_measured"] = ceil
    if args.copy_probe:
        n = args.copy_probe << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        res["copy_probe"] = {"bytes_each_way": n, "gbps": 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9}
        del a, b
    case = c["case"]
    del c
    torch.cuda.empty_cache()
    if args.workload == "m3" and args.secondary != "none":
        # the largest workload, fp8 at 128K tokens, timed in the same run
        c2 = prepare(args.secondary, args.seed, args.mode, dev)
        sec = run_forward(c2, max(5, args.steps // 2), max(1, args.warmup), ceil)
        res["secondary"] = {k: sec[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup",
                                                "dtype", "config", "kernel_ms", "roofline",
                                                "kernels", "main_attn_tflops",
                                                "main_attn_mfma_frac", "useful_gflop", "nsb",
                                                "entries", "gen_seconds")}
        del c2
        torch.cuda.empty_cache()
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
