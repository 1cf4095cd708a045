"""Benchmark: bidirectional linear attention, forward + backward, one MI355X.

One step is one pass of the whole path over one batch: la_fwd_state (phi, split-T
state reduction, combine), la_fwd_output (O), la_bwd_dq (dQ and the dS, dz
state), la_bwd_dkv (dK, dV) -- exactly the launches of la_fwd then la_bwd, on
torch's current stream. HIP events bracket every launch, so each kernel's
duration is measured live. Before every step (outside the events) the 256 MB
infinity cache and the L2s are flushed by reading a 1 GiB scratch buffer: a
read leaves them holding clean lines, so every input is fetched from HBM and
no write-back of the flush's own data is charged to the step (a writing flush
would leave 256 MB of dirty lines to evict during the next kernel).

Prints one JSON line. `value` is the forward's algorithmic HBM rate (Q, K, V
read and O written once) in GB/s; fwd/bwd/fwd+bwd milliseconds ride along.
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

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import non_causal_linear_amd as la  # noqa: E402
from synth import HEAD_SIZE_WORKLOADS, HEADLINE, WORKLOADS, make_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# FBi-LA README, "Benchmarks" (A800 80G, B8-H16-D64, T = 16384), in ms.
PAGE_A800_FWD_MS = 0.980992
PAGE_A800_BWD_MS = 5.022208

KERNELS = ("fwd_state", "fwd_output", "bwd_dq", "bwd_dkv")
ALL_WORKLOADS = {**WORKLOADS, **HEAD_SIZE_WORKLOADS}


def launch_bytes(w) -> dict:
    """Algorithmic HBM bytes per launch: each tensor read or written once.
    Q-side tensors (Q, K, dQ, dK) hold B*H*T*D elements, V-side ones (V, O,
    dO, dV) B*H*T*Dv. state reads K, V; output reads Q, writes O; dq reads Q,
    dO, writes dQ; dkv reads K, V, writes dK, dV."""
    nk, nv = w.numel * w.elem_bytes, w.numel_v * w.elem_bytes
    return {"fwd_state": nk + nv, "fwd_output": nk + nv, "bwd_dq": 2 * nk + nv, "bwd_dkv": 2 * nk + 2 * nv}


def launch_flops(w) -> dict:
    """Algorithmic FLOPs per launch (a multiply-add counts 2), per token:
    state S += phi(k) v^T and z += phi(k): 2 D (Dv + 1); output phi(q) S and
    phi(q) . z: 2 D (Dv + 1); bwd Q side u = S dO, phi(q) . u, dS += phi(q) g^T
    and dz += c phi(q): 2 D (2 Dv + 2); bwd K/V side dS v + dz and dS^T phi(k):
    2 D (2 Dv + 1)."""
    n, D, Dv = w.B * w.H * w.T, w.D, w.dv
    return {"fwd_state": 2 * n * D * (Dv + 1), "fwd_output": 2 * n * D * (Dv + 1),
            "bwd_dq": 2 * n * D * (2 * Dv + 2), "bwd_dkv": 2 * n * D * (2 * Dv + 1)}


# Dense MFMA peaks of MI355X (published; no sparsity), TFLOP/s per operand type
MFMA_PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0, "bf16": 2500.0}
DTYPE_NAME = {"f32": "f32", "f16": "f16", "bf16": "bf16"}


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def cpu_baseline(w, x, max_heads: int, gpu_out: dict | None = None) -> dict:
    """The fp64 oracle as it stands, forward then backward, per head on a
    thread pool of the host's cores (at most 16: one GPU's share of the box).

    The oracle's outputs for the sampled heads are then held against the
    GPU's outputs of the timed steps (gpu_out: device tensors O, dQ, dK, dV),
    outside every timed region: the bench line carries the normwise max
    relative error of each tensor over those heads."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    import oracle

    n = w.B * w.H
    heads = min(n, max_heads)
    available = len(os.sched_getaffinity(0))
    cores = max(1, min(available, 16))
    qh, kh = (x[nm].reshape(n, w.T, w.D) for nm in ("q", "k"))
    vh, dh = (x[nm].reshape(n, w.T, w.dv) for nm in ("v", "do"))

    def fwd_one(h):
        return oracle.fwd_head(oracle.decode(qh[h], w.dtype), oracle.decode(kh[h], w.dtype),
                               oracle.decode(vh[h], w.dtype), w.eps, w.simple)[0]

    def bwd_one(h):
        return oracle.bwd_head(oracle.decode(qh[h], w.dtype), oracle.decode(kh[h], w.dtype),
                               oracle.decode(vh[h], w.dtype), oracle.decode(dh[h], w.dtype),
                               w.eps, w.simple)

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=cores) as pool:
        list(pool.map(fwd_one, range(min(heads, cores))))  # warm-up
        t0 = time.perf_counter()
        o_ref = list(pool.map(fwd_one, range(heads)))
        t1 = time.perf_counter()
        g_ref = list(pool.map(bwd_one, range(heads)))
        t2 = time.perf_counter()
    fwd_bytes = 2 * heads * w.T * (w.D + w.dv) * w.elem_bytes
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    res = {
        "value": fwd_bytes / (t1 - t0) / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "cores_available": available,
        "kind": "oracle",
        "sample": f"{heads} of {n} heads at T={w.T}, D={w.D}, Dv={w.dv}: fp64 forward then backward, "
                  f"one head per thread on {cores} threads",
        "fwd_ms_sample": (t1 - t0) * 1e3,
        "bwd_ms_sample": (t2 - t1) * 1e3,
        "cpu": model,
    }
    if gpu_out is not None:
        res["parity_vs_oracle"] = parity(w, heads, gpu_out, o_ref, g_ref)
    return res


def parity(w, heads: int, gpu_out: dict, o_ref, g_ref) -> dict:
    """Normwise max relative error max|X - R| / max|R| per tensor and head
    (the worst head reported) of the timed steps' outputs against the oracle."""
    import oracle

    n = w.B * w.H
    worst = {}
    for name, refs, width in (("O", o_ref, w.dv), ("dQ", [g[0] for g in g_ref], w.D),
                              ("dK", [g[1] for g in g_ref], w.D), ("dV", [g[2] for g in g_ref], w.dv)):
        t = gpu_out.get(name)
        if t is None:
            continue
        t = t.reshape(n, w.T, width)
        e = 0.0
        for h in range(heads):
            got = oracle.decode(storage(t[h]), w.dtype)
            r = refs[h]
            e = max(e, float(np.max(np.abs(got - r)) / max(float(np.max(np.abs(r))), 1e-300)))
        worst[name] = float(f"{e:.3e}")
    tol = 2e-2 if w.dtype == "bf16" else 5e-3
    return {"max_rel_err": worst, "heads": heads, "tolerance": tol,
            "pass": all(v <= tol for v in worst.values()),
            "metric": "per tensor, the worst over the heads of max|X - R| / max|R|"}


def storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor to the host storage format the oracle decodes."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def versions() -> dict:
    """Toolchain and library versions of this run (no child process: the
    compiler that built libla.so is read from the file the build wrote beside
    it, the HIP runtime's version from the runtime torch has loaded)."""
    import ctypes

    out = {"torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
           "la_version": int(la.lib().la_version())}
    try:
        out["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        out["rocm"] = None
    try:
        out["hipcc"] = json.load(open(os.path.join(ROOT, "non_causal_linear_amd", "libla.build.json")))["hipcc"]
    except (OSError, ValueError, KeyError):
        out["hipcc"] = None
    try:
        rt = ctypes.c_int(0)
        if ctypes.CDLL("libamdhip64.so").hipRuntimeGetVersion(ctypes.byref(rt)) == 0:
            out["hip_runtime"] = rt.value
    except OSError:
        pass
    try:
        out["gpu"] = torch.cuda.get_device_properties(0).gcnArchName
    except (AttributeError, RuntimeError):
        out["gpu"] = None
    return out


def copy_bandwidth(reps: int = 10) -> float:
    """GB/s of a plain 1 GiB device-to-device copy (read + write bytes over the
    mean time): what a streaming kernel can reach on this machine. Context, not
    the target."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    del src, dst
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


def torch_eager(w, q, k, v, do, do_flush, reps: int = 3) -> dict:
    """The same formula in plain torch ops, fp32, forward and forward + backward
    (autograd), on the same inputs and with the same flush: the eager
    baseline a torch user would write. Context only."""
    def forward(q32, k32, v32):
        qt = torch.nn.functional.elu(q32) + 1
        kt = torch.nn.functional.elu(k32) + 1
        s_ = torch.matmul(kt.transpose(-1, -2).contiguous(), v32)
        num = torch.matmul(qt, s_)
        if w.simple:
            return num
        z = kt.sum(dim=-2, keepdim=True)
        return num / ((qt * z).sum(dim=-1, keepdim=True) + w.eps)

    def once(bwd):
        q32, k32, v32 = (x.float().requires_grad_(bwd) for x in (q, k, v))
        o = forward(q32, k32, v32)
        if bwd:
            o.backward(do.float())
        return o

    with torch.no_grad():
        once(False)
    once(True)
    torch.cuda.synchronize()
    out = {}
    for key, bwd in (("fwd_ms", False), ("fwd_bwd_ms", True)):
        ts = []
        for _ in range(reps):
            do_flush("read")
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if bwd:
                once(True)
            else:
                with torch.no_grad():
                    once(False)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        out[key] = round(float(np.mean(ts)), 3)
    torch.cuda.empty_cache()
    return out


def causal_bench(args, w, t, do_flush) -> int:
    """The causal path: one la_fwd call (segment states, their prefixes, the
    chunked scan), then one la_bwd call with LA_REUSE_PREFIX on the same
    workspace (the forward-order dQ scan from the prefixes the forward left
    there, the suffixes of its segment sums, the reverse-order dK, dV scan),
    as a training step runs them. Rates count the algorithmic minimum: one
    pass over Q, K, V and O forward, over Q, K, V, dO and dQ, dK, dV backward;
    the forward reads K and V once more (the segment states)."""
    q, k, v, do, o, dq, dk, dv = (t[n] for n in ("q", "k", "v", "do", "o", "dq", "dk", "dv"))
    prob = la.make_problem(q.shape, q.dtype, w.eps, w.simple, dv=w.dv, causal=True)
    state = la.new_state(prob, q.device)
    ws = la.workspace(prob, q.device)

    def step(ev):
        ev[0].record()
        la.fwd(q, k, v, eps=w.eps, simple=w.simple, out=o, state=state, ws=ws, causal=True)
        ev[1].record()
        la.bwd(q, k, v, do, None, eps=w.eps, simple=w.simple, dq=dq, dk=dk, dv=dv, ws=ws, causal=True,
               reuse_prefix=True)
        ev[2].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3)]  # noqa: E731
    for _ in range(args.warmup):
        do_flush(args.flush)
        step(mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        do_flush(args.flush)
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.array([ev[0].elapsed_time(ev[1]) for ev in events])
    bwd_ms = np.array([ev[1].elapsed_time(ev[2]) for ev in events])
    lb = launch_bytes(w)
    alg_f = lb["fwd_state"] + lb["fwd_output"]  # Q, K, V in, O out
    alg_b = lb["bwd_dq"] + lb["bwd_dkv"]  # Q, K, V, dO in, dQ, dK, dV out
    value = alg_f / (float(np.mean(fwd_ms)) * 1e-3) / 1e9
    bwd_rate = alg_b / (float(np.mean(bwd_ms)) * 1e-3) / 1e9
    line = {
        "metric": "causal LA fwd GB/s (algorithmic Q, K, V, O bytes) and ms",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(fwd_ms + bwd_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.dtype],
        "data": "synthetic: seeded N(0, sigma^2) Q, K, V, dO rounded to the dtype",
        "config": {"workload": w.name + "-causal", "B": w.B, "H": w.H, "T": w.T, "D": w.D, "Dv": w.dv,
                   "mode": ("simple_la" if w.simple else "normalised") + ", causal", "pass": "fwd+bwd"},
        "fwd_ms": round(float(np.mean(fwd_ms)), 4),
        "fwd_ms_min": round(float(np.min(fwd_ms)), 4),
        "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
        "fwd_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "bwd_ms": round(float(np.mean(bwd_ms)), 4),
        "bwd_ms_median": round(float(np.median(bwd_ms)), 4),
        "bwd_reuses_forward_prefixes": True,
        "split": la.split_of(prob),
        "bwd_GBps_algorithmic": round(bwd_rate, 1),
        "bwd_frac_of_hbm_peak": round(bwd_rate / HBM_PEAK_GBS, 4),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "roofline": {"kernel": "la_fwd causal (state, prefix, chunked scan)", "bound": "hbm",
                     "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None},
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(ALL_WORKLOADS))
    ap.add_argument("--flush", choices=("read", "write", "none"), default="read",
                    help="cache flush before each step: read 1 GiB (default), write 1 GiB, or none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=128, help="heads in the oracle sample")
    ap.add_argument("--all-cache-conditions", action="store_true",
                    help="also time the step after a writing flush and with no flush")
    ap.add_argument("--causal", action="store_true",
                    help="time the causal forward and backward (LA_CAUSAL) instead of the bidirectional path")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements (device copy bandwidth, torch eager baseline)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards over heads with no communication; see the design notes)",
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is a single-process, single-GPU benchmark", file=sys.stderr)
        return 2
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    w = ALL_WORKLOADS[args.workload]
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    prob = la.make_problem(q.shape, q.dtype, w.eps, w.simple, dv=w.dv)
    state = la.new_state(prob, q.device)
    ws = la.workspace(prob, q.device)
    o, dv = torch.empty_like(v), torch.empty_like(v)
    dq, dk = torch.empty_like(q), torch.empty_like(q)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB

    def do_flush(mode):
        if mode == "read":
            flush.sum()
        elif mode == "write":
            flush.fill_(1.0)

    def step(ev):
        ev[0].record()
        la.fwd_state(k, v, eps=w.eps, simple=w.simple, state=state, ws=ws)
        ev[1].record()
        la.fwd_output(q, state, eps=w.eps, simple=w.simple, out=o)
        ev[2].record()
        if w.bwd:
            la.bwd_dq(q, do, state, eps=w.eps, simple=w.simple, dq=dq, ws=ws)
            ev[3].record()
            la.bwd_dkv(k, v, eps=w.eps, simple=w.simple, dk=dk, dv=dv, ws=ws)
        else:
            ev[3].record()
        ev[4].record()

    if args.causal:
        return causal_bench(args, w, {"q": q, "k": k, "v": v, "do": do, "o": o, "dq": dq, "dk": dk, "dv": dv},
                            do_flush)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(5)]  # noqa: E731
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        do_flush(args.flush)
        step(mk())
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    events = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        do_flush(args.flush)  # evict the infinity cache and L2s, outside the events
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # The same step under the other two cache conditions, for context: a
    # writing flush (what L2-flushing benchmark helpers usually do) and none
    # (back-to-back steps: each pays the write-back of the previous one's
    # outputs that the 256 MB infinity cache still holds).
    other = {}
    for mode in ("read", "write", "none") if args.all_cache_conditions else ():
        if mode == args.flush:
            continue
        evs = [mk() for _ in range(min(args.steps, 10))]
        for ev in evs:
            do_flush(mode)
            step(ev)
        torch.cuda.synchronize()
        f = np.mean([ev[0].elapsed_time(ev[2]) for ev in evs])
        other[mode] = {"fwd_ms": round(float(f), 4),
                       "fwd_bwd_ms": round(float(np.mean([ev[0].elapsed_time(ev[4]) for ev in evs])), 4)}

    per = {kname: np.array([ev[j].elapsed_time(ev[j + 1]) for ev in events])
           for j, kname in enumerate(KERNELS)}
    if not w.bwd:
        per = {kname: per[kname] for kname in ("fwd_state", "fwd_output")}
    step_ms = np.array([ev[0].elapsed_time(ev[4]) for ev in events])
    fwd_ms = per["fwd_state"] + per["fwd_output"]
    lb = launch_bytes(w)
    fwd_bytes = lb["fwd_state"] + lb["fwd_output"]
    value = fwd_bytes / (float(np.mean(fwd_ms)) * 1e-3) / 1e9

    avg = {kname: float(np.mean(a)) for kname, a in per.items()}
    dominant = max(avg, key=avg.get)
    dom_bytes = lb[dominant]
    achieved = dom_bytes / (avg[dominant] * 1e-3) / 1e9
    # the dominant kernel's bound: the larger of its HBM and MFMA fractions
    # (fp32 operands run MFMA at 157.3 TFLOP/s, below what 8 TB/s would feed)
    tflops = launch_flops(w)[dominant] / (avg[dominant] * 1e-3) / 1e12
    mfma_frac = tflops / MFMA_PEAK_TFLOPS[w.dtype]
    if mfma_frac > achieved / HBM_PEAK_GBS:
        roof = {"kernel": dominant, "bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": round(mfma_frac, 4), "traffic": None,
                "hbm_GBps": round(achieved, 1), "hbm_frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "mfma_TFLOPs": round(tflops, 2), "mfma_frac": round(mfma_frac, 4)}

    # one more step after the timed ones (untimed): its outputs must equal the
    # last timed step's byte for byte
    outs = {"O": o, "state": state}
    if w.bwd:
        outs.update({"dQ": dq, "dK": dk, "dV": dv})
    kept = {nm: t.clone() for nm, t in outs.items()}
    do_flush(args.flush)
    step(mk())
    torch.cuda.synchronize()
    bit_identical = all(torch.equal(kept[nm].view(torch.uint8), outs[nm].view(torch.uint8)) for nm in outs)
    del kept

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    line = {
        "metric": "non-causal LA fwd GB/s & ms (B8-H16-T16384-D64 fp16); fwd+bwd ms",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.dtype],
        "data": "synthetic: seeded N(0, sigma^2) Q, K, V, dO rounded to the dtype",
        "config": {
            "workload": w.name + ("-simple" if w.simple and "simple" not in w.name else ""),
            "B": w.B, "H": w.H, "T": w.T, "D": w.D, "Dv": w.dv,
            "mode": "simple_la" if w.simple else "normalised",
            "eps": w.eps,
            "pass": "fwd+bwd" if w.bwd else "fwd",
            "cache_flush_before_step": {"read": "read 1 GiB", "write": "write 1 GiB",
                                        "none": "none"}[args.flush],
        },
        "fwd_ms": round(float(np.mean(fwd_ms)), 4),
        "fwd_ms_min": round(float(np.min(fwd_ms)), 4),
        "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
        "fwd_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernel_ms": {kname: round(a, 4) for kname, a in avg.items()},
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        **({"other_cache_conditions": other} if other else {}),
        "bit_identical_rerun": bit_identical,
        "split": la.split_of(prob),
        "versions": versions(),
        "roofline": roof,
    }
    # HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    # (scaled by a 1 GiB copy), valid only while the kernels are unchanged
    tpath = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tpath):
        t = json.load(open(tpath))
        src = os.path.join(ROOT, "non_causal_linear_amd", "csrc", "la_kernels.hip")
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if t.get("kernel_source_sha256_prefix") == h and dominant in t.get("per_step_call_bytes", {}):
            tb = t["per_step_call_bytes"][dominant]
            line["roofline"]["traffic"] = round(tb)
            line["roofline"]["traffic_unit"] = "bytes/launch"
            line["roofline"]["traffic_over_algorithmic"] = round(tb / dom_bytes, 4)
            line["roofline"]["traffic_source"] = (f"stored rocprofv3 FETCH_SIZE and WRITE_SIZE runs on this "
                                                  f"kernel source (sha256 {h}), profiles/traffic_{w.name}.json")
    if w.bwd:
        bwd_ms = per["bwd_dq"] + per["bwd_dkv"]
        line["bwd_ms"] = round(float(np.mean(bwd_ms)), 4)
        line["fwd_bwd_ms"] = round(float(np.mean(step_ms)), 4)
        line["fwd_bwd_ms_min"] = round(float(np.min(step_ms)), 4)
        line["fwd_bwd_ms_median"] = round(float(np.median(step_ms)), 4)
    if w.name == HEADLINE:
        line["context_pages_a800_triton"] = {"fwd_ms": PAGE_A800_FWD_MS, "bwd_ms": PAGE_A800_BWD_MS,
                                             "note": "another GPU, dtype unstated: context only"}
    if not args.no_context:
        print("[bench] context: device copy, torch eager", file=sys.stderr, flush=True)
        line["context_copy_1GiB_GBps"] = round(copy_bandwidth(), 1)
        if w.bwd:
            line["context_torch_eager_fp32"] = torch_eager(w, q, k, v, do, do_flush)
    if not args.no_cpu_baseline:
        print("[bench] oracle on host cores", file=sys.stderr, flush=True)
        gpu_out = {"O": o}
        if w.bwd:
            gpu_out.update({"dQ": dq, "dK": dk, "dV": dv})
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_heads, gpu_out)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
