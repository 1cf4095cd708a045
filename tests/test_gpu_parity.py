"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every element; they span several tiles and slices and end
on ragged tails. The five named workloads run at full size in the launch
configuration the benchmark times: the fp32 state (S, z) is checked for every
head, O/dQ/dK/dV completely on four heads (first, last, two seeded picks), O on
sampled rows of every other head, and dQ/dK/dV on the same sampled rows of every
head (slice boundaries included). Results must also be bit-identical
across reruns.
"""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import WORKLOADS, Workload, make_inputs
from tests.la_testutil import (TIGHT, TOL, TORCH_DTYPE, bytes_equal, decode, max_rel_err,
                               split_state, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    torch.manual_seed(0)


def run(w: Workload, x: dict, bwd: bool):
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    o, state = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=w.simple)
    out = {"o": o, "state": state}
    if bwd:
        out["dq"], out["dk"], out["dv"] = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], state,
                                                 eps=w.eps, simple=w.simple)
    torch.cuda.synchronize()
    return dev, out


def check(name, got, ref, dtype, where="", scale=None):
    """Normwise max relative error; ``scale`` (if given) replaces max|ref| when larger:
    the size of summands that cancel in an ill-conditioned result."""
    err = max_rel_err(got, ref)
    if scale is not None and scale > np.max(np.abs(ref)):
        err = float(np.max(np.abs(got - ref)) / scale)
        where += " (vs leading terms)"
    print(f"  {name}{where}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}{where}: non-finite output"
    assert err <= TOL[dtype], f"{name}{where}: {err:.3e} > {TOL[dtype]}"
    if dtype in TIGHT:
        assert err <= TIGHT[dtype], f"{name}{where}: {err:.3e} > {TIGHT[dtype]} (fp32 bar)"
    return err


def heads_of(x, dtype):
    d = oracle.decode(x, dtype)
    return d.reshape(-1, d.shape[-2], d.shape[-1])


# ------------------------------------------------------------- small, full compare

SMALL_T = [1, 129, 1000, 4097]


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", SMALL_T)
def test_small_fwd_bwd_all_elements(T, D, dtype, simple):
    seed = 10_000 + 97 * T + D + 7 * ["f32", "f16", "bf16"].index(dtype) + (3 if simple else 0)
    w = Workload("small", 2, 3, T, D, dtype, simple=simple, seed=seed)
    print(f"case T={T} D={D} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w)
    _, out = run(w, x, bwd=True)
    o_ref, s_ref, z_ref = oracle.fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], dtype, w.eps, simple)
    s_got, z_got = split_state(out["state"], w.B, w.H, D)
    check("S", s_got, s_ref, dtype)
    check("z", z_got, z_ref, dtype)
    check("O", decode(out["o"], dtype), o_ref, dtype)
    sq = sk = None
    if T == 1 and not simple:
        # the exact dQ, dK are O(eps): two O(1) summands cancel; measure the
        # error against those summands instead of the result
        sc = [oracle.bwd_leading_terms_head(*(oracle.decode(x[n], dtype)[b, h]
                                              for n in ("q", "k", "v", "do")), w.eps)
              for b in range(w.B) for h in range(w.H)]
        sq, sk = max(a for a, _ in sc), max(b for _, b in sc)
    check("dQ", decode(out["dq"], dtype), dq_ref, dtype, scale=sq)
    check("dK", decode(out["dk"], dtype), dk_ref, dtype, scale=sk)
    check("dV", decode(out["dv"], dtype), dv_ref, dtype)


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_many_heads_single_slice_ragged(D, dtype, simple):
    """640 heads of 300 tokens: enough heads that every step runs one slice or
    chunk per head (the state and dS go straight to their outputs, no
    partials), each ending on a ragged tail inside its first rounds."""
    seed = 20_000 + D + 7 * ["f16", "bf16"].index(dtype) + (3 if simple else 0)
    w = Workload("many-heads", 4, 160, 300, D, dtype, simple=simple, seed=seed)
    print(f"case B4 H160 T300 D={D} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w)
    _, out = run(w, x, bwd=True)
    o_ref, s_ref, z_ref = oracle.fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], dtype, w.eps, simple)
    s_got, z_got = split_state(out["state"], w.B, w.H, D)
    check("S", s_got, s_ref, dtype)
    check("z", z_got, z_ref, dtype)
    check("O", decode(out["o"], dtype), o_ref, dtype)
    check("dQ", decode(out["dq"], dtype), dq_ref, dtype)
    check("dK", decode(out["dk"], dtype), dk_ref, dtype)
    check("dV", decode(out["dv"], dtype), dv_ref, dtype)


@pytest.mark.parametrize("D,dtype", [(64, "f16"), (128, "bf16")])
def test_max_head_size_periodic(D, dtype):
    """The largest head the library accepts (T * D * 2 bytes just below 2^31),
    one head, ragged against every tile and slice size. The inputs repeat a
    seeded 4096-row block, so the exact state is n S(block) + S(first r rows)
    and dS, dz likewise (given the full S, z), and any output row follows from
    its own inputs and the states: the state and sampled rows of O, dQ, dK,
    dV are compared with the oracle."""
    from synth import normal
    T = (1 << 31) // (D * 2) - 1
    period, eps = 4096, 1e-6
    nfull, rem = divmod(T, period)
    seed = 30_000 + D
    sigma = 1.0 if D == 64 else 0.5
    blk = {n: normal((period, D), seed + i, sigma, dtype) for i, n in enumerate(("q", "k", "v", "do"))}
    print(f"case B1 H1 T={T} D={D} {dtype} period={period} seed={seed}", flush=True)
    dev = {n: to_device(np.resize(a, (T, D)), dtype).view(1, 1, T, D) for n, a in blk.items()}
    o, state = la.fwd(dev["q"], dev["k"], dev["v"], eps=eps)
    dq, dk, dv = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], state, eps=eps)
    torch.cuda.synchronize()
    x = {n: oracle.decode(a, dtype) for n, a in blk.items()}
    s1, z1 = oracle.state_head(x["k"], x["v"])
    s2, z2 = oracle.state_head(x["k"][:rem], x["v"][:rem])
    s_ref, z_ref = nfull * s1 + s2, nfull * z1 + z2
    s_got, z_got = split_state(state, 1, 1, D)
    check("S", s_got[0, 0], s_ref, dtype)
    check("z", z_got[0, 0], z_ref, dtype)
    _, ds1, dz1 = oracle.bwd_q_side_head(x["q"], x["do"], s_ref, z_ref, eps, False)
    _, ds2, dz2 = oracle.bwd_q_side_head(x["q"][:rem], x["do"][:rem], s_ref, z_ref, eps, False)
    ds_ref, dz_ref = nfull * ds1 + ds2, nfull * dz1 + dz2
    rng = np.random.default_rng(seed)
    rows = sorted(set([0, 1, period - 1, period, T // 2, T - rem - 1, T - rem, T - 2, T - 1]
                      + [int(t) for t in rng.integers(0, T, size=48)]))
    idx = torch.tensor(rows, device="cuda")
    b = [t % period for t in rows]
    got = {n: decode(t[0, 0].index_select(0, idx), dtype) for n, t in
           (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv))}
    dq_ref, _, _ = oracle.bwd_q_side_head(x["q"][b], x["do"][b], s_ref, z_ref, eps, False)
    dk_ref, dv_ref = oracle.bwd_kv_side_head(x["k"][b], x["v"][b], ds_ref, dz_ref, False)
    check("O", got["O"], oracle.output_head(x["q"][b], s_ref, z_ref, eps, False), dtype, " (sampled rows)")
    check("dQ", got["dQ"], dq_ref, dtype, " (sampled rows)")
    check("dK", got["dK"], dk_ref, dtype, " (sampled rows)")
    check("dV", got["dV"], dv_ref, dtype, " (sampled rows)")


# ------------------------------------------------------------- full-size workloads

def grad_rows(T, seed, extra=40):
    """Rows at both sides of every boundary of a power-of-two split of T into
    up to 64 pieces, the first and last rows, and seeded picks."""
    rows = {0, 1, T - 2, T - 1}
    for p in (2, 4, 8, 16, 32, 64):
        for i in range(1, p):
            b = i * T // p
            rows.update((b - 1, b))
    rows.update(int(t) for t in np.random.default_rng(seed).integers(0, T, size=extra))
    return sorted(r for r in rows if 0 <= r < T)


def sampled_heads(n, seed):
    rng = np.random.default_rng(seed)
    picks = [0, n - 1] + [int(h) for h in rng.choice(np.arange(1, max(n - 1, 2)), size=2)]
    return sorted(set(h for h in picks if 0 <= h < n))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    w = WORKLOADS[name]
    modes = [False, True] if name.startswith("B1-H2-T128") else [w.simple]
    print(f"workload {name}", flush=True)
    x = make_inputs(w, with_grad=True)
    for simple in modes:
        wm = Workload(w.name, w.B, w.H, w.T, w.D, w.dtype, w.sigma, simple, w.eps, w.bwd, w.seed)
        dev, out = run(wm, x, bwd=w.bwd)
        n = w.B * w.H
        qh, kh, vh = heads_of(x["q"], w.dtype), heads_of(x["k"], w.dtype), heads_of(x["v"], w.dtype)
        s_got, z_got = split_state(out["state"], w.B, w.H, w.D)
        s_got, z_got = s_got.reshape(n, w.D, w.D), z_got.reshape(n, w.D)
        # the same sampled rows of dQ, dK, dV on every head: the slice and
        # chunk boundaries of every power-of-two split up to 64 (either side),
        # the ends, and seeded picks
        if w.bwd:
            rows = grad_rows(w.T, w.seed + 41)
            idx = torch.tensor(rows, device="cuda")
            g_rows = {nm: decode(out[nm].reshape(n, w.T, w.D).index_select(1, idx), w.dtype)
                      for nm in ("dq", "dk", "dv")}
            dh_all = heads_of(x["do"], w.dtype)
        # state of every head, and its gradient rows from the oracle's two
        # halves of the backward with that head's own S, z, dS, dz
        worst_s = worst_z = 0.0
        worst_g = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
        for h in range(n):
            s_ref, z_ref = oracle.state_head(kh[h], vh[h])
            worst_s = max(worst_s, max_rel_err(s_got[h], s_ref))
            worst_z = max(worst_z, max_rel_err(z_got[h], z_ref))
            if w.bwd:
                dq_ref, ds_ref, dz_ref = oracle.bwd_q_side_head(qh[h], dh_all[h], s_ref, z_ref, w.eps, simple)
                dk_ref, dv_ref = oracle.bwd_kv_side_head(kh[h][rows], vh[h][rows], ds_ref, dz_ref, simple)
                for nm, ref in (("dq", dq_ref[rows]), ("dk", dk_ref), ("dv", dv_ref)):
                    worst_g[nm] = max(worst_g[nm], max_rel_err(g_rows[nm][h], ref))
        print(f"  state, all {n} heads: S {worst_s:.3e}  z {worst_z:.3e}", flush=True)
        assert worst_s <= TOL[w.dtype] and worst_z <= TOL[w.dtype]
        if w.bwd:
            print(f"  gradients, {len(rows)} rows on all {n} heads: dQ {worst_g['dq']:.3e}  "
                  f"dK {worst_g['dk']:.3e}  dV {worst_g['dv']:.3e}", flush=True)
            for nm, e in worst_g.items():
                assert e <= TOL[w.dtype], f"{nm} sampled rows, all heads: {e:.3e} > {TOL[w.dtype]}"
            del g_rows, dh_all
        o_all = out["o"].reshape(n, w.T, w.D)
        # complete tensors on sampled heads
        heads = sampled_heads(n, w.seed + 17)
        for h in heads:
            o_ref, _, _ = oracle.fwd_head(qh[h], kh[h], vh[h], w.eps, simple)
            check("O", decode(o_all[h], w.dtype), o_ref, w.dtype, f" head {h}")
            if w.bwd:
                dh = heads_of(x["do"], w.dtype)[h]
                refs = oracle.bwd_head(qh[h], kh[h], vh[h], dh, w.eps, simple)
                for nm, ref in zip(("dq", "dk", "dv"), refs):
                    got = decode(out[nm].reshape(n, w.T, w.D)[h], w.dtype)
                    check(nm, got, ref, w.dtype, f" head {h}")
        # sampled rows of O on every other head (first and last row included)
        rng = np.random.default_rng(w.seed + 29)
        worst = 0.0
        for h in range(n):
            if h in heads:
                continue
            rows = sorted(set([0, w.T - 1] + [int(r) for r in rng.integers(0, w.T, size=6)]))
            ref = oracle.sampled_rows_head(qh[h], kh[h], vh[h], rows, w.eps, simple)
            got = decode(o_all[h][rows], w.dtype)
            worst = max(worst, max_rel_err(got, ref))
        print(f"  O sampled rows, other heads: {worst:.3e}", flush=True)
        assert worst <= TOL[w.dtype]
        # bit-identical across reruns
        _, out2 = run(wm, x, bwd=w.bwd)
        for nm in out:
            assert bytes_equal(out[nm], out2[nm]), f"{nm} differs between runs"
        del dev, out, out2
        torch.cuda.empty_cache()


# ------------------------------------------------------------- invariants and edges

def test_v_ones_gives_ones():
    w = Workload("v1", 2, 2, 3000, 64, "f16", seed=321)
    x = make_inputs(w, with_grad=False)
    x["v"] = np.ones_like(x["v"])
    _, out = run(w, x, bwd=False)
    o = decode(out["o"], "f16")
    err = float(np.max(np.abs(o - 1.0)))
    print(f"  V=ones: max |O-1| = {err:.3e}", flush=True)
    assert err <= 2.0 ** -10


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_joint_kv_permutation_within_tolerance(dtype):
    w = Workload("perm", 1, 2, 2048, 64, dtype, seed=654)
    x = make_inputs(w, with_grad=False)
    perm = np.random.default_rng(3).permutation(w.T)
    xp = dict(x, k=np.ascontiguousarray(x["k"][:, :, perm]), v=np.ascontiguousarray(x["v"][:, :, perm]))
    _, a = run(w, x, bwd=False)
    _, b = run(w, xp, bwd=False)
    oa, ob = decode(a["o"], dtype), decode(b["o"], dtype)
    assert max_rel_err(ob, oa) <= TOL[dtype]


def test_q_row_permutation_permutes_output():
    w = Workload("qperm", 1, 2, 1024, 64, "f16", seed=987)
    x = make_inputs(w, with_grad=False)
    perm = np.random.default_rng(4).permutation(w.T)
    xp = dict(x, q=np.ascontiguousarray(x["q"][:, :, perm]))
    _, a = run(w, x, bwd=False)
    _, b = run(w, xp, bwd=False)
    oa, ob = decode(a["o"], "f16"), decode(b["o"], "f16")
    assert max_rel_err(ob, oa[:, :, perm]) <= TOL["f16"]
    print(f"  Q-row permutation bitwise: {np.array_equal(ob, oa[:, :, perm])}", flush=True)


def test_large_eps_matters():
    # eps comparable to phi(q).z: a misplaced eps would show
    w = Workload("eps", 1, 2, 256, 64, "f32", eps=3000.0, seed=111)
    x = make_inputs(w)
    _, out = run(w, x, bwd=True)
    o_ref, _, _ = oracle.fwd(x["q"], x["k"], x["v"], "f32", w.eps, False)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], "f32", w.eps, False)
    check("O", decode(out["o"], "f32"), o_ref, "f32")
    check("dQ", decode(out["dq"], "f32"), dq_ref, "f32")
    check("dK", decode(out["dk"], "f32"), dk_ref, "f32")
    check("dV", decode(out["dv"], "f32"), dv_ref, "f32")


def test_t_zero_writes_zero_state():
    q = torch.zeros(2, 3, 0, 64, dtype=torch.float16, device="cuda")
    state = torch.full((2 * 3 * (64 * 64 + 64),), 7.0, device="cuda")
    o, st = la.fwd(q, q.clone(), q.clone(), state=state)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.count_nonzero(st).item() == 0
    dq, dk, dv = la.bwd(q, q.clone(), q.clone(), q.clone(), st)
    assert dq.numel() == dk.numel() == dv.numel() == 0


def test_underflowing_features_give_zero_output():
    # every phi(q) underflows (q = -120): den = eps, O = 0; simple mode also 0
    w = Workload("uf", 1, 1, 300, 64, "f32", seed=5)
    x = make_inputs(w, with_grad=False)
    x["q"] = np.full_like(x["q"], -120.0)
    for simple in (False, True):
        wm = Workload("uf", 1, 1, 300, 64, "f32", simple=simple, seed=5)
        _, out = run(wm, x, bwd=False)
        o = decode(out["o"], "f32")
        assert np.all(np.isfinite(o)) and np.max(np.abs(o)) < 1e-30


def test_step_calls_compose_to_fwd_bwd():
    w = Workload("steps", 2, 4, 3333, 64, "bf16", seed=42)
    x = make_inputs(w)
    dev, out = run(w, x, bwd=True)
    st = la.fwd_state(dev["k"], dev["v"], eps=w.eps)
    o = la.fwd_output(dev["q"], st, eps=w.eps)
    dq = la.bwd_dq(dev["q"], dev["do"], st, eps=w.eps)
    dk, dv = la.bwd_dkv(dev["k"], dev["v"], eps=w.eps)
    torch.cuda.synchronize()
    for a, b in ((st, out["state"]), (o, out["o"]), (dq, out["dq"]), (dk, out["dk"]), (dv, out["dv"])):
        assert bytes_equal(a, b)


def test_reruns_bit_identical_many_slices():
    # B*H = 2 makes the planner split each head into many slices
    w = Workload("det", 1, 2, 50_000, 64, "f16", seed=77)
    x = make_inputs(w)
    _, a = run(w, x, bwd=True)
    for _ in range(2):
        _, b = run(w, x, bwd=True)
        for nm in a:
            assert bytes_equal(a[nm], b[nm]), nm


def test_non_default_stream():
    w = Workload("stream", 1, 2, 777, 128, "f16", seed=9)
    x = make_inputs(w)
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    ref_o, ref_st = la.fwd(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, st = la.fwd(dev["q"], dev["k"], dev["v"])
    s.synchronize()
    assert bytes_equal(o, ref_o) and bytes_equal(st, ref_st)


def test_earlier_hip_error_is_not_reported():
    """A HIP error that an earlier, unrelated call left in this thread (here
    an attribute query for a device that does not exist) is not mistaken for
    a failed launch of the library's kernels."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    val = ctypes.c_int(0)
    status = hip.hipDeviceGetAttribute(ctypes.byref(val), ctypes.c_int(0), ctypes.c_int(1 << 20))
    assert status != 0, "the query for a nonexistent device was expected to fail"
    w = Workload("stale-error", 1, 2, 300, 64, "f16", seed=11)
    x = make_inputs(w, with_grad=True)
    _, out = run(w, x, bwd=True)
    o_ref, _, _ = oracle.fwd(x["q"], x["k"], x["v"], w.dtype, w.eps, False)
    check("O", decode(out["o"], w.dtype), o_ref, w.dtype)
    hip.hipGetLastError()


def _digest_of_run(B, H, T, D, dtype, seed):
    """sha256 over O, state, dQ, dK, dV of one fixed problem (used in two processes)."""
    import hashlib
    w = Workload("proc", B, H, T, D, dtype, seed=seed)
    x = make_inputs(w, with_grad=True)
    _, out = run(w, x, bwd=True)
    h = hashlib.sha256()
    for n in ("o", "state", "dq", "dk", "dv"):
        h.update(out[n].contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def test_outputs_identical_across_processes():
    """The work split is a pure function of the shape and no reduction uses
    atomics, so a second process computes the same bytes."""
    import os
    import subprocess
    import sys
    args = (4, 8, 5000, 64, "f16", 77)
    mine = _digest_of_run(*args)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r); import torch; import non_causal_linear_amd as la; la.lib(); "
            "from tests.test_gpu_parity import _digest_of_run; print(_digest_of_run%r)" % (root, args))
    print("case: second process, B4 H8 T5000 D64 f16 seed 77", flush=True)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=root)
    assert res.returncode == 0, res.stderr[-2000:]
    assert res.stdout.strip().splitlines()[-1] == mine


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
def test_autograd_wrapper_matches_oracle(simple):
    """linear_attention under torch.autograd: the output and the gradients of
    sum(O * dO) for q, k, v against the oracle."""
    w = Workload("autograd", 2, 3, 777, 64, "bf16", simple=simple, seed=51)
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = la.linear_attention(q, k, v, eps=w.eps, simple=simple)
    (o.float() * dev["do"].float()).sum().backward()
    torch.cuda.synchronize()
    o_ref, _, _ = oracle.fwd(x["q"], x["k"], x["v"], w.dtype, w.eps, simple)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], w.dtype, w.eps, simple)
    check("O", decode(o, w.dtype), o_ref, w.dtype)
    check("dQ", decode(q.grad, w.dtype), dq_ref, w.dtype)
    check("dK", decode(k.grad, w.dtype), dk_ref, w.dtype)
    check("dV", decode(v.grad, w.dtype), dv_ref, w.dtype)


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [129, 4097])
def test_token_major_layout(T, D, dtype, simple):
    """[B, T, H, D] tensors (layout "bthd"): the same kernels address the rows
    H * D apart, so every output equals, byte for byte, the [B, H, T, D] run
    on the same values; and it matches the oracle."""
    seed = 40_000 + 97 * T + D + 7 * ["f32", "f16", "bf16"].index(dtype) + (3 if simple else 0)
    w = Workload("bthd", 2, 3, T, D, dtype, simple=simple, seed=seed)
    print(f"case bthd T={T} D={D} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    dev, ref = run(w, x, bwd=True)
    tm = {n: t.transpose(1, 2).contiguous() for n, t in dev.items()}
    o, state = la.fwd(tm["q"], tm["k"], tm["v"], eps=w.eps, simple=simple, layout="bthd")
    dq, dk, dv = la.bwd(tm["q"], tm["k"], tm["v"], tm["do"], state, eps=w.eps, simple=simple, layout="bthd")
    torch.cuda.synchronize()
    assert bytes_equal(state, ref["state"])
    for name, got in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bytes_equal(got.transpose(1, 2).contiguous(), ref[name]), name
    o_ref, _, _ = oracle.fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple)
    check("O", decode(o.transpose(1, 2).contiguous(), dtype), o_ref, dtype)


def test_autograd_wrapper_token_major():
    w = Workload("autograd-bthd", 2, 4, 500, 128, "f16", seed=53)
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, w.dtype).transpose(1, 2).contiguous() for n, a in x.items()}
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = la.linear_attention(q, k, v, eps=w.eps, layout="bthd")
    (o.float() * dev["do"].float()).sum().backward()
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], w.dtype, w.eps, False)
    for name, g, ref in (("dQ", q.grad, dq_ref), ("dK", k.grad, dk_ref), ("dV", v.grad, dv_ref)):
        check(name, decode(g.transpose(1, 2).contiguous(), w.dtype), ref, w.dtype)


@pytest.mark.parametrize("fm,simple", [("relu", False), ("relu", True), ("identity", True), ("identity", False)],
                         ids=["relu-norm", "relu-simple", "identity-simple", "identity-norm"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [129, 4097])
def test_other_feature_maps(T, D, dtype, fm, simple):
    """phi = relu or identity (LA_PHI_RELU, LA_PHI_IDENTITY) against the oracle,
    every element. With the identity map a normalised denominator can vanish,
    so that case takes positive Q and K."""
    from synth import to_storage
    seed = 50_000 + 97 * T + D + 7 * ["f32", "f16", "bf16"].index(dtype) + 3 * ["relu", "identity"].index(fm)
    w = Workload("maps", 2, 3, T, D, dtype, simple=simple, seed=seed)
    print(f"case phi={fm} simple={simple} T={T} D={D} {dtype} seed={seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    if fm == "identity" and not simple:
        for n in ("q", "k"):
            x[n] = to_storage((np.abs(oracle.decode(x[n], dtype)) + 0.5).astype(np.float32), dtype)
    dev = {n: to_device(a, dtype) for n, a in x.items()}
    o, state = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=simple, phi=fm)
    dq, dk, dv = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], state, eps=w.eps, simple=simple, phi=fm)
    torch.cuda.synchronize()
    o_ref, s_ref, z_ref = oracle.fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple, fm)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], dtype, w.eps, simple, fm)
    s_got, z_got = split_state(state, w.B, w.H, D)
    check("S", s_got, s_ref, dtype)
    check("z", z_got, z_ref, dtype)
    check("O", decode(o, dtype), o_ref, dtype)
    check("dQ", decode(dq, dtype), dq_ref, dtype)
    check("dK", decode(dk, dtype), dk_ref, dtype)
    check("dV", decode(dv, dtype), dv_ref, dtype)
