"""GPU parity of the optional query scale (la_problem.scale: phi(q) becomes
scale * phi(q)) against the fp64 oracle with the same scale: the bidirectional
and causal paths, forward and backward, both modes, the step calls, autograd,
a full-size simple_la case; scale 1 is byte-identical to no scale. eps is
large in normalised mode so that eps / scale visibly moves the result."""
import ctypes

import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs
from tests.la_testutil import TOL, bytes_equal, decode, max_rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def check(name, got, ref, dtype):
    err = max_rel_err(got, ref)
    print(f"  {name}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert err <= TOL[dtype], f"{name}: {err:.3e} > {TOL[dtype]}"


def workload(T, D, Dv, dtype, simple, seed):
    return Workload("scale", 2, 3, T, D, dtype, simple=simple, seed=seed, Dv=Dv, eps=0.0 if simple else 1000.0)


@pytest.mark.parametrize("scale", [0.125, 3.0])
@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D,Dv", [(64, 64), (32, 96)], ids=["D64", "D32-Dv96"])
def test_scale_bidirectional(D, Dv, dtype, simple, scale):
    seed = 96_000 + D + Dv + 7 * ["f32", "f16", "bf16"].index(dtype) + (3 if simple else 0) + int(8 * scale)
    w = workload(1000, D, Dv, dtype, simple, seed)
    print(f"case scale={scale} D={D} Dv={Dv} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, dtype) for n, a in x.items()}
    o, st = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=simple, scale=scale)
    g = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], st, eps=w.eps, simple=simple, scale=scale)
    torch.cuda.synchronize()
    o_ref, _, _ = oracle.fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple, scale=scale)
    check("O", decode(o, dtype), o_ref, dtype)
    for name, a, r in zip(("dQ", "dK", "dV"), g, oracle.bwd(x["q"], x["k"], x["v"], x["do"], dtype, w.eps, simple,
                                                          scale=scale)):
        check(name, decode(a, dtype), r, dtype)
    # the step calls give the same bytes
    st2 = la.fwd_state(dev["k"], dev["v"], eps=w.eps, simple=simple)
    o2 = la.fwd_output(dev["q"], st2, eps=w.eps, simple=simple, scale=scale, dv=Dv)
    ws = la.workspace(la.make_problem(dev["q"].shape, dev["q"].dtype, w.eps, simple, dv=Dv), dev["q"].device)
    dq2 = la.bwd_dq(dev["q"], dev["do"], st2, eps=w.eps, simple=simple, scale=scale, ws=ws)
    dk2, dv2 = la.bwd_dkv(dev["k"], dev["v"], eps=w.eps, simple=simple, ws=ws)
    torch.cuda.synchronize()
    for a, b in zip((o2, dq2, dk2, dv2), (o,) + tuple(g)):
        assert bytes_equal(a, b)


@pytest.mark.parametrize("scale", [0.125, 3.0])
@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,Dv", [(64, 64), (128, 64)], ids=["D64", "D128-Dv64"])
def test_scale_causal(D, Dv, dtype, simple, scale):
    seed = 97_000 + D + Dv + 7 * ["f16", "bf16"].index(dtype) + (3 if simple else 0) + int(8 * scale)
    w = workload(1000, D, Dv, dtype, simple, seed)
    print(f"case causal scale={scale} D={D} Dv={Dv} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, dtype) for n, a in x.items()}
    o, _ = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=simple, scale=scale, causal=True)
    g = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], None, eps=w.eps, simple=simple, scale=scale, causal=True)
    torch.cuda.synchronize()
    o_ref, _, _ = oracle.causal_fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple, scale=scale)
    check("O", decode(o, dtype), o_ref, dtype)
    for name, a, r in zip(("dQ", "dK", "dV"), g, oracle.causal_bwd(x["q"], x["k"], x["v"], x["do"], dtype, w.eps,
                                                                 simple, scale=scale)):
        check(name, decode(a, dtype), r, dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_one_is_no_scale(causal):
    w = workload(777, 64, 64, "f16", False, 98_000 + int(causal))
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, "f16") for n, a in x.items()}
    outs = []
    for sc in (None, 1.0):
        o, st = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, scale=sc, causal=causal)
        g = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], None if causal else st, eps=w.eps, scale=sc,
                   causal=causal)
        outs.append((o,) + tuple(g))
    # a zero scale in the C struct stands for 1 (the binding refuses 0 itself)
    prob = la.make_problem(dev["q"].shape, dev["q"].dtype, w.eps, False, causal=causal)
    prob.scale = 0.0
    o0 = torch.empty_like(outs[0][0])
    ws = la.workspace(prob, dev["q"].device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    status = la.lib().la_fwd(ctypes.byref(prob), ptr(dev["q"]), ptr(dev["k"]), ptr(dev["v"]), ptr(o0), None,
                             ptr(ws), ctypes.c_size_t(ws.numel()), stream)
    assert status == 0
    torch.cuda.synchronize()
    assert bytes_equal(o0, outs[0][0])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert bytes_equal(a, b)


def test_scale_full_size_simple_sampled_rows():
    """B8 H16 T16384 D64 f16, simple_la, scale 1/8: sampled output rows of four
    heads against the oracle's per-row form."""
    w = Workload("scale-long", 8, 16, 16384, 64, "f16", simple=True, seed=98_100)
    x = make_inputs(w, with_grad=False)
    dev = {n: to_device(a, "f16") for n, a in x.items()}
    o, _ = la.fwd(dev["q"], dev["k"], dev["v"], simple=True, scale=0.125)
    torch.cuda.synchronize()
    n = w.B * w.H
    hd = {nm: oracle.decode(a, "f16").reshape(n, w.T, -1) for nm, a in x.items()}
    rng = np.random.default_rng(w.seed)
    worst = 0.0
    for h in (0, 41, 90, n - 1):
        rows = sorted({0, w.T - 1} | {int(t) for t in rng.integers(0, w.T, size=16)})
        ref = oracle.sampled_rows_head(hd["q"][h], hd["k"][h], hd["v"][h], rows, w.eps, True, scale=0.125)
        worst = max(worst, max_rel_err(decode(o.reshape(n, w.T, -1)[h][rows], "f16"), ref))
    print(f"  O sampled rows: {worst:.3e}", flush=True)
    assert worst <= TOL["f16"]


@pytest.mark.parametrize("causal", [False, True])
def test_scale_autograd(causal):
    w = workload(300, 64, 64, "bf16", False, 98_200 + int(causal))
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, "bf16").requires_grad_(n != "do") for n, a in x.items()}
    o = la.linear_attention(dev["q"], dev["k"], dev["v"], eps=w.eps, causal=causal, scale=0.5)
    (o.float() * dev["do"].float()).sum().backward()
    torch.cuda.synchronize()
    fb = oracle.causal_bwd if causal else oracle.bwd
    for name, r in zip(("q", "k", "v"), fb(x["q"], x["k"], x["v"], x["do"], "bf16", w.eps, False, scale=0.5)):
        check("d" + name.upper(), decode(dev[name].grad, "bf16"), r, "bf16")
