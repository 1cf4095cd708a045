"""GPU parity at head size 256 (D = Dv = 256, f16 and bf16: the wide kernels)
against the fp64 oracle: every element at small sizes (several slices and
blocks, ragged tails, T = 1), the other feature maps and the optional scale,
token-major and strided views byte-identical to the dense call, the step
calls, the allocation-free forward, reruns; and B8-H16-T4096 on every head
(the state completely, O and dQ, dK, dV on sampled rows, two heads whole)."""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs, normal
from tests.la_testutil import TOL, bytes_equal, decode, max_rel_err, split_state, to_device

pytestmark = pytest.mark.gpu

D = 256
SIGMA = {"f16": 1.0, "bf16": 0.5}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def check(name, got, ref, dtype, where="", scale=None):
    err = max_rel_err(got, ref)
    if scale is not None and scale > np.max(np.abs(ref)):
        err = float(np.max(np.abs(got - ref)) / scale)
        where += " (vs leading terms)"
    print(f"  {name}{where}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}{where}: non-finite output"
    assert err <= TOL[dtype], f"{name}{where}: {err:.3e} > {TOL[dtype]}"


def run(w, x, simple, phi="elu1", scale=None):
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    o, st = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=simple, phi=phi, scale=scale)
    g = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], st, eps=w.eps, simple=simple, phi=phi, scale=scale)
    torch.cuda.synchronize()
    return dev, o, st, g


def check_all(w, x, o, st, g, simple, fm="elu1", scale=1.0):
    o_ref, s_ref, z_ref = oracle.fwd(x["q"], x["k"], x["v"], w.dtype, w.eps, simple, fm, scale)
    s_got, z_got = split_state(st, w.B, w.H, D)
    check("S", s_got, s_ref, w.dtype)
    check("z", z_got, z_ref, w.dtype)
    check("O", decode(o, w.dtype), o_ref, w.dtype)
    refs = oracle.bwd(x["q"], x["k"], x["v"], x["do"], w.dtype, w.eps, simple, fm, scale)
    scales = [None, None, None]
    if w.T == 1 and not simple:
        # one token: dQ, dK are O(eps), two O(1) summands cancelling; measure
        # the error against those summands
        sc = [oracle.bwd_leading_terms_head(*(oracle.decode(x[n], w.dtype)[b, h] for n in ("q", "k", "v", "do")),
                                            w.eps, fm)
              for b in range(w.B) for h in range(w.H)]
        scales[:2] = [max(a for a, _ in sc), max(b for _, b in sc)]
    for name, t, r, sc in zip(("dQ", "dK", "dV"), g, refs, scales):
        check(name, decode(t, w.dtype), r, w.dtype, scale=sc)


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T", [1, 100, 1000, 4097])
def test_all_elements(T, dtype, simple):
    seed = 99_000 + 7 * T + (1 if dtype == "bf16" else 0) + (3 if simple else 0)
    # simple_la has no normaliser: with 256 features O grows like T^(1/2) D
    # and leaves f16's range at sigma = 1 (test_simple_overflow_is_inf)
    sigma = 0.25 if simple else SIGMA[dtype]
    w = Workload("d256", 2, 2, T, D, dtype, sigma=sigma, simple=simple, seed=seed)
    print(f"case D256 B2 H2 T={T} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w)
    _, o, st, g = run(w, x, simple)
    check_all(w, x, o, st, g, simple)


def test_simple_overflow_is_inf():
    """simple_la, f16, sigma = 1, T = 4097: where the exact O leaves f16's
    range the library returns inf of the right sign (round to nearest), and
    elsewhere it matches the oracle."""
    w = Workload("d256-ovf", 2, 2, 4097, D, "f16", simple=True, seed=99_050)
    x = make_inputs(w, with_grad=False)
    dev = {n: to_device(a, "f16") for n, a in x.items()}
    o, _ = la.fwd(dev["q"], dev["k"], dev["v"], simple=True)
    torch.cuda.synchronize()
    got = decode(o, "f16")
    ref = oracle.fwd(x["q"], x["k"], x["v"], "f16", w.eps, True)[0]
    big = np.abs(ref) > 66000.0  # past the largest f16 (65504) by more than the fp32 error
    small = np.abs(ref) < 65000.0
    print(f"  {int(big.sum())} of {ref.size} outputs beyond f16", flush=True)
    assert big.any()
    assert np.all(np.isinf(got[big])) and np.all(np.sign(got[big]) == np.sign(ref[big]))
    assert np.all(np.isfinite(got[small]))
    err = float(np.max(np.abs(got[small] - ref[small])) / np.max(np.abs(ref[small])))
    print(f"  O within range: max rel err {err:.3e}", flush=True)
    assert err <= TOL["f16"]


@pytest.mark.parametrize("fm,simple", [("relu", False), ("relu", True), ("identity", True), ("identity", False)])
def test_other_feature_maps(fm, simple):
    from synth import to_storage
    w = Workload("d256-maps", 1, 3, 777, D, "f16", simple=simple, seed=99_100 + 3 * ["relu", "identity"].index(fm))
    print(f"case D256 phi={fm} simple={simple} seed={w.seed}", flush=True)
    x = make_inputs(w)
    if fm == "identity" and not simple:
        for n in ("q", "k"):
            x[n] = to_storage((np.abs(oracle.decode(x[n], "f16")) + 0.5).astype(np.float32), "f16")
    _, o, st, g = run(w, x, simple, fm)
    check_all(w, x, o, st, g, simple, fm)


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
def test_query_scale(simple):
    w = Workload("d256-scale", 1, 2, 600, D, "bf16", sigma=0.5, simple=simple, seed=99_200 + simple)
    x = make_inputs(w)
    _, o, st, g = run(w, x, simple, scale=0.0625)
    check_all(w, x, o, st, g, simple, scale=0.0625)


def test_layouts_and_strides_match_dense():
    """[B, T, H, D] tensors and the q, k, v views of a packed [B, T, 3, H, D]
    buffer give the dense call's bytes."""
    B, T, H = 2, 900, 3
    buf = to_device(normal((B, T, 3, H, D), 99_300, 1.0, "f16"), "f16")
    q, k, v = buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
    do = to_device(normal((B, T, H, D), 99_301, 1.0, "f16"), "f16")
    o, st = la.fwd(q, k, v, layout="bthd")
    g = la.bwd(q, k, v, do, st, layout="bthd")
    dense = [x.transpose(1, 2).contiguous() for x in (q, k, v, do)]
    o2, st2 = la.fwd(*dense[:3])
    g2 = la.bwd(*dense, st2)
    torch.cuda.synchronize()
    assert bytes_equal(st, st2)
    assert bytes_equal(o.transpose(1, 2).contiguous(), o2)
    for a, b in zip(g, g2):
        assert bytes_equal(a.transpose(1, 2).contiguous(), b)


def test_step_calls_noalloc_and_reruns():
    w = Workload("d256-steps", 2, 3, 2100, D, "bf16", sigma=0.5, seed=99_400)
    x = make_inputs(w)
    dev, o, st, g = run(w, x, False)
    st1 = la.fwd_state(dev["k"], dev["v"], eps=w.eps)
    o1 = la.fwd_output(dev["q"], st1, eps=w.eps)
    dq1 = la.bwd_dq(dev["q"], dev["do"], st1, eps=w.eps)
    dk1, dv1 = la.bwd_dkv(dev["k"], dev["v"], eps=w.eps)
    out = torch.full_like(o, float("nan"))
    st_na = torch.full_like(st, float("nan"))
    la.fwd_noalloc(dev["q"], dev["k"], dev["v"], out=out, state=st_na, eps=w.eps)
    _, o3, st3, g3 = run(w, x, False)
    torch.cuda.synchronize()
    for a, b in ((st1, st), (o1, o), (dq1, g[0]), (dk1, g[1]), (dv1, g[2]), (out, o), (st_na, st), (o3, o), (st3, st)):
        assert bytes_equal(a, b)
    for a, b in zip(g3, g):
        assert bytes_equal(a, b)


def test_full_size_every_head():
    """B8-H16-T4096-D256 f16: S, z of every head; O, dQ, dK, dV on sampled
    rows of every head (slice and block boundaries included) from the
    oracle's halves of the backward with that head's S, z, dS, dz; two heads
    completely."""
    w = Workload("B8-H16-T4096-D256-f16", 8, 16, 4096, D, "f16", seed=6600)
    print(f"case {w.name} seed={w.seed}", flush=True)
    x = make_inputs(w)
    dev, o, st, g = run(w, x, False)
    n = w.B * w.H
    hd = {nm: oracle.decode(a, "f16").reshape(n, w.T, D) for nm, a in x.items()}
    s_got, z_got = split_state(st, w.B, w.H, D)
    s_got, z_got = s_got.reshape(n, D, D), z_got.reshape(n, D)
    rows = sorted(set([0, 1, w.T - 2, w.T - 1] + [b + d for p in (2, 4, 8, 16, 32, 64) for i in range(1, p)
                                                  for b in [i * w.T // p] for d in (-1, 0)]
                      + [int(t) for t in np.random.default_rng(w.seed + 5).integers(0, w.T, size=40)]))
    idx = torch.tensor(rows, device="cuda")
    got = {nm: decode(t.reshape(n, w.T, D).index_select(1, idx), "f16")
           for nm, t in (("O", o), ("dQ", g[0]), ("dK", g[1]), ("dV", g[2]))}
    worst = {k_: 0.0 for k_ in ("S", "z", "O", "dQ", "dK", "dV")}
    for h in range(n):
        s_ref, z_ref = oracle.state_head(hd["k"][h], hd["v"][h])
        worst["S"] = max(worst["S"], max_rel_err(s_got[h], s_ref))
        worst["z"] = max(worst["z"], max_rel_err(z_got[h], z_ref))
        o_ref = oracle.output_head(hd["q"][h][rows], s_ref, z_ref, w.eps, False)
        dq_ref, ds_ref, dz_ref = oracle.bwd_q_side_head(hd["q"][h], hd["do"][h], s_ref, z_ref, w.eps, False)
        dk_ref, dv_ref = oracle.bwd_kv_side_head(hd["k"][h][rows], hd["v"][h][rows], ds_ref, dz_ref, False)
        for nm, r in (("O", o_ref), ("dQ", dq_ref[rows]), ("dK", dk_ref), ("dV", dv_ref)):
            worst[nm] = max(worst[nm], max_rel_err(got[nm][h], r))
    print("  all heads: " + "  ".join(f"{k_} {v_:.3e}" for k_, v_ in worst.items()), flush=True)
    for k_, v_ in worst.items():
        assert v_ <= TOL["f16"], f"{k_}: {v_:.3e}"
    for h in (0, n - 1):
        o_ref, _, _ = oracle.fwd_head(hd["q"][h], hd["k"][h], hd["v"][h], w.eps, False)
        check("O", decode(o.reshape(n, w.T, D)[h], "f16"), o_ref, "f16", f" head {h}")
        refs = oracle.bwd_head(hd["q"][h], hd["k"][h], hd["v"][h], hd["do"][h], w.eps, False)
        for nm, t, r in zip(("dQ", "dK", "dV"), g, refs):
            check(nm, decode(t.reshape(n, w.T, D)[h], "f16"), r, "f16", f" head {h}")
