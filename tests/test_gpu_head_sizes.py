"""GPU parity for every head size: D (of Q, K) and Dv (of V) each in
{32, 64, 96, 128}, in all sixteen combinations, against the fp64 oracle.

Small cases compare every element and end on ragged tails inside several
slices; a long case per shape family checks the state of every head and
complete outputs on sampled heads in the launch configuration of a full-size
run. The token-major layout, the other feature maps, the step calls and the
autograd wrapper are exercised with D != Dv as well.
"""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs, to_storage
from tests.la_testutil import TIGHT, TOL, bytes_equal, decode, max_rel_err, split_state, to_device

pytestmark = pytest.mark.gpu

SIZES = [32, 64, 96, 128]
PAIRS = [(d, dv) for d in SIZES for dv in SIZES]
DTYPES = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def check(name, got, ref, dtype, where=""):
    err = max_rel_err(got, ref)
    print(f"  {name}{where}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}{where}: non-finite output"
    assert err <= TOL[dtype], f"{name}{where}: {err:.3e} > {TOL[dtype]}"
    if dtype in TIGHT:
        assert err <= TIGHT[dtype], f"{name}{where}: {err:.3e} > {TIGHT[dtype]} (fp32 bar)"


def seed_of(base, T, D, Dv, dtype, simple):
    return base + 97 * T + 13 * D + Dv + 7 * DTYPES.index(dtype) + (3 if simple else 0)


def run_all(w, x, simple, layout="bhtd", phi="elu1"):
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    o, state = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=simple, layout=layout, phi=phi)
    dq, dk, dv = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], state, eps=w.eps, simple=simple,
                        layout=layout, phi=phi)
    torch.cuda.synchronize()
    return dev, {"o": o, "state": state, "dq": dq, "dk": dk, "dv": dv}


def compare_all(w, x, out, simple, phi="elu1"):
    dtype = w.dtype
    o_ref, s_ref, z_ref = oracle.fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple, phi)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], dtype, w.eps, simple, phi)
    assert tuple(out["o"].shape) == w.shape_v and tuple(out["dv"].shape) == w.shape_v
    assert tuple(out["dq"].shape) == w.shape and tuple(out["dk"].shape) == w.shape
    s_got, z_got = split_state(out["state"], w.B, w.H, w.D, w.dv)
    check("S", s_got, s_ref, dtype)
    check("z", z_got, z_ref, dtype)
    check("O", decode(out["o"], dtype), o_ref, dtype)
    check("dQ", decode(out["dq"], dtype), dq_ref, dtype)
    check("dK", decode(out["dk"], dtype), dk_ref, dtype)
    check("dV", decode(out["dv"], dtype), dv_ref, dtype)


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D,Dv", PAIRS, ids=[f"D{d}-Dv{dv}" for d, dv in PAIRS])
def test_head_sizes_all_elements(D, Dv, dtype, simple):
    """B2 H3 T1000: every step splits each head into a few slices or chunks,
    the last one ragged."""
    T = 1000
    seed = seed_of(60_000, T, D, Dv, dtype, simple)
    w = Workload("sizes", 2, 3, T, D, dtype, simple=simple, seed=seed, Dv=Dv)
    print(f"case T={T} D={D} Dv={Dv} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w)
    _, out = run_all(w, x, simple)
    compare_all(w, x, out, simple)


@pytest.mark.parametrize("T", [1, 4097])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D,Dv", [(32, 32), (96, 96), (32, 128), (128, 96)],
                         ids=["D32-Dv32", "D96-Dv96", "D32-Dv128", "D128-Dv96"])
def test_head_sizes_lengths(D, Dv, dtype, T):
    """One token, and a length one past a power of two (many slices, a
    one-token tail), normalised mode. At T = 1 the exact dQ and dK are O(eps):
    two O(1) summands cancel, so their error is measured against the size of
    those summands rather than of the result."""
    seed = seed_of(61_000, T, D, Dv, dtype, False)
    w = Workload("lengths", 2, 3, T, D, dtype, seed=seed, Dv=Dv)
    print(f"case T={T} D={D} Dv={Dv} {dtype} seed={seed}", flush=True)
    x = make_inputs(w)
    _, out = run_all(w, x, False)
    if T > 1:
        compare_all(w, x, out, False)
        return
    o_ref, s_ref, z_ref = oracle.fwd(x["q"], x["k"], x["v"], dtype, w.eps, False)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], dtype, w.eps, False)
    s_got, z_got = split_state(out["state"], w.B, w.H, D, Dv)
    check("S", s_got, s_ref, dtype)
    check("z", z_got, z_ref, dtype)
    check("O", decode(out["o"], dtype), o_ref, dtype)
    check("dV", decode(out["dv"], dtype), dv_ref, dtype)
    sc = [oracle.bwd_leading_terms_head(*(oracle.decode(x[n], dtype)[b, h] for n in ("q", "k", "v", "do")),
                                        w.eps) for b in range(w.B) for h in range(w.H)]
    for name, got, ref, scale in (("dQ", out["dq"], dq_ref, max(a for a, _ in sc)),
                                  ("dK", out["dk"], dk_ref, max(c for _, c in sc))):
        err = float(np.max(np.abs(decode(got, dtype) - ref)) / scale)
        print(f"  {name} (vs leading terms): {err:.3e}", flush=True)
        assert err <= TOL[dtype], f"{name}: {err:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,Dv", [(32, 32), (96, 64), (64, 128)], ids=["D32-Dv32", "D96-Dv64", "D64-Dv128"])
def test_head_sizes_many_heads_single_slice(D, Dv, dtype):
    """640 heads of 300 tokens: one slice or chunk per head in every step
    (states written directly, no partials), each ending on a ragged tail."""
    seed = seed_of(62_000, 300, D, Dv, dtype, False)
    w = Workload("many-heads", 4, 160, 300, D, dtype, seed=seed, Dv=Dv)
    print(f"case B4 H160 T300 D={D} Dv={Dv} {dtype} seed={seed}", flush=True)
    x = make_inputs(w)
    _, out = run_all(w, x, False)
    compare_all(w, x, out, False)


@pytest.mark.parametrize("D,Dv,dtype,simple", [(32, 32, "f16", False), (96, 96, "bf16", False),
                                                (128, 64, "f16", False), (64, 32, "bf16", True)],
                         ids=["D32-f16", "D96-bf16", "D128-Dv64-f16", "D64-Dv32-bf16-simple"])
def test_head_sizes_long_sequence(D, Dv, dtype, simple):
    """B8 H16 T16384: the state of every head against the oracle, complete
    O, dQ, dK, dV on four heads, and bit-identical reruns."""
    w = Workload("long", 8, 16, 16384, D, dtype, simple=simple, seed=seed_of(63_000, 0, D, Dv, dtype, simple),
                 Dv=Dv)
    print(f"case B8 H16 T16384 D={D} Dv={Dv} {dtype} simple={simple} seed={w.seed}", flush=True)
    x = make_inputs(w)
    _, out = run_all(w, x, simple)
    n = w.B * w.H
    hd = {nm: oracle.decode(a, dtype).reshape(n, w.T, -1) for nm, a in x.items()}
    s_got, z_got = split_state(out["state"], w.B, w.H, D, Dv)
    s_got, z_got = s_got.reshape(n, D, Dv), z_got.reshape(n, D)
    worst = 0.0
    for h in range(n):
        s_ref, z_ref = oracle.state_head(hd["k"][h], hd["v"][h])
        worst = max(worst, max_rel_err(s_got[h], s_ref), max_rel_err(z_got[h], z_ref))
    print(f"  state, all {n} heads: {worst:.3e}", flush=True)
    assert worst <= TOL[dtype]
    for h in (0, 37, 90, n - 1):
        o_ref, _, _ = oracle.fwd_head(hd["q"][h], hd["k"][h], hd["v"][h], w.eps, simple)
        refs = oracle.bwd_head(hd["q"][h], hd["k"][h], hd["v"][h], hd["do"][h], w.eps, simple)
        check("O", decode(out["o"].reshape(n, w.T, Dv)[h], dtype), o_ref, dtype, f" head {h}")
        for nm, ref, width in zip(("dq", "dk", "dv"), refs, (D, D, Dv)):
            check(nm, decode(out[nm].reshape(n, w.T, width)[h], dtype), ref, dtype, f" head {h}")
    _, out2 = run_all(w, x, simple)
    for nm in out:
        assert bytes_equal(out[nm], out2[nm]), f"{nm} differs between runs"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D,Dv", [(32, 96), (128, 32), (96, 96)], ids=["D32-Dv96", "D128-Dv32", "D96-Dv96"])
def test_head_sizes_token_major(D, Dv, dtype):
    """[B, T, H, D] and [B, T, H, Dv] tensors give, byte for byte, the outputs
    of the [B, H, T, *] run on the same values."""
    T = 777
    seed = seed_of(64_000, T, D, Dv, dtype, False)
    w = Workload("bthd", 2, 3, T, D, dtype, seed=seed, Dv=Dv)
    print(f"case bthd T={T} D={D} Dv={Dv} {dtype} seed={seed}", flush=True)
    x = make_inputs(w)
    dev, ref = run_all(w, x, False)
    tm = {n: t.transpose(1, 2).contiguous() for n, t in dev.items()}
    o, state = la.fwd(tm["q"], tm["k"], tm["v"], eps=w.eps, layout="bthd")
    dq, dk, dv = la.bwd(tm["q"], tm["k"], tm["v"], tm["do"], state, eps=w.eps, layout="bthd")
    torch.cuda.synchronize()
    assert bytes_equal(state, ref["state"])
    for name, got in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bytes_equal(got.transpose(1, 2).contiguous(), ref[name]), name
    compare_all(w, x, ref, False)


@pytest.mark.parametrize("fm,simple", [("relu", False), ("identity", True)], ids=["relu-norm", "identity-simple"])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D,Dv", [(32, 64), (96, 128)], ids=["D32-Dv64", "D96-Dv128"])
def test_head_sizes_other_feature_maps(D, Dv, dtype, fm, simple):
    T = 1000
    seed = seed_of(65_000, T, D, Dv, dtype, simple)
    w = Workload("maps", 2, 3, T, D, dtype, simple=simple, seed=seed, Dv=Dv)
    print(f"case phi={fm} simple={simple} T={T} D={D} Dv={Dv} {dtype} seed={seed}", flush=True)
    x = make_inputs(w)
    _, out = run_all(w, x, simple, phi=fm)
    compare_all(w, x, out, simple, phi=fm)


def test_head_sizes_step_calls_compose():
    w = Workload("steps", 2, 4, 3333, 96, "bf16", seed=66_001, Dv=32)
    x = make_inputs(w)
    dev, out = run_all(w, x, False)
    st = la.fwd_state(dev["k"], dev["v"], eps=w.eps)
    o = la.fwd_output(dev["q"], st, eps=w.eps, dv=32)
    dq = la.bwd_dq(dev["q"], dev["do"], st, eps=w.eps)
    dk, dv = la.bwd_dkv(dev["k"], dev["v"], eps=w.eps)
    torch.cuda.synchronize()
    assert tuple(o.shape) == w.shape_v and tuple(dv.shape) == w.shape_v
    for a, b in ((st, out["state"]), (o, out["o"]), (dq, out["dq"]), (dk, out["dk"]), (dv, out["dv"])):
        assert bytes_equal(a, b)


def test_head_sizes_autograd_wrapper():
    w = Workload("autograd", 2, 4, 500, 64, "f16", seed=66_002, Dv=96)
    x = make_inputs(w)
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = la.linear_attention(q, k, v, eps=w.eps)
    assert tuple(o.shape) == w.shape_v
    (o.float() * dev["do"].float()).sum().backward()
    torch.cuda.synchronize()
    o_ref, _, _ = oracle.fwd(x["q"], x["k"], x["v"], w.dtype, w.eps, False)
    dq_ref, dk_ref, dv_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], w.dtype, w.eps, False)
    check("O", decode(o.detach(), w.dtype), o_ref, w.dtype)
    for name, g, ref in (("dQ", q.grad, dq_ref), ("dK", k.grad, dk_ref), ("dV", v.grad, dv_ref)):
        check(name, decode(g, w.dtype), ref, w.dtype)


def test_head_sizes_binding_rejects_mismatched_tensors():
    """Shapes are checked in the binding before any call into the library."""
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16, device="cuda")
    v = torch.zeros(1, 2, 8, 32, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        la.fwd(q, q, torch.zeros(1, 2, 9, 32, dtype=torch.float16, device="cuda"))
    _, st = la.fwd(q, q, v)
    with pytest.raises(ValueError):
        la.bwd(q, q, v, q, st)  # dO must have v's head size
    with pytest.raises(ValueError):
        la.fwd_output(q, st, dv=64)  # the state holds 64 x 32 blocks, too small for 64 x 64
    with pytest.raises(la.LAError):
        la.fwd(torch.zeros(1, 2, 8, 48, dtype=torch.float16, device="cuda"),
               torch.zeros(1, 2, 8, 48, dtype=torch.float16, device="cuda"), v)
