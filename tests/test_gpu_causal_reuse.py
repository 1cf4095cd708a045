"""The causal backward with LA_REUSE_PREFIX: la_bwd reads the segment
prefixes the causal la_fwd left in the same workspace instead of recomputing
them. Its gradients must be the bytes of the recomputing backward (the same
kernels produce the same prefixes), for every dtype, padded head sizes, one
segment and many; the reusing path also matches the oracle, and the autograd
wrapper (which reuses) gives the explicit backward's gradients, a second time
through a retained graph as well."""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs
from tests.la_testutil import TOL, bytes_equal, decode, max_rel_err, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, T, D, Dv, simple
    ("f16", 2, 4, 20000, 64, 64, False),
    ("bf16", 1, 3, 9000, 128, 128, True),
    ("f32", 1, 2, 6000, 64, 64, False),
    ("f16", 1, 2, 5000, 32, 96, False),
    ("bf16", 2, 2, 7000, 96, 64, False),
    ("f16", 1, 1, 100, 64, 64, False),
]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def inputs(dtype, B, H, T, D, Dv, simple, seed):
    w = Workload("reuse", B, H, T, D, dtype, sigma=0.5 if dtype == "bf16" else 1.0, simple=simple, seed=seed, Dv=Dv)
    x = make_inputs(w, with_grad=True)
    return w, x, {n: to_device(a, dtype) for n, a in x.items()}


def fresh_ws(prob, device):
    return torch.empty(max(la.workspace_bytes(prob), 256), dtype=torch.uint8, device=device)


@pytest.mark.parametrize("dtype,B,H,T,D,Dv,simple", CASES,
                         ids=[f"{c[0]}-B{c[1]}H{c[2]}T{c[3]}-D{c[4]}-Dv{c[5]}{'-simple' if c[6] else ''}" for c in CASES])
def test_reuse_equals_recompute(dtype, B, H, T, D, Dv, simple):
    w, _, dev = inputs(dtype, B, H, T, D, Dv, simple, 140_000 + T + D)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    prob = la.make_problem(q.shape, q.dtype, w.eps, simple, dv=Dv, causal=True)
    print(f"case {dtype} B{B} H{H} T{T} D{D} Dv{Dv} simple={simple} split {la.split_of(prob)}", flush=True)
    ws = fresh_ws(prob, q.device)
    la.fwd(q, k, v, eps=w.eps, simple=simple, causal=True, ws=ws)
    got = la.bwd(q, k, v, do, None, eps=w.eps, simple=simple, causal=True, ws=ws, reuse_prefix=True)
    # a second reusing call on the same workspace: the backward leaves the prefixes as they were
    again = la.bwd(q, k, v, do, None, eps=w.eps, simple=simple, causal=True, ws=ws, reuse_prefix=True)
    ref = la.bwd(q, k, v, do, None, eps=w.eps, simple=simple, causal=True, ws=fresh_ws(prob, q.device))
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dQ", "dK", "dV"), got, again, ref):
        assert bytes_equal(a, c), f"{name}: reusing backward differs from the recomputing one"
        assert bytes_equal(b, c), f"{name}: second reusing backward differs"


def test_reuse_matches_oracle():
    """Several segments (P > 1) and ragged tails, every element."""
    w, x, dev = inputs("f16", 1, 2, 3001, 64, 64, False, 141_000)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    prob = la.make_problem(q.shape, q.dtype, w.eps, False, causal=True)
    assert la.split_of(prob)["P"] > 1
    ws = fresh_ws(prob, q.device)
    la.fwd(q, k, v, eps=w.eps, causal=True, ws=ws)
    g = la.bwd(q, k, v, do, None, eps=w.eps, causal=True, ws=ws, reuse_prefix=True)
    torch.cuda.synchronize()
    refs = oracle.causal_bwd(x["q"], x["k"], x["v"], x["do"], "f16", w.eps, False)
    for name, got, ref in zip(("dQ", "dK", "dV"), g, refs):
        err = max_rel_err(decode(got, "f16"), ref)
        print(f"  {name}: max rel err {err:.3e}", flush=True)
        assert np.all(np.isfinite(decode(got, "f16")))
        assert err <= TOL["f16"], f"{name}: {err:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_autograd_reuses_forward_prefixes(dtype):
    w, _, dev = inputs(dtype, 2, 3, 6000, 64, 64, False, 142_000 + (dtype == "bf16"))
    leaves = {n: dev[n].clone().requires_grad_(True) for n in ("q", "k", "v")}
    o = la.linear_attention(leaves["q"], leaves["k"], leaves["v"], eps=w.eps, causal=True)
    o.backward(dev["do"], retain_graph=True)
    first = [leaves[n].grad.clone() for n in ("q", "k", "v")]
    for t in leaves.values():
        t.grad = None
    o.backward(dev["do"])  # through the retained graph: the kept workspace still holds the prefixes
    second = [leaves[n].grad for n in ("q", "k", "v")]
    ref = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], None, eps=w.eps, causal=True)
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dQ", "dK", "dV"), first, second, ref):
        assert bytes_equal(a, c), f"{name}: autograd differs from the explicit backward"
        assert bytes_equal(b, c), f"{name}: second backward through the retained graph differs"
