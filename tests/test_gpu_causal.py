"""GPU parity of the causal forward (LA_CAUSAL) against the fp64 oracle's
causal forms: every element at small sizes (several segments and chunks,
ragged tails), sampled rows at full size, the token-major layout, the other
feature maps; the state equals that of the non-causal call (byte for byte
where the segments are its slices), and reruns are bit-identical."""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs, to_storage
from tests.la_testutil import TOL, bytes_equal, decode, max_rel_err, split_state, to_device

pytestmark = pytest.mark.gpu

PAIRS = [(64, 64), (128, 128), (64, 128), (128, 64)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def decode_state(st):
    return st.detach().cpu().numpy().astype(np.float64)


def check(name, got, ref, dtype, where=""):
    err = max_rel_err(got, ref)
    print(f"  {name}{where}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}{where}: non-finite output"
    assert err <= TOL[dtype], f"{name}{where}: {err:.3e} > {TOL[dtype]}"


def run(w, x, simple, layout="bhtd", phi="elu1", causal=True):
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    if layout == "bthd":
        dev = {n: t.transpose(1, 2).contiguous() for n, t in dev.items()}
    o, st = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=simple, layout=layout, phi=phi, causal=causal)
    torch.cuda.synchronize()
    return o, st


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,Dv", PAIRS, ids=[f"D{a}-Dv{b}" for a, b in PAIRS])
@pytest.mark.parametrize("T", [1, 100, 1000, 4097])
def test_causal_all_elements(T, D, Dv, dtype, simple):
    seed = 80_000 + 97 * T + 13 * D + Dv + 7 * ["f16", "bf16"].index(dtype) + (3 if simple else 0)
    w = Workload("causal", 2, 3, T, D, dtype, simple=simple, seed=seed, Dv=Dv)
    print(f"case causal T={T} D={D} Dv={Dv} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w, with_grad=False)
    o, st = run(w, x, simple)
    o_ref, s_ref, z_ref = oracle.causal_fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple)
    check("O", decode(o, dtype), o_ref, dtype)
    s_got, z_got = split_state(st, w.B, w.H, D, Dv)
    check("S", s_got, s_ref, dtype)
    check("z", z_got, z_ref, dtype)
    _, st_nc = run(w, x, simple, causal=False)
    if (D, Dv) == (64, 64):
        # the causal form sums twice as many segments as the non-causal call
        # sums slices at this size: the same values up to the order of the
        # fp32 additions
        assert max_rel_err(decode_state(st), decode_state(st_nc)) <= 1e-6
    else:
        assert bytes_equal(st, st_nc), "causal state differs from the non-causal state"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_many_heads_one_segment(dtype):
    """640 heads of 300 tokens: one segment per head, no prefix pass."""
    w = Workload("causal-many", 4, 160, 300, 64, dtype, seed=81_000 + ["f16", "bf16"].index(dtype))
    print(f"case causal B4 H160 T300 {dtype} seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=False)
    o, _ = run(w, x, False)
    o_ref, _, _ = oracle.causal_fwd(x["q"], x["k"], x["v"], dtype, w.eps, False)
    check("O", decode(o, dtype), o_ref, dtype)


@pytest.mark.parametrize("D,dtype,simple", [(64, "f16", False), (128, "bf16", False), (64, "bf16", True)],
                         ids=["D64-f16", "D128-bf16", "D64-bf16-simple"])
def test_causal_long_sequence_sampled_rows(D, dtype, simple):
    """B8 H16 T16384: rows around every segment and chunk boundary of four
    heads, and rows sampled on every head, against the per-row causal form;
    bit-identical reruns."""
    w = Workload("causal-long", 8, 16, 16384, D, dtype, simple=simple, seed=82_000 + D + (3 if simple else 0))
    print(f"case causal B8 H16 T16384 D={D} {dtype} simple={simple} seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=False)
    o, st = run(w, x, simple)
    n = w.B * w.H
    hd = {nm: oracle.decode(a, dtype).reshape(n, w.T, -1) for nm, a in x.items()}
    og = o.reshape(n, w.T, D)
    rng = np.random.default_rng(w.seed)
    edges = sorted({r for b in range(0, w.T + 1, 64) for r in (b - 1, b) if 0 <= r < w.T})
    worst = 0.0
    for h in range(n):
        rows = sorted(set(edges[:: 16]) | {0, w.T - 1} | {int(t) for t in rng.integers(0, w.T, size=4)})
        if h in (0, 37, 90, n - 1):
            rows = sorted(set(rows) | set(edges))
        ref = oracle.causal_sampled_rows_head(hd["q"][h], hd["k"][h], hd["v"][h], rows, w.eps, simple)
        got = decode(og[h][rows], dtype)
        worst = max(worst, max_rel_err(got, ref))
    print(f"  O sampled rows, all heads: {worst:.3e}", flush=True)
    assert worst <= TOL[dtype]
    o2, st2 = run(w, x, simple)
    assert bytes_equal(o, o2) and bytes_equal(st, st2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,Dv", [(64, 64), (128, 64)], ids=["D64", "D128-Dv64"])
def test_causal_token_major(D, Dv, dtype):
    w = Workload("causal-bthd", 2, 3, 777, D, dtype, seed=83_000 + D + Dv, Dv=Dv)
    x = make_inputs(w, with_grad=False)
    o_ref, st_ref = run(w, x, False)
    o, st = run(w, x, False, layout="bthd")
    assert bytes_equal(st, st_ref)
    assert bytes_equal(o.transpose(1, 2).contiguous(), o_ref)


@pytest.mark.parametrize("fm,simple", [("relu", False), ("identity", True)], ids=["relu-norm", "identity-simple"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_other_feature_maps(dtype, fm, simple):
    w = Workload("causal-maps", 2, 3, 1000, 64, dtype, simple=simple, seed=84_000 + ["f16", "bf16"].index(dtype))
    print(f"case causal phi={fm} simple={simple} {dtype} seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=False)
    o, _ = run(w, x, simple, phi=fm)
    o_ref, _, _ = oracle.causal_fwd(x["q"], x["k"], x["v"], dtype, w.eps, simple, fm)
    check("O", decode(o, dtype), o_ref, dtype)


def test_causal_rejects_unsupported():
    """The causal form has no head size 256 (the wide kernels are
    bidirectional only): refused before any launch."""
    y = torch.zeros(1, 2, 8, 256, dtype=torch.float16, device="cuda")
    with pytest.raises(la.LAError):
        la.fwd(y, y, y, causal=True)