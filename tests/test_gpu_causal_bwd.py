"""GPU parity of the causal backward (la_bwd with LA_CAUSAL) against the fp64
oracle's chain rule through the recurrent form: every element at small sizes
(several segments and chunks, ragged tails), whole heads at B8 H16 T16384, the
last-row property against the non-causal backward at that size, the
token-major layout, the other feature maps, and bit-identical reruns."""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs
from tests import oracle_pool
from tests.la_testutil import TOL, bytes_equal, decode, max_rel_err, to_device

pytestmark = pytest.mark.gpu

PAIRS = [(64, 64), (128, 128), (64, 128), (128, 64)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def check(name, got, ref, dtype, where="", scale=None):
    err = max_rel_err(got, ref) if scale is None else float(np.max(np.abs(got - ref))) / scale
    print(f"  {name}{where}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}{where}: non-finite output"
    assert err <= TOL[dtype], f"{name}{where}: {err:.3e} > {TOL[dtype]}"


def run(w, x, simple, layout="bhtd", phi="elu1", causal=True):
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    if layout == "bthd":
        dev = {n: t.transpose(1, 2).contiguous() for n, t in dev.items()}
    state = None
    if not causal:
        _, state = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=simple, layout=layout, phi=phi)
    g = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], state, eps=w.eps, simple=simple, layout=layout, phi=phi,
               causal=causal)
    torch.cuda.synchronize()
    return g


def check_all(w, x, grads, simple, fm="elu1"):
    ref = oracle.causal_bwd(x["q"], x["k"], x["v"], x["do"], w.dtype, w.eps, simple, fm)
    scales = [None, None, None]
    if w.T == 1 and not simple:
        # one token: the exact dQ, dK are O(eps), two O(1) summands cancelling
        # (the causal and non-causal forms coincide); measure the error
        # against those summands instead of the result
        sc = [oracle.bwd_leading_terms_head(*(oracle.decode(x[n], w.dtype)[b, h] for n in ("q", "k", "v", "do")),
                                            w.eps)
              for b in range(w.B) for h in range(w.H)]
        scales[:2] = [max(a for a, _ in sc), max(b for _, b in sc)]
    for name, g, r, sc in zip(("dQ", "dK", "dV"), grads, ref, scales):
        check(name, decode(g, w.dtype), r, w.dtype, scale=sc)


@pytest.mark.parametrize("simple", [False, True], ids=["norm", "simple"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,Dv", PAIRS, ids=[f"D{a}-Dv{b}" for a, b in PAIRS])
@pytest.mark.parametrize("T", [1, 100, 1000, 4097])
def test_causal_bwd_all_elements(T, D, Dv, dtype, simple):
    seed = 90_000 + 97 * T + 13 * D + Dv + 7 * ["f16", "bf16"].index(dtype) + (3 if simple else 0)
    w = Workload("causal-bwd", 2, 3, T, D, dtype, simple=simple, seed=seed, Dv=Dv)
    print(f"case causal bwd T={T} D={D} Dv={Dv} {dtype} simple={simple} seed={seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    check_all(w, x, run(w, x, simple), simple)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_bwd_many_heads_one_segment(dtype):
    """640 heads of 300 tokens: one segment per head, no prefix or suffix pass."""
    w = Workload("causal-bwd-many", 4, 160, 300, 64, dtype, seed=91_000 + ["f16", "bf16"].index(dtype))
    print(f"case causal bwd B4 H160 T300 {dtype} seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    check_all(w, x, run(w, x, False), False)


def boundary_rows(T, seed, extra=24):
    """Both sides of every boundary of a power-of-two split of T into up to 64
    segments, both sides of every 64-token chunk boundary near them, the ends,
    and seeded picks."""
    rows = {0, 1, T - 2, T - 1}
    for p in (2, 4, 8, 16, 32, 64):
        for i in range(1, p):
            b = i * T // p
            rows.update((b - 1, b, b + 63, b + 64))
    rows.update(int(t) for t in np.random.default_rng(seed).integers(0, T, size=extra))
    return sorted(r for r in rows if 0 <= r < T)


def head_slices(x, n, T):
    return {nm: a.reshape(n, T, -1) for nm, a in x.items()}


@pytest.mark.parametrize("D,Dv,dtype,simple", [(64, 64, "f16", False), (128, 128, "bf16", False),
                                              (64, 64, "bf16", True), (64, 128, "f16", False)],
                         ids=["D64-f16", "D128-bf16", "D64-bf16-simple", "D64-Dv128-f16"])
def test_causal_bwd_long_sequence_whole_heads(D, Dv, dtype, simple):
    """B8 H16 T16384 (every segment boundary of the split): three whole heads
    against the oracle, sampled rows (segment and chunk boundaries included)
    of every head; bit-identical reruns."""
    w = Workload("causal-bwd-long", 8, 16, 16384, D, dtype, simple=simple, seed=92_000 + D + Dv + (3 if simple else 0),
                 Dv=Dv)
    print(f"case causal bwd B8 H16 T16384 D={D} Dv={Dv} {dtype} simple={simple} seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    g = run(w, x, simple)
    n = w.B * w.H
    hx = head_slices(x, n, w.T)
    whole = (0, 77, n - 1)
    for h in whole:
        ref = oracle.causal_bwd(*(hx[nm][h][None, None] for nm in ("q", "k", "v", "do")), dtype, w.eps, simple)
        for name, gg, r in zip(("dQ", "dK", "dV"), g, ref):
            check(name, decode(gg.reshape(n, w.T, -1)[h], dtype), r[0, 0], dtype, f" head {h}")
    # every other head: sampled rows, the oracle run in a process pool
    rows = boundary_rows(w.T, w.seed + 5)
    idx = torch.tensor(rows, device="cuda")
    got = [decode(gg.reshape(n, w.T, -1).index_select(1, idx), dtype) for gg in g]
    dec = {nm: oracle.decode(hx[nm], dtype) for nm in ("q", "k", "v", "do")}
    others = [h for h in range(n) if h not in whole]
    jobs = [(dec["q"][h], dec["k"][h], dec["v"][h], dec["do"][h], rows, w.eps, simple, "elu1") for h in others]
    res = oracle_pool.map_heads(oracle_pool.causal_bwd_rows, jobs)
    for i, name in enumerate(("dQ", "dK", "dV")):
        worst = max(max_rel_err(got[i][h], r[i]) for h, r in zip(others, res))
        print(f"  {name}, {len(rows)} rows on all {len(others)} other heads: max rel err {worst:.3e}", flush=True)
        assert worst <= TOL[dtype], f"{name} sampled rows: {worst:.3e} > {TOL[dtype]}"
    g2 = run(w, x, simple)
    for a, b in zip(g, g2):
        assert bytes_equal(a, b)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_bwd_last_row_equals_noncausal(dtype):
    """With dO zero except on the last token of every head, that token sees the
    whole sequence: the causal gradients equal the non-causal ones
    (B8 H16 T16384 D64)."""
    w = Workload("causal-bwd-last", 8, 16, 16384, 64, dtype, seed=93_000 + ["f16", "bf16"].index(dtype))
    print(f"case causal bwd last-row B8 H16 T16384 {dtype} seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    do = x["do"].copy()
    do[:, :, :-1, :] = 0
    x["do"] = do
    gc = run(w, x, False)
    gn = run(w, x, False, causal=False)
    for name, a, b in zip(("dQ", "dK", "dV"), gc, gn):
        check(name, decode(a, dtype), decode(b, dtype).astype(np.float64), dtype, " vs non-causal")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,Dv", [(64, 64), (128, 64)], ids=["D64", "D128-Dv64"])
def test_causal_bwd_token_major(D, Dv, dtype):
    w = Workload("causal-bwd-bthd", 2, 3, 777, D, dtype, seed=94_000 + D + Dv, Dv=Dv)
    x = make_inputs(w, with_grad=True)
    ref = run(w, x, False)
    got = run(w, x, False, layout="bthd")
    for a, b in zip(got, ref):
        assert bytes_equal(a.transpose(1, 2).contiguous(), b)


@pytest.mark.parametrize("fm,simple", [("relu", False), ("identity", True)], ids=["relu-norm", "identity-simple"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_bwd_other_feature_maps(dtype, fm, simple):
    w = Workload("causal-bwd-maps", 2, 3, 1000, 64, dtype, simple=simple, seed=95_000 + ["f16", "bf16"].index(dtype))
    print(f"case causal bwd phi={fm} simple={simple} {dtype} seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    check_all(w, x, run(w, x, simple, phi=fm), simple, fm)


def test_causal_bwd_rejects_unsupported():
    """The causal form has no head size 256 (the wide kernels are
    bidirectional only): refused before any launch."""
    y = torch.zeros(1, 2, 8, 256, dtype=torch.float16, device="cuda")
    with pytest.raises(la.LAError):
        la.bwd(y, y, y, y, causal=True)


def test_causal_long_sequence_few_heads():
    """B2 H8 T262144 D64 bf16 simple_la (16 heads, 64 segments each): the
    forward and backward of one whole head against the oracle, sampled output
    rows of every head, and bit-identical reruns."""
    w = Workload("causal-c5", 2, 8, 262144, 64, "bf16", simple=True, seed=99_000)
    print(f"case causal B2 H8 T262144 bf16 simple seed={w.seed}", flush=True)
    x = make_inputs(w, with_grad=True)
    dev = {n: to_device(a, "bf16") for n, a in x.items()}
    o, _ = la.fwd(dev["q"], dev["k"], dev["v"], simple=True, causal=True)
    g = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], None, simple=True, causal=True)
    torch.cuda.synchronize()
    n = w.B * w.H
    hx = head_slices(x, n, w.T)
    h = 11
    args = [hx[nm][h][None, None] for nm in ("q", "k", "v", "do")]
    o_ref, _, _ = oracle.causal_fwd(*args[:3], "bf16", w.eps, True)
    check("O", decode(o.reshape(n, w.T, -1)[h], "bf16"), o_ref[0, 0], "bf16", f" head {h}")
    for name, gg, r in zip(("dQ", "dK", "dV"), g, oracle.causal_bwd(*args, "bf16", w.eps, True)):
        check(name, decode(gg.reshape(n, w.T, -1)[h], "bf16"), r[0, 0], "bf16", f" head {h}")
    rng = np.random.default_rng(w.seed)
    hd = {nm: oracle.decode(a, "bf16").reshape(n, w.T, -1) for nm, a in x.items() if nm != "do"}
    worst = 0.0
    for hh in range(n):
        rows = sorted({0, w.T - 1} | {int(t) for t in rng.integers(0, w.T, size=6)})
        ref = oracle.causal_sampled_rows_head(hd["q"][hh], hd["k"][hh], hd["v"][hh], rows, w.eps, True)
        worst = max(worst, max_rel_err(decode(o.reshape(n, w.T, -1)[hh][rows], "bf16"), ref))
    print(f"  O sampled rows, all heads: {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]
    o2, _ = la.fwd(dev["q"], dev["k"], dev["v"], simple=True, causal=True)
    g2 = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], None, simple=True, causal=True)
    torch.cuda.synchronize()
    assert bytes_equal(o, o2)
    for a, b in zip(g, g2):
        assert bytes_equal(a, b)


@pytest.mark.parametrize("D,Dv", [(64, 64), (128, 64)], ids=["D64", "D128-Dv64"])
def test_causal_empty_sequence(D, Dv):
    """T = 0: the causal forward writes a zero state (as the bidirectional one
    does) and the backward returns at once."""
    q = torch.zeros(2, 3, 0, D, dtype=torch.float16, device="cuda")
    v = torch.zeros(2, 3, 0, Dv, dtype=torch.float16, device="cuda")
    prob = la.make_problem(q.shape, q.dtype, 1e-6, False, dv=Dv, causal=True)
    state = torch.full((la.state_bytes(prob) // 4,), 7.0, device="cuda")
    o, st = la.fwd(q, q, v, causal=True, state=state)
    dq, dk, dv = la.bwd(q, q, v, v, None, causal=True)
    torch.cuda.synchronize()
    assert o.numel() == 0 and dq.numel() == 0 and dk.numel() == 0 and dv.numel() == 0
    assert torch.count_nonzero(st).item() == 0
