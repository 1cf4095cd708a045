"""Pins of the fp64 oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, eps in the wrong place, the wrong
branch of phi) fails at least one of them:
  * pure-Python brute force of the quadratic form (a different formula, no numpy)
  * the hand-worked example in tests/golden/ (exact rationals)
  * torch's elu for phi, torch fp64 autograd of the quadratic form for the VJP
  * central finite differences of L = sum(O * dO)
  * invariants: V = ones, joint K/V permutation, Q-row permutation, linearity
    in V, the T = 1 closed form, sum_t dV_t and V = c*1 identities.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_T2_D2.json")


def frac_array(rows):
    return np.array([[float(Fraction(x)) for x in r] for r in rows]) if isinstance(rows[0], list) \
        else np.array([float(Fraction(x)) for x in rows])


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- phi

def test_phi_matches_torch_elu_plus_one():
    torch = pytest.importorskip("torch")
    x = np.concatenate([rand(1000, 1) * 4, [0.0, -0.0, 1e-300, -1e-300, -50.0, 30.0]])
    ref = (torch.nn.functional.elu(torch.from_numpy(x)) + 1).numpy()
    # torch forms expm1(x) + 1, which loses up to half an ulp of 1 for x < 0
    np.testing.assert_allclose(oracle.phi(x), ref, rtol=1e-15, atol=2.3e-16)


def test_phi_special_values_and_derivative():
    assert oracle.phi(np.array([0.0]))[0] == 1.0
    assert oracle.phi(np.array([1.0]))[0] == 2.0
    assert oracle.phi(np.array([2.5]))[0] == 3.5
    assert abs(oracle.phi(np.array([-math.log(2)]))[0] - 0.5) < 1e-16
    # no cancellation for very negative x: phi(-40) = e^-40, not 0
    assert oracle.phi(np.array([-40.0]))[0] == pytest.approx(math.exp(-40), rel=1e-15)
    # phi' from central differences, away from the kink of phi'' at 0
    x = np.array([-3.0, -0.5, -1e-3, 1e-3, 0.7, 4.0])
    h = 1e-6
    fd = (oracle.phi(x + h) - oracle.phi(x - h)) / (2 * h)
    np.testing.assert_allclose(oracle.dphi(x), fd, rtol=1e-8)
    assert oracle.dphi(np.array([0.0]))[0] == 1.0


# ---------------------------------------------------------------- forward

def brute_force(q, k, v, eps, simple, fm="elu1", scale=1.0):
    """Pure-Python quadratic form: O_t = sum_s a_ts v_s / (sum_s a_ts + eps),
    a_ts = (scale phi(q_t)) . phi(k_s)."""
    def ph(x):
        if fm == "relu":
            return x if x > 0 else 0.0
        if fm == "identity":
            return x
        return x + 1.0 if x > 0 else math.exp(x)
    T, D, Dv = len(q), len(q[0]), len(v[0])
    out = []
    for t in range(T):
        a = [sum(scale * ph(q[t][i]) * ph(k[s][i]) for i in range(D)) for s in range(T)]
        row = [sum(a[s] * v[s][j] for s in range(T)) for j in range(Dv)]
        if not simple:
            den = sum(a) + eps
            row = [x / den for x in row]
        out.append(row)
    return np.array(out)


@pytest.mark.parametrize("simple", [False, True])
@pytest.mark.parametrize("T,D,Dv", [(1, 5, 5), (7, 5, 5), (16, 8, 8), (40, 64, 64),
                                    (7, 5, 3), (16, 8, 12), (40, 32, 96)])
def test_linear_form_matches_brute_force(T, D, Dv, simple):
    q, k, v = rand((T, D), 1), rand((T, D), 2), rand((T, Dv), 3)
    eps = 0.3  # large enough that a misplaced eps shows
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), eps, simple)
    o, _, _ = oracle.fwd_head(q, k, v, eps, simple)
    assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))
    oq = oracle.quadratic_head(q, k, v, eps, simple)
    assert np.max(np.abs(oq - ref)) <= 1e-12 * np.max(np.abs(ref))
    rows = [0, T // 2, T - 1]
    os_ = oracle.sampled_rows_head(q, k, v, rows, eps, simple)
    assert np.max(np.abs(os_ - ref[rows])) <= 1e-12 * np.max(np.abs(ref))


def test_golden_hand_worked_forward():
    g = json.load(open(GOLDEN))
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    o, s, z = oracle.fwd_head(q, k, v, g["eps"], simple=False)
    np.testing.assert_allclose(o, frac_array(g["normalised"]["o"]), rtol=1e-15)
    np.testing.assert_allclose(s, frac_array(g["normalised"]["S"]), rtol=1e-15)
    np.testing.assert_allclose(z, frac_array(g["normalised"]["z"]), rtol=1e-15)
    o, _, _ = oracle.fwd_head(q, k, v, g["eps"], simple=True)
    np.testing.assert_allclose(o, frac_array(g["simple"]["o"]), rtol=1e-15)
    e = g["exp_branch_T1"]
    q1, k1, v1 = (np.array([e[n]]) for n in ("q", "k", "v"))
    o, _, _ = oracle.fwd_head(q1, k1, v1, e["eps"], simple=False)
    np.testing.assert_allclose(o[0], frac_array(e["o_normalised"]), rtol=1e-15)
    o, _, _ = oracle.fwd_head(q1, k1, v1, e["eps"], simple=True)
    np.testing.assert_allclose(o[0], frac_array(e["o_simple"]), rtol=1e-15)


def test_v_ones_gives_ones_normalised():
    T, D = 64, 16
    q, k = rand((T, D), 4), rand((T, D), 5)
    v = np.ones((T, D))
    o, _, z = oracle.fwd_head(q, k, v, 0.0, simple=False)
    np.testing.assert_allclose(o, 1.0, rtol=1e-14)
    # with eps: O_t = a_t / (a_t + eps) * 1, a_t = phi(q_t) . z; eps = 5 makes it visible
    eps = 5.0
    o, _, _ = oracle.fwd_head(q, k, v, eps, simple=False)
    a = np.array([sum(oracle.phi(q[t]) * z) for t in range(T)])
    np.testing.assert_allclose(o, np.repeat((a / (a + eps))[:, None], D, axis=1), rtol=1e-14)
    assert np.all(o < 1.0)


@pytest.mark.parametrize("simple", [False, True])
def test_joint_kv_permutation_invariance(simple):
    T, D = 100, 16
    q, k, v = rand((T, D), 6), rand((T, D), 7), rand((T, D), 8)
    perm = np.random.default_rng(9).permutation(T)
    o1, s1, z1 = oracle.fwd_head(q, k, v, 1e-6, simple)
    o2, s2, z2 = oracle.fwd_head(q, k[perm], v[perm], 1e-6, simple)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13 * np.abs(o1).max())
    # permuting only V (not K) must change the result: pins pairing of k_t with v_t
    o3, _, _ = oracle.fwd_head(q, k, v[perm], 1e-6, simple)
    assert np.max(np.abs(o3 - o1)) > 1e-3 * np.abs(o1).max()


@pytest.mark.parametrize("simple", [False, True])
def test_q_row_permutation_equivariance(simple):
    T, D = 50, 8
    q, k, v = rand((T, D), 10), rand((T, D), 11), rand((T, D), 12)
    perm = np.random.default_rng(13).permutation(T)
    o1, _, _ = oracle.fwd_head(q, k, v, 1e-6, simple)
    o2, _, _ = oracle.fwd_head(q[perm], k, v, 1e-6, simple)
    np.testing.assert_allclose(o2, o1[perm], rtol=1e-14)


@pytest.mark.parametrize("simple", [False, True])
def test_t1_closed_form(simple):
    D = 6
    q, k, v = rand((1, D), 14), rand((1, D), 15), rand((1, D), 16)
    eps = 0.25
    a = sum((qi + 1 if qi > 0 else math.exp(qi)) * (ki + 1 if ki > 0 else math.exp(ki))
            for qi, ki in zip(q[0], k[0]))
    expect = a * v[0] if simple else a / (a + eps) * v[0]
    o, _, _ = oracle.fwd_head(q, k, v, eps, simple)
    np.testing.assert_allclose(o[0], expect, rtol=1e-14)


@pytest.mark.parametrize("simple", [False, True])
def test_linearity_in_v(simple):
    T, D = 30, 8
    q, k = rand((T, D), 17), rand((T, D), 18)
    v1, v2 = rand((T, D), 19), rand((T, D), 20)
    a, b = 0.7, -2.5
    o1, _, _ = oracle.fwd_head(q, k, v1, 1e-3, simple)
    o2, _, _ = oracle.fwd_head(q, k, v2, 1e-3, simple)
    o3, _, _ = oracle.fwd_head(q, k, a * v1 + b * v2, 1e-3, simple)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-13 * np.abs(o3).max())


def test_batched_fwd_matches_per_head_and_decodes():
    from synth import Workload
    w = Workload("t", 2, 3, 20, 8, "bf16", seed=77)
    x = make_inputs(w, with_grad=False)
    o, s, z = oracle.fwd(x["q"], x["k"], x["v"], "bf16", 1e-6, False)
    assert o.shape == (2, 3, 20, 8) and s.shape == (2, 3, 8, 8) and z.shape == (2, 3, 8)
    wr = Workload("t", 2, 3, 20, 8, "bf16", seed=77, Dv=12)
    xr = make_inputs(wr, with_grad=False)
    assert xr["q"].shape == (2, 3, 20, 8) and xr["v"].shape == (2, 3, 20, 12)
    orr, sr, zr = oracle.fwd(xr["q"], xr["k"], xr["v"], "bf16", 1e-6, False)
    assert orr.shape == (2, 3, 20, 12) and sr.shape == (2, 3, 8, 12) and zr.shape == (2, 3, 8)
    qd = oracle.decode(x["q"], "bf16")
    # bf16 values decode to float32-representable numbers with 8-bit mantissas
    m, _ = np.frexp(qd)
    assert np.all((m * 256) == np.round(m * 256))
    o11, s11, _ = oracle.fwd_head(qd[1, 1], oracle.decode(x["k"], "bf16")[1, 1],
                                  oracle.decode(x["v"], "bf16")[1, 1], 1e-6, False)
    np.testing.assert_array_equal(o[1, 1], o11)
    np.testing.assert_array_equal(s[1, 1], s11)


# ---------------------------------------------------------------- backward

def loss(q, k, v, do, eps, simple, fm="elu1", scale=1.0):
    o, _, _ = oracle.fwd_head(q, k, v, eps, simple, fm, scale)
    return float(np.sum(o * do))


def finite_difference(q, k, v, do, eps, simple, which, coords, h=1e-6, fm="elu1", scale=1.0):
    arrs = {"q": q, "k": k, "v": v}
    out = []
    for (t, d) in coords:
        plus = {n: a.copy() for n, a in arrs.items()}
        minus = {n: a.copy() for n, a in arrs.items()}
        plus[which][t, d] += h
        minus[which][t, d] -= h
        out.append((loss(plus["q"], plus["k"], plus["v"], do, eps, simple, fm, scale)
                    - loss(minus["q"], minus["k"], minus["v"], do, eps, simple, fm, scale)) / (2 * h))
    return np.array(out)


def away_from_zero(x, margin):
    return np.where(np.abs(x) < margin, np.sign(x + 1e-30) * margin * 3, x)


@pytest.mark.parametrize("simple", [False, True])
@pytest.mark.parametrize("T,D,Dv", [(5, 3, 3), (16, 8, 8), (6, 3, 5), (9, 7, 2)])
def test_bwd_matches_finite_differences_all_coords(T, D, Dv, simple):
    # inputs kept away from 0 where phi'' jumps; eps large enough to matter
    q = away_from_zero(rand((T, D), 21), 1e-4)
    k = away_from_zero(rand((T, D), 22), 1e-4)
    v, do = rand((T, Dv), 23), rand((T, Dv), 24)
    eps = 0.5
    dq, dk, dv = oracle.bwd_head(q, k, v, do, eps, simple)
    assert dq.shape == (T, D) and dk.shape == (T, D) and dv.shape == (T, Dv)
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        cols = Dv if name == "v" else D
        coords = [(t, d) for t in range(T) for d in range(cols)]
        fd = finite_difference(q, k, v, do, eps, simple, name, coords).reshape(T, cols)
        assert np.max(np.abs(g - fd)) <= 1e-6 * max(1.0, np.abs(fd).max()), name


@pytest.mark.parametrize("simple", [False, True])
def test_bwd_finite_differences_sampled_tiny_config_shape(simple):
    T, D = 128, 64
    q = away_from_zero(rand((T, D), 31), 1e-4)
    k = away_from_zero(rand((T, D), 32), 1e-4)
    v, do = rand((T, D), 33), rand((T, D), 34)
    eps = 1e-6
    dq, dk, dv = oracle.bwd_head(q, k, v, do, eps, simple)
    rng = np.random.default_rng(35)
    coords = [(int(rng.integers(T)), int(rng.integers(D))) for _ in range(24)]
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        fd = finite_difference(q, k, v, do, eps, simple, name, coords, h=1e-5)
        got = np.array([g[t, d] for t, d in coords])
        assert np.max(np.abs(got - fd)) <= 1e-5 * max(np.abs(fd).max(), 1e-12), name


@pytest.mark.parametrize("simple", [False, True])
@pytest.mark.parametrize("D,Dv", [(16, 16), (16, 24)])
def test_bwd_matches_torch_autograd_of_quadratic_form(D, Dv, simple):
    torch = pytest.importorskip("torch")
    T = 48
    q, k = rand((T, D), 41), rand((T, D), 42)
    v, do = rand((T, Dv), 43), rand((T, Dv), 44)
    eps = 0.05
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    fq = torch.nn.functional.elu(tq) + 1
    fk = torch.nn.functional.elu(tk) + 1
    a = fq @ fk.T
    o = a @ tv
    if not simple:
        o = o / (a.sum(dim=1, keepdim=True) + eps)
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv = oracle.bwd_head(q, k, v, do, eps, simple)
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        ref = t.grad.numpy()
        assert np.max(np.abs(g - ref)) <= 1e-12 * np.abs(ref).max()


def test_golden_hand_worked_backward():
    g = json.load(open(GOLDEN))
    q, k, v, do = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v", "do"))
    for mode, simple in (("normalised", False), ("simple", True)):
        dq, dk, dv = oracle.bwd_head(q, k, v, do, g["eps"], simple)
        np.testing.assert_allclose(dq, frac_array(g[mode]["dq"]), rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(dk, frac_array(g[mode]["dk"]), rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(dv, frac_array(g[mode]["dv"]), rtol=1e-14, atol=1e-16)


def test_bwd_dv_column_sum_identity():
    # sum_t dV_t = sum_s dO_s * a_s / (a_s + eps), a_s = phi(q_s) . z
    T, D = 70, 12
    q, k, v, do = (rand((T, D), s) for s in (51, 52, 53, 54))
    eps = 2.0
    _, dk, dv = oracle.bwd_head(q, k, v, do, eps, simple=False)
    _, _, z = oracle.fwd_head(q, k, v, eps, simple=False)
    a = np.array([np.dot(oracle.phi(q[s]), z) for s in range(T)])
    np.testing.assert_allclose(dv.sum(axis=0), (do * (a / (a + eps))[:, None]).sum(axis=0),
                               rtol=1e-12)


def test_bwd_constant_v_gives_zero_dq_dk():
    # V = c*1 makes O_t = c a_t/(a_t+eps): with eps = 0 O is constant, so dQ = dK = 0
    T, D = 40, 8
    q, k, do = rand((T, D), 61), rand((T, D), 62), rand((T, D), 63)
    v = np.full((T, D), -1.75)
    dq, dk, dv = oracle.bwd_head(q, k, v, do, 0.0, simple=False)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.abs(dv).max() > 1e-2


def test_batched_bwd_matches_per_head():
    from synth import Workload
    for dv_ in (0, 16):
        w = Workload("t", 1, 2, 33, 8, "f16", seed=88, Dv=dv_)
        x = make_inputs(w)
        dq, dk, dv = oracle.bwd(x["q"], x["k"], x["v"], x["do"], "f16", 1e-6, False)
        assert dq.shape == dk.shape == w.shape and dv.shape == w.shape_v
        ref = oracle.bwd_head(*(oracle.decode(x[n], "f16")[0, 1] for n in ("q", "k", "v", "do")),
                              1e-6, False)
        for a, b in zip((dq[0, 1], dk[0, 1], dv[0, 1]), ref):
            np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible slips in a copy of the oracle's forward and check that the
    pins above would fail on each one (the pins compare against brute force)."""
    T, D = 9, 4
    q, k, v = rand((T, D), 71), rand((T, D), 72), rand((T, D), 73)
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.3, False)

    def variant(kind):
        qt, kt = oracle.phi(q), oracle.phi(k)
        if kind == "elu_no_plus_one":
            qt, kt = qt - 1, kt - 1
        s = kt.T @ v
        if kind == "transposed_state":
            s = s.T
        z = kt.sum(0)
        den = qt @ z + (0.0 if kind == "no_eps" else 0.3)
        if kind == "eps_multiplied":
            den = (qt @ z) * (1 + 0.3)
        return (qt @ s) / den[:, None]

    for kind in ("elu_no_plus_one", "transposed_state", "no_eps", "eps_multiplied"):
        bad = variant(kind)
        assert np.max(np.abs(bad - ref)) > 1e-6 * np.abs(ref).max(), kind
    assert np.max(np.abs(variant("none") - ref)) <= 1e-12 * np.abs(ref).max()


def test_workloads_inputs_are_seeded_and_rounded():
    w = WORKLOADS["B1-H2-T128-D64-f32"]
    a = make_inputs(w)
    b = make_inputs(w)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
    assert a["q"].dtype == np.float32 and a["q"].shape == (1, 2, 128, 64)
    assert not np.array_equal(a["q"], a["k"])


def test_leading_terms_cancel_at_t1():
    # T = 1, normalised: dQ = phi'(q) k~ (v.dO) eps / den^2, tiny next to u/den
    q, k, v, do = (rand((1, 8), s) for s in (81, 82, 83, 84))
    eps = 1e-6
    dq, dk, _ = oracle.bwd_head(q, k, v, do, eps, simple=False)
    sq, sk = oracle.bwd_leading_terms_head(q, k, v, do, eps)
    assert np.abs(dq).max() < 1e-4 * sq and np.abs(dk).max() < 1e-4 * sk
    kt, qt = oracle.phi(k[0]), oracle.phi(q[0])
    den = qt @ kt + eps
    np.testing.assert_allclose(dq[0], oracle.dphi(q[0]) * kt * (v[0] @ do[0]) * eps / den**2,
                               rtol=1e-6, atol=1e-300)


def leading_terms_loop(q, k, v, do, eps, fm="elu1"):
    """Pure-Python loops over both summands of the normalised gradients, one
    element at a time (no numpy), from the definitions
      dphi(q_t)[i] = u_t[i] / den_t + c_t z[i],   u_t[i] = sum_j S[i][j] dO_t[j],
      dphi(k_s)[i] = (dS v_s)[i] + dz[i],          dS[i][j] = sum_t phi(q_t)[i] dO_t[j] / den_t,
    returning the largest |u_t[i] / den_t * phi'(q_t[i])| and the largest
    |(dS v_s)[i] * phi'(k_s[i])|: the first summand of each, times phi'."""
    def ph(x):
        if fm == "relu":
            return max(x, 0.0)
        return x + 1.0 if x > 0 else math.exp(x)

    def dph(x):
        if fm == "relu":
            return 1.0 if x > 0 else 0.0
        return 1.0 if x > 0 else math.exp(x)

    T, D, Dv = len(q), len(q[0]), len(v[0])
    S = [[sum(ph(k[s][i]) * v[s][j] for s in range(T)) for j in range(Dv)] for i in range(D)]
    z = [sum(ph(k[s][i]) for s in range(T)) for i in range(D)]
    den = [sum(ph(q[t][i]) * z[i] for i in range(D)) + eps for t in range(T)]
    mq = 0.0
    for t in range(T):
        for i in range(D):
            u = sum(S[i][j] * do[t][j] for j in range(Dv))
            mq = max(mq, abs(u / den[t] * dph(q[t][i])))
    dS = [[sum(ph(q[t][i]) * do[t][j] / den[t] for t in range(T)) for j in range(Dv)] for i in range(D)]
    mk = 0.0
    for s in range(T):
        for i in range(D):
            g = sum(dS[i][j] * v[s][j] for j in range(Dv))
            mk = max(mk, abs(g * dph(k[s][i])))
    return mq, mk


@pytest.mark.parametrize("fm", ["elu1", "relu"])
@pytest.mark.parametrize("T,D,Dv,eps", [(1, 8, 8, 1e-6), (1, 5, 3, 0.7), (6, 4, 4, 1e-6), (9, 5, 7, 2.0)])
def test_leading_terms_match_elementwise_loop(T, D, Dv, eps, fm):
    """bwd_leading_terms_head (the error scale of the T = 1 normalised gradient
    checks) against a pure-Python element-by-element loop over its summands."""
    q, k, do = rand((T, D), 130 + T), rand((T, D), 131 + T), rand((T, Dv), 132 + T)
    v = rand((T, Dv), 133 + T)
    if fm == "relu":  # keep every row's denominator away from eps alone
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    got = oracle.bwd_leading_terms_head(q, k, v, do, eps, fm)
    ref = leading_terms_loop(q.tolist(), k.tolist(), v.tolist(), do.tolist(), eps, fm)
    np.testing.assert_allclose(got, ref, rtol=1e-12)


def test_leading_terms_pins_catch_planted_mistakes():
    """Slips planted in a copy of bwd_leading_terms_head (phi' dropped from
    either term, a sum over elements for the max, eps left out of den, the
    dS of simple_la) each fail the element-by-element loop. Q and K are all
    negative here, so phi' < 1 on every element and dropping it changes each
    maximum; eps is of the size of den, so leaving it out shows."""
    T, D, Dv, eps = 5, 4, 6, 1.5
    q, k = -np.abs(rand((T, D), 141)) - 0.3, -np.abs(rand((T, D), 142)) - 0.3
    v, do = rand((T, Dv), 143), rand((T, Dv), 144)
    ref = np.array(leading_terms_loop(q.tolist(), k.tolist(), v.tolist(), do.tolist(), eps))

    def variant(kind):
        qt, kt = oracle.phi(q), oracle.phi(k)
        s, z = kt.T @ v, kt.sum(axis=0)
        den = qt @ z + (0.0 if kind == "no_eps" else eps)
        u = do @ s.T
        ds = qt.T @ (do if kind == "simple_ds" else do / den[:, None])
        dq_term = u / den[:, None] * (1.0 if kind == "no_dphi_q" else oracle.dphi(q))
        dk_term = (v @ ds.T) * (1.0 if kind == "no_dphi_k" else oracle.dphi(k))
        red = (lambda a: float(np.sum(np.abs(a)))) if kind == "sum_not_max" else (lambda a: float(np.max(np.abs(a))))
        return np.array([red(dq_term), red(dk_term)])

    np.testing.assert_allclose(variant("none"), ref, rtol=1e-12)
    np.testing.assert_allclose(oracle.bwd_leading_terms_head(q, k, v, do, eps), ref, rtol=1e-12)
    for kind in ("no_eps", "simple_ds", "no_dphi_q", "no_dphi_k", "sum_not_max"):
        bad = variant(kind)
        assert np.max(np.abs(bad - ref) / ref) > 1e-3, kind


@pytest.mark.parametrize("simple", [False, True])
def test_causal_batched_bwd_matches_per_head(simple):
    """The batched causal backward is causal_bwd_head on each decoded head,
    in place, bitwise, with D != Dv and heads that differ."""
    from synth import Workload
    w = Workload("t", 2, 3, 21, 6, "bf16", seed=151, Dv=10)
    x = make_inputs(w)
    dq, dk, dv = oracle.causal_bwd(x["q"], x["k"], x["v"], x["do"], "bf16", 0.2, simple)
    assert dq.shape == dk.shape == w.shape and dv.shape == w.shape_v
    d = {n: oracle.decode(x[n], "bf16") for n in ("q", "k", "v", "do")}
    for b in range(2):
        for h in range(3):
            ref = oracle.causal_bwd_head(d["q"][b, h], d["k"][b, h], d["v"][b, h], d["do"][b, h], 0.2, simple)
            for got, r in zip((dq[b, h], dk[b, h], dv[b, h]), ref):
                np.testing.assert_array_equal(got, r)
    assert not np.array_equal(dq[0, 0], dq[1, 2])


@pytest.mark.parametrize("simple", [False, True])
def test_backward_halves_compose_and_add_over_tokens(simple):
    """The Q side and K/V side of the backward, taken one at a time: with the
    full state they give bwd_head's dQ, their dS and dz add up over any split
    of the tokens (a sum over t), and the K/V side then gives bwd_head's dK, dV."""
    T, D = 23, 6
    q, k, v, do = (rand((T, D), 91 + i) for i in range(4))
    dq_ref, dk_ref, dv_ref = oracle.bwd_head(q, k, v, do, 0.25, simple)
    s, z = oracle.state_head(k, v)
    dq, ds, dz = oracle.bwd_q_side_head(q, do, s, z, 0.25, simple)
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-13, atol=1e-13)
    _, ds_a, dz_a = oracle.bwd_q_side_head(q[:9], do[:9], s, z, 0.25, simple)
    dq_b, ds_b, dz_b = oracle.bwd_q_side_head(q[9:], do[9:], s, z, 0.25, simple)
    np.testing.assert_allclose(ds_a + ds_b, ds, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dz_a + dz_b, dz, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dq_b, dq_ref[9:], rtol=1e-13, atol=1e-13)
    dk, dv = oracle.bwd_kv_side_head(k, v, ds, dz, simple)
    np.testing.assert_allclose(dk, dk_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dv, dv_ref, rtol=1e-13, atol=1e-13)
    o = oracle.output_head(q, s, z, 0.25, simple)
    np.testing.assert_allclose(o, oracle.quadratic_head(q, k, v, 0.25, simple), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- relu and identity maps

def test_relu_and_identity_maps():
    torch = pytest.importorskip("torch")
    x = np.concatenate([rand((1000,), 61, 3.0), [0.0, -0.0, 1e-300, -1e-300]])
    np.testing.assert_array_equal(oracle.phi(x, "relu"), torch.relu(torch.tensor(x)).numpy())
    np.testing.assert_array_equal(oracle.phi(x, "identity"), x)
    np.testing.assert_array_equal(oracle.dphi(x, "relu"), (x > 0).astype(np.float64))
    assert oracle.dphi(np.array([0.0]), "relu")[0] == 0.0
    np.testing.assert_array_equal(oracle.dphi(x, "identity"), np.ones_like(x))
    assert np.isnan(oracle.phi(np.array([np.nan]), "relu")[0])


CASES_OTHER_MAPS = [("relu", False), ("relu", True), ("identity", True), ("identity", False)]


def positive_if_identity_normalised(x, fm, simple):
    # with the identity map a normalised denominator can vanish; keep it away
    return np.abs(x) + 0.5 if (fm == "identity" and not simple) else x


@pytest.mark.parametrize("fm,simple", CASES_OTHER_MAPS)
@pytest.mark.parametrize("T,D", [(1, 5), (7, 5), (16, 8)])
def test_other_maps_linear_form_matches_brute_force(T, D, fm, simple):
    q, k, v = (rand((T, D), 71 + i) for i in range(3))
    q, k = (positive_if_identity_normalised(a, fm, simple) for a in (q, k))
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.3, simple, fm)
    o, _, _ = oracle.fwd_head(q, k, v, 0.3, simple, fm)
    assert np.max(np.abs(o - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("fm,simple", CASES_OTHER_MAPS)
def test_other_maps_bwd_matches_finite_differences(fm, simple):
    T, D = 9, 6
    q = away_from_zero(rand((T, D), 81), 1e-3)
    k = away_from_zero(rand((T, D), 82), 1e-3)
    q, k = (positive_if_identity_normalised(a, fm, simple) for a in (q, k))
    v, do = rand((T, D), 83), rand((T, D), 84)
    eps = 0.5
    grads = dict(zip("qkv", oracle.bwd_head(q, k, v, do, eps, simple, fm)))
    coords = [(t, d) for t in range(T) for d in range(D)]
    for name, g in grads.items():
        fd = finite_difference(q, k, v, do, eps, simple, name, coords, fm=fm).reshape(T, D)
        assert np.max(np.abs(g - fd)) <= 1e-6 * max(1.0, np.abs(fd).max()), (fm, name)


@pytest.mark.parametrize("simple", [False, True])
def test_relu_bwd_matches_torch_autograd_of_quadratic_form(simple):
    torch = pytest.importorskip("torch")
    T, D = 40, 12
    q, k, v, do = (rand((T, D), s) for s in (91, 92, 93, 94))
    eps = 0.05
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    a = torch.relu(tq) @ torch.relu(tk).T
    o = a @ tv
    if not simple:
        o = o / (a.sum(dim=1, keepdim=True) + eps)
    (o * torch.tensor(do)).sum().backward()
    for g, t in zip(oracle.bwd_head(q, k, v, do, eps, simple, "relu"), (tq, tk, tv)):
        ref = t.grad.numpy()
        assert np.max(np.abs(g - ref)) <= 1e-12 * np.abs(ref).max()


# ---------------------------------------------------------------- causal form

def causal_brute_force(q, k, v, eps, simple, fm="elu1", scale=1.0):
    """Pure-Python masked quadratic form: O_t = sum_{s<=t} a_ts v_s / (sum_{s<=t} a_ts + eps)."""
    def ph(x):
        if fm == "relu":
            return x if x > 0 else 0.0
        if fm == "identity":
            return x
        return x + 1.0 if x > 0 else math.exp(x)
    T, D, Dv = len(q), len(q[0]), len(v[0])
    out = []
    for t in range(T):
        a = [sum(scale * ph(q[t][i]) * ph(k[s][i]) for i in range(D)) for s in range(t + 1)]
        row = [sum(a[s] * v[s][j] for s in range(t + 1)) for j in range(Dv)]
        if not simple:
            den = sum(a) + eps
            row = [x / den for x in row]
        out.append(row)
    return np.array(out)


@pytest.mark.parametrize("fm", ["elu1", "relu"])
@pytest.mark.parametrize("simple", [False, True])
@pytest.mark.parametrize("T,D,Dv", [(1, 4, 4), (9, 5, 5), (17, 6, 3), (33, 8, 12)])
def test_causal_forms_match_brute_force(T, D, Dv, simple, fm):
    q, k, v = rand((T, D), 81), rand((T, D), 82), rand((T, Dv), 83)
    eps = 0.3
    ref = causal_brute_force(q.tolist(), k.tolist(), v.tolist(), eps, simple, fm)
    scale = np.max(np.abs(ref))
    oq = oracle.causal_quadratic_head(q, k, v, eps, simple, fm)
    orr, s, z = oracle.causal_recurrent_head(q, k, v, eps, simple, fm)
    assert np.max(np.abs(oq - ref)) <= 1e-12 * scale
    assert np.max(np.abs(orr - ref)) <= 1e-12 * scale
    rows = sorted({0, T // 2, T - 1})
    osr = oracle.causal_sampled_rows_head(q, k, v, rows, eps, simple, fm)
    assert np.max(np.abs(osr - ref[rows])) <= 1e-12 * scale
    # the recurrent form's final state is the non-causal state
    s_ref, z_ref = oracle.state_head(k, v, fm)
    np.testing.assert_allclose(s, s_ref, rtol=1e-12, atol=1e-12 * np.abs(s_ref).max())
    np.testing.assert_allclose(z, z_ref, rtol=1e-12)


@pytest.mark.parametrize("simple", [False, True])
def test_causal_last_row_is_the_noncausal_row(simple):
    """The last token sees every token: its causal output equals the
    non-causal output row (pinned independently above)."""
    T, D = 50, 16
    q, k, v = rand((T, D), 84), rand((T, D), 85), rand((T, D), 86)
    o_c, _, _ = oracle.causal_recurrent_head(q, k, v, 1e-6, simple)
    o_n, _, _ = oracle.fwd_head(q, k, v, 1e-6, simple)
    np.testing.assert_allclose(o_c[-1], o_n[-1], rtol=1e-12, atol=1e-12 * np.abs(o_n).max())
    assert np.max(np.abs(o_c[0] - o_n[0])) > 1e-3 * np.abs(o_n).max()  # the first row differs


@pytest.mark.parametrize("simple", [False, True])
def test_causal_first_row_closed_form(simple):
    """O_0 = a v_0 / (a + eps) (simple_la: a v_0) with a = phi(q_0) . phi(k_0)."""
    T, D = 7, 6
    q, k, v = rand((T, D), 87), rand((T, D), 88), rand((T, D), 89)
    eps = 0.25
    a = float(oracle.phi(q[0]) @ oracle.phi(k[0]))
    want = a * v[0] if simple else a * v[0] / (a + eps)
    o, _, _ = oracle.causal_recurrent_head(q, k, v, eps, simple)
    np.testing.assert_allclose(o[0], want, rtol=1e-14)


def test_causal_rows_ignore_later_tokens():
    """Changing K and V after position t leaves rows 0..t unchanged."""
    T, D, t = 40, 8, 23
    q, k, v = rand((T, D), 90), rand((T, D), 91), rand((T, D), 92)
    o1, _, _ = oracle.causal_recurrent_head(q, k, v, 1e-6, False)
    k2, v2 = k.copy(), v.copy()
    k2[t + 1:] = rand((T - t - 1, D), 93)
    v2[t + 1:] = rand((T - t - 1, D), 94)
    o2, _, _ = oracle.causal_recurrent_head(q, k2, v2, 1e-6, False)
    np.testing.assert_array_equal(o1[: t + 1], o2[: t + 1])
    assert np.max(np.abs(o1[t + 1:] - o2[t + 1:])) > 1e-3


def test_causal_v_ones_gives_ones():
    T, D = 30, 8
    q, k = rand((T, D), 95), rand((T, D), 96)
    eps = 1e-6
    o, _, _ = oracle.causal_recurrent_head(q, k, np.ones((T, 5)), eps, False)
    a = np.cumsum(oracle.phi(k) @ oracle.phi(q).T, axis=0).diagonal()  # sum_{s<=t} a_ts
    np.testing.assert_allclose(o, np.repeat((a / (a + eps))[:, None], 5, axis=1), rtol=1e-13)


def test_causal_batched_matches_per_head_and_quadratic():
    from synth import Workload
    w = Workload("t", 2, 3, 70, 8, "f16", seed=97, Dv=12)
    x = make_inputs(w, with_grad=False)
    o, s, z = oracle.causal_fwd(x["q"], x["k"], x["v"], "f16", 1e-6, False)
    assert o.shape == w.shape_v and s.shape == (2, 3, 8, 12) and z.shape == (2, 3, 8)
    d = {n: oracle.decode(x[n], "f16") for n in ("q", "k", "v")}
    oq = oracle.causal_quadratic_head(d["q"][1, 2], d["k"][1, 2], d["v"][1, 2], 1e-6, False)
    np.testing.assert_allclose(o[1, 2], oq, rtol=1e-12, atol=1e-12 * np.abs(oq).max())


def test_causal_pins_catch_planted_mistakes():
    """Slips planted in a copy of the causal form (mask excluding the diagonal,
    mask transposed, the non-causal form) each fail the brute-force pin."""
    T, D = 12, 4
    q, k, v = rand((T, D), 98), rand((T, D), 99), rand((T, D), 100)
    ref = causal_brute_force(q.tolist(), k.tolist(), v.tolist(), 0.3, False)
    a_full = oracle.phi(q) @ oracle.phi(k).T
    for kind, a in (("strict_mask", np.tril(a_full, -1)), ("upper_mask", np.triu(a_full)),
                    ("no_mask", a_full), ("none", np.tril(a_full))):
        o = (a @ v) / (a.sum(axis=1) + 0.3)[:, None]
        err = np.max(np.abs(o - ref)) / np.abs(ref).max()
        if kind == "none":
            assert err <= 1e-12
        else:
            assert err > 1e-3, kind


def causal_loss(q, k, v, do, eps, simple, fm="elu1"):
    return float(np.sum(oracle.causal_quadratic_head(q, k, v, eps, simple, fm) * do))


@pytest.mark.parametrize("simple", [False, True])
@pytest.mark.parametrize("D,Dv", [(16, 16), (8, 12)])
def test_causal_bwd_matches_torch_autograd(D, Dv, simple):
    torch = pytest.importorskip("torch")
    T = 40
    q, k = rand((T, D), 110), rand((T, D), 111)
    v, do = rand((T, Dv), 112), rand((T, Dv), 113)
    eps = 0.05
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    a = torch.tril((torch.nn.functional.elu(tq) + 1) @ (torch.nn.functional.elu(tk) + 1).T)
    o = a @ tv
    if not simple:
        o = o / (a.sum(dim=1, keepdim=True) + eps)
    (o * torch.tensor(do)).sum().backward()
    got = oracle.causal_bwd_head(q, k, v, do, eps, simple)
    for g, t in zip(got, (tq, tk, tv)):
        ref = t.grad.numpy()
        assert np.max(np.abs(g - ref)) <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("fm", ["elu1", "relu"])
@pytest.mark.parametrize("simple", [False, True])
def test_causal_bwd_matches_finite_differences(simple, fm):
    T, D, Dv = 7, 3, 4
    q = away_from_zero(rand((T, D), 114), 1e-4)
    k = away_from_zero(rand((T, D), 115), 1e-4)
    v, do = rand((T, Dv), 116), rand((T, Dv), 117)
    eps = 0.5
    got = oracle.causal_bwd_head(q, k, v, do, eps, simple, fm)
    arrs = {"q": q, "k": k, "v": v}
    h = 1e-6
    for name, g in zip(("q", "k", "v"), got):
        cols = Dv if name == "v" else D
        fd = np.empty((T, cols))
        for t in range(T):
            for d in range(cols):
                plus = {n: a.copy() for n, a in arrs.items()}
                minus = {n: a.copy() for n, a in arrs.items()}
                plus[name][t, d] += h
                minus[name][t, d] -= h
                fd[t, d] = (causal_loss(plus["q"], plus["k"], plus["v"], do, eps, simple, fm)
                            - causal_loss(minus["q"], minus["k"], minus["v"], do, eps, simple, fm)) / (2 * h)
        assert np.max(np.abs(g - fd)) <= 1e-6 * max(1.0, np.abs(fd).max()), name


@pytest.mark.parametrize("simple", [False, True])
def test_causal_bwd_last_row_gradient_is_noncausal(simple):
    """With dO zero except on the last row, only that row (which sees every
    token) carries a gradient: the causal VJP equals the non-causal one."""
    T, D = 30, 8
    q, k, v = rand((T, D), 118), rand((T, D), 119), rand((T, D), 120)
    do = np.zeros((T, D))
    do[-1] = rand((1, D), 121)[0]
    got = oracle.causal_bwd_head(q, k, v, do, 0.1, simple)
    ref = oracle.bwd_head(q, k, v, do, 0.1, simple)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-12 * np.abs(r).max())


def test_causal_bwd_dv_column_sum():
    """sum_s dV_s = sum_t dO_t a_t / (a_t + eps), a_t = sum_{s <= t} a_ts."""
    T, D = 25, 6
    q, k, v, do = (rand((T, D), s_) for s_ in (122, 123, 124, 125))
    eps = 0.2
    _, _, dv = oracle.causal_bwd_head(q, k, v, do, eps, False)
    a = np.tril(oracle.phi(q) @ oracle.phi(k).T).sum(axis=1)
    np.testing.assert_allclose(dv.sum(axis=0), (do * (a / (a + eps))[:, None]).sum(axis=0), rtol=1e-12)


# ------------------------------------------------------------- optional scale
# The scale multiplies phi(q) (flash-linear-attention's kernels scale the
# feature-mapped query the same way); 1 is the method as stated.

@pytest.mark.parametrize("scale", [0.125, 3.0])
@pytest.mark.parametrize("simple", [False, True])
def test_scale_matches_brute_force(simple, scale):
    T, D, Dv = 9, 5, 4
    q, k, v = rand((T, D), 130), rand((T, D), 131), rand((T, Dv), 132)
    eps = 0.3
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), eps, simple, scale=scale)
    o, _, _ = oracle.fwd_head(q, k, v, eps, simple, scale=scale)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    np.testing.assert_allclose(oracle.quadratic_head(q, k, v, eps, simple, scale=scale), ref, rtol=1e-12,
                               atol=1e-12 * np.abs(ref).max())
    cref = causal_brute_force(q.tolist(), k.tolist(), v.tolist(), eps, simple, scale=scale)
    co, _, _ = oracle.causal_recurrent_head(q, k, v, eps, simple, scale=scale)
    np.testing.assert_allclose(co, cref, rtol=1e-12, atol=1e-12 * np.abs(cref).max())


def test_scale_invariants():
    """simple_la is homogeneous of degree 1 in the scale (O and every
    gradient); in normalised mode scale s with eps equals scale 1 with eps/s
    (O and every gradient, eps held constant)."""
    T, D, Dv = 30, 6, 5
    q, k, v, do = rand((T, D), 133), rand((T, D), 134), rand((T, Dv), 135), rand((T, Dv), 136)
    s_, eps = 0.37, 0.05
    for fwd, bwd in ((oracle.fwd_head, oracle.bwd_head), (oracle.causal_recurrent_head, oracle.causal_bwd_head)):
        o1 = fwd(q, k, v, eps, True)[0]
        os_ = fwd(q, k, v, eps, True, scale=s_)[0]
        np.testing.assert_allclose(os_, s_ * o1, rtol=1e-12)
        for a, b in zip(bwd(q, k, v, do, eps, True, scale=s_), bwd(q, k, v, do, eps, True)):
            np.testing.assert_allclose(a, s_ * b, rtol=1e-11, atol=1e-12 * np.abs(b).max())
        np.testing.assert_allclose(fwd(q, k, v, eps, False, scale=s_)[0], fwd(q, k, v, eps / s_, False)[0],
                                   rtol=1e-12)
        for a, b in zip(bwd(q, k, v, do, eps, False, scale=s_), bwd(q, k, v, do, eps / s_, False)):
            np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12 * np.abs(b).max())


@pytest.mark.parametrize("simple", [False, True])
def test_scale_bwd_matches_finite_differences(simple):
    T, D, Dv = 6, 3, 4
    q = away_from_zero(rand((T, D), 137), 1e-4)
    k = away_from_zero(rand((T, D), 138), 1e-4)
    v, do = rand((T, Dv), 139), rand((T, Dv), 140)
    eps, s_ = 0.5, 2.5
    got = oracle.bwd_head(q, k, v, do, eps, simple, scale=s_)
    coords = {"q": [(t, d) for t in range(T) for d in range(D)], "k": [(t, d) for t in range(T) for d in range(D)],
              "v": [(t, d) for t in range(T) for d in range(Dv)]}
    for name, g in zip(("q", "k", "v"), got):
        fd = finite_difference(q, k, v, do, eps, simple, name, coords[name], scale=s_)
        np.testing.assert_allclose(g.reshape(-1), fd, rtol=1e-6, atol=1e-6 * np.abs(fd).max())


@pytest.mark.parametrize("simple", [False, True])
def test_scale_causal_bwd_matches_torch_autograd(simple):
    torch = pytest.importorskip("torch")
    T, D, Dv = 24, 8, 6
    q, k = rand((T, D), 141), rand((T, D), 142)
    v, do = rand((T, Dv), 143), rand((T, Dv), 144)
    eps, s_ = 0.05, 0.3
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    a = torch.tril(s_ * (torch.nn.functional.elu(tq) + 1) @ (torch.nn.functional.elu(tk) + 1).T)
    o = a @ tv
    if not simple:
        o = o / (a.sum(dim=1, keepdim=True) + eps)
    (o * torch.tensor(do)).sum().backward()
    got = oracle.causal_bwd_head(q, k, v, do, eps, simple, scale=s_)
    for g, t in zip(got, (tq, tk, tv)):
        ref = t.grad.numpy()
        assert np.max(np.abs(g - ref)) <= 1e-12 * np.abs(ref).max()
