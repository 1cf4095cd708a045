"""fp64 CPU oracle: plain definitions of non-causal linear attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path. All arithmetic is numpy float64; no blocking, splitting or
reordering beyond the definitions written out below.
"""
from __future__ import annotations

import numpy as np


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs.

    f32 and f16 widen exactly; bf16 is stored as uint16 bit patterns, whose
    value is the float32 with those bits in the upper half.
    """
    if dtype in ("f32", "f16"):
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        b = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


FEATURE_MAPS = ("elu1", "relu", "identity")


def phi(x: np.ndarray, fm: str = "elu1") -> np.ndarray:
    """Feature map. "elu1" (the method's statement): elu(x) + 1, written
    piecewise, x + 1 for x > 0 and exp(x) else (the piecewise form avoids
    exp(x) - 1 + 1, which cancels for x << 0). The pages' models vary the
    kernelised map (FBi-LA README, "Models"); "relu" (max(x, 0)) and
    "identity" (x) are the two plain alternatives offered."""
    x = np.asarray(x, dtype=np.float64)
    if fm == "relu":
        return np.maximum(x, 0.0)
    if fm == "identity":
        return x.copy()
    assert fm == "elu1", fm
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def qfeat(q: np.ndarray, fm: str = "elu1", scale: float = 1.0) -> np.ndarray:
    """The query feature scale * phi(q). The optional scale multiplies phi(q),
    as flash-linear-attention's kernels multiply the (feature-mapped) query by
    their `scale` argument; 1 leaves the method as stated."""
    return scale * phi(q, fm)


def dphi(x: np.ndarray, fm: str = "elu1") -> np.ndarray:
    """Derivative of phi. elu1: 1 for x > 0, exp(x) for x <= 0 (both sides are
    1 at 0). relu: 1 for x > 0, 0 for x <= 0 (0 at the kink). identity: 1."""
    x = np.asarray(x, dtype=np.float64)
    if fm == "relu":
        return np.where(x > 0, 1.0, 0.0)
    if fm == "identity":
        return np.ones_like(x)
    assert fm == "elu1", fm
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def quadratic_head(q, k, v, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0) -> np.ndarray:
    """Quadratic ("parallel") form for one (batch, head): Q, K [T, Dk] and
    V [T, Dv] -> O [T, Dv].

    A = phi(Q) phi(K)^T (T x T); normalised: O = (A V) / (A 1 + eps),
    simple_la: O = A V. flash-linear-attention README, "Different forms of
    linear attention", Parallel. Cost O(T^2 D): tiny T only.
    """
    a = qfeat(q, fm, scale) @ phi(k, fm).T
    num = a @ np.asarray(v, dtype=np.float64)
    if simple:
        return num
    return num / (a.sum(axis=1) + eps)[:, None]


def output_head(q, s, z, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0) -> np.ndarray:
    """Last step of the forward for one (batch, head), from a given state:
    O = phi(Q) S / (phi(Q) z + eps), or phi(Q) S for simple_la (FBi-LA
    README, intro and "Update" 2024-12-28)."""
    qt = qfeat(q, fm, scale)
    num = qt @ s
    if simple:
        return num
    den = qt @ z + eps
    return num / den[:, None]


def fwd_head(q, k, v, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Linear form for one (batch, head): returns (O, S, z).

    S = phi(K)^T V (Dk x Dv, S[i, j] = sum_t phi(k_t)[i] v_t[j]),
    z = sum_t phi(k_t), then O from output_head.
    """
    s, z = state_head(k, v, fm)
    return output_head(q, s, z, eps, simple, fm, scale), s, z


def bwd_q_side_head(q, do, s, z, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Q side of the backward for one (batch, head), from the forward state.

    The chain rule applied to the formula of fwd_head (the FBi-LA README's
    "Update" 2024-12-30 names an optimised backward; it prints no formula).
    Returns (dQ, dS, dz) for the rows given (dS and dz summed over them):
      u_t   = S dO_t
      den_t = phi(q_t) . z + eps,  r_t = phi(q_t) . u_t,  c_t = -r_t / den_t^2
      dphi(q_t) = u_t / den_t + c_t z            (simple_la: u_t)
      dS    = sum_t phi(q_t) (dO_t / den_t)^T    (simple_la: sum phi(q_t) dO_t^T)
      dz    = sum_t c_t phi(q_t)                 (simple_la: 0)
      dQ = dphi(q) * phi'(q)
    """
    do = np.asarray(do, dtype=np.float64)
    qt = qfeat(q, fm, scale)
    u = do @ s.T  # row t is S dO_t
    dq_of = scale * dphi(q, fm)  # d(scale phi(q)) / dq
    if simple:
        return u * dq_of, qt.T @ do, np.zeros_like(z)
    den = qt @ z + eps
    r = np.einsum("td,td->t", qt, u)
    c = -r / den**2
    dqt = u / den[:, None] + c[:, None] * z[None, :]
    return dqt * dq_of, qt.T @ (do / den[:, None]), c @ qt


def bwd_kv_side_head(k, v, ds, dz, simple: bool, fm: str = "elu1"):
    """K/V side of the backward for one (batch, head), from (dS, dz), by the
    chain rule through S = phi(K)^T V and z = sum_t phi(k_t) (FBi-LA README,
    "Update" 2024-12-30; no formula printed there):
    dphi(k_t) = dS v_t + dz (simple_la: dS v_t), dK = dphi(k) * phi'(k),
    dV_t = dS^T phi(k_t). Returns (dK, dV)."""
    v = np.asarray(v, dtype=np.float64)
    kt = phi(k, fm)
    dkt = v @ ds.T if simple else v @ ds.T + dz[None, :]
    return dkt * dphi(k, fm), kt @ ds


def bwd_head(q, k, v, do, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Vector-Jacobian product of L = sum(O * dO) for one (batch, head).

    Returns (dQ, dK, dV). eps is a constant. Derived by the chain rule from
    fwd_head (the FBi-LA README's "Update" 2024-12-30 names an optimised
    backward; it prints no formula): the state, then bwd_q_side_head, then
    bwd_kv_side_head.
    """
    s, z = state_head(k, v, fm)
    dq, ds, dz = bwd_q_side_head(q, do, s, z, eps, simple, fm, scale)
    dk, dv = bwd_kv_side_head(k, v, ds, dz, simple, fm)
    return dq, dk, dv


def bwd_leading_terms_head(q, k, v, do, eps: float, fm: str = "elu1"):
    """Largest summands of dQ and dK in normalised mode, for error scaling.

    dphi(q_t) = u_t / den_t + c_t z and dphi(k_t) = dS v_t + dz add terms that
    cancel almost exactly when the output hardly depends on Q or K (T = 1:
    O_t = a_t v / (a_t + eps), so both gradients are O(eps)). Returns
    (max |u/den * phi'(q)|, max |dS v * phi'(k)|): the scale rounding errors of
    the summands are measured against.
    """
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    qt, kt = phi(q, fm), phi(k, fm)
    s = kt.T @ v
    z = kt.sum(axis=0)
    den = qt @ z + eps
    u = do @ s.T
    ds = qt.T @ (do / den[:, None])
    return (float(np.max(np.abs(u / den[:, None] * dphi(q, fm)))),
            float(np.max(np.abs((v @ ds.T) * dphi(k, fm)))))


def state_head(k, v, fm: str = "elu1"):
    """The state alone for one (batch, head): S = phi(K)^T V and z = sum_t phi(k_t)."""
    kt = phi(k, fm)
    return kt.T @ np.asarray(v, dtype=np.float64), kt.sum(axis=0)


def sampled_rows_head(q, k, v, rows, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0) -> np.ndarray:
    """Output rows O_t, t in ``rows``, computed one by one from the quadratic form.

    O_t = sum_s a_ts v_s / (sum_s a_ts + eps) with a_ts = phi(q_t) . phi(k_s);
    cost O(T D) per row, so it serves full-size sequences.
    """
    kt = phi(k, fm)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), v.shape[1]))
    for n, t in enumerate(rows):
        a = kt @ qfeat(q[t], fm, scale)
        out[n] = a @ v
        if not simple:
            out[n] /= a.sum() + eps
    return out


def _heads(x: np.ndarray, dtype: str):
    """Decode a [B, H, T, D] storage array to a float64 [B*H, T, D] view."""
    d = decode(x, dtype)
    return d.reshape(-1, d.shape[-2], d.shape[-1])


def fwd(q, k, v, dtype: str, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Forward over storage arrays Q, K [B, H, T, Dk] and V [B, H, T, Dv]:
    (O [B,H,T,Dv], S [B,H,Dk,Dv], z [B,H,Dk])."""
    lead = q.shape[:-1]
    qh, kh, vh = _heads(q, dtype), _heads(k, dtype), _heads(v, dtype)
    n, dk, dv = qh.shape[0], q.shape[-1], v.shape[-1]
    o = np.empty(vh.shape)
    s = np.empty((n, dk, dv))
    z = np.empty((n, dk))
    for h in range(n):
        o[h], s[h], z[h] = fwd_head(qh[h], kh[h], vh[h], eps, simple, fm, scale)
    return (o.reshape(lead + (dv,)), s.reshape(lead[:-1] + (dk, dv)),
            z.reshape(lead[:-1] + (dk,)))


def bwd(q, k, v, do, dtype: str, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Backward over storage arrays Q, K [B, H, T, Dk] and V, dO [B, H, T, Dv]:
    (dQ, dK, dV), float64, shaped like Q, K, V."""
    qh, kh, vh, dh = (_heads(x, dtype) for x in (q, k, v, do))
    dq, dk, dv = np.empty(qh.shape), np.empty(kh.shape), np.empty(vh.shape)
    for h in range(qh.shape[0]):
        dq[h], dk[h], dv[h] = bwd_head(qh[h], kh[h], vh[h], dh[h], eps, simple, fm, scale)
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


# ---------------------------------------------------------------- causal form
# flash-linear-attention README, "Different forms of linear attention": the
# causal (autoregressive) variant, where token t attends to tokens s <= t. Its
# Parallel form is the quadratic form with a causal mask; its FusedRecurrent
# form carries the state S_t = S_{t-1} + phi(k_t) v_t^T from token to token.

def causal_quadratic_head(q, k, v, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0) -> np.ndarray:
    """Causal Parallel form for one (batch, head): A = phi(Q) phi(K)^T with
    A[t, s] = 0 for s > t; normalised O = (A V) / (A 1 + eps), simple_la
    O = A V. Cost O(T^2 D): tiny T only."""
    a = np.tril(qfeat(q, fm, scale) @ phi(k, fm).T)
    num = a @ np.asarray(v, dtype=np.float64)
    if simple:
        return num
    return num / (a.sum(axis=1) + eps)[:, None]


def causal_recurrent_head(q, k, v, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Causal Recurrent form for one (batch, head), token by token:
    S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t) (S_0 = 0, z_0 = 0),
    O_t = phi(q_t) S_t / (phi(q_t) . z_t + eps), or phi(q_t) S_t for simple_la.
    Returns (O, S_T, z_T); S_T, z_T are the non-causal state of the head."""
    qt, kt = qfeat(q, fm, scale), phi(k, fm)
    v = np.asarray(v, dtype=np.float64)
    T, dk = kt.shape
    s = np.zeros((dk, v.shape[1]))
    z = np.zeros(dk)
    o = np.empty((T, v.shape[1]))
    for t in range(T):
        s += np.outer(kt[t], v[t])
        z += kt[t]
        o[t] = qt[t] @ s
        if not simple:
            o[t] /= qt[t] @ z + eps
    return o, s, z


def causal_sampled_rows_head(q, k, v, rows, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0) -> np.ndarray:
    """Causal output rows O_t, t in ``rows``, one by one from the masked
    quadratic form: O_t = sum_{s <= t} a_ts v_s / (sum_{s <= t} a_ts + eps),
    a_ts = phi(q_t) . phi(k_s). Cost O(t D) per row, for full-size sequences."""
    kt = phi(k, fm)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows), v.shape[1]))
    for n, t in enumerate(rows):
        a = kt[: t + 1] @ qfeat(q[t], fm, scale)
        out[n] = a @ v[: t + 1]
        if not simple:
            out[n] /= a.sum() + eps
    return out


def causal_fwd(q, k, v, dtype: str, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Causal forward over storage arrays Q, K [B, H, T, Dk], V [B, H, T, Dv]:
    (O [B,H,T,Dv], S [B,H,Dk,Dv], z [B,H,Dk]) by the recurrent form; S and z are
    the full-sequence state."""
    lead = q.shape[:-1]
    qh, kh, vh = _heads(q, dtype), _heads(k, dtype), _heads(v, dtype)
    n, dk, dv = qh.shape[0], q.shape[-1], v.shape[-1]
    o = np.empty(vh.shape)
    s = np.empty((n, dk, dv))
    z = np.empty((n, dk))
    for h in range(n):
        o[h], s[h], z[h] = causal_recurrent_head(qh[h], kh[h], vh[h], eps, simple, fm, scale)
    return (o.reshape(lead + (dv,)), s.reshape(lead[:-1] + (dk, dv)),
            z.reshape(lead[:-1] + (dk,)))


def causal_bwd_head(q, k, v, do, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Vector-Jacobian product of L = sum(O * dO) for the causal form of one
    (batch, head), eps held constant: the chain rule through the recurrent
    form (causal_recurrent_head). With the inclusive prefixes S_t, z_t,
      den_t = phi(q_t) . z_t + eps,  u_t = S_t dO_t,  r_t = phi(q_t) . u_t,
      c_t = -r_t / den_t^2,  w_t = dO_t / den_t,
      dphi(q_t) = u_t / den_t + c_t z_t           (simple_la: u_t)
    and with the suffixes G_s = sum_{t >= s} phi(q_t) w_t^T (simple_la: dO_t),
    g_s = sum_{t >= s} c_t phi(q_t) (simple_la: 0),
      dphi(k_s) = G_s v_s + g_s,  dV_s = G_s^T phi(k_s).
    dQ = dphi(q) * phi'(q), dK = dphi(k) * phi'(k). Returns (dQ, dK, dV).
    With a scale, phi(q) stands for scale * phi(q) throughout and dQ gains
    the factor scale."""
    qt, kt = qfeat(q, fm, scale), phi(k, fm)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    T, dk = kt.shape
    dv_ = v.shape[1]
    s = np.zeros((dk, dv_))
    z = np.zeros(dk)
    dqt = np.empty((T, dk))
    w = np.empty((T, dv_))
    c = np.zeros(T)
    for t in range(T):  # forward over the prefix
        s += np.outer(kt[t], v[t])
        z += kt[t]
        u = s @ do[t]
        if simple:
            dqt[t] = u
            w[t] = do[t]
        else:
            den = qt[t] @ z + eps
            c[t] = -(qt[t] @ u) / den**2
            dqt[t] = u / den + c[t] * z
            w[t] = do[t] / den
    g = np.zeros((dk, dv_))
    gz = np.zeros(dk)
    dkt = np.empty((T, dk))
    dv = np.empty((T, dv_))
    for t in range(T - 1, -1, -1):  # backward over the suffix
        g += np.outer(qt[t], w[t])
        gz += c[t] * qt[t]
        dkt[t] = g @ v[t] + gz
        dv[t] = g.T @ kt[t]
    return dqt * (scale * dphi(q, fm)), dkt * dphi(k, fm), dv


def causal_bwd(q, k, v, do, dtype: str, eps: float, simple: bool, fm: str = "elu1", scale: float = 1.0):
    """Causal backward over storage arrays Q, K [B, H, T, Dk] and V, dO
    [B, H, T, Dv]: (dQ, dK, dV), float64, shaped like Q, K, V."""
    qh, kh, vh, dh = (_heads(x, dtype) for x in (q, k, v, do))
    dq, dk, dv = np.empty(qh.shape), np.empty(kh.shape), np.empty(vh.shape)
    for h in range(qh.shape[0]):
        dq[h], dk[h], dv[h] = causal_bwd_head(qh[h], kh[h], vh[h], dh[h], eps, simple, fm, scale)
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)
