"""GPU parity of strided views (la_problem.strides): tensors that are views
into larger buffers run without a copy and give the same bytes as the dense
call on contiguous copies of the same values (the work split is a function of
the shape alone), within the oracle's tolerance as well. Covers the Q, K, V
views of a packed [B, T, 3, H, D] projection, feature slices of wider rows,
K and V shared by every head (head stride 0), strided outputs (the bytes
around them untouched), both paths (bidirectional and causal), the step
calls, and autograd through a packed buffer."""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs, normal
from tests.la_testutil import TOL, bytes_equal, decode, max_rel_err, to_device

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def packed_qkv(B, T, H, D, dtype, seed):
    """A [B, T, 3, H, D] buffer of seeded values and its q, k, v views [B, T, H, D]."""
    buf = to_device(normal((B, T, 3, H, D), seed, 1.0, dtype), dtype)
    return buf, buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]


def check_vs_oracle(name, got, ref, dtype):
    err = max_rel_err(decode(got, dtype), ref)
    print(f"  {name}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(decode(got, dtype))) and err <= TOL[dtype], f"{name}: {err:.3e}"


def host(x, dtype):
    """[B, T, H, D] device view -> contiguous [B, H, T, D] storage array."""
    t = x.transpose(1, 2).contiguous().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@pytest.mark.parametrize("causal", [False, True], ids=["bidir", "causal"])
@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64)])
def test_packed_qkv_forward_backward(dtype, D, causal):
    B, T, H = 2, 1500, 4
    seed = 98_000 + D + 7 * ["f32", "f16", "bf16"].index(dtype) + (1 if causal else 0)
    print(f"case packed qkv B{B} T{T} H{H} D{D} {dtype} causal={causal} seed={seed}", flush=True)
    buf, q, k, v = packed_qkv(B, T, H, D, dtype, seed)
    assert not q.is_contiguous()
    do = to_device(normal((B, T, H, D), seed + 9, 1.0, dtype), dtype)
    o, st = la.fwd(q, k, v, layout="bthd", causal=causal)
    g = la.bwd(q, k, v, do, None if causal else st, layout="bthd", causal=causal)
    qc, kc, vc = (x.contiguous() for x in (q, k, v))
    o2, st2 = la.fwd(qc, kc, vc, layout="bthd", causal=causal)
    g2 = la.bwd(qc, kc, vc, do, None if causal else st2, layout="bthd", causal=causal)
    torch.cuda.synchronize()
    assert bytes_equal(o, o2) and bytes_equal(st, st2)
    for a, b in zip(g, g2):
        assert bytes_equal(a, b)
    x = {n: host(t, dtype) for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}
    if causal:
        o_ref = oracle.causal_fwd(x["q"], x["k"], x["v"], dtype, 1e-6, False)[0]
        g_ref = oracle.causal_bwd(x["q"], x["k"], x["v"], x["do"], dtype, 1e-6, False)
    else:
        o_ref = oracle.fwd(x["q"], x["k"], x["v"], dtype, 1e-6, False)[0]
        g_ref = oracle.bwd(x["q"], x["k"], x["v"], x["do"], dtype, 1e-6, False)
    check_vs_oracle("O", o.transpose(1, 2), o_ref, dtype)
    for name, a, r in zip(("dQ", "dK", "dV"), g, g_ref):
        check_vs_oracle(name, a.transpose(1, 2), r, dtype)


@pytest.mark.parametrize("causal", [False, True], ids=["bidir", "causal"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_feature_slices_and_strided_outputs(dtype, causal):
    """[B, H, T, D] views taking D = 64 features out of 128-wide rows, with
    O and the gradients written into the other half of wider buffers, whose
    untouched bytes keep their guard value (the causal scans store their
    outputs as 8-byte row pieces straight from the MFMA results)."""
    B, H, T, D = 2, 3, 2100, 64
    seed = 98_100 + ["f16", "bf16"].index(dtype) + (2 if causal else 0)
    print(f"case feature slices B{B} H{H} T{T} D{D} {dtype} causal={causal} seed={seed}", flush=True)
    wide = {n: to_device(normal((B, H, T, 2 * D), seed + i, 1.0, dtype), dtype)
            for i, n in enumerate(("q", "k", "v", "do"))}
    view = {n: t[..., D:] for n, t in wide.items()}
    outs = {n: torch.full((B, H, T, 2 * D), 7.0, dtype=TDT[dtype], device="cuda") for n in ("o", "dq", "dk", "dv")}
    ov = {n: t[..., :D] for n, t in outs.items()}
    _, st = la.fwd(view["q"], view["k"], view["v"], out=ov["o"], causal=causal)
    la.bwd(view["q"], view["k"], view["v"], view["do"], None if causal else st, dq=ov["dq"], dk=ov["dk"],
           dv=ov["dv"], causal=causal)
    dense = {n: t.contiguous() for n, t in view.items()}
    o2, st2 = la.fwd(dense["q"], dense["k"], dense["v"], causal=causal)
    g2 = la.bwd(dense["q"], dense["k"], dense["v"], dense["do"], None if causal else st2, causal=causal)
    torch.cuda.synchronize()
    assert bytes_equal(st, st2)
    for n, ref in zip(("o", "dq", "dk", "dv"), (o2,) + tuple(g2)):
        assert bytes_equal(ov[n].contiguous(), ref), n
        assert torch.all(outs[n][..., D:] == 7.0), f"{n}: bytes outside the view were written"
    x = {n: np.ascontiguousarray(decode(t, dtype)) for n, t in dense.items()}
    if causal:
        o_ref = oracle.causal_fwd(x["q"], x["k"], x["v"], "f32", 1e-6, False)[0]
        g_ref = oracle.causal_bwd(x["q"], x["k"], x["v"], x["do"], "f32", 1e-6, False)
        for name, a, r in zip(("dQ", "dK", "dV"), (ov["dq"], ov["dk"], ov["dv"]), g_ref):
            check_vs_oracle(name, a, r, dtype)
    else:
        o_ref = oracle.fwd(x["q"], x["k"], x["v"], "f32", 1e-6, False)[0]
    check_vs_oracle("O", ov["o"], o_ref, dtype)


@pytest.mark.parametrize("causal", [False, True], ids=["bidir", "causal"])
def test_kv_shared_by_every_head(causal):
    """K and V given once and read by every head (head stride 0): each head's
    result is the oracle's with that one K, V."""
    B, H, T, D = 2, 4, 1200, 64
    w = Workload("shared-kv", B, 1, T, D, "f16", seed=98_200 + (1 if causal else 0))
    x = make_inputs(w)
    q = to_device(normal((B, H, T, D), w.seed + 10, 1.0, "f16"), "f16")
    do = to_device(normal((B, H, T, D), w.seed + 11, 1.0, "f16"), "f16")
    k1, v1 = to_device(x["k"], "f16"), to_device(x["v"], "f16")
    k, v = k1.expand(B, H, T, D), v1.expand(B, H, T, D)
    assert k.stride(1) == 0
    print(f"case shared K, V B{B} H{H} T{T} causal={causal} seed={w.seed}", flush=True)
    o, st = la.fwd(q, k, v, causal=causal)
    dq, dk, dv = la.bwd(q, k, v, do, None if causal else st, causal=causal)
    kc, vc = k.contiguous(), v.contiguous()
    o2, _ = la.fwd(q, kc, vc, causal=causal)
    torch.cuda.synchronize()
    assert bytes_equal(o, o2)
    qh, dh = decode(q, "f16"), decode(do, "f16")
    kh, vh = oracle.decode(x["k"], "f16"), oracle.decode(x["v"], "f16")
    for b in range(B):
        for h in range(H):
            if causal:
                o_ref = oracle.causal_recurrent_head(qh[b, h], kh[b, 0], vh[b, 0], 1e-6, False)[0]
                g_ref = oracle.causal_bwd_head(qh[b, h], kh[b, 0], vh[b, 0], dh[b, h], 1e-6, False)
            else:
                o_ref = oracle.fwd_head(qh[b, h], kh[b, 0], vh[b, 0], 1e-6, False)[0]
                g_ref = oracle.bwd_head(qh[b, h], kh[b, 0], vh[b, 0], dh[b, h], 1e-6, False)
            assert max_rel_err(decode(o[b, h], "f16"), o_ref) <= TOL["f16"]
            for a, r in zip((dq, dk, dv), g_ref):
                assert max_rel_err(decode(a[b, h], "f16"), r) <= TOL["f16"]


def test_step_calls_with_strides_and_separate_v_width():
    """The four step calls on packed q, k views (D = 64) and a V of width 128
    sliced from a wider buffer, against the dense composition, byte for byte."""
    B, T, H, D, Dv = 2, 900, 3, 64, 128
    buf, q, k, _ = packed_qkv(B, T, H, D, "bf16", 98_300)
    vw = to_device(normal((B, T, H, 2 * Dv), 98_301, 1.0, "bf16"), "bf16")
    v = vw[..., Dv:]
    do = to_device(normal((B, T, H, Dv), 98_302, 1.0, "bf16"), "bf16")
    st = la.fwd_state(k, v, layout="bthd")
    o = la.fwd_output(q, st, layout="bthd", dv=Dv)
    dq = la.bwd_dq(q, do, st, layout="bthd")
    dk, dv = la.bwd_dkv(k, v, layout="bthd")
    qc, kc, vc = q.contiguous(), k.contiguous(), v.contiguous()
    o2, st2 = la.fwd(qc, kc, vc, layout="bthd")
    g2 = la.bwd(qc, kc, vc, do, st2, layout="bthd")
    torch.cuda.synchronize()
    for a, b in ((st, st2), (o, o2), (dq, g2[0]), (dk, g2[1]), (dv, g2[2])):
        assert bytes_equal(a, b)


def test_autograd_through_packed_buffer():
    """linear_attention on the q, k, v views of a packed buffer that requires
    grad: the buffer's gradient holds dQ, dK, dV in its three slots."""
    B, T, H, D = 2, 700, 2, 64
    buf, _, _, _ = packed_qkv(B, T, H, D, "f16", 98_400)
    buf = buf.float().half().requires_grad_(True)
    q, k, v = buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
    o = la.linear_attention(q, k, v, layout="bthd")
    do = to_device(normal((B, T, H, D), 98_401, 1.0, "f16"), "f16")
    o.backward(do)
    with torch.no_grad():
        qc, kc, vc = (x.detach().contiguous() for x in (q, k, v))
        _, st = la.fwd(qc, kc, vc, layout="bthd")
        g = la.bwd(qc, kc, vc, do, st, layout="bthd")
    torch.cuda.synchronize()
    for i in range(3):
        assert bytes_equal(buf.grad[:, :, i].contiguous(), g[i])
