"""Host-side tests of the C ABI: no GPU needed, no kernel is launched.

Every call here is either a pure query (sizes, strings, version) or carries an
argument error, which include/la.h promises to report before any HIP call.
Pointers are fake addresses: they are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

import non_causal_linear_amd as la
from non_causal_linear_amd import Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")

OK, NULL, SHAPE, DTYPE, HEAD_DIM, FLAGS, EPS, WORKSPACE, ALIGN, ALIAS, DEVICE, SCALE, SCRATCH, STRIDE = range(14)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(la.LIB_PATH):
        from non_causal_linear_amd import build
        build.build()
    return la.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_declares_what_binding_expects():
    assert header_functions() == sorted(la.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(la_\w+)$", out, flags=re.M))
    for name in header_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_version_and_status_strings(L):
    assert L.la_version() == 9
    for s in range(14):
        txt = L.la_status_str(s).decode()
        assert txt.startswith("LA_"), txt
    assert L.la_status_str(99).decode() == "unknown la_status"
    assert "HEAD_DIM" in L.la_status_str(HEAD_DIM).decode()


def prob(B=2, H=3, T=100, D=64, dtype=1, flags=0, eps=1e-6, Dv=0, scale=0.0):
    return Problem(B, H, T, D, Dv, dtype, flags, eps, scale)


def test_problem_struct_matches_header():
    # int64 B, H, T, D, Dv; int32 dtype; uint32 flags; float eps, scale; pointer strides
    assert ctypes.sizeof(Problem) == 64
    assert [f[0] for f in Problem._fields_] == ["B", "H", "T", "D", "Dv", "dtype", "flags", "eps", "scale",
                                                "strides"]
    assert ctypes.sizeof(la.Strides) == 8 * 3 * 8
    assert [f[0] for f in la.Strides._fields_] == ["q", "k", "v", "o", "dout", "dq", "dk", "dv"]


def test_state_bytes_formula(L):
    for (B, H, D, Dv) in ((1, 2, 64, 0), (8, 16, 64, 64), (8, 32, 128, 0), (2, 3, 32, 96), (2, 3, 128, 32)):
        p = prob(B=B, H=H, D=D, Dv=Dv)
        assert L.la_state_bytes(ctypes.byref(p)) == B * H * (D * (Dv or D) + D) * 4


def test_workspace_bytes_covers_state_and_partials(L):
    # B8-H16-T16384-D64: 128 heads, each split into several token slices whose
    # partial (S, z) blocks live in the workspace next to two full states
    p = prob(B=8, H=16, T=16384, D=64)
    ws = L.la_workspace_bytes(ctypes.byref(p))
    E = 64 * 64 + 64
    assert 128 * 2 * E * 4 + 2 * 128 * E * 4 <= ws <= 128 * 64 * E * 4
    assert ws % 256 == 0
    # one head, long sequence: more slices, more partials
    one = L.la_workspace_bytes(ctypes.byref(prob(B=1, H=1, T=1 << 20, D=64)))
    assert one >= 64 * E * 4
    # invalid problems report 0
    assert L.la_workspace_bytes(ctypes.byref(prob(D=256, dtype=0))) == 0
    assert L.la_workspace_bytes(ctypes.byref(prob(D=256, Dv=64))) == 0
    assert L.la_workspace_bytes(ctypes.byref(prob(Dv=48))) == 0
    assert L.la_state_bytes(ctypes.byref(prob(dtype=7))) == 0
    assert L.la_workspace_bytes(None) == 0


def test_workspace_is_pure_function_of_shape(L):
    a = L.la_workspace_bytes(ctypes.byref(prob(B=2, H=8, T=262144, D=64, dtype=2, flags=1)))
    b = L.la_workspace_bytes(ctypes.byref(prob(B=2, H=8, T=262144, D=64, dtype=2, flags=1)))
    assert a == b > 0


def test_split_query(L):
    """la_split_of: each step's pieces cover the head's tokens exactly (the
    last piece may be short, none is empty), the answer is a pure function of
    the problem, and invalid problems or NULL pointers return the error and
    leave the output untouched."""
    for kw in (dict(B=8, H=16, T=16384, D=64), dict(B=1, H=1, T=1 << 20, D=128, dtype=2),
               dict(B=4, H=3, T=1, D=32, Dv=96, dtype=0), dict(B=8, H=16, T=4096, D=256),
               dict(B=2, H=8, T=262144, D=64, flags=0x10), dict(B=3, H=5, T=0, D=64)):
        p = prob(**kw)
        out = la.Split()
        assert L.la_split_of(ctypes.byref(p), ctypes.byref(out)) == 0, kw
        T = kw["T"]
        for n, length in (("P", "L"), ("PB", "LB"), ("NQ", "LQ"), ("NK", "LK")):
            pieces, size = getattr(out, n), getattr(out, length)
            assert pieces >= 1, (kw, n)
            if T > 0:
                assert pieces * size >= T and (pieces - 1) * size < T, (kw, n, pieces, size)
        again = la.Split()
        L.la_split_of(ctypes.byref(p), ctypes.byref(again))
        assert bytes(again) == bytes(out)
    # the long single head is cut into more slices than one
    out = la.Split()
    L.la_split_of(ctypes.byref(prob(B=1, H=1, T=1 << 20, D=64)), ctypes.byref(out))
    assert out.P > 1 and out.PB > 1
    sentinel = la.Split(*([-7] * 8))
    assert L.la_split_of(ctypes.byref(prob(D=48)), ctypes.byref(sentinel)) == HEAD_DIM
    assert L.la_split_of(ctypes.byref(prob(dtype=9)), ctypes.byref(sentinel)) == DTYPE
    assert list(bytes(sentinel)) == list(bytes(la.Split(*([-7] * 8))))
    assert L.la_split_of(None, ctypes.byref(sentinel)) == NULL
    assert L.la_split_of(ctypes.byref(prob()), None) == NULL


A = 0x100000  # fake, 256-aligned, never dereferenced
TB = 2 * 3 * 100 * 64 * 2  # bytes of one tensor of prob()


def addrs(n, stride=1 << 24):
    return [ctypes.c_void_p(A + i * stride) for i in range(n)]


def fwd_call(L, p, q=None, k=None, v=None, o=None, state=None, ws=None, ws_bytes=None):
    d = addrs(6)
    q = d[0] if q is None else q
    k = d[1] if k is None else k
    v = d[2] if v is None else v
    o = d[3] if o is None else o
    state = d[4] if state is None else state
    ws = d[5] if ws is None else ws
    if ws_bytes is not None:
        need = ws_bytes
    else:
        need = L.la_workspace_bytes(ctypes.byref(p)) if p is not None else 1 << 20
    return L.la_fwd(ctypes.byref(p) if p is not None else None, q, k, v, o, state, ws, need, None)


def test_fwd_rejects_bad_problems(L):
    assert fwd_call(L, None) == NULL
    assert fwd_call(L, prob(dtype=3)) == DTYPE
    assert fwd_call(L, prob(dtype=-1)) == DTYPE
    for d, dv in ((48, 0), (256, 128), (0, 64), (16, 0), (64, 256), (64, 16), (64, -64), (96, 160), (512, 0)):
        assert fwd_call(L, prob(D=d, Dv=dv)) == HEAD_DIM, (d, dv)
    assert fwd_call(L, prob(B=-1)) == SHAPE
    assert fwd_call(L, prob(T=-5)) == SHAPE
    assert fwd_call(L, prob(H=1 << 30)) == SHAPE
    # one head's rows must stay below 2^31 bytes (32-bit buffer offsets)
    assert fwd_call(L, prob(T=(1 << 31) // (128 * 2), D=128)) == SHAPE
    assert L.la_workspace_bytes(ctypes.byref(prob(T=(1 << 31) // (128 * 2) - 1, D=128))) > 0
    assert L.la_workspace_bytes(ctypes.byref(prob(T=(1 << 31) // (64 * 4), D=64, dtype=0))) == 0
    # the wider of the two head sizes sets the limit
    assert fwd_call(L, prob(T=(1 << 31) // (128 * 2), D=32, Dv=128)) == SHAPE
    assert fwd_call(L, prob(T=(1 << 31) // (128 * 2), D=128, Dv=32)) == SHAPE
    assert L.la_workspace_bytes(ctypes.byref(prob(T=(1 << 31) // (128 * 2) - 1, D=32, Dv=128))) > 0
    assert fwd_call(L, prob(flags=0x40)) == FLAGS
    assert fwd_call(L, prob(flags=0x80000000)) == FLAGS
    assert fwd_call(L, prob(flags=0x4 | 0x8)) == FLAGS  # two feature maps
    assert fwd_call(L, prob(eps=-1e-3)) == EPS
    assert fwd_call(L, prob(eps=float("nan"))) == EPS
    assert fwd_call(L, prob(eps=float("inf"))) == EPS
    assert fwd_call(L, prob(scale=float("nan"))) == SCALE
    assert fwd_call(L, prob(scale=float("-inf"))) == SCALE
    assert "SCALE" in L.la_status_str(SCALE).decode()


def test_fwd_rejects_bad_buffers(L):
    p = prob()
    need = L.la_workspace_bytes(ctypes.byref(p))
    assert fwd_call(L, p, ws_bytes=need - 1) == WORKSPACE
    assert fwd_call(L, p, q=ctypes.c_void_p(0)) == NULL
    assert fwd_call(L, p, o=ctypes.c_void_p(0)) == NULL
    assert fwd_call(L, p, q=ctypes.c_void_p(A + 8)) == ALIGN
    assert fwd_call(L, p, o=ctypes.c_void_p(A + (3 << 24) + 4)) == ALIGN
    assert fwd_call(L, p, ws=ctypes.c_void_p(A + (5 << 24) + 16)) == ALIGN
    # output aliasing an input, fully or partly
    assert fwd_call(L, p, o=ctypes.c_void_p(A)) == ALIAS
    assert fwd_call(L, p, o=ctypes.c_void_p(A + (1 << 24) + TB - 16)) == ALIAS
    # state overlapping the output
    assert fwd_call(L, p, state=ctypes.c_void_p(A + (3 << 24) + 256)) == ALIAS
    # workspace overlapping an input
    assert fwd_call(L, p, ws=ctypes.c_void_p(A + (2 << 24))) == ALIAS


def test_buffer_checks_use_each_tensors_head_size(L):
    """With D != Dv, q/k/dq/dk span T*D and v/o/dout/dv span T*Dv elements per
    head: overlaps are checked on those spans. Every call below is rejected."""
    p = prob(D=32, Dv=128)
    tk, tv = 2 * 3 * 100 * 32 * 2, 2 * 3 * 100 * 128 * 2
    need = L.la_workspace_bytes(ctypes.byref(p))
    assert L.la_state_bytes(ctypes.byref(p)) == 6 * (32 * 128 + 32) * 4
    # o placed tk bytes after v: apart if v spanned tk bytes, but v spans tv
    v = ctypes.c_void_p(A + (2 << 24))
    assert fwd_call(L, p, v=v, o=ctypes.c_void_p(A + (2 << 24) + tk)) == ALIAS
    # the state placed inside o's tv bytes, past its first tk bytes
    assert fwd_call(L, p, state=ctypes.c_void_p(A + (3 << 24) + tk + 256)) == ALIAS
    d = addrs(9)

    def bwd_call(**kw):
        args = dict(q=d[0], k=d[1], v=d[2], do=d[3], state=d[4], dq=d[5], dk=d[6], dv=d[7], ws=d[8])
        args.update(kw)
        return L.la_bwd(ctypes.byref(p), args["q"], args["k"], args["v"], args["do"], args["state"],
                        args["dq"], args["dk"], args["dv"], args["ws"], need, None)

    # dq (tk bytes) placed inside dout's tv bytes, past its first tk bytes
    assert bwd_call(dq=ctypes.c_void_p(A + (3 << 24) + tk + 256)) == ALIAS
    # dv (tv bytes) starting just before dk ends
    assert bwd_call(dv=ctypes.c_void_p(A + (6 << 24) + tk - 16)) == ALIAS
    # dk (tk bytes) starting inside v's tv bytes
    assert bwd_call(dk=ctypes.c_void_p(A + (2 << 24) + tv - 16)) == ALIAS


def test_empty_problems_need_no_device(L):
    # B*H = 0: nothing to compute, nothing launched, NULL tensors accepted
    p = prob(B=0)
    z = ctypes.c_void_p(0)
    assert L.la_fwd(ctypes.byref(p), z, z, z, z, z, ctypes.c_void_p(A), 256, None) == OK
    assert L.la_bwd(ctypes.byref(p), z, z, z, z, z, z, z, z, ctypes.c_void_p(A), 256, None) == OK
    # T = 0 backward and output: no rows, nothing launched
    p = prob(T=0)
    need = L.la_workspace_bytes(ctypes.byref(p))
    assert L.la_fwd_output(ctypes.byref(p), z, ctypes.c_void_p(A), z, None) == OK
    assert L.la_bwd(ctypes.byref(p), z, z, z, z, ctypes.c_void_p(A), z, z, z,
                    ctypes.c_void_p(A + (1 << 24)), need, None) == OK


def test_bwd_rejects_bad_buffers(L):
    p = prob()
    need = L.la_workspace_bytes(ctypes.byref(p))
    d = addrs(9)

    def call(**kw):
        args = dict(q=d[0], k=d[1], v=d[2], do=d[3], state=d[4], dq=d[5], dk=d[6], dv=d[7], ws=d[8])
        args.update(kw)
        return L.la_bwd(ctypes.byref(p), args["q"], args["k"], args["v"], args["do"], args["state"],
                        args["dq"], args["dk"], args["dv"], args["ws"], kw.get("nbytes", need), None)

    assert call(state=ctypes.c_void_p(0)) == NULL
    assert call(do=ctypes.c_void_p(0)) == NULL
    assert call(nbytes=need - 256) == WORKSPACE
    assert call(dk=d[5]) == ALIAS          # two outputs on one buffer
    assert call(dv=d[3]) == ALIAS          # output on an input
    assert call(dq=d[4]) == ALIAS          # output on the state
    assert call(dq=ctypes.c_void_p(A + (5 << 24) + 2)) == ALIGN
    assert L.la_bwd(ctypes.byref(prob(D=256, Dv=128)), *d[:9], need, None) == HEAD_DIM


def test_step_calls_validate(L):
    p = prob()
    need = L.la_workspace_bytes(ctypes.byref(p))
    d = addrs(6)
    z = ctypes.c_void_p(0)
    assert L.la_fwd_state(ctypes.byref(p), d[0], d[1], z, d[3], need, None) == NULL
    assert L.la_fwd_state(ctypes.byref(p), d[0], d[1], d[2], d[3], need - 1, None) == WORKSPACE
    assert L.la_fwd_state(ctypes.byref(p), d[0], d[1], d[0], d[3], need, None) == ALIAS
    assert L.la_fwd_output(ctypes.byref(p), d[0], d[1], d[0], None) == ALIAS
    assert L.la_fwd_output(ctypes.byref(prob(flags=0x40)), d[0], d[1], d[2], None) == FLAGS
    assert L.la_bwd_dq(ctypes.byref(p), d[0], d[1], z, d[3], d[4], need, None) == NULL
    assert L.la_bwd_dq(ctypes.byref(p), d[0], d[1], d[2], d[1], d[4], need, None) == ALIAS
    assert L.la_bwd_dkv(ctypes.byref(p), d[0], d[1], d[2], d[2], d[4], need, None) == ALIAS
    assert L.la_bwd_dkv(ctypes.byref(p), d[0], d[1], d[2], d[3], d[4], 0, None) == WORKSPACE


def test_binding_marshalling_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        la.fwd(x, x, x)
    with pytest.raises(ValueError):
        la.make_problem((1, 4, 64), torch.float16, 1e-6, False)
    with pytest.raises(ValueError):
        la.make_problem((1, 1, 4, 64), torch.int32, 1e-6, False)
    # a zero scale would read as "no scale" in the C struct: the binding refuses it
    with pytest.raises(ValueError):
        la.make_problem((1, 1, 4, 64), torch.float16, 1e-6, False, scale=0.0)
    assert la.make_problem((1, 1, 4, 64), torch.float16, 1e-6, False, scale=-0.5).scale == -0.5


def test_binding_validates_state_buffers():
    """A caller-supplied state must be contiguous fp32 on the tensors' device and
    hold la_state_bytes(); the check runs before any call into the library."""
    torch = pytest.importorskip("torch")
    dev = torch.device("cpu")
    prob = la.make_problem((2, 3, 100, 64), torch.float16, 1e-6, False)
    need = la.state_bytes(prob) // 4
    assert la._state(torch.zeros(need), prob, dev).numel() == need
    for bad in (torch.zeros(need - 1), torch.zeros(need, dtype=torch.float64),
                torch.zeros(2 * need)[::2], torch.zeros(need, dtype=torch.float16)):
        with pytest.raises(ValueError):
            la._state(bad, prob, dev)
    with pytest.raises(TypeError):
        la._state(None, prob, dev)


def test_token_major_layout_limits(L):
    """[B, T, H, D] (LA_LAYOUT_BTHD): the flag is accepted, the workspace does not
    depend on the layout, and a head's span (T + 1024 rows of H * D elements)
    must stay below 2^31 bytes."""
    BTHD = 2
    base = L.la_workspace_bytes(ctypes.byref(prob(B=2, H=3, T=1000)))
    assert L.la_workspace_bytes(ctypes.byref(prob(B=2, H=3, T=1000, flags=BTHD))) == base
    assert L.la_workspace_bytes(ctypes.byref(prob(B=2, H=3, T=1000, flags=BTHD | 1))) > 0
    H, D, elt = 16, 64, 2
    t_max = ((1 << 31) - 1) // (H * D * elt) - 1024
    assert L.la_workspace_bytes(ctypes.byref(prob(B=1, H=H, T=t_max, D=D, flags=BTHD))) > 0
    assert fwd_call(L, prob(B=1, H=H, T=t_max + 1, D=D, flags=BTHD)) == SHAPE
    # the same T is fine in [B, H, T, D], where only T * D * elt counts
    assert L.la_workspace_bytes(ctypes.byref(prob(B=1, H=H, T=t_max + 1, D=D))) > 0
    # B = 0 stays an empty problem (nothing launched) in either layout
    assert fwd_call(L, prob(B=0, flags=BTHD)) == 0


def test_causal_flag_accepted_by_la_fwd_and_la_bwd_only(L):
    """LA_CAUSAL: la_fwd and la_bwd take it for every dtype and for D, Dv in
    {32, 64, 96, 128} (not 256); the step calls reject it before any HIP call.
    Every call here ends in an argument error."""
    CAUSAL = 0x10
    p = prob(flags=CAUSAL)
    need = L.la_workspace_bytes(ctypes.byref(p))
    assert need > L.la_workspace_bytes(ctypes.byref(prob())), "causal backward scratch not counted"
    assert L.la_state_bytes(ctypes.byref(p)) > 0
    d = addrs(9)
    for dt in (0, 1, 2):
        for dd, dv in ((32, 0), (96, 0), (64, 32), (128, 96), (64, 0), (128, 64)):
            pc = prob(flags=CAUSAL, D=dd, Dv=dv, dtype=dt)
            n = L.la_workspace_bytes(ctypes.byref(pc))
            assert n > 0, (dt, dd, dv)
            # accepted: the short workspace is the error reported
            assert fwd_call(L, pc, ws_bytes=n - 1) == WORKSPACE, (dt, dd, dv)
            assert L.la_bwd(ctypes.byref(pc), *d[:9], n - 1, None) == WORKSPACE, (dt, dd, dv)
    for dd, dv in ((256, 0), (256, 64), (64, 256)):
        assert fwd_call(L, prob(flags=CAUSAL, D=dd, Dv=dv, dtype=1), ws_bytes=1 << 30) == HEAD_DIM, (dd, dv)
    # the causal backward reads no state: NULL passes that check and the
    # workspace check reports; without the flag NULL is reported first
    args = [d[0], d[1], d[2], d[3], None, d[5], d[6], d[7], d[8]]
    assert L.la_bwd(ctypes.byref(p), *args, need - 1, None) == WORKSPACE
    assert L.la_bwd(ctypes.byref(prob()), *args, need - 1, None) == NULL
    assert L.la_fwd_state(ctypes.byref(p), d[0], d[1], d[2], d[3], need, None) == FLAGS
    assert L.la_fwd_output(ctypes.byref(p), d[0], d[1], d[2], None) == FLAGS
    assert L.la_bwd_dq(ctypes.byref(p), d[0], d[1], d[2], d[3], d[4], need, None) == FLAGS
    assert L.la_bwd_dkv(ctypes.byref(p), d[0], d[1], d[2], d[3], d[4], need, None) == FLAGS
    # an accepted causal call with an argument error still reports that error
    assert fwd_call(L, p, ws_bytes=need - 1) == WORKSPACE
    assert fwd_call(L, prob(flags=CAUSAL | 0x40)) == FLAGS


def test_reuse_prefix_flag(L):
    """LA_REUSE_PREFIX: accepted with LA_CAUSAL by la_fwd (which ignores it)
    and la_bwd, with the same workspace size and split as without it;
    refused without LA_CAUSAL, by la_fwd_noalloc and by the step calls.
    Every call here ends in an argument error."""
    CAUSAL, REUSE = 0x10, 0x20
    assert la.LA_REUSE_PREFIX == REUSE
    d = addrs(9)
    for dt, dd, dv in ((1, 64, 0), (2, 128, 0), (0, 64, 0), (1, 32, 96)):
        pc, pr = prob(flags=CAUSAL, D=dd, Dv=dv, dtype=dt), prob(flags=CAUSAL | REUSE, D=dd, Dv=dv, dtype=dt)
        n = L.la_workspace_bytes(ctypes.byref(pc))
        assert L.la_workspace_bytes(ctypes.byref(pr)) == n > 0
        assert la.split_of(pr) == la.split_of(pc)
        assert fwd_call(L, pr, ws_bytes=n - 1) == WORKSPACE
        assert L.la_bwd(ctypes.byref(pr), *d[:4], None, *d[5:9], n - 1, None) == WORKSPACE
        assert L.la_fwd_noalloc(ctypes.byref(pr), *d[:5], None) == FLAGS
    pr = prob(flags=CAUSAL | REUSE)
    need = L.la_workspace_bytes(ctypes.byref(pr))
    assert L.la_fwd_state(ctypes.byref(pr), d[0], d[1], d[2], d[3], need, None) == FLAGS
    assert L.la_bwd_dq(ctypes.byref(pr), d[0], d[1], d[2], d[3], d[4], need, None) == FLAGS
    p = prob(flags=REUSE)
    assert L.la_workspace_bytes(ctypes.byref(p)) == 0
    assert fwd_call(L, p) == FLAGS
    assert L.la_bwd(ctypes.byref(p), *d[:9], need, None) == FLAGS
    assert L.la_fwd_noalloc(ctypes.byref(p), *d[:5], None) == FLAGS


def test_fwd_noalloc_validates_before_any_hip_call(L):
    """la_fwd_noalloc rejects a missing state, bad buffers and a problem whose
    partials exceed the static scratch, before it looks up the scratch or
    launches anything (fake, never-dereferenced addresses)."""
    f = L.la_fwd_noalloc
    base = 1 << 40
    ptrs = [ctypes.c_void_p(base + i * (1 << 36)) for i in range(5)]
    q, k, v, o, st = ptrs
    assert f(None, q, k, v, o, st, None) == NULL
    assert f(ctypes.byref(prob(D=48)), q, k, v, o, st, None) == HEAD_DIM
    assert f(ctypes.byref(prob()), q, k, v, o, None, None) == NULL
    assert f(ctypes.byref(prob()), q, k, v, q, st, None) == ALIAS
    assert f(ctypes.byref(prob()), ctypes.c_void_p(base + 8), k, v, o, st, None) == ALIGN
    assert f(ctypes.byref(prob(flags=0x10, D=256)), q, k, v, o, st, None) == HEAD_DIM
    # fp32, D = Dv = 128, one head of 2^18 tokens: split into 1024 slices whose
    # partials (1024 * (128 * 128 + 128) * 4 bytes) exceed 64 MiB
    big = prob(B=1, H=1, T=1 << 18, D=128, dtype=0)
    assert 1024 * (128 * 128 + 128) * 4 > la.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), q, k, v, o, st, None) == SCRATCH
    assert "SCRATCH" in L.la_status_str(SCRATCH).decode()


def strided(B=2, H=3, T=100, D=64, dtype=1, flags=0, **over):
    """A problem with explicit strides: every tensor dense [B, H, T, D] unless
    overridden (name -> (batch, head, token))."""
    st = la.Strides()
    for n in la.STRIDED:
        setattr(st, n, la.TensorStrides(*over.get(n, (H * T * D, T * D, D))))
    p = prob(B=B, H=H, T=T, D=D, dtype=dtype, flags=flags)
    p.strides = ctypes.pointer(st)
    p._keep = st
    return p


def test_strides_validated_before_any_hip_call(L):
    base = 1 << 40
    q, k, v, o, st_ = (ctypes.c_void_p(base + i * (1 << 34)) for i in range(5))
    ws = ctypes.c_void_p(base + 6 * (1 << 34))

    def fwd(p, ws_bytes=0, out=o):
        return L.la_fwd(ctypes.byref(p), q, k, v, out, st_, ws, ctypes.c_size_t(ws_bytes), None)

    B, H, T, D = 2, 3, 100, 64
    # dense strides given explicitly pass the checks (then the workspace is too small)
    assert fwd(strided()) == WORKSPACE
    # the layout flag with strides is ambiguous
    assert fwd(strided(flags=0x2)) == FLAGS
    # negative, unaligned (f16: 4 elements = 8 bytes), token below the row width
    assert fwd(strided(q=(-H * T * D, T * D, D))) == STRIDE
    assert fwd(strided(k=(H * T * D, T * D, D + 4))) == STRIDE
    assert fwd(strided(v=(H * T * D, T * D, D - 8))) == STRIDE
    # a head's rows must stay addressable with 32-bit offsets
    assert fwd(strided(v=(0, 0, 1 << 26))) == STRIDE
    # inputs may share rows across heads (head stride 0) and interleave with
    # each other, as the q, k, v views of a packed [B, T, 3, H, D] buffer do
    assert fwd(strided(k=(H * T * D, 0, D), v=(H * T * D, 0, D))) == WORKSPACE
    pk = (T * 3 * H * D, D, 3 * H * D)
    assert fwd(strided(q=pk, k=pk, v=pk)) == WORKSPACE
    # an output whose heads overlap each other, or whose rows overlap
    assert fwd(strided(o=(H * T * D, 0, D))) == STRIDE
    assert fwd(strided(o=(H * T * D, D, D))) == STRIDE
    # an output interleaved with an input (compared by byte spans): o starts
    # one f16 row (2 D bytes) into q's span
    p = strided(q=pk, k=pk, v=pk, o=pk)
    need = L.la_workspace_bytes(ctypes.byref(p))
    assert L.la_fwd(ctypes.byref(p), q, k, v, ctypes.c_void_p(q.value + 2 * D), st_, ws,
                    ctypes.c_size_t(need), None) == ALIAS
    # the backward's packed outputs interleave: rejected, nothing launched
    pd = strided(dq=pk, dk=pk, dv=pk)
    need = L.la_workspace_bytes(ctypes.byref(pd))
    g = base + 9 * (1 << 34)
    assert L.la_bwd(ctypes.byref(pd), q, k, v, o, st_, ctypes.c_void_p(g), ctypes.c_void_p(g + 2 * D),
                    ctypes.c_void_p(g + 4 * D), ws, ctypes.c_size_t(need), None) == ALIAS


def test_strides_span_and_workspace_unchanged(L):
    # strides change no sizes: state and workspace are functions of the shape
    for p_dense, p_str in ((prob(), strided()), (prob(B=8, H=16, T=16384), strided(B=8, H=16, T=16384))):
        assert L.la_workspace_bytes(ctypes.byref(p_dense)) == L.la_workspace_bytes(ctypes.byref(p_str))
        assert L.la_state_bytes(ctypes.byref(p_dense)) == L.la_state_bytes(ctypes.byref(p_str))


def test_head_size_256_rules(L):
    """D = Dv = 256 is built for 16-bit inputs; fp32, a mixed pair with 256,
    and the causal form at 256 are refused before any HIP call."""
    base = 1 << 40
    q, k, v, o, st_, ws = (ctypes.c_void_p(base + i * (1 << 36)) for i in range(6))

    def fwd(p):
        return L.la_fwd(ctypes.byref(p), q, k, v, o, st_, ws, ctypes.c_size_t(0), None)

    for dt in (1, 2):
        p = prob(D=256, dtype=dt)
        assert L.la_state_bytes(ctypes.byref(p)) == 2 * 3 * (256 * 256 + 256) * 4
        assert fwd(p) == WORKSPACE  # accepted; the workspace is too small
        assert fwd(prob(D=256, Dv=128, dtype=dt)) == HEAD_DIM
        assert fwd(prob(D=64, Dv=256, dtype=dt)) == HEAD_DIM
        assert fwd(prob(D=256, dtype=dt, flags=0x10)) == HEAD_DIM
    assert fwd(prob(D=256, dtype=0)) == HEAD_DIM
    # B8-H16-T4096-D256: two slices per head, their 263 KB partials in the workspace
    p = prob(B=8, H=16, T=4096, D=256)
    E = 256 * 256 + 256
    assert L.la_workspace_bytes(ctypes.byref(p)) >= 128 * 2 * E * 4 + 2 * 128 * E * 4
