"""Python binding of libla.so: bidirectional (non-causal) linear attention on gfx950.

Argument marshalling only. Every step of the computation runs in the HIP
kernels behind the C ABI declared in include/la.h; this module turns torch
tensors into device pointers, passes torch's current HIP stream, allocates
outputs and a workspace, and turns status codes into exceptions.
There is no fallback: if libla.so is missing or a call fails, it raises.

torch is imported before the library is loaded so that libla.so binds to the
HIP runtime torch already has in the process (both carry the SONAME
libamdhip64.so.7), which keeps torch's stream handles valid in the library.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LAError", "lib", "fwd", "bwd", "fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "Strides", "TensorStrides", "fwd_state", "fwd_output", "bwd_dq", "bwd_dkv", "linear_attention",
    "state_bytes", "workspace_bytes", "split_of", "Split", "new_state", "workspace", "Problem",
    "LA_F32", "LA_F16", "LA_BF16", "LA_SIMPLE", "LA_LAYOUT_BTHD", "LA_PHI_RELU", "LA_PHI_IDENTITY", "LA_CAUSAL",
    "LA_REUSE_PREFIX", "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libla.so")

LA_F32, LA_F16, LA_BF16 = 0, 1, 2
LA_SIMPLE = 0x1
LA_LAYOUT_BTHD = 0x2
LA_PHI_RELU, LA_PHI_IDENTITY = 0x4, 0x8
LA_CAUSAL = 0x10
LA_REUSE_PREFIX = 0x20
LAYOUTS = ("bhtd", "bthd")
FEATURE_MAPS = {"elu1": 0, "relu": LA_PHI_RELU, "identity": LA_PHI_IDENTITY}
DTYPE_CODE = {torch.float32: LA_F32, torch.float16: LA_F16, torch.bfloat16: LA_BF16}

# Every symbol include/la.h declares.
EXPORTS = ("la_version", "la_status_str", "la_state_bytes", "la_workspace_bytes", "la_fwd",
           "la_bwd", "la_fwd_state", "la_fwd_output", "la_bwd_dq", "la_bwd_dkv", "la_fwd_noalloc",
           "la_split_of")
# Size of the static device scratch behind la_fwd_noalloc (LA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


class Split(ctypes.Structure):
    """Mirror of la_split: P slices of L tokens (forward reduction), PB of LB
    (backward Q side), NQ chunks of LQ (output), NK of LK (backward K/V side)."""
    _fields_ = [(n, ctypes.c_int64) for n in ("P", "L", "PB", "LB", "NQ", "LQ", "NK", "LK")]


class TensorStrides(ctypes.Structure):
    """Mirror of la_tensor_strides (elements)."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


STRIDED = ("q", "k", "v", "o", "dout", "dq", "dk", "dv")


class Strides(ctypes.Structure):
    """Mirror of la_strides."""
    _fields_ = [(n, TensorStrides) for n in STRIDED]


class Problem(ctypes.Structure):
    """Mirror of la_problem."""
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("D", ctypes.c_int64), ("Dv", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("eps", ctypes.c_float), ("scale", ctypes.c_float),
                ("strides", ctypes.POINTER(Strides))]


class LAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libla.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m non_causal_linear_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.la_version.restype = ctypes.c_int
    L.la_version.argtypes = []
    L.la_status_str.restype = ctypes.c_char_p
    L.la_status_str.argtypes = [ctypes.c_int]
    L.la_state_bytes.restype = sz
    L.la_state_bytes.argtypes = [P]
    L.la_workspace_bytes.restype = sz
    L.la_workspace_bytes.argtypes = [P]
    sigs = {
        "la_fwd": [P, vp, vp, vp, vp, vp, vp, sz, vp],
        "la_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "la_fwd_state": [P, vp, vp, vp, vp, sz, vp],
        "la_fwd_output": [P, vp, vp, vp, vp],
        "la_bwd_dq": [P, vp, vp, vp, vp, vp, sz, vp],
        "la_bwd_dkv": [P, vp, vp, vp, vp, vp, sz, vp],
        "la_fwd_noalloc": [P, vp, vp, vp, vp, vp, vp],
        "la_split_of": [P, ctypes.POINTER(Split)],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise LAError(status, lib().la_status_str(status).decode())


def make_problem(shape, dtype: torch.dtype, eps: float, simple: bool, layout: str = "bhtd",
                 phi: str = "elu1", dv: int | None = None, causal: bool = False,
                 scale: float | None = None) -> Problem:
    """Problem for Q/K-side tensors of ``shape``: [B, H, T, D] (layout "bhtd")
    or [B, T, H, D] (layout "bthd"), V-side tensors with head size ``dv``
    (None: D); feature map phi "elu1" (elu(x) + 1), "relu" or "identity";
    ``scale`` multiplies phi(q) (None: 1). A zero scale is refused here: in
    the C struct 0 stands for 1 (a zero-initialised problem), which a caller
    who asks for 0 would not expect."""
    if scale is not None and float(scale) == 0.0:
        raise ValueError("scale must be non-zero (None for no scale)")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {LAYOUTS}, got {layout!r}")
    if phi not in FEATURE_MAPS:
        raise ValueError(f"phi must be one of {tuple(FEATURE_MAPS)}, got {phi!r}")
    if len(shape) != 4:
        raise ValueError(f"expected a 4-d tensor ({layout}), got shape {tuple(shape)}")
    if dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dtype}")
    if layout == "bhtd":
        B, H, T, D = (int(x) for x in shape)
    else:
        B, T, H, D = (int(x) for x in shape)
    flags = ((LA_SIMPLE if simple else 0) | (LA_LAYOUT_BTHD if layout == "bthd" else 0) | FEATURE_MAPS[phi]
             | (LA_CAUSAL if causal else 0))
    return Problem(B, H, T, D, D if dv is None else int(dv), DTYPE_CODE[dtype], flags, float(eps),
                   1.0 if scale is None else float(scale))


def _tensor(x: torch.Tensor, like: torch.Tensor | None, name: str, last: int | None = None) -> torch.Tensor:
    """x must be a GPU tensor whose last (feature) dimension is contiguous;
    given ``like``, with its dtype, device and leading three dimensions, and a
    last dimension of ``last`` (None: like's). The other dimensions may be
    strided (a view into a larger buffer): the library takes their strides."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {x.device}")
    if x.dim() != 4 or (x.shape[-1] > 1 and x.stride(-1) != 1):
        raise ValueError(f"{name} must be a 4-d tensor with a contiguous last dimension")
    if like is not None:
        want = tuple(like.shape[:-1]) + ((like.shape[-1] if last is None else last),)
        if tuple(x.shape) != want or x.dtype != like.dtype or x.device != like.device:
            raise ValueError(f"{name} must be {want} {like.dtype} on {like.device}, got "
                             f"{tuple(x.shape)} {x.dtype} on {x.device}")
    return x


def _new_like(x: torch.Tensor, last: int) -> torch.Tensor:
    return torch.empty(tuple(x.shape[:-1]) + (last,), dtype=x.dtype, device=x.device)


def _state(state, prob: Problem, device: torch.device, name: str = "state") -> torch.Tensor:
    """A state buffer: contiguous fp32 on the tensors' device, large enough."""
    if not isinstance(state, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if state.dtype != torch.float32 or state.device != device or not state.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor on {device}")
    if state.numel() * 4 < state_bytes(prob):
        raise ValueError(f"{name} holds {state.numel() * 4} bytes; the problem needs {state_bytes(prob)}")
    return state


def _tensor_strides(x: torch.Tensor, layout: str) -> TensorStrides:
    """Batch, head and token strides of a [B, H, T, D] ("bhtd") or [B, T, H, D]
    ("bthd") tensor. A dimension of extent 1 has no meaningful stride: it is
    given as 0 (batch, head) or the row width (token)."""
    if layout == "bhtd":
        (B, H, T, W), (sb, sh, st) = x.shape, x.stride()[:3]
    else:
        (B, T, H, W), (sb, st, sh) = x.shape, x.stride()[:3]
    return TensorStrides(sb if B > 1 else 0, sh if H > 1 else 0, st if T > 1 else W)


def _attach_strides(prob: Problem, layout: str, tensors: dict) -> Problem:
    """Describe the call's tensors by their strides when any of them is not
    dense in ``layout`` (a dense call keeps strides NULL and runs exactly as
    before). tensors: la_strides field name -> tensor."""
    if all(t.is_contiguous() for t in tensors.values()):
        return prob
    st = Strides()
    for name, t in tensors.items():
        setattr(st, name, _tensor_strides(t, layout))
    prob.flags &= ~LA_LAYOUT_BTHD
    prob.strides = ctypes.pointer(st)
    prob._strides_keepalive = st
    return prob


def _ptr(x: torch.Tensor | None):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def split_of(prob: Problem) -> dict:
    """The library's token split for this problem, per step (la_split_of)."""
    out = Split()
    _check(lib().la_split_of(ctypes.byref(prob), ctypes.byref(out)))
    return {name: int(getattr(out, name)) for name, _ in Split._fields_}


def state_bytes(prob: Problem) -> int:
    return int(lib().la_state_bytes(ctypes.byref(prob)))


def workspace_bytes(prob: Problem) -> int:
    return int(lib().la_workspace_bytes(ctypes.byref(prob)))


def new_state(prob: Problem, device) -> torch.Tensor:
    """fp32 state buffer: B*H blocks of S (D*Dv) followed by B*H blocks of z (D)."""
    return torch.empty(state_bytes(prob) // 4, dtype=torch.float32, device=device)


_ws_cache: dict = {}


def workspace(prob: Problem, device) -> torch.Tensor:
    """A workspace for this device and its current stream, reused across calls.

    Reuse in stream order is valid; a different stream gets its own workspace.
    """
    device = torch.device(device)
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    need = max(workspace_bytes(prob), 256)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _ws(prob, device, ws):
    if ws is None:
        ws = workspace(prob, device)
    elif not isinstance(ws, torch.Tensor) or ws.device != torch.device(device) or not ws.is_contiguous():
        raise ValueError(f"ws must be a contiguous tensor on {device}")
    return ws, ctypes.c_size_t(ws.numel() * ws.element_size())


def fwd_state(k, v, *, eps=1e-6, simple=False, layout="bhtd", phi="elu1", state=None, ws=None):
    """Steps 1-3: the fp32 state (S, z) of phi(K), V."""
    _tensor(k, None, "k")
    _tensor(v, k, "v", v.shape[-1] if isinstance(v, torch.Tensor) else None)
    prob = make_problem(k.shape, k.dtype, eps, simple, layout, phi, v.shape[-1])
    _attach_strides(prob, layout, {"k": k, "v": v})
    state = new_state(prob, k.device) if state is None else _state(state, prob, k.device)
    ws, wsb = _ws(prob, k.device, ws)
    _check(lib().la_fwd_state(ctypes.byref(prob), _ptr(k), _ptr(v), _ptr(state), _ptr(ws), wsb,
                              _stream(k.device)))
    return state


def fwd_output(q, state, *, eps=1e-6, simple=False, layout="bhtd", phi="elu1", out=None, dv=None, scale=None):
    """Step 4: O from Q and a complete state; dv is the head size of V and O
    (None: that of out if given, else D)."""
    _tensor(q, None, "q")
    if dv is None:
        dv = out.shape[-1] if isinstance(out, torch.Tensor) else q.shape[-1]
    prob = make_problem(q.shape, q.dtype, eps, simple, layout, phi, dv, scale=scale)
    _state(state, prob, q.device)
    out = _new_like(q, dv) if out is None else _tensor(out, q, "out", dv)
    _attach_strides(prob, layout, {"q": q, "o": out})
    _check(lib().la_fwd_output(ctypes.byref(prob), _ptr(q), _ptr(state), _ptr(out), _stream(q.device)))
    return out


def fwd(q, k, v, *, eps=1e-6, simple=False, layout="bhtd", phi="elu1", out=None, state=None, ws=None,
        causal=False, scale=None):
    """O = phi(Q) S / (phi(Q) z + eps) (or phi(Q) S); returns (O, state).
    causal=True: token t attends to tokens s <= t (D and Dv up to 128); the
    state is still that of the whole sequence."""
    _tensor(q, None, "q")
    _tensor(k, q, "k")
    dv = v.shape[-1] if isinstance(v, torch.Tensor) else None
    _tensor(v, q, "v", dv)
    prob = make_problem(q.shape, q.dtype, eps, simple, layout, phi, dv, causal, scale)
    out = _new_like(q, dv) if out is None else _tensor(out, q, "out", dv)
    _attach_strides(prob, layout, {"q": q, "k": k, "v": v, "o": out})
    state = new_state(prob, q.device) if state is None else _state(state, prob, q.device)
    ws, wsb = _ws(prob, q.device, ws)
    _check(lib().la_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state),
                        _ptr(ws), wsb, _stream(q.device)))
    return out, state


def fwd_noalloc(q, k, v, *, out, state, eps=1e-6, simple=False, layout="bhtd", phi="elu1", causal=False,
                scale=None):
    """fwd through la_fwd_noalloc: the library call allocates nothing (its
    partials go into the library's static device scratch), so the caller
    passes both outputs, ``out`` and ``state``; writes and returns them. The
    same bits as fwd. Calls that overlap in time on one GPU race on the
    scratch."""
    _tensor(q, None, "q")
    _tensor(k, q, "k")
    dv = v.shape[-1] if isinstance(v, torch.Tensor) else None
    _tensor(v, q, "v", dv)
    prob = make_problem(q.shape, q.dtype, eps, simple, layout, phi, dv, causal, scale)
    _tensor(out, q, "out", dv)
    _attach_strides(prob, layout, {"q": q, "k": k, "v": v, "o": out})
    _state(state, prob, q.device)
    _check(lib().la_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state),
                                _stream(q.device)))
    return out, state


def bwd_dq(q, do, state, *, eps=1e-6, simple=False, layout="bhtd", phi="elu1", dq=None, ws=None, scale=None):
    """Steps 5-6: dQ; leaves dS, dz in the workspace for bwd_dkv."""
    _tensor(q, None, "q")
    dv = do.shape[-1] if isinstance(do, torch.Tensor) else None
    _tensor(do, q, "do", dv)
    prob = make_problem(q.shape, q.dtype, eps, simple, layout, phi, dv, scale=scale)
    _state(state, prob, q.device)
    dq = _new_like(q, q.shape[-1]) if dq is None else _tensor(dq, q, "dq")
    _attach_strides(prob, layout, {"q": q, "dout": do, "dq": dq})
    ws, wsb = _ws(prob, q.device, ws)
    _check(lib().la_bwd_dq(ctypes.byref(prob), _ptr(q), _ptr(do), _ptr(state), _ptr(dq), _ptr(ws), wsb,
                           _stream(q.device)))
    return dq


def bwd_dkv(k, v, *, eps=1e-6, simple=False, layout="bhtd", phi="elu1", dk=None, dv=None, ws=None):
    """Step 7: dK, dV from the backward state bwd_dq left in the same workspace."""
    _tensor(k, None, "k")
    hv = v.shape[-1] if isinstance(v, torch.Tensor) else None
    _tensor(v, k, "v", hv)
    prob = make_problem(k.shape, k.dtype, eps, simple, layout, phi, hv)
    dk = _new_like(k, k.shape[-1]) if dk is None else _tensor(dk, k, "dk")
    dv = _new_like(k, hv) if dv is None else _tensor(dv, k, "dv", hv)
    _attach_strides(prob, layout, {"k": k, "v": v, "dk": dk, "dv": dv})
    ws, wsb = _ws(prob, k.device, ws)
    _check(lib().la_bwd_dkv(ctypes.byref(prob), _ptr(k), _ptr(v), _ptr(dk), _ptr(dv), _ptr(ws), wsb,
                            _stream(k.device)))
    return dk, dv


def bwd(q, k, v, do, state=None, *, eps=1e-6, simple=False, layout="bhtd", phi="elu1", dq=None, dk=None, dv=None,
        ws=None, causal=False, scale=None, reuse_prefix=False):
    """dQ, dK, dV of L = sum(O * dO), from the state fwd returned.
    causal=True: the backward of the causal form (D and Dv up to 128); no
    state is read (pass None). reuse_prefix=True (causal only): ``ws`` still
    holds the segment prefixes the causal fwd on the same problem and K, V
    wrote into it, and the backward reads them instead of recomputing them
    (LA_REUSE_PREFIX; the library cannot check this)."""
    _tensor(q, None, "q")
    _tensor(k, q, "k")
    hv = v.shape[-1] if isinstance(v, torch.Tensor) else None
    _tensor(v, q, "v", hv)
    _tensor(do, q, "do", hv)
    prob = make_problem(q.shape, q.dtype, eps, simple, layout, phi, hv, causal, scale)
    if reuse_prefix:
        prob.flags |= LA_REUSE_PREFIX
    if not causal or state is not None:
        _state(state, prob, q.device)
    dq = _new_like(q, q.shape[-1]) if dq is None else _tensor(dq, q, "dq")
    dk = _new_like(q, q.shape[-1]) if dk is None else _tensor(dk, q, "dk")
    dv = _new_like(q, hv) if dv is None else _tensor(dv, q, "dv", hv)
    _attach_strides(prob, layout, {"q": q, "k": k, "v": v, "dout": do, "dq": dq, "dk": dk, "dv": dv})
    ws, wsb = _ws(prob, q.device, ws)
    _check(lib().la_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(state),
                        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), wsb, _stream(q.device)))
    return dq, dk, dv


class _LinearAttention(torch.autograd.Function):
    """Autograd node over la_fwd / la_bwd. The forward keeps the fp32 state
    (S, z) for the backward, which therefore reads Q, K, V, dO and the state
    and does not recompute S. The causal forward runs in a workspace of its
    own, kept for the backward, which reads the segment prefixes from it
    (LA_REUSE_PREFIX) instead of recomputing them; nothing else writes to it
    in between."""

    @staticmethod
    def forward(ctx, q, k, v, eps, simple, layout, phi, causal, scale):
        ws = None
        if causal:
            dv = v.shape[-1] if isinstance(v, torch.Tensor) else None
            prob = make_problem(q.shape, q.dtype, eps, simple, layout, phi, dv, causal, scale)
            ws = torch.empty(max(workspace_bytes(prob), 256), dtype=torch.uint8, device=q.device)
        o, state = fwd(q, k, v, eps=eps, simple=simple, layout=layout, phi=phi, causal=causal, scale=scale, ws=ws)
        if causal:
            state = None  # the causal backward does not read it
            ctx.save_for_backward(q, k, v)
        else:
            ctx.save_for_backward(q, k, v, state)
        ctx.ws = ws
        ctx.eps, ctx.simple, ctx.layout, ctx.phi, ctx.causal, ctx.scale = eps, simple, layout, phi, causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        saved = ctx.saved_tensors
        q, k, v = saved[:3]
        state = saved[3] if len(saved) > 3 else None
        if do.shape[-1] > 1 and do.stride(-1) != 1:
            do = do.contiguous()
        dq, dk, dv = bwd(q, k, v, do, state, eps=ctx.eps, simple=ctx.simple, layout=ctx.layout,
                         phi=ctx.phi, causal=ctx.causal, scale=ctx.scale, ws=ctx.ws,
                         reuse_prefix=ctx.causal)
        return dq, dk, dv, None, None, None, None, None, None


def linear_attention(q, k, v, *, eps: float = 1e-6, simple: bool = False, layout: str = "bhtd",
                     phi: str = "elu1", causal: bool = False, scale: float | None = None) -> torch.Tensor:
    """O = phi(Q) S / (phi(Q) z + eps) (or phi(Q) S with simple=True), with
    gradients for q, k and v through the library's backward. Tensors are
    [B, H, T, D] (layout "bhtd") or [B, T, H, D] (layout "bthd") on a GPU in
    float32, float16 or bfloat16, with D (of q, k) and Dv (of v) each in
    {32, 64, 96, 128}; phi is "elu1" (elu + 1),
    "relu" or "identity". causal=True: token t attends to tokens s <= t
    (any dtype, D and Dv up to 128). scale multiplies phi(q) (None: 1; 0 is refused)."""
    return _LinearAttention.apply(q, k, v, float(eps), bool(simple), layout, phi, bool(causal),
                                  None if scale is None else float(scale))
