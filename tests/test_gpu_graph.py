"""The library under HIP graph capture: la_fwd and la_bwd allocate nothing and
enqueue only kernels, so a captured forward + backward replays like the eager
calls. Every replay is compared bit for bit with the eager result, with eager
work in between that overwrites the outputs."""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
from synth import Workload, make_inputs
from tests.la_testutil import bytes_equal, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def eager(dev, w, causal=False):
    o, st = la.fwd(dev["q"], dev["k"], dev["v"], eps=w.eps, simple=w.simple, causal=causal)
    dq, dk, dv = la.bwd(dev["q"], dev["k"], dev["v"], dev["do"], None if causal else st, eps=w.eps,
                        simple=w.simple, causal=causal)
    torch.cuda.synchronize()
    return {"o": o, "state": st, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("D,Dv,dtype,simple,causal,reuse", [(64, 64, "f16", False, False, False),
                                                             (128, 128, "bf16", False, False, False),
                                                             (96, 32, "f16", True, False, False),
                                                             (64, 64, "f16", False, True, False),
                                                             (128, 64, "bf16", True, True, False),
                                                             (64, 64, "f16", False, True, True)],
                         ids=["D64-f16", "D128-bf16", "D96-Dv32-f16-simple", "causal-D64-f16",
                              "causal-D128-Dv64-bf16-simple", "causal-D64-f16-reuse-prefix"])
def test_graph_replays_match_eager(D, Dv, dtype, simple, causal, reuse):
    """reuse: the captured backward reads the segment prefixes the captured
    forward left in the workspace (LA_REUSE_PREFIX); the workspace is
    overwritten between replays, so each replay's forward must refill them."""
    w = Workload("graph", 2, 4, 3000, D, dtype, simple=simple, seed=70_000 + D + Dv, Dv=Dv)
    print(f"case graph D={D} Dv={Dv} {dtype} simple={simple} causal={causal} reuse={reuse} seed={w.seed}",
          flush=True)
    x = make_inputs(w)
    dev = {n: to_device(a, w.dtype) for n, a in x.items()}
    ref = eager(dev, w, causal)

    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    prob = la.make_problem(q.shape, q.dtype, w.eps, simple, dv=Dv, causal=causal)
    out = {"o": torch.empty_like(v), "state": la.new_state(prob, q.device), "dq": torch.empty_like(q),
           "dk": torch.empty_like(k), "dv": torch.empty_like(v)}
    ws = torch.empty(la.workspace_bytes(prob), dtype=torch.uint8, device=q.device)

    def calls():
        la.fwd(q, k, v, eps=w.eps, simple=simple, out=out["o"], state=out["state"], ws=ws, causal=causal)
        la.bwd(q, k, v, do, None if causal else out["state"], eps=w.eps, simple=simple, dq=out["dq"], dk=out["dk"],
               dv=out["dv"], ws=ws, causal=causal, reuse_prefix=reuse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    for i in range(4):
        for t in list(out.values()) + [ws]:
            t.view(torch.uint8).fill_(0xFF)  # eager overwrite between replays (NaN patterns)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for nm in ref:
            assert bytes_equal(out[nm], ref[nm]), f"replay {i}: {nm} differs from the eager run"

    # the graph reads the buffers it captured: new values in them, new results
    x2 = make_inputs(Workload("graph2", 2, 4, 3000, D, dtype, simple=simple, seed=w.seed + 1, Dv=Dv))
    for n, a in x2.items():
        dev[n].copy_(to_device(a, w.dtype))
    ref2 = eager(dev, w, causal)
    g.replay()
    torch.cuda.synchronize()
    for nm in ref2:
        assert bytes_equal(out[nm], ref2[nm]), f"after new inputs: {nm} differs"
    assert not bytes_equal(ref2["o"], ref["o"])
