"""la_fwd_noalloc (the forward whose partials go into the library's static
device scratch) against la_fwd with a caller workspace: three calls in a row,
each smaller than the one before, byte-identical outputs and states, and the
oracle's bar on top. The outputs are filled with NaN before each call, so a
stale value would show."""
import numpy as np
import pytest
import torch

import non_causal_linear_amd as la
import oracle
from synth import Workload, make_inputs
from tests.la_testutil import TOL, bytes_equal, decode, max_rel_err, to_device

pytestmark = pytest.mark.gpu

# largest first: B2 H8 T20000 splits each head into 64 slices (partials in the
# scratch); then a bf16 case with fewer, smaller slices; then a causal one
CASES = [
    (Workload("noalloc-1", 2, 8, 20000, 64, "f16", seed=97_001), False),
    (Workload("noalloc-2", 1, 3, 2500, 128, "bf16", seed=97_002, Dv=64), False),
    (Workload("noalloc-3", 1, 2, 1500, 64, "f16", seed=97_003), True),
]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()


def test_fwd_noalloc_matches_fwd_on_calls_in_a_row():
    for w, causal in CASES:
        print(f"case la_fwd_noalloc {w.name} B{w.B} H{w.H} T{w.T} D{w.D} Dv{w.dv} {w.dtype} causal={causal}",
              flush=True)
        x = make_inputs(w, with_grad=False)
        d = {n: to_device(a, w.dtype) for n, a in x.items()}
        o_ref, st_ref = la.fwd(d["q"], d["k"], d["v"], eps=w.eps, causal=causal)
        prob = la.make_problem(d["q"].shape, d["q"].dtype, w.eps, False, dv=w.dv, causal=causal)
        out = torch.full_like(o_ref, float("nan"))
        state = torch.full((la.state_bytes(prob) // 4,), float("nan"), device="cuda")
        la.fwd_noalloc(d["q"], d["k"], d["v"], out=out, state=state, eps=w.eps, causal=causal)
        torch.cuda.synchronize()
        assert bytes_equal(out, o_ref), f"{w.name}: O differs from la_fwd"
        assert bytes_equal(state, st_ref), f"{w.name}: state differs from la_fwd"
        ref = (oracle.causal_fwd if causal else oracle.fwd)(x["q"], x["k"], x["v"], w.dtype, w.eps, False)[0]
        err = max_rel_err(decode(out, w.dtype), ref)
        print(f"  O: byte-identical to la_fwd; max rel err vs oracle {err:.3e}", flush=True)
        assert np.all(np.isfinite(decode(out, w.dtype))) and err <= TOL[w.dtype]


def test_fwd_noalloc_rejects_oversized_problem_and_enqueues_nothing():
    # fp32, D = Dv = 128, one head of 2^18 tokens: 1024 partial states of
    # 66 KB, more than the 64 MiB scratch; the call must fail before any launch
    T, D = 1 << 18, 128
    q = torch.zeros(1, 1, T, D, device="cuda")
    out = torch.full_like(q, 3.0)
    prob = la.make_problem(q.shape, q.dtype, 1e-6, False)
    state = torch.full((la.state_bytes(prob) // 4,), 5.0, device="cuda")
    with pytest.raises(la.LAError) as e:
        la.fwd_noalloc(q, q.clone(), q.clone(), out=out, state=state)
    assert e.value.status == 12
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(state == 5.0)
