"""fp64 CPU oracle for bidirectional (non-causal) linear attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py use it. It shares no code with the HIP library or its Python binding.

Every function cites the passage it follows. The method is named on the FBi-LA
README (page "flash-bidirectional-linear-attention", intro: bi-directional
linear attention for non-causal modelling; "Update" 2024-12-28: simple_la is
linear attention without the norm term). The pages print no formula; the one
used here is the plain statement of the method: with phi(x) = elu(x) + 1,
  S = sum_t phi(k_t) v_t^T,  z = sum_t phi(k_t),
  O_t = phi(q_t) S / (phi(q_t) . z + eps)   (normalised)
  O_t = phi(q_t) S                          (simple_la)
which equals, by associativity, the quadratic "parallel" form listed on the
flash-linear-attention README ("Different forms of linear attention",
Parallel): O = rownorm(phi(Q) phi(K)^T) V.

The causal variant (token t attends to tokens s <= t; flash-linear-attention
README, "Different forms of linear attention") is given by its masked
quadratic form and its recurrent form.

Every function takes an optional `scale` that multiplies phi(q) (default 1:
the method as stated).

Pins (tests/test_oracle.py): brute-force quadratic form in pure Python, a
hand-worked example (tests/golden/), V = ones, joint K/V permutation, Q-row
permutation, the T = 1 closed form, linearity in V, central finite
differences of the loss, torch fp64 autograd of the quadratic form, and two
backward identities; for the causal form, a pure-Python masked brute force,
agreement of the two causal forms, the last row against the non-causal form,
the first row's closed form, and independence of earlier rows from later
tokens; for the causal backward, torch fp64 autograd of the masked quadratic
form, central finite differences, the non-causal backward when only the last
row has a gradient, and the dV column-sum identity. No function here is
"parity unpinned".
"""
from .la_oracle import (  # noqa: F401
    causal_bwd,
    causal_bwd_head,
    causal_fwd,
    causal_quadratic_head,
    causal_recurrent_head,
    causal_sampled_rows_head,
    decode,
    dphi,
    fwd,
    fwd_head,
    output_head,
    bwd,
    bwd_head,
    bwd_kv_side_head,
    bwd_leading_terms_head,
    bwd_q_side_head,
    phi,
    qfeat,
    quadratic_head,
    sampled_rows_head,
    state_head,
)
