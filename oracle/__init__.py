"""CPU oracle for the Matryoshka multi-exit hot path (test infrastructure).

Plain, slow, float64 NumPy definitions of what the path computes.  It is
test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline may import it; the product path never calls it.  It shares no code
with the HIP library and imports nothing from it.

Sources (the paper's equations are referenced but not printed on the pages;
each function states the reading it implements):

* "Matryoshka Language Model Suites" (agihunt summary) -- paragraph on the
  junction, paragraph on distillation, paragraph on speculative decoding.
* "Visualizing Core ideas" (main-visual explainer) -- panels (b) and (c).
* "Visualizing the core idea of Matryoshka LM Suites" (key-visual
  explainer) -- bottom panel: the junction.
* "Editing the methods of ...": copyedit of Sec. 2 "Modeling" -- the
  notation x, e_m in R^{V x (D_m - D_{m-1})}, D_0 = 0, W^m in R^{V x D_m}.
* "Is nesting the cheapest way to build a model suite?" -- follow-up 4:
  the 0.7 next-token / 0.3 teacher cross-entropy mix, beta = sum min(p, q),
  and the reverse-KL / Jensen-Shannon / acceptance-loss swaps; follow-up 2,
  arm (B): the stop-gradient at the junction.

Pins: every function is checked by ``tests/test_oracle_pins.py`` and
``tests/test_golden.py`` against closed forms, brute force and library
special cases.  What no pin can reach is whether the paper's printed
Eq. 1 and Eqs. 2-3 hold more than the prose says (an epsilon, a width
factor, a temperature): against the paper itself the oracle is
"parity unpinned"; it is pinned to the reading stated in each docstring.
"""
from .matryoshka import (  # noqa: F401
    junction, junction_backward, JUNCTION_RESCALE, JUNCTION_NO_RESCALE, JUNCTION_ZERO_FILL,
    divergence, divergence_grad, DIV_FORWARD, DIV_REVERSE_KL, DIV_JS, DIV_TV, heads, head_backward, logsumexp, softmax, matryoshka_loss, matryoshka_grad,
    argmax_lowest, accept_prefix, forward_tokens, nucleus, sample_inverse_cdf,
    speculative_verify, working_precision, loss_backward,
)
