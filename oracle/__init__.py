"""fp64 CPU oracle for the single-pass fused cascaded-reduction attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The library under ``attention_pass_cascaded_amd`` never imports, links or
calls anything here, and this package imports nothing from there: the two
share no code.  Inputs come from ``workloads`` (random draws only).

Contents
  cascade.py    the unfused three-pass cascade (max pass, exp-sum pass,
                P.V pass), the incremental (m, l, O) form, split-KV partials
                and the log-sum-exp merge, RoPE.  numpy, float64.
  brute.py      pure-Python scalar reference for tiny inputs (math.exp,
                math.fsum), written from the textbook softmax definition.
  backward.py   gradients dq, dk, dv of the forward by the chain rule
                (softmax Jacobian row term, inverse RoPE rotation, GQA sums).
  layernorm.py  a second cascaded reduction: LayerNorm mean -> variance ->
                normalise, three-pass and incremental (n, mean, M2) forms.
  topk.py       softmax followed by TopK (the max/+ row of RedFuser Table 1),
                three-pass and incremental (m, l, k best) forms.

Every function is pinned by ``tests/test_oracle.py``,
``tests/test_oracle_backward.py``, ``tests/test_oracle_layernorm.py`` and
``tests/test_oracle_topk.py`` (brute force, finite differences of the
brute force, closed forms, invariants and library routines the definition
reduces to).
"""
from .cascade import (  # noqa: F401
    attention,
    attention_incremental,
    attention_rows,
    lse_merge,
    query_positions,
    rope_rotate,
    split_partials,
    visible_mask,
    softmax_probs,
)
from .backward import attention_backward, row_terms  # noqa: F401
from .layernorm import layer_norm, layer_norm_incremental  # noqa: F401
from .topk import softmax_topk, softmax_topk_incremental  # noqa: F401
