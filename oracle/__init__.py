"""CPU oracle for the greedy speculative-decoding verify round.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import anything here.  The product path (``weight_bound_verify_amd``) never imports
this package, and this package never imports the product path: the two share no code.
The only inputs both sides see are the bytes made by ``weight_bound_verify_amd.synth``.

Plain, slow, obviously-correct numpy in fp64.  Each function names the page and section
it follows (pages of the "Core AI model zoo" knowledge base):

* "Stream C - Speculative decoding: feasibility verdict + implementation plan"
  (the spec-decode feasibility page): the delta section (accept/reject indexing, n-gram
  drafter), the C-value speedup model, the control-logic proof, implementation status.
* "Spec-decode on GDN hybrids (Qwen3.5/3.6 family) - static-S verify design"
  (the hybrid verify-design page): static S=K+1 verify graph, hybrid state discipline
  (correction/bonus unified), harness lessons (draft past the anchor).
* "Riding Apple's pipelined GPU engine" (the pipelined-engine page): quantization on the
  GPU delegate (per-block-32 absmax int8 head), numerics gating (margin rule).
* "Flagship dramatic-speedup plan - the full stackable tuning set" (the tuning-stack
  page): baseline byte model, axis 4 (fused RMSNorm/SwiGLU).

Tree verify (``tree.py``) follows the feasibility page's EAGLE-3 + tree handoff and deferred
list (tree drafts, tree-mask verify, a walk down the tree instead of the linear accept).
Sampling verify (``sampling.py``) follows the feasibility page's deferred list and the
published speculative-sampling rule it refers to; its random numbers come from
Philox4x32-10, implemented here from its published definition.

Parity status of every function is stated in its module docstring; all are pinned by the
``-m "not gpu"`` tests (brute force, closed forms, invariants, the pages' printed tables).
"""
from .verify import (  # noqa: F401
    dequantize, head_logits, dequantize_q4b32, head_logits_q4b32, argmax_lowest, top2_gap, admissible_sets, accept_length,
    accept, propose_scan, NgramIndex, expected_tokens_per_round, greedy_decode,
    spec_decode, verify_round,
)
from .stack import rmsnorm_fp16, silu, linear_q8b32, mlp_block, stack_forward  # noqa: F401
from .tree import tree_accept, propose_tree, path_tokens, tree_spec_decode  # noqa: F401
from .sampling import (  # noqa: F401
    philox4, philox4x32_np, uniform01, noise_uniforms, accept_uniforms, probabilities, residual,
    gumbel_sample, sampling_verify, sample_decode, spec_sample_decode,
)
