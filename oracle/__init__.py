"""Float64 CPU oracle of the MoE layer: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package. It shares no code with the GPU library.

Parity status of each function (the pins are the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py``):
  router_logits, select_topk, gates_selected, gates_all, route  - pinned
  load_fractions, mean_probs, aux_loss, coverage_fraction         - pinned
  logsumexp_rows, z_loss, router_entropy, mean_max_prob, top_gap  - pinned
  bias_update                                                     - pinned
  ep_group_ids, ep_permutation, ep_group_expert, ep_send_rows,
  ep_dispatch_bytes, forward(ep=n)                                - pinned
  silu_grad, swiglu_backward, aux_loss_logit_grad, backward       - pinned
  token_input_grad, expert_unit_grads                             - pinned
  capacity, assign_rows, permutation_by_prefix_sum                - pinned
  swiglu, expert_ffn, combine, forward, dense_all_experts,
  token_output                                                    - pinned
  params.counts                                                   - pinned
"""
from . import moe, params  # noqa: F401
