"""fp64 CPU oracle of the MoE layer.  TEST INFRASTRUCTURE ONLY: imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the GPU path."""
from . import mx
from .moe import (Backward, Dispatch, ExpertGrad, Forward, Routing, backward, backward_mx,
                  backward_tokens, brute_force, expert_backward_mx, token_quant, combine, dispatch, expert_backward, expert_ffn, forward,
                  forward_tokens, from_bf16_bits, from_f32, max_abs_rel, ring_fill, route,
                  router_logit_grad, router_weight_grad_rows, segment_slots, sigmoid, softmax_rows,
                  swiglu, weights_from_arrays)
