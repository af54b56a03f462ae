"""Pins for the oracle's backward pass of the tree-masked attention (CPU only).

Independent references: torch autograd through its float64
scaled_dot_product_attention (math path) with a dense mask built here by a
parent chase; central finite differences of that same library forward; sum
rules of the softmax Jacobian; the subtree structure of the mask; and a
two-node case solved by hand.
"""
import numpy as np

import oracle
from tests import pins


def test_backward_equals_torch_autograd():
    pins.check_backward_autograd(oracle.tree_attention_backward)


def test_backward_matches_finite_differences():
    pins.check_backward_finite_differences(oracle.tree_attention_backward)


def test_backward_sum_rules_and_unread_rows():
    pins.check_backward_invariants(oracle.tree_attention_backward)


def test_backward_gradient_reaches_only_ancestors():
    pins.check_backward_subtree_locality(oracle.tree_attention_backward)


def test_backward_closed_form_two_nodes():
    pins.check_backward_closed_form(oracle.tree_attention_backward)


def test_backward_bf16_inputs_are_upcast_exactly():
    """bf16 bit patterns in, the same gradients as their exact float32 values."""
    rng = np.random.default_rng(14)
    parents, prefix, q, k, v = pins.rand_case(rng, 2, 5, 4, 2, 8, [3, 6])
    d_out = rng.standard_normal(q.shape).astype(np.float32)
    import torch

    def bits(x):
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def back(x):
        return torch.from_numpy(x).to(torch.bfloat16).float().numpy()

    got = oracle.tree_attention_backward(bits(q), bits(k), bits(v), prefix, parents, bits(d_out), 0.3,
                                         q_fmt="bf16", kv_fmt="bf16")
    ref = oracle.tree_attention_backward(back(q), back(k), back(v), prefix, parents, back(d_out), 0.3,
                                         q_fmt="f32", kv_fmt="f32")
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
