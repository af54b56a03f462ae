"""Pins for the oracle's tree-masked attention (CPU only).

Independent references: torch's scaled_dot_product_attention (CPU, float64,
math path) with explicit masks, closed forms, and torch's own bf16 / e4m3fn
conversions for the exact upcasts.
"""
import numpy as np
import torch

import oracle
from tests import pins


def test_chain_equals_causal_attention():
    pins.check_attention_chain_is_causal(oracle.tree_attention)


def test_one_node_tree_equals_decode_attention():
    pins.check_attention_one_node_is_decode(oracle.tree_attention)


def test_each_node_equals_its_own_chain():
    pins.check_attention_node_locality(oracle.tree_attention)


def test_gqa_equals_mha_with_repeated_kv():
    pins.check_attention_gqa_is_mha(oracle.tree_attention)


def test_closed_form_two_and_three_nodes():
    pins.check_attention_closed_form(oracle.tree_attention)


def test_one_request_one_head_call():
    pins.check_attention_bh(oracle.tree_attention_bh, oracle.tree_attention)


def test_rows_past_the_tree_are_ignored():
    pins.check_attention_ignores_rows_past_tree(oracle.tree_attention)


def test_dense_mask_layout():
    A = oracle.dense_tree_mask([-1, 0, 0, 1], 3)
    want = np.array([[1, 1, 1, 1, 0, 0, 0],
                     [1, 1, 1, 1, 1, 0, 0],
                     [1, 1, 1, 1, 0, 1, 0],
                     [1, 1, 1, 1, 1, 0, 1]], dtype=bool)
    np.testing.assert_array_equal(A, want)


def test_bf16_upcast_is_exact():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal(4096).astype(np.float32) * 37).to(torch.bfloat16)
    x = torch.cat([x, torch.tensor([0.0, -0.0, 1e-40, -3e38], dtype=torch.bfloat16)])
    got = oracle.bf16_bits_to_f64(x.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(got, x.double().numpy())


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    tab = oracle.e4m3_decode_table()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(tab[ok], ref[ok])
    assert np.nanmax(tab) == 448.0 and np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])


def test_bf16_and_fp8_paths_equal_f32_path_on_exact_values():
    """Feeding the same values as f32, as bf16 bits and as e4m3 codes (scale 1)
    gives identical float64 outputs."""
    rng = np.random.default_rng(8)
    parents, prefix, q, k, v = pins.rand_case(rng, 2, 5, 4, 2, 8, [6, 2])
    codes_k = rng.integers(0, 126, size=k.shape).astype(np.uint8)
    codes_v = rng.integers(0, 126, size=v.shape).astype(np.uint8)
    codes_k |= (rng.random(k.shape) < 0.5).astype(np.uint8) << 7
    kf = oracle.decode_e4m3(codes_k, 1.0).astype(np.float32)
    vf = oracle.decode_e4m3(codes_v, 1.0).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    qf = qb.float().numpy()
    qbits = qb.view(torch.int16).numpy().view(np.uint16)
    o1, l1 = oracle.tree_attention(qf, kf, vf, prefix, parents, 0.2, q_fmt="f32", kv_fmt="f32")
    o2, l2 = oracle.tree_attention(qbits, codes_k, codes_v, prefix, parents, 0.2, q_fmt="bf16",
                                   kv_fmt="e4m3", k_scale=np.ones(2), v_scale=np.ones(2))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    kb = torch.from_numpy(kf).to(torch.bfloat16)          # e4m3 values are exact in bf16
    vb = torch.from_numpy(vf).to(torch.bfloat16)
    o3, _ = oracle.tree_attention(qbits, kb.view(torch.int16).numpy().view(np.uint16),
                                  vb.view(torch.int16).numpy().view(np.uint16), prefix, parents, 0.2,
                                  q_fmt="bf16", kv_fmt="bf16")
    np.testing.assert_array_equal(o1, o3)


def test_fp8_scale_multiplies_values():
    rng = np.random.default_rng(10)
    parents, prefix, q, k, v = pins.rand_case(rng, 1, 3, 2, 2, 4, 5)
    ck = rng.integers(0, 120, size=k.shape).astype(np.uint8)
    cv = rng.integers(0, 120, size=v.shape).astype(np.uint8)
    ks, vs = np.array([0.5, 2.0]), np.array([4.0, 0.25])
    o, _ = oracle.tree_attention(q, ck, cv, prefix, parents, 0.3, q_fmt="f32", kv_fmt="e4m3",
                                 k_scale=ks, v_scale=vs)
    kf = oracle.decode_e4m3(ck, 1.0) * ks[None, :, None, None]
    vf = oracle.decode_e4m3(cv, 1.0) * vs[None, :, None, None]
    o2, _ = oracle.tree_attention(q, kf.astype(np.float32), vf.astype(np.float32), prefix, parents, 0.3,
                                  q_fmt="f32", kv_fmt="f32")
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
