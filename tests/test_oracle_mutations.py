"""Planted mistakes in the oracle (on the CPU): each mutation below is a
plausible slip -- a dropped term, a wrong index, a transposed rule -- applied
to a fresh copy of the oracle's source.  The pins must reject every one.
"""
import importlib.util
import os
import sys
import types

import pytest

from tests import pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def load_mutant(edits):
    """Load a private copy of the oracle package with textual edits applied.
    edits: list of (file, old, new); each old string must occur."""
    name = "oracle_mutant_%d" % id(edits)
    pkg = types.ModuleType(name)
    pkg.__path__ = []
    sys.modules[name] = pkg
    try:
        for mod in ("tree", "attention", "argmax", "step", "commit", "attention_bwd"):
            with open(os.path.join(ORACLE_DIR, mod + ".py")) as f:
                src = f.read()
            for (fname, old, new) in edits:
                if fname == mod:
                    assert old in src, (fname, old)
                    src = src.replace(old, new)
            m = types.ModuleType(f"{name}.{mod}")
            m.__package__ = name
            sys.modules[m.__name__] = m
            exec(compile(src, f"<mutant {mod}>", "exec"), m.__dict__)
            setattr(pkg, mod, m)
        return pkg
    finally:
        for k in [k for k in sys.modules if k == name or k.startswith(name + ".")]:
            del sys.modules[k]


MUTANTS = {
    # ancestor masks
    "mask_drops_self": ([("tree", "    out = [i]\n", "    out = [int(p[i])] if p[i] != -1 else [i]\n")],
                        lambda o: pins.check_mask_closed_forms(o.tree.build_masks)),
    "mask_parent_only": ([("tree", "    while p[out[-1]] != -1:\n        out.append(int(p[out[-1]]))",
                           "    if p[i] != -1:\n        out.append(int(p[i]))")],
                         lambda o: pins.check_mask_brute_force(o.tree.build_masks, 5)),
    "depth_counts_nodes": ([("tree", "depth[b, i] = len(a) - 1", "depth[b, i] = len(a)")],
                           lambda o: pins.check_mask_golden(o.tree.build_masks)),
    # accept walk
    "walk_compares_own_target": ([("tree", "return d[c] == t[p[c]]", "return d[c] == t[c]")],
                                 lambda o: pins.check_walk_brute_force(o.tree.accept_walk, 4, 2)),
    "walk_greedy_first_child": ([("tree", "                    r = walk(c, depth_u + 1)\n"
                                          "                    if r[0] > best[0] or (r[0] == best[0] and r[1] < best[1]):\n"
                                          "                        best = r",
                                  "                    return walk(c, depth_u + 1)")],
                                lambda o: pins.check_walk_golden(o.tree.accept_walk)),
    "walk_tie_to_higher_index": ([("tree", "r[1] < best[1]", "r[1] > best[1]")],
                                 lambda o: pins.check_walk_brute_force(o.tree.accept_walk, 5, 3)),
    "walk_outputs_drafts": ([("tree", "out_tokens[b, k] = t[node]", "out_tokens[b, k] = d[node]")],
                            lambda o: pins.check_walk_golden(o.tree.accept_walk)),
    "walk_counts_root": ([("tree", "accept_len[b] = L", "accept_len[b] = L + 1")],
                         lambda o: pins.check_walk_chain_closed_forms(o.tree.accept_walk)),
    # argmax
    "argmax_last_max": ([("argmax", "np.flatnonzero(row == best)[0]", "np.flatnonzero(row == best)[-1]")],
                        lambda o: pins.check_argmax_constructed(o.argmax.vocab_argmax)),
    "argmax_abs": ([("argmax", "best = row.max()\n        out[r] = np.flatnonzero(row == best)[0]",
                     "best = np.abs(row).max()\n        out[r] = np.flatnonzero(np.abs(row) == best)[0]")],
                   lambda o: pins.check_argmax_brute_force(o.argmax.vocab_argmax)),
    # attention
    "attn_no_self": ([("attention", "        for j in ancestors(p, i):\n            A[i, P + j] = True",
                       "        for j in ancestors(p, i)[1:]:\n            A[i, P + j] = True")],
                     lambda o: pins.check_attention_chain_is_causal(o.attention.tree_attention)),
    "attn_sees_siblings": ([("attention", "        for j in ancestors(p, i):\n            A[i, P + j] = True",
                             "        A[i, P:P + i + 1] = True")],
                           lambda o: pins.check_attention_node_locality(o.attention.tree_attention)),
    "attn_tree_rows_off_by_one": ([("attention", "A[i, P + j] = True", "A[i, P + j - 1] = True")],
                                  lambda o: pins.check_attention_chain_is_causal(o.attention.tree_attention)),
    "attn_kv_head_mod": ([("attention", "for h in range(kvh * g, (kvh + 1) * g):", "for h in range(kvh, Hq, Hkv):")],
                         lambda o: pins.check_attention_chain_is_causal(o.attention.tree_attention)),
    "attn_bh_kv_head_mod": ([("attention", "    kvh = h // g\n", "    kvh = h % k_cache.shape[1]\n")],
                            lambda o: pins.check_attention_bh(o.attention.tree_attention_bh,
                                                              o.attention.tree_attention)),
    "attn_bh_query_of_kv_head": ([("attention", "Q = _as_f64(np.asarray(q[b, :, h, :]), q_fmt)            # [N][D]",
                                   "Q = _as_f64(np.asarray(q[b, :, kvh, :]), q_fmt)            # [N][D]")],
                                 lambda o: pins.check_attention_bh(o.attention.tree_attention_bh,
                                                                   o.attention.tree_attention)),
    "attn_no_scale": ([("attention", "s = float(sm_scale) * (Q @ Kf.T)                         # [N][L]", "s = Q @ Kf.T")],
                      lambda o: pins.check_attention_chain_is_causal(o.attention.tree_attention)),
    "attn_k_for_v": ([("attention", "out = w @ Vf", "out = w @ Kf")],
                     lambda o: pins.check_attention_one_node_is_decode(o.attention.tree_attention)),
    "attn_lse_without_max": ([("attention", "lse = (m + np.log(den))[:, 0]", "lse = np.log(den)[:, 0]")],
                             lambda o: pins.check_attention_chain_is_causal(o.attention.tree_attention)),
    "attn_prefix_short": ([("attention", "    A[:, :P] = True", "    A[:, :max(P - 1, 0)] = True")],
                          lambda o: pins.check_attention_one_node_is_decode(o.attention.tree_attention)),
    "e4m3_bias_8": ([("attention", "2.0 ** (e - 7)", "2.0 ** (e - 8)")],
                    lambda o: _check_e4m3(o)),
    "e2m1_bias_2": ([("attention", "(1.0 + m / 2.0) * 2.0 ** (e - 1)", "(1.0 + m / 2.0) * 2.0 ** (e - 2)")],
                    lambda o: pins.check_e2m1_table(o.attention.e2m1_decode_table)),
    "e2m1_high_nibble_first": ([("attention", "out = np.stack([lo, hi], axis=-1)", "out = np.stack([hi, lo], axis=-1)")],
                               lambda o: pins.check_e2m1_packing(o.attention.decode_e2m1_packed)),
    "e4m3_subnormal_dropped": ([("attention", "tab[code] = s * (m / 8.0) * 2.0 ** -6", "tab[code] = 0.0")],
                               lambda o: _check_e4m3(o)),
    # commit step
    "commit_dst_off_by_one": ([("commit", "k_new[b, :, P + k] = k_cache[b, :, src]", "k_new[b, :, P + k - 1] = k_cache[b, :, src]")],
                              lambda o: pins.check_commit_golden(o.commit.commit_accepted)),
    "commit_prefix_drops_root": ([("commit", "new_prefix[b] = P + 1 + L", "new_prefix[b] = P + L")],
                                 lambda o: pins.check_commit_golden(o.commit.commit_accepted)),
    "commit_root_labelled_accepted": ([("commit", "labels[b, 0] = LABEL_ROOT", "labels[b, 0] = LABEL_ACCEPTED")],
                                      lambda o: pins.check_commit_against_parent_chase(o.commit.commit_accepted,
                                                                                       o.tree.accept_walk)),
    "commit_source_by_depth": ([("commit", "src = P + path[k]", "src = P + k")],
                               lambda o: pins.check_commit_against_parent_chase(o.commit.commit_accepted,
                                                                                o.tree.accept_walk)),
    # backward pass
    "bwd_no_softmax_mean": ([("attention_bwd", "ds = w * (dw - (w * dw).sum(axis=1, keepdims=True))", "ds = w * dw")],
                            lambda o: pins.check_backward_invariants(o.attention_bwd.tree_attention_backward)),
    "bwd_dw_from_k": ([("attention_bwd", "dw = dO @ Vf.T", "dw = dO @ Kf.T")],
                      lambda o: pins.check_backward_autograd(o.attention_bwd.tree_attention_backward)),
    "bwd_dq_unscaled": ([("attention_bwd", "dQ = float(sm_scale) * (ds @ Kf)", "dQ = ds @ Kf")],
                        lambda o: pins.check_backward_finite_differences(o.attention_bwd.tree_attention_backward)),
    "bwd_dk_from_weights": ([("attention_bwd", "dK = float(sm_scale) * (ds.T @ Q)", "dK = float(sm_scale) * (w.T @ Q)")],
                            lambda o: pins.check_backward_invariants(o.attention_bwd.tree_attention_backward)),
    "bwd_unmasked_weights": ([("attention_bwd", "    s = np.where(A, s, -np.inf)\n", "")],
                             lambda o: pins.check_backward_subtree_locality(o.attention_bwd.tree_attention_backward)),
    "bwd_dv_last_head_only": ([("attention_bwd", "dv[b, kvh, :L] += dVh", "dv[b, kvh, :L] = dVh")],
                              lambda o: pins.check_backward_invariants(o.attention_bwd.tree_attention_backward)),
}


def _check_e4m3(o):
    import numpy as np
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    tab = o.attention.e4m3_decode_table()
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(tab[ok], ref[ok])


def test_unmutated_oracle_passes_every_mutation_pin():
    o = load_mutant([])
    for name, (_, pin) in MUTANTS.items():
        pin(o)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pin_rejects_planted_mistake(name):
    edits, pin = MUTANTS[name]
    o = load_mutant(edits)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        pin(o)
