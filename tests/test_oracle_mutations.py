"""Planted mistakes in the oracle must fail its pins.

Each case swaps one oracle function for a plausible wrong variant (a dropped
term, a wrong sign or index, an off-by-one) on the CPU, runs the pin tests
that are meant to guard it, and requires at least one of them to fail.  This
checks the pins themselves, not the GPU path.
"""

import numpy as np
import pytest

import test_oracle_accept_commit as PAC
import test_oracle_attention as PA
import test_oracle_sampling as PS
import test_oracle_tree as PT
from oracle import accept as AC
from oracle import sampling as SM
from oracle import attention as A
from oracle import commit as CM
from oracle import tree as T


def _fails(*pins):
    """True if at least one pin raises AssertionError."""
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return True
    return False


def test_unmutated_oracle_passes_these_pins():
    assert not _fails(PT.test_packed_table_pin, PT.test_positions_pin, PA.test_rope_golden,
                      PA.test_chain_is_causal_attention, PA.test_star_sees_context_and_self,
                      PAC.test_verify_tree_example_pin, PAC.test_argmax_ties_and_signed_zero)


def test_dropped_self_bit_is_caught(monkeypatch):
    orig = T.ancestor_path
    monkeypatch.setattr(T, "ancestor_path", lambda i, parents: orig(i, parents)[:-1])
    assert _fails(PT.test_packed_table_pin)


def test_one_based_depth_is_caught(monkeypatch):
    orig = T.depth_of
    monkeypatch.setattr(T, "depth_of", lambda i, parents: orig(i, parents) + 1)
    assert _fails(PT.test_positions_pin, PT.test_packed_table_pin)


def test_rope_sign_error_is_caught(monkeypatch):
    orig = A.rope
    # rotating by the opposite angle flips the sign of the sin terms
    monkeypatch.setattr(A, "rope", lambda x, pos, base=10000.0: orig(x, -np.asarray(pos), base))
    assert _fails(PA.test_rope_golden, PA.test_rope_matches_complex_rotation)


def test_rope_ignoring_base_is_caught(monkeypatch):
    orig = A.rope
    # a rope that always uses the default base passes every base-10000 case,
    # so only the goldens at bases 16, 100 and 500000 can catch it
    monkeypatch.setattr(A, "rope", lambda x, pos, base=10000.0: orig(x, pos, 10000.0))
    assert _fails(PA.test_rope_golden)


def test_rope_base_exponent_off_by_two_is_caught(monkeypatch):
    def rope_wrong_exponent(x, pos, base=10000.0):
        # inv_freq base^(-m/D) instead of base^(-2m/D)
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        inv = float(base) ** (-np.arange(D // 2) / D)
        ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
        c, s = np.cos(ang), np.sin(ang)
        out = np.empty_like(x)
        out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        out[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
        return out
    monkeypatch.setattr(A, "rope", rope_wrong_exponent)
    assert _fails(PA.test_rope_golden)


def test_rope_half_split_variant_is_caught(monkeypatch):
    def rope_neox(x, pos, base=10000.0):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        inv = base ** (-np.arange(D // 2) * 2.0 / D)
        ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[..., :D // 2], x[..., D // 2:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    monkeypatch.setattr(A, "rope", rope_neox)
    assert _fails(PA.test_rope_golden, PA.test_rope_matches_complex_rotation)


def test_missing_sqrt_in_scale_is_caught(monkeypatch):
    orig = A.softmax_attend
    monkeypatch.setattr(A, "softmax_attend",
                        lambda qg, kc, vc, kp, vp, scale: orig(qg, kc, vc, kp, vp, scale * scale))
    assert _fails(PA.test_chain_is_causal_attention)


def test_sibling_leak_is_caught(monkeypatch):
    # every earlier node visible (a lower-triangular mask) instead of ancestors only
    monkeypatch.setattr(A, "ancestor_path", lambda i, parents: list(range(i + 1)))
    assert _fails(PA.test_star_sees_context_and_self)


def test_argmax_last_tie_is_caught(monkeypatch):
    def last_argmax(rows):
        out = []
        for r in rows:
            r = np.asarray(r, dtype=np.float64)
            out.append(int(len(r) - 1 - np.argmax(r[::-1])))
        return out
    monkeypatch.setattr(AC, "row_argmax", last_argmax)
    assert _fails(PAC.test_argmax_ties_and_signed_zero)


def test_walk_without_bonus_row_is_caught(monkeypatch):
    orig = AC.greedy_walk

    def walk_bonus_from_parent_row(choice, tokens, parents, max_accept):
        w = orig(choice, tokens, parents, max_accept)
        acc = w["accepted"]
        # bonus taken from the row before the stop node (an off-by-one in the row index)
        w["bonus"] = choice[acc[-1]] if acc else choice[0]
        return w
    monkeypatch.setattr(AC, "greedy_walk", walk_bonus_from_parent_row)
    assert _fails(PAC.test_verify_tree_example_pin)


def test_commit_off_by_one_slot_is_caught(monkeypatch):
    def commit_shifted(k_cache, v_cache, ctx_lens, accept_len, accepted_nodes):
        k = np.array(k_cache, copy=True)
        v = np.array(v_cache, copy=True)
        new_lens = []
        for b, (ctx, a) in enumerate(zip(ctx_lens, accept_len)):
            for d in range(a):
                i = accepted_nodes[b][d]
                k[b, :, ctx + d] = k_cache[b, :, ctx + i - 1 if i > 0 else ctx + i]
                v[b, :, ctx + d] = v_cache[b, :, ctx + i - 1 if i > 0 else ctx + i]
            new_lens.append(ctx + a)
        return k, v, new_lens
    monkeypatch.setattr(CM, "commit_contiguous", commit_shifted)
    assert _fails(PAC.test_verify_tree_example_pin)


# ---- sampled walks ----

def test_sampling_without_noise_is_caught(monkeypatch):
    orig = SM.perturbed_rows
    monkeypatch.setattr(SM, "perturbed_rows", lambda x, T, g: orig(x, T, np.zeros_like(g)))
    assert _fails(PS.test_gumbel_max_frequencies_match_softmax, PS.test_hand_computed_row)


def test_sampling_ignoring_temperature_is_caught(monkeypatch):
    orig = SM.perturbed_rows
    monkeypatch.setattr(SM, "perturbed_rows", lambda x, T, g: orig(x, 1.0, g))
    assert _fails(PS.test_gumbel_max_frequencies_match_softmax)


def test_sampling_dividing_noise_by_temperature_is_caught(monkeypatch):
    # (x + g) / T samples from softmax(x / T) only when T = 1
    monkeypatch.setattr(SM, "perturbed_rows",
                        lambda x, T, g: ((np.asarray(x, np.float32) + np.asarray(g, np.float32)) /
                                         np.float32(T)).astype(np.float32))
    assert _fails(PS.test_gumbel_max_frequencies_match_softmax)


def _walk_variant(residual=True, ratio_swapped=False):
    """A copy of the stochastic walk with one step changed."""
    def walk(rows_f32, T, q_rows, u, g_rows, tokens, parents, max_accept):
        tokens = [int(t) for t in tokens]
        parents = [int(p) for p in parents]
        accepted, cur, row = [], -1, 0
        r = SM.softmax_f64(rows_f32[0], T)
        while True:
            q = np.asarray(q_rows[row], dtype=np.float64)
            nxt = None
            for j in [j for j in range(len(parents)) if parents[j] == cur]:
                x = tokens[j]
                ok = (u[j] * r[x] < q[x]) if ratio_swapped else (u[j] * q[x] < r[x])
                if ok:
                    nxt = j
                    break
                if residual:
                    res = np.maximum(r - q, 0.0)
                    if res.sum() > 0:
                        r = res / res.sum()
            if nxt is None:
                return dict(accepted=accepted, accepted_tokens=[tokens[j] for j in accepted],
                            bonus=SM.gumbel_sample(r, g_rows[row]), err=0)
            accepted.append(nxt)
            cur, row = nxt, 1 + nxt
            r = SM.softmax_f64(rows_f32[row], T)
    return walk


def test_stochastic_walk_copy_passes():
    import test_oracle_sampling as P
    orig = SM.stochastic_walk
    try:
        SM.stochastic_walk = _walk_variant()
        assert not _fails(P.test_stochastic_hand_computed, P.test_q_equal_p_accepts_first_children)
    finally:
        SM.stochastic_walk = orig


def test_stochastic_walk_without_residual_is_caught(monkeypatch):
    monkeypatch.setattr(SM, "stochastic_walk", _walk_variant(residual=False))
    assert _fails(PS.test_stochastic_hand_computed, lambda: PS.test_stochastic_walk_is_lossless(3))


def test_stochastic_walk_with_swapped_ratio_is_caught(monkeypatch):
    monkeypatch.setattr(SM, "stochastic_walk", _walk_variant(ratio_swapped=True))
    assert _fails(PS.test_stochastic_hand_computed, PS.test_q_equal_p_accepts_first_children)


# ---- DDTree construction ----

def test_ddtree_without_sibling_push_is_caught(monkeypatch):
    import heapq
    import test_oracle_ddtree as PD
    from oracle import ddtree as DD

    def no_siblings(logq, budget):
        heap = [(-logq[0][0], (0,))]
        popped = []
        while heap and len(popped) < budget:
            negs, ranks = heapq.heappop(heap)
            popped.append(ranks)
            d = len(ranks) - 1
            if d + 1 < len(logq):
                heapq.heappush(heap, (-(-negs + logq[d + 1][0]), ranks + (0,)))
        return popped
    monkeypatch.setattr(DD, "best_first", no_siblings)
    assert _fails(PD.test_worked_example_tree, lambda: PD.test_top_b_against_brute_force(0, 5, 3, 8))


def test_ddtree_unsorted_topk_is_caught(monkeypatch):
    import test_oracle_ddtree as PD
    from oracle import ddtree as DD
    orig = DD.depth_topk

    def first_k(z_row, K):  # the first K tokens instead of the K largest
        z = np.asarray(z_row, dtype=np.float64)
        toks, _ = orig(z, len(z))
        sel = np.sort(toks[:K])
        lq = z[sel] - np.log(np.exp(z[sel]).sum())
        return sel, lq
    monkeypatch.setattr(DD, "depth_topk", first_k)
    assert _fails(PD.test_depth_topk_order_and_normalisation, PD.test_worked_example_tree)
