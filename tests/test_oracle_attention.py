"""Pins of the attention oracle.

The oracle computes, per node, causal attention over its linearised path.
It is checked against (a) hand-derived RoPE values, (b) the page's claim
that one packed pass with the ancestry mask gives the same numbers, done
here with torch's own scaled_dot_product_attention in float64 and a mask
built from the reflexive-transitive closure of the parent relation,
(c) the page's negative result that a lower-triangular mask leaks between
siblings, and (d) textbook causal attention for a chain.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import attention as A
from oracle import bf16 as OB
from conftest import golden


def rope_complex(x, pos, base=10000.0):
    """RoPE written as complex rotation of (x0 + i x1) pairs, for cross-checking."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-np.arange(D // 2) * 2.0 / D)
    w = z * np.exp(1j * theta)
    out = np.empty_like(x)
    out[..., 0::2] = w.real
    out[..., 1::2] = w.imag
    return out


def test_rope_golden():
    for c in golden("rope_cases.json")["cases"]:
        got = A.rope(np.array(c["x"]), c["position"], c["base"])
        np.testing.assert_allclose(got, c["expected"], rtol=0, atol=1e-15)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 128))
    pos = rng.integers(0, 40000, size=(5, 1))
    np.testing.assert_allclose(A.rope(x, pos), rope_complex(x, pos), rtol=0, atol=1e-10)


def closure(parents):
    n = len(parents)
    R = np.eye(n, dtype=bool)
    for i in range(n):
        j = parents[i]
        while j != -1:
            R[i, j] = True
            j = parents[j]
    return R


def depths_by_closure(parents):
    return closure(parents).sum(1) - 1


def random_bf16(rng, shape):
    return synth.bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))


def packed_sdpa(q, k_new, v_new, k_ctx, v_ctx, parents, ctx, mask_tree=None, base=10000.0):
    """One packed pass with torch SDPA (float64), GQA by repeating KV heads per group."""
    N, Hq, D = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    pos = ctx + depths_by_closure(parents)
    qr = rope_complex(OB.to_f64(q), pos[:, None], base)                 # [N, Hq, D]
    kr = rope_complex(OB.to_f64(k_new), pos[:, None], base)             # [N, Hkv, D]
    K = np.concatenate([OB.to_f64(k_ctx).transpose(1, 0, 2), kr], 0)   # [ctx+N, Hkv, D]
    V = np.concatenate([OB.to_f64(v_ctx).transpose(1, 0, 2), OB.to_f64(v_new)], 0)
    K = np.repeat(K, G, axis=1)
    V = np.repeat(V, G, axis=1)
    if mask_tree is None:
        mask_tree = closure(parents)
    mask = np.concatenate([np.ones((N, ctx), dtype=bool), mask_tree], 1)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(t(qr), t(K), t(V), attn_mask=torch.from_numpy(mask))
    return o[0].numpy().transpose(1, 0, 2)


def case(rng, parents, ctx, Hq, Hkv, D):
    N = len(parents)
    return dict(q=random_bf16(rng, (N, Hq, D)), k_new=random_bf16(rng, (N, Hkv, D)),
                v_new=random_bf16(rng, (N, Hkv, D)), k_ctx=random_bf16(rng, (Hkv, ctx, D)),
                v_ctx=random_bf16(rng, (Hkv, ctx, D)))


def test_packed_equals_branch_on_page_tree():
    """Page experiment: B=1, H=2, P=2, N=8, D=8; packed == branch within 1e-12; wrong mask leaks."""
    g = golden("packed_table.json")
    rng = np.random.default_rng(233)
    par = g["parents"]
    c = case(rng, par, g["prefix_length"], 2, 2, 8)
    ref = A.attention_request(c["q"], c["k_new"], c["v_new"], c["k_ctx"], c["v_ctx"], par, g["prefix_length"])
    packed = packed_sdpa(parents=par, ctx=g["prefix_length"], **c)
    assert np.abs(packed - ref).max() <= g["packed_vs_branch_tolerance"]
    wrong = packed_sdpa(parents=par, ctx=g["prefix_length"], mask_tree=np.tril(np.ones((8, 8), bool)), **c)
    assert np.abs(wrong - ref).max() > g["wrong_mask_leak_lower_bound"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_packed_equals_branch_random_trees(seed):
    rng = np.random.default_rng(seed)
    par = synth.random_tree(rng, 37, max_parent_depth=5).tolist()
    c = case(rng, par, 50, 8, 2, 64)
    ref = A.attention_request(c["q"], c["k_new"], c["v_new"], c["k_ctx"], c["v_ctx"], par, 50)
    packed = packed_sdpa(parents=par, ctx=50, **c)
    assert np.abs(packed - ref).max() <= 1e-12


def test_chain_is_causal_attention():
    rng = np.random.default_rng(7)
    ctx, N, H, D = 20, 12, 2, 32
    par = [-1] + list(range(N - 1))
    c = case(rng, par, ctx, H, H, D)
    ref = A.attention_request(c["q"], c["k_new"], c["v_new"], c["k_ctx"], c["v_ctx"], par, ctx)
    # Textbook: one causal sequence ctx ++ chain; chain token i sits at position ctx + i.
    L = ctx + N
    qfull = np.zeros((L, H, D))
    qfull[ctx:] = rope_complex(OB.to_f64(c["q"]), (ctx + np.arange(N))[:, None])
    K = np.concatenate([OB.to_f64(c["k_ctx"]).transpose(1, 0, 2),
                        rope_complex(OB.to_f64(c["k_new"]), (ctx + np.arange(N))[:, None])], 0)
    V = np.concatenate([OB.to_f64(c["v_ctx"]).transpose(1, 0, 2), OB.to_f64(c["v_new"])], 0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(t(qfull), t(K), t(V), is_causal=True)[0].numpy().transpose(1, 0, 2)
    assert np.abs(o[ctx:] - ref).max() <= 1e-12


def test_star_sees_context_and_self():
    rng = np.random.default_rng(8)
    ctx, N, D = 9, 6, 16
    par = [-1] * N
    c = case(rng, par, ctx, 1, 1, D)
    ref = A.attention_request(c["q"], c["k_new"], c["v_new"], c["k_ctx"], c["v_ctx"], par, ctx)
    for i in range(N):
        q = rope_complex(OB.to_f64(c["q"][i, 0]), ctx)
        K = np.concatenate([OB.to_f64(c["k_ctx"][0]), rope_complex(OB.to_f64(c["k_new"][i:i + 1, 0]), np.array([[ctx]])[0])], 0)
        V = np.concatenate([OB.to_f64(c["v_ctx"][0]), OB.to_f64(c["v_new"][i:i + 1, 0])], 0)
        s = K @ q / np.sqrt(D)
        p = np.exp(s - s.max())
        np.testing.assert_allclose(ref[i, 0], (p / p.sum()) @ V, rtol=0, atol=1e-13)


def test_no_context_and_single_node():
    rng = np.random.default_rng(9)
    c = case(rng, [-1], 0, 2, 1, 8)
    ref = A.attention_request(c["q"], c["k_new"], c["v_new"], c["k_ctx"], c["v_ctx"], [-1], 0)
    # One key only: the output is that key's value exactly, for every head.
    np.testing.assert_array_equal(ref[0, 0], OB.to_f64(c["v_new"][0, 0]))
    np.testing.assert_array_equal(ref[0, 1], OB.to_f64(c["v_new"][0, 0]))


def test_node_subset_matches_full():
    rng = np.random.default_rng(10)
    par = synth.random_tree(rng, 20).tolist()
    c = case(rng, par, 30, 4, 2, 32)
    full = A.attention_request(c["q"], c["k_new"], c["v_new"], c["k_ctx"], c["v_ctx"], par, 30)
    sub = A.attention_request(c["q"], c["k_new"], c["v_new"], c["k_ctx"], c["v_ctx"], par, 30, nodes=[19, 3])
    np.testing.assert_array_equal(sub, full[[19, 3]])


def test_paged_context_gather():
    rng = np.random.default_rng(11)
    ctx, Hkv, D, bs = 45, 2, 8, 16
    kc = random_bf16(rng, (Hkv, ctx, D))
    vc = random_bf16(rng, (Hkv, ctx, D))
    nblk = -(-ctx // bs)
    perm = rng.permutation(10)[:nblk]
    pool_k = np.zeros((10, Hkv, bs, D), np.uint16)
    pool_v = np.zeros((10, Hkv, bs, D), np.uint16)
    for lb in range(nblk):
        seg = slice(lb * bs, min(ctx, lb * bs + bs))
        w = seg.stop - seg.start
        pool_k[perm[lb], :, :w] = kc[:, seg]
        pool_v[perm[lb], :, :w] = vc[:, seg]
    table = np.full((1, 4), -1, np.int32)
    table[0, :nblk] = perm
    gk, gv = A.context_of(pool_k, pool_v, 0, ctx, "paged", table, bs)
    np.testing.assert_array_equal(gk, kc)
    np.testing.assert_array_equal(gv, vc)


def test_tentative_k_is_rotation_at_tree_positions():
    rng = np.random.default_rng(12)
    par = [-1, 0, 0, 1, -1]
    k = random_bf16(rng, (5, 2, 16))
    got = A.tentative_k(k, par, 100)
    pos = 100 + np.array([0, 1, 1, 2, 0])
    np.testing.assert_allclose(got, rope_complex(OB.to_f64(k), pos[:, None]), rtol=0, atol=1e-12)
