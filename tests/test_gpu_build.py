"""tree_build on the GPU against the oracle: bit-exact."""

import itertools

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import host, require_gpu, say
from parity import check_build

pytestmark = pytest.mark.gpu


def run_build(tb, n_max=None, mask_words=None):
    import torch
    n_max = tb.n_max if n_max is None else n_max
    bt = tta.Batch(torch.from_numpy(tb.node_offsets).cuda(), torch.from_numpy(tb.ctx_lens).cuda(),
                   n_max, total_nodes=tb.total_nodes)
    parents = torch.from_numpy(np.ascontiguousarray(tb.parents, dtype=np.int32)).cuda()
    out = None
    if mask_words is not None:
        T, B = tb.total_nodes, tb.batch
        i32 = dict(dtype=torch.int32, device="cuda")
        out = {"mask": torch.full((T, mask_words), -7, **i32)}
        for k in ("depth", "positions", "retrieve_index", "retrieve_next_token", "retrieve_next_sibling"):
            out[k] = torch.full((T,), -7, **i32)
        out["err"] = torch.full((B,), -7, **i32)
        import ctypes
        st = tta.load_library().tree_build(ctypes.byref(bt._c), parents.data_ptr(), out["mask"].data_ptr(),
                                           mask_words, out["depth"].data_ptr(), out["positions"].data_ptr(),
                                           out["retrieve_index"].data_ptr(),
                                           out["retrieve_next_token"].data_ptr(),
                                           out["retrieve_next_sibling"].data_ptr(), out["err"].data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
        assert st == 0
    else:
        out = tta.tree_build(bt, parents)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def tree_batch(parent_lists, ctx):
    sizes = [len(p) for p in parent_lists]
    offs = np.zeros(len(sizes) + 1, np.int32)
    offs[1:] = np.cumsum(sizes)
    par = np.concatenate([np.asarray(p, np.int32) for p in parent_lists]) if offs[-1] else np.zeros(0, np.int32)
    return synth.TreeBatch(par, np.zeros_like(par), offs, np.asarray(ctx, np.int32),
                           np.zeros(len(sizes)), list(parent_lists), [])


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5])
def test_build_configs(cfg):
    require_gpu()
    tb = synth.make_trees(cfg, 0)
    say(f"tree_build cfg={cfg} B={tb.batch} T={tb.total_nodes} n_max={tb.n_max}")
    check_build(tb, run_build(tb))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_build_all_parent_lists(n):
    require_gpu()
    lists = [list(p) for p in itertools.product(*[range(-1, i) for i in range(n)])]
    tb = tree_batch(lists, [(7 * i) % 11 for i in range(len(lists))])
    say(f"tree_build all parent lists n={n} B={tb.batch}")
    check_build(tb, run_build(tb))


def test_build_large_shapes():
    require_gpu()
    chain = list(range(-1, 1023))
    star = [-1] * 1024
    rng = np.random.default_rng(5)
    rnd = synth.random_tree(rng, 1024, max_parent_depth=1000).tolist()
    comb = [-1] + [i - 1 if i % 2 else i - 2 for i in range(1, 1024)]
    comb = [max(-1, min(p, i - 1)) for i, p in enumerate(comb)]
    tb = tree_batch([chain, star, rnd, comb, [], [-1]], [0, 5, 100000, 3, 9, 0])
    say("tree_build 1024-node chain/star/random/comb + empty + single")
    check_build(tb, run_build(tb, n_max=1024))


def test_build_errors_and_wide_stride():
    require_gpu()
    lists = [[-1, 1, 0], [-1, 0, 0, 0, 0, 0], [-1, -2], [-1, 0]]
    tb = tree_batch(lists, [4, 4, 4, -3])
    say("tree_build error bits")
    out = run_build(tb, n_max=5, mask_words=3)
    assert out["err"].tolist() == [tta.ERR_BAD_PARENT, tta.ERR_TOO_MANY_NODES, tta.ERR_BAD_PARENT,
                                   tta.ERR_BAD_LENGTH]
    # stride wider than needed: unused words are written as zero
    good = tree_batch([[-1, 0, 1], [-1, -1]], [2, 3])
    out = run_build(good, n_max=3, mask_words=3)
    assert (out["mask"][:, 1:] == 0).all()
    check_build(good, out, n_max=3)
