"""The C ABI library on the host (no GPU needed): it loads, exports every
function the headers declare, and rejects bad arguments before launching."""

import ctypes
import glob
import os
import re

import pytest

import token_tree_attention_amd as tta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        names += re.findall(r"TTV_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tta.library_path()):
        pytest.skip("library not built (run python -m token_tree_attention_amd.build)")
    return tta.load_library()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("tree_build", "tree_attention_verify", "tree_greedy_accept", "tree_kv_commit",
              "tree_attention_workspace_bytes", "tree_greedy_accept_workspace_bytes"):
        assert n in names
    assert sorted(tta.EXPORTED_SYMBOLS) == names


def test_every_declared_symbol_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_debug_build_exports_and_release_reports_none(lib):
    """The release library answers ttv_debug_report with TTV_EINVAL (None from
    the binding); the debug build, when built, exports the same symbols."""
    if os.environ.get("TTV_DEBUG", "") in ("", "0") and not os.environ.get("TTV_LIBRARY"):
        assert tta.ttv_debug_report() is None
    dbg = os.path.join(ROOT, "token_tree_attention_amd", "libtreeverify_debug.so")
    if not os.path.exists(dbg):
        pytest.skip("debug library not built (python -m token_tree_attention_amd.build --debug)")
    d = ctypes.CDLL(dbg)
    for n in declared_functions():
        assert hasattr(d, n), n
    count, site = ctypes.c_uint32(7), ctypes.c_int32(7)
    assert d.ttv_debug_report(None, ctypes.byref(site), 0) == tta.TTV_EINVAL  # null output: rejected


def test_version_and_status(lib):
    assert tta.ttv_version() >= 100
    assert "invalid" in tta.ttv_status_string(tta.TTV_EINVAL)
    assert "workspace" in tta.ttv_status_string(tta.TTV_ENOSPC)


def _batch(B=2, n_max=8, T=10, offs=0x1000, ctx=0x2000):
    return tta._CBatch(B, n_max, T, offs, ctx)


def _cache(layout=0, hkv=2, D=128, cap=64, table=None, max_blocks=0, bs=0, nb=0):
    return tta._CCache(0x10000, 0x20000, layout, hkv, D, cap, table, max_blocks, bs, nb)


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def test_tree_build_rejects(lib):
    b = _batch()
    args = [FAKE] * 6
    assert lib.tree_build(None, FAKE, FAKE, 1, *args[:5], FAKE, None) == tta.TTV_EINVAL
    bad = _batch(n_max=2000)
    assert lib.tree_build(ctypes.byref(bad), FAKE, FAKE, 63, *args[:5], FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_build(ctypes.byref(b), FAKE, FAKE, 0, *args[:5], FAKE, None) == tta.TTV_EINVAL  # mask_words
    assert lib.tree_build(ctypes.byref(b), None, FAKE, 1, *args[:5], FAKE, None) == tta.TTV_EINVAL
    over = _batch(B=1, n_max=4, T=5)
    assert lib.tree_build(ctypes.byref(over), FAKE, FAKE, 1, *args[:5], FAKE, None) == tta.TTV_EINVAL
    empty = _batch(B=0, T=0)
    assert lib.tree_build(ctypes.byref(empty), None, None, 1, None, None, None, None, None, None, None) == tta.TTV_OK


def test_attention_rejects_and_sizes(lib):
    b = _batch()
    ok = _cache()
    ws = lib.tree_attention_workspace_bytes(ctypes.byref(b), ctypes.byref(ok), 8)
    assert ws > 0 and ws % 256 == 0
    assert lib.tree_attention_workspace_bytes(ctypes.byref(b), ctypes.byref(_cache(D=96)), 8) == 0
    assert lib.tree_attention_workspace_bytes(ctypes.byref(b), ctypes.byref(ok), 7) == 0  # 7 % 2
    paged_bad = _cache(layout=1, bs=32, max_blocks=4, nb=10, table=FAKE)
    assert lib.tree_attention_workspace_bytes(ctypes.byref(b), ctypes.byref(paged_bad), 8) == 0

    def call(bt=b, cache=ok, heads=8, base=10000.0, scale=0.0, ws_ptr=FAKE * 16, ws_bytes=ws, words=1,
             q=FAKE):
        return lib.tree_attention_verify(ctypes.byref(bt), q, FAKE, FAKE, FAKE, words, FAKE,
                                         ctypes.byref(cache), heads, base, scale, FAKE, ws_ptr, ws_bytes,
                                         FAKE, None)

    assert call(heads=3) == tta.TTV_EINVAL
    assert call(base=0.0) == tta.TTV_EINVAL
    assert call(scale=-1.0) == tta.TTV_EINVAL
    assert call(words=0) == tta.TTV_EINVAL
    assert call(q=None) == tta.TTV_EINVAL
    assert call(ws_ptr=FAKE * 16 + 8) == tta.TTV_EINVAL          # workspace not 256-aligned
    assert call(ws_bytes=ws - 1) == tta.TTV_ENOSPC
    assert call(cache=_cache(D=64 + 32)) == tta.TTV_EINVAL
    assert call(bt=_batch(B=5000, T=10)) == tta.TTV_EINVAL


def test_accept_rejects_and_sizes(lib):
    b = _batch()
    need = lib.tree_greedy_accept_workspace_bytes(ctypes.byref(b), 128256)
    assert need >= 8 * (10 + 2)
    assert lib.tree_greedy_accept_workspace_bytes(ctypes.byref(b), 0) == 0

    def call(dtype=1, vocab=128256, max_accept=16, ws_bytes=need, logits=FAKE):
        return lib.tree_greedy_accept(ctypes.byref(b), logits, dtype, vocab, FAKE, FAKE, FAKE, max_accept,
                                      FAKE, FAKE, FAKE, None, FAKE, ws_bytes, FAKE, None)

    assert call(dtype=7) == tta.TTV_EINVAL
    assert call(vocab=0) == tta.TTV_EINVAL
    assert call(max_accept=0) == tta.TTV_EINVAL
    assert call(logits=None) == tta.TTV_EINVAL
    assert call(ws_bytes=need - 1) == tta.TTV_ENOSPC


def test_commit_rejects(lib):
    b = _batch()

    def call(cache, max_accept=16, rel=FAKE, nrel=FAKE):
        return lib.tree_kv_commit(ctypes.byref(b), ctypes.byref(cache), FAKE, FAKE, max_accept, FAKE, rel,
                                  nrel, FAKE, None)

    assert call(_cache(D=80)) == tta.TTV_EINVAL
    assert call(_cache(), max_accept=0) == tta.TTV_EINVAL
    assert call(_cache(layout=1, bs=16, max_blocks=4, nb=10, table=None)) == tta.TTV_EINVAL
    assert call(_cache(layout=1, bs=16, max_blocks=4, nb=10, table=FAKE), rel=None) == tta.TTV_EINVAL
    assert call(_cache(layout=5)) == tta.TTV_EINVAL


def test_attention_rejects_oversized_mask_stride(lib):
    b = _batch()
    ok = _cache()
    ws = lib.tree_attention_workspace_bytes(ctypes.byref(b), ctypes.byref(ok), 8)
    # a mask row stride above 32 words (1024 nodes) is refused before any launch
    assert lib.tree_attention_verify(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 33, FAKE, ctypes.byref(ok), 8,
                                     10000.0, 0.0, FAKE, FAKE * 16, ws, FAKE, None) == tta.TTV_EINVAL


# ---- the Python binding checks shapes before anything reaches the library ----

def _fake_batch(B=2, T=10, n_max=8):
    from types import SimpleNamespace
    return SimpleNamespace(batch=B, total_nodes=T, n_max=n_max, mask_words=max(1, (n_max + 31) // 32))


def _fake_cache(B=2, hkv=2, D=128, paged=False, table_rows=2):
    import torch
    from types import SimpleNamespace
    k = torch.zeros((B, hkv, 4, D), dtype=torch.bfloat16)
    return SimpleNamespace(k=k, v=k, n_kv_heads=hkv, head_dim=D,
                           layout=tta.KV_PAGED if paged else tta.KV_CONTIGUOUS,
                           block_table=torch.zeros((table_rows, 3), dtype=torch.int32) if paged else None)


def _attn_args(T=10, Hq=8, D=128, W=1):
    import torch
    bf = dict(dtype=torch.bfloat16)
    return dict(q=torch.zeros((T, Hq, D), **bf), k_new=torch.zeros((T, 2, 128), **bf),
                v_new=torch.zeros((T, 2, 128), **bf), mask=torch.zeros((T, W), dtype=torch.int32),
                positions=torch.zeros(T, dtype=torch.int32), err=torch.zeros(2, dtype=torch.int32))


@pytest.mark.parametrize("bad, match", [
    (dict(q=(10, 8, 64)), "q must be"),          # head_dim differs from the cache's
    (dict(q=(9, 8, 128)), "q must be"),          # rows differ from T
    (dict(mask=(9, 1)), "mask must be"),         # mask rows differ from T
    (dict(mask=(10, 33)), "mask must be"),       # stride over 32 words
    (dict(out=(10, 8, 64)), "out must have"),    # out smaller than q
])
def test_binding_attention_shape_mismatch_raises(lib, bad, match):
    import torch
    a = _attn_args()
    out = None
    for k, shape in bad.items():
        t = torch.zeros(shape, dtype=torch.int32 if k == "mask" else torch.bfloat16)
        if k == "out":
            out = t
        else:
            a[k] = t
    with pytest.raises(ValueError, match=match):
        tta.tree_attention_verify(_fake_batch(), a["q"], a["k_new"], a["v_new"], a["mask"], a["positions"],
                                  _fake_cache(), a["err"], out=out)


def test_binding_cache_rows_must_match_batch(lib):
    a = _attn_args()
    with pytest.raises(ValueError, match="contiguous cache"):
        tta.tree_attention_verify(_fake_batch(), a["q"], a["k_new"], a["v_new"], a["mask"], a["positions"],
                                  _fake_cache(B=3), a["err"])
    with pytest.raises(ValueError, match="block_table"):
        tta.tree_attention_verify(_fake_batch(), a["q"], a["k_new"], a["v_new"], a["mask"], a["positions"],
                                  _fake_cache(paged=True, table_rows=5), a["err"])


def test_binding_commit_shapes(lib):
    import torch
    z = lambda *s: torch.zeros(s, dtype=torch.int32)
    with pytest.raises(ValueError, match="accepted_nodes"):
        tta.tree_kv_commit(_fake_batch(), _fake_cache(), z(2), z(3, 4), z(2))
    with pytest.raises(ValueError, match="block_table"):
        tta.tree_kv_commit(_fake_batch(), _fake_cache(paged=True, table_rows=1), z(2), z(2, 4), z(2))


def test_binding_refuses_host_tensors(lib):
    a = _attn_args()
    with pytest.raises(ValueError, match="ROCm device"):
        tta.tree_attention_verify(_fake_batch(), a["q"], a["k_new"], a["v_new"], a["mask"], a["positions"],
                                  _fake_cache(), a["err"])


def test_accept_noalloc_rejects_beyond_its_scratch(lib):
    # 1000 requests of up to 1024 nodes: (T + B) keys of 8 bytes exceed the 4 MiB scratch
    big = _batch(B=1000, n_max=1024, T=1000 * 1024)
    assert lib.tree_greedy_accept_workspace_bytes(ctypes.byref(big), 32000) > (4 << 20)
    assert lib.tree_greedy_accept_noalloc(ctypes.byref(big), FAKE, 1, 32000, FAKE, FAKE, FAKE, 16,
                                          FAKE, FAKE, FAKE, None, FAKE, None) == tta.TTV_ENOSPC
    b = _batch()
    assert lib.tree_greedy_accept_noalloc(ctypes.byref(b), FAKE, 7, 32000, FAKE, FAKE, FAKE, 16,
                                          FAKE, FAKE, FAKE, None, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_greedy_accept_noalloc(ctypes.byref(b), None, 1, 32000, FAKE, FAKE, FAKE, 16,
                                          FAKE, FAKE, FAKE, None, FAKE, None) == tta.TTV_EINVAL


def test_sampled_walks_reject(lib):
    b = _batch()
    need = lib.tree_greedy_accept_workspace_bytes(ctypes.byref(b), 1000)

    def sample(T=1.0, gumbel=FAKE, ws_bytes=need):
        return lib.tree_sample_accept(ctypes.byref(b), FAKE, 1, 1000, T, gumbel, FAKE, FAKE, FAKE, 16, FAKE, FAKE,
                                      FAKE, None, FAKE, ws_bytes, FAKE, None)

    assert sample(T=0.0) == tta.TTV_EINVAL
    assert sample(T=-2.0) == tta.TTV_EINVAL
    assert sample(T=float("inf")) == tta.TTV_EINVAL
    assert sample(T=1e-45) == tta.TTV_EINVAL        # 1 / T overflows float32
    assert sample(gumbel=None) == tta.TTV_EINVAL
    assert sample(ws_bytes=need - 1) == tta.TTV_ENOSPC
    sneed = lib.tree_stochastic_accept_workspace_bytes(ctypes.byref(b), 1000)
    # two float64 vocab buffers per request (padded to 256 bytes), then a
    # 1024-byte record per request for the reductions of a request's workgroups
    assert sneed == (2 * 2 * 1000 * 8 + 255) // 256 * 256 + 2 * 1024

    def stoch(T=1.0, q=FAKE, u=FAKE, ws_bytes=sneed):
        return lib.tree_stochastic_accept(ctypes.byref(b), FAKE, 1, 1000, T, q, u, FAKE, FAKE, FAKE, FAKE, 16,
                                          FAKE, FAKE, FAKE, FAKE, ws_bytes, FAKE, None)

    assert stoch(T=0.0) == tta.TTV_EINVAL
    assert stoch(q=None) == tta.TTV_EINVAL
    assert stoch(u=None) == tta.TTV_EINVAL
    assert stoch(ws_bytes=sneed - 1) == tta.TTV_ENOSPC


def test_mask_interop_rejects(lib):
    b = _batch()
    assert lib.tree_expand_mask(ctypes.byref(b), FAKE, 1, 2, FAKE, 64, FAKE, None) == tta.TTV_EINVAL   # mode
    assert lib.tree_expand_mask(ctypes.byref(b), FAKE, 0, 0, FAKE, 64, FAKE, None) == tta.TTV_EINVAL   # words
    assert lib.tree_expand_mask(ctypes.byref(b), FAKE, 33, 0, FAKE, 64, FAKE, None) == tta.TTV_EINVAL  # words > 32
    assert lib.tree_expand_mask(ctypes.byref(b), FAKE, 1, 0, FAKE, 4, FAKE, None) == tta.TTV_EINVAL    # stride < n_max
    assert lib.tree_expand_mask(ctypes.byref(b), None, 1, 0, FAKE, 64, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_pack_mask(ctypes.byref(b), FAKE, 64, 5, FAKE, 1, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_pack_mask(ctypes.byref(b), None, 64, 1, FAKE, 1, FAKE, None) == tta.TTV_EINVAL
    empty = _batch(B=0, T=0)
    assert lib.tree_pack_mask(ctypes.byref(empty), None, 64, 1, None, 1, None, None) == tta.TTV_OK


def test_ddtree_build_rejects(lib):
    assert lib.tree_ddtree_workspace_bytes(4, 16, 151936, 1024) == 4 * 16 * 1024 * 12 + 256
    assert lib.tree_ddtree_workspace_bytes(4, 21, 1000, 64) == 0      # depths > 20
    assert lib.tree_ddtree_workspace_bytes(4, 16, 1000, 1025) == 0    # budget > 1024
    need = lib.tree_ddtree_workspace_bytes(2, 3, 50, 20)
    assert lib.tree_ddtree_build(2, 3, 50, 20, None, FAKE, FAKE, FAKE, FAKE * 16, need, None) == tta.TTV_EINVAL
    assert lib.tree_ddtree_build(2, 3, 50, 20, FAKE, FAKE, FAKE, FAKE, FAKE * 16 + 8, need, None) == tta.TTV_EINVAL
    assert lib.tree_ddtree_build(2, 3, 50, 20, FAKE, FAKE, FAKE, FAKE, FAKE * 16, need - 1, None) == tta.TTV_ENOSPC
    assert lib.tree_ddtree_build(0, 3, 50, 20, None, None, None, None, None, 0, None) == tta.TTV_OK


def test_merge_sequences_rejects(lib):
    assert lib.tree_merge_sequences(1, 1025, 4, FAKE, 64, FAKE, FAKE, FAKE, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_merge_sequences(1, 4, 4, FAKE, 1025, FAKE, FAKE, FAKE, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_merge_sequences(1, 4, 4, None, 64, FAKE, FAKE, FAKE, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_merge_sequences(0, 4, 4, None, 64, None, None, None, None, None) == tta.TTV_OK


def test_eagle_grow_rejects(lib):
    assert lib.tree_eagle_grow(1, 17, 6, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_eagle_grow(1, 4, 17, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_eagle_grow(1, 4, 6, FAKE, FAKE, FAKE, FAKE, 1025, FAKE, FAKE, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_eagle_grow(1, 4, 6, FAKE, FAKE, None, FAKE, 64, FAKE, FAKE, FAKE, None) == tta.TTV_EINVAL
    assert lib.tree_eagle_grow(0, 4, 6, None, None, None, None, 64, None, None, None, None) == tta.TTV_OK
