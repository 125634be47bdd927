"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces on the host, and rejects bad arguments with the
documented status before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uniprefill.h")

UP_OK, UP_EINVAL, UP_EUNSUPPORTED, UP_EWORKSPACE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def L():
    from block_wise_token_amd import lib
    return lib()


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(up_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    syms = _declared_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(L, s), f"{s} declared in include/uniprefill.h but not exported"


def test_status_strings(L):
    assert L.up_status_string(UP_OK) == b"UP_OK"
    for st in (UP_EINVAL, UP_EUNSUPPORTED, UP_EWORKSPACE, -4):
        assert L.up_status_string(st).startswith(b"UP_E")
    assert L.up_abi_version() == 1


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def test_workspace_sizes(L):
    cu = _cu([131072])
    ws = L.up_block_scores_workspace(_p(cu), 1, 32, 8, 128, 128, 64)
    # at least the per-(row, block) statistics: 2048 blocks x 4096 rows x 8 bytes
    assert ws >= 2048 * 4096 * 8
    assert ws % 256 == 0
    assert L.up_block_scores_workspace(_p(cu), 1, 32, 7, 128, 128, 64) == 0     # Hq % Hkv
    assert L.up_block_scores_workspace(_p(cu), 1, 32, 8, 96, 128, 64) == 0      # d unsupported
    assert L.up_block_scores_workspace(_p(cu), 1, 32, 8, 128, 128, 16) == 0     # G unsupported
    cw = L.up_expand_compact_workspace(_p(cu), 1, 64)
    assert cw >= 3 * 2048 * 4
    vl = _cu([8192, 0, 65536, 77])
    assert L.up_block_scores_workspace(_p(vl), 4, 32, 8, 128, 128, 64) > 0
    # the given-lse pass needs only the plan and one float per (block, kv head, row tile)
    lw = L.up_block_scores_lse_workspace(_p(cu), 1, 32, 8, 128, 128, 64)
    assert 2048 * 8 * 4 <= lw < ws // 100 and lw % 256 == 0
    assert L.up_block_scores_lse_workspace(_p(cu), 1, 32, 8, 96, 128, 64) == 0
    bad = np.array([0, 10, 5], np.int32)
    assert L.up_expand_compact_workspace(_p(bad), 2, 64) == 0


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first


def test_block_scores_rejects_bad_arguments(L):
    cu = _cu([4096])
    f = L.up_block_scores

    def call(cu_h=cu, B=1, Hq=8, Hkv=2, d=64, n=128, G=64, ws=FAKE, wsb=1 << 40, q=FAKE):
        return f(q, FAKE, FAKE, _p(cu_h), B, Hq, Hkv, d, n, G, ctypes.c_float(0.0), FAKE, None,
                 ws, ctypes.c_size_t(wsb), None)

    assert call(Hkv=3) == UP_EINVAL
    assert call(Hq=0) == UP_EINVAL
    assert call(n=0) == UP_EINVAL
    assert call(d=80) == UP_EUNSUPPORTED
    assert call(G=48) == UP_EUNSUPPORTED
    assert call(G=2048) == UP_EUNSUPPORTED
    assert call(Hq=4096, Hkv=4096, d=256) == UP_EUNSUPPORTED   # 1024 key rows reach 2 GiB
    assert call(cu_h=np.array([0, 5, 3], np.int32), B=2) == UP_EINVAL
    assert call(cu_h=np.array([1, 5], np.int32)) == UP_EINVAL
    assert call(q=None) == UP_EINVAL
    assert call(q=ctypes.c_void_p(0x100002)) == UP_EINVAL           # qwin not 16-byte aligned
    assert call(wsb=16) == UP_EWORKSPACE
    assert call(ws=None) == UP_EWORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == UP_EWORKSPACE      # not 256-byte aligned
    # nothing to do is not an error
    assert call(cu_h=np.array([0], np.int32), B=0) == UP_OK
    assert call(cu_h=np.array([0, 0, 0], np.int32), B=2) == UP_OK


def test_select_rejects_bad_arguments(L):
    cu = _cu([4096])
    for p in (0.0, -0.5, 1.5, float("nan")):
        assert L.up_topp_select(FAKE, FAKE, _p(cu), 1, 128, 64, ctypes.c_float(p), FAKE, FAKE,
                                None) == UP_EINVAL
    assert L.up_topk_select(FAKE, FAKE, _p(cu), 1, 128, 64, -1, FAKE, FAKE, None) == UP_EINVAL
    assert L.up_topp_select(FAKE, FAKE, _p(cu), 1, 0, 64, ctypes.c_float(0.9), FAKE, FAKE,
                            None) == UP_EINVAL
    assert L.up_topp_select(FAKE, FAKE, _p(cu), 1, 128, 64, ctypes.c_float(0.9), FAKE, None,
                            None) == UP_EINVAL
    huge = _cu([64 * 16384 + 1])                                       # 16385 blocks
    assert L.up_topp_select(FAKE, FAKE, _p(huge), 1, 128, 64, ctypes.c_float(0.9), FAKE, FAKE,
                            None) == UP_EUNSUPPORTED
    assert L.up_topp_select(FAKE, FAKE, _p(np.array([0, 3, 2], np.int32)), 2, 128, 64,
                            ctypes.c_float(0.9), FAKE, FAKE, None) == UP_EINVAL


def test_expand_compact_and_compose_reject_bad_arguments(L):
    cu = _cu([4096])
    f = L.up_expand_compact

    def call(H=1024, eb=2, ws=FAKE, wsb=1 << 30, hidden=FAKE, pos=FAKE, pos_out=FAKE, G=64,
             prev=None, orig=None):
        return f(hidden, H, eb, pos, FAKE, FAKE, FAKE, _p(cu), 1, G, FAKE, FAKE, pos_out, prev,
                 orig, ws, ctypes.c_size_t(wsb), None)

    assert call(H=0) == UP_EINVAL
    assert call(eb=0) == UP_EINVAL
    assert call(G=0) == UP_EINVAL
    assert call(hidden=None) == UP_EINVAL
    assert call(pos=None) == UP_EINVAL          # pos_out requested without pos
    assert call(orig=FAKE) == UP_EINVAL         # orig_out requested without prev_orig
    assert call(wsb=8) == UP_EWORKSPACE
    assert call(ws=None) == UP_EWORKSPACE
    g = L.up_compose_drops
    assert g(FAKE, 10, FAKE, FAKE, -1, FAKE, None) == UP_EINVAL
    assert g(FAKE, -1, FAKE, FAKE, 4, FAKE, None) == UP_EINVAL
    assert g(FAKE, 10, None, FAKE, 4, FAKE, None) == UP_EINVAL
    assert g(None, 0, None, None, 0, None, None) == UP_OK                # empty: nothing to do


def test_no_cpu_fallback_in_the_product_path():
    """The binding has no route to the oracle or any CPU implementation."""
    pkg = os.path.join(ROOT, "block_wise_token_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src, fn
            assert "uniprefill_oracle" not in src, fn


def test_block_scores_lse_rejects_bad_arguments(L):
    cu = _cu([4096])
    f = L.up_block_scores_lse

    def call(lse=FAKE, B=1, Hkv=2, d=64, G=64, ws=FAKE, wsb=1 << 40):
        return f(FAKE, FAKE, lse, FAKE, _p(cu), B, 8, Hkv, d, 128, G, ctypes.c_float(0.0), FAKE,
                 ws, ctypes.c_size_t(wsb), None)

    assert call(Hkv=3) == UP_EINVAL
    assert call(d=80) == UP_EUNSUPPORTED
    assert call(G=48) == UP_EUNSUPPORTED
    assert call(lse=None) == UP_EINVAL
    assert call(lse=ctypes.c_void_p(0x100002)) == UP_EINVAL      # row_lse not 4-byte aligned
    assert call(wsb=16) == UP_EWORKSPACE
    assert call(ws=None) == UP_EWORKSPACE


def test_score_chunks_are_not_tiny_for_mixed_lengths(L):
    """The score pass's key chunks must amortise a workgroup's fixed cost: for the
    8-request pack (8K-64K tokens) the chunk statistics ([chunks][Hkv][rows] pairs)
    stay a small fraction of the per-block statistics ([blocks][Hkv][rows] pairs),
    which they would match with one-block chunks."""
    lens = [56971, 44718, 37503, 23662, 25844, 10541, 12506, 9139]
    cu = _cu(lens)
    Hq, Hkv, d, n, G = 32, 8, 128, 128, 64
    ws = L.up_block_scores_workspace(_p(cu), len(lens), Hq, Hkv, d, n, G)
    per_block = sum((x + G - 1) // G for x in lens) * Hq * n * 8     # (m, l) pairs, bytes
    assert per_block < ws < 1.2 * per_block


def test_statistics_chunks_depend_on_the_request_alone(L):
    """A request's statistics chunks (where the score pass restarts its softmax
    reference) come from its own length and the call's shape only: the same whether it
    is scored alone or packed with others, so its scores can be bit-identical."""
    lens = [56971, 44718, 37503, 23662, 25844, 10541, 12506, 9139, 0, 1, 700]
    Hq, Hkv, d, n, G = 32, 8, 128, 128, 64
    packed = (ctypes.c_int32 * len(lens))()
    assert L.up_block_scores_chunks(_p(_cu(lens)), len(lens), Hq, Hkv, d, n, G, packed) == UP_OK
    for i, x in enumerate(lens):
        alone = (ctypes.c_int32 * 1)()
        assert L.up_block_scores_chunks(_p(_cu([x])), 1, Hq, Hkv, d, n, G, alone) == UP_OK
        assert alone[0] == packed[i], (i, x)
        assert 1 <= packed[i] <= 256
    # a lone 128K request of the Llama-3.1-8B shape: 64-block chunks (256 workgroups)
    one = (ctypes.c_int32 * 1)()
    assert L.up_block_scores_chunks(_p(_cu([131072])), 1, Hq, Hkv, d, n, G, one) == UP_OK
    assert one[0] == 64
    # the same argument checks as the score pass
    assert L.up_block_scores_chunks(_p(_cu([100])), 1, 32, 7, d, n, G, one) == UP_EINVAL
    assert L.up_block_scores_chunks(_p(_cu([100])), 1, 32, 8, 96, n, G, one) == UP_EUNSUPPORTED
    assert L.up_block_scores_chunks(_p(_cu([100])), 1, 32, 8, d, n, G, None) == UP_EINVAL


def test_block_scores_paged_rejects_bad_arguments(L):
    cu = _cu([1000, 24])
    f = L.up_block_scores_paged

    def call(ps=16, maxp=63, table=FAKE, npages=100, B=2):
        return f(FAKE, FAKE, ctypes.c_int64(npages), ps, table, maxp, FAKE, _p(cu), B, 8, 2, 64,
                 128, 64, ctypes.c_float(0.0), FAKE, None, FAKE, ctypes.c_size_t(1 << 40), None)

    assert call(ps=24) == UP_EUNSUPPORTED          # not a power of two
    assert call(ps=8) == UP_EUNSUPPORTED           # below 16
    assert call(ps=2048) == UP_EUNSUPPORTED
    assert call(maxp=62) == UP_EINVAL              # 1000 tokens need 63 pages of 16
    assert call(table=None) == UP_EINVAL
    assert call(npages=0) == UP_EINVAL
    assert call(npages=-1) == UP_EINVAL


def test_block_scores_lse_paged_rejects_bad_arguments(L):
    cu = _cu([1000, 24])
    f = L.up_block_scores_lse_paged

    def call(ps=16, maxp=63, table=FAKE, npages=100, lse=FAKE, wsb=1 << 40):
        return f(FAKE, FAKE, ctypes.c_int64(npages), ps, table, maxp, lse, FAKE, _p(cu), 2, 8, 2,
                 64, 128, 64, ctypes.c_float(0.0), FAKE, FAKE, ctypes.c_size_t(wsb), None)

    assert call(ps=24) == UP_EUNSUPPORTED
    assert call(maxp=62) == UP_EINVAL
    assert call(table=None) == UP_EINVAL
    assert call(npages=0) == UP_EINVAL
    assert call(lse=None) == UP_EINVAL
    assert call(lse=ctypes.c_void_p(0x100002)) == UP_EINVAL
    assert call(wsb=16) == UP_EWORKSPACE


def test_rope_attention_workspace_and_arguments(L):
    f = L.up_rope_attention_workspace
    f.restype = ctypes.c_size_t
    cu = _cu([100, 0, 64, 1])
    Rp = 128 + 0 + 64 + 64
    ws = f(_p(cu), 4, 8, 2, 128)
    # rotated q (Hq) and k (Hkv), transposed v (Hkv), all over 64-row padded requests
    assert ws >= (8 + 2 + 2) * Rp * 128 * 2 and ws % 256 == 0
    assert f(_p(cu), 4, 8, 2, 192) == 0      # d unsupported
    assert f(_p(cu), 4, 8, 2, 256) >= (8 + 2 + 2) * Rp * 256 * 2   # d = 256 supported
    assert f(_p(cu), 4, 8, 3, 128) == 0      # Hq % Hkv
    bad = _cu([5, 3])
    bad[1] = 9; bad[2] = 4                   # decreasing offsets
    assert f(_p(bad), 2, 8, 2, 128) == 0
    a = L.up_rope_attention
    a.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 4 + [ctypes.c_float] * 2 + \
                 [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    dummy = ctypes.c_void_p(4096)
    args = lambda **kw: dict(dict(q=dummy, k=dummy, v=dummy, pos=dummy, cu=dummy, cu_h=_p(cu),
                                  B=4, Hq=8, Hkv=2, d=128, scale=0.0, theta=500000.0, out=dummy,
                                  ws=None, wsb=0, st=None), **kw)
    call = lambda kw: a(*args(**kw).values())
    assert call(dict(d=96)) == UP_EUNSUPPORTED
    assert call(dict(theta=1.0)) == UP_EINVAL
    assert call(dict(q=None)) == UP_EINVAL
    assert call(dict(out=ctypes.c_void_p(4098))) == UP_EINVAL     # misaligned
    assert call(dict()) == UP_EWORKSPACE                         # no workspace
    assert call(dict(ws=ctypes.c_void_p(4096), wsb=ws - 1)) == UP_EWORKSPACE
    assert call(dict(B=0, cu_h=_p(np.zeros(1, np.int32)))) == UP_OK   # nothing to do


@pytest.fixture(scope="module")
def LL():
    from block_wise_token_amd._binding import layer_lib
    return layer_lib()


LAYER_HEADER = os.path.join(ROOT, "include", "uniprefill_layer.h")


def test_layer_library_exports_its_header_and_decision_library_links_no_blas(LL):
    text = re.sub(r"/\*.*?\*/", "", open(LAYER_HEADER).read(), flags=re.S)
    syms = sorted(set(re.findall(r"\b(up_[a-z0-9_]+)\s*\(", text)))
    assert syms == ["up_linear", "up_swiglu_ffn", "up_swiglu_ffn_workspace"]
    for s_ in syms:
        assert hasattr(LL, s_)
    # the decision library needs no vendor GEMM library
    import subprocess
    from block_wise_token_amd._binding import LIB_PATH
    out = subprocess.run(["readelf", "-d", LIB_PATH], capture_output=True, text=True).stdout
    needed = re.findall(r"NEEDED.*\[(.*?)\]", out)
    assert needed and not [n for n in needed if "blas" in n.lower()], needed


def test_linear_swiglu_ffn_reject_bad_arguments(L, LL):
    L_gate = L
    L = LL
    L.up_linear.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_size_t, ctypes.c_void_p]
    d = ctypes.c_void_p(4096)
    assert L.up_linear(d, d, None, -1, 16, 16, d, None, 0, None) == UP_EINVAL
    assert L.up_linear(d, d, None, 8, 0, 16, d, None, 0, None) == UP_EINVAL
    assert L.up_linear(None, d, None, 8, 16, 16, d, None, 0, None) == UP_EINVAL
    assert L.up_linear(d, d, None, 8, 16, 16, d, None, 64, None) == UP_EINVAL   # bytes, no ptr
    assert L.up_linear(d, d, None, 8, 16, 16, d, ctypes.c_void_p(4100), 64, None) == UP_EWORKSPACE
    assert L.up_linear(d, d, None, 0, 16, 16, d, None, 0, None) == UP_OK
    L_gate.up_swiglu.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    assert L_gate.up_swiglu(d, 4, 12, d, None) == UP_EUNSUPPORTED               # F % 8
    assert L_gate.up_swiglu(None, 4, 16, d, None) == UP_EINVAL
    L.up_swiglu_ffn_workspace.restype = ctypes.c_size_t
    L.up_swiglu_ffn_workspace.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    w = L.up_swiglu_ffn_workspace(1000, 4096, 14336)
    assert w >= 1000 * 3 * 14336 * 2 and w % 256 == 0
    L.up_swiglu_ffn.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_void_p, ctypes.c_void_p,
                                                        ctypes.c_size_t, ctypes.c_void_p]
    assert L.up_swiglu_ffn(d, d, d, None, 1000, 4096, 14336, d, d, w - 1, None) == UP_EWORKSPACE
    assert L.up_swiglu_ffn(d, d, d, None, 1000, 4096, 14330, d, d, w, None) == UP_EUNSUPPORTED
    # operands of 2^32 elements or more are refused before any launch
    assert L.up_linear(d, d, None, 1 << 20, 4096, 4096, d, None, 0, None) == UP_EUNSUPPORTED
    assert L.up_linear(d, d, None, 149797, 4096, 28672, d, None, 0, None) == UP_EUNSUPPORTED
    assert L.up_swiglu_ffn(d, d, d, None, 220884, 4096, 14336, d, d, 1 << 62, None) == \
        UP_EUNSUPPORTED
    # the largest layer that has run: 131,072 rows at width 15,360 (4.03e9 elements)
    big = L.up_swiglu_ffn_workspace(131072, 3840, 15360)
    assert L.up_swiglu_ffn(d, d, d, None, 131072, 3840, 15360, d, d, big - 1, None) == \
        UP_EWORKSPACE


def test_layer_decision_workspace_and_arguments(L):
    f = L.up_layer_decision_workspace
    f.restype = ctypes.c_size_t
    cu = _cu([131072])
    ws = f(_p(cu), 1, 32, 8, 128, 128, 64)
    # the score workspace, the compaction workspace and one int32 per block (the fused
    # select's request index), 256-byte aligned
    L.up_block_scores_workspace.restype = ctypes.c_size_t
    L.up_expand_compact_workspace.restype = ctypes.c_size_t
    nb = 131072 // 64
    parts = (L.up_block_scores_workspace(_p(cu), 1, 32, 8, 128, 128, 64) +
             L.up_expand_compact_workspace(_p(cu), 1, 64) + (nb * 4 + 255) // 256 * 256)
    assert ws == parts and ws % 256 == 0
    assert f(_p(cu), 1, 32, 8, 96, 128, 64) == 0      # d unsupported
    a = L.up_layer_decision
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    a.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, cf, vp, ci, ci, vp, vp, vp, vp, vp,
                  vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    d = ctypes.c_void_p(4096)
    base = dict(qwin=d, k=d, cu=d, cu_h=_p(cu), B=1, Hq=32, Hkv=8, dd=128, n=128, G=64, scale=0.0,
                p=0.99, hidden=d, H=4096, eb=2, pos=d, prev=None, scores=d, keep=d, cu_out=d,
                idx=d, hout=d, pos_out=d, orig=None, ws=None, wsb=0, st=None)
    call = lambda **kw: a(*dict(base, **kw).values())
    assert call(p=0.0) == UP_EINVAL
    assert call(p=1.5) == UP_EINVAL
    assert call(H=0) == UP_EINVAL
    assert call(dd=96) == UP_EUNSUPPORTED
    assert call() == UP_EWORKSPACE                               # no workspace
    assert call(ws=ctypes.c_void_p(4096), wsb=ws - 1) == UP_EWORKSPACE
    assert call(ws=ctypes.c_void_p(4096), wsb=ws, scores=None) == UP_EINVAL
    assert call(ws=ctypes.c_void_p(4096), wsb=ws, orig=d) == UP_EINVAL   # orig_out without prev_orig
    assert call(ws=ctypes.c_void_p(4096), wsb=ws, pos=None) == UP_EINVAL  # pos_out without pos
    assert call(B=0, cu_h=_p(np.zeros(1, np.int32))) == UP_OK


def test_rope_attention_rejects_more_than_65535_tiles(L):
    """Workgroup tiles are the grid's y dimension: 65535 tiles are accepted, one more is
    UP_EUNSUPPORTED.  With 4 query heads per kv head a tile is one token tile per
    head: 64 tokens for the 8-wave kernel (d = 64, 128 with at most 256 kv heads), 32
    for the 4-wave kernel (d = 256, or more kv heads); with one query head per kv head
    a tile spans 4 token tiles."""
    f = L.up_rope_attention_workspace
    f.restype = ctypes.c_size_t
    for d, tok in ((64, 64), (128, 64), (256, 32)):
        assert f(_p(_cu([tok * 65535])), 1, 8, 2, d) > 0
        assert f(_p(_cu([tok * 65535 + 1])), 1, 8, 2, d) == 0
    assert f(_p(_cu([256 * 65535])), 1, 2, 2, 128) > 0
    assert f(_p(_cu([256 * 65535 + 1])), 1, 2, 2, 128) == 0
    assert f(_p(_cu([32 * 65535])), 1, 2048, 512, 128) > 0     # 512 kv heads: 4-wave kernel
    assert f(_p(_cu([32 * 65535 + 1])), 1, 2048, 512, 128) == 0
    a = L.up_rope_attention
    a.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 4 + [ctypes.c_float] * 2 + \
                 [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    d = ctypes.c_void_p(4096)
    cu = _cu([64 * 65535 + 1])
    assert a(d, d, d, d, d, _p(cu), 1, 8, 2, 128, 0.0, 500000.0, d, None, 0, None) == UP_EUNSUPPORTED


def test_rope_attention_scores_sizes_and_rejections(L):
    """up_rope_attention_scores: the workspace holds the attention's and the score
    pass's; unsupported block sizes and head dimensions, a missing scores pointer and a
    short workspace are refused before any launch."""
    f = L.up_rope_attention_scores_workspace
    f.restype = ctypes.c_size_t
    cu = _cu([131072])
    att = L.up_rope_attention_workspace
    att.restype = ctypes.c_size_t
    sw = L.up_block_scores_workspace(_p(cu), 1, 32, 8, 128, 128, 64)
    assert f(_p(cu), 1, 32, 8, 128, 128, 64) >= att(_p(cu), 1, 32, 8, 128) + sw
    assert f(_p(cu), 1, 32, 8, 128, 128, 48) == 0      # G not a multiple of 32
    assert f(_p(cu), 1, 32, 8, 96, 128, 64) == 0       # d unsupported
    assert f(_p(cu), 1, 32, 8, 128, 0, 64) == 0        # n = 0
    a = L.up_rope_attention_scores
    a.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 4 + [ctypes.c_float] * 2 + \
                 [ctypes.c_int] * 2 + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]
    c4 = _cu([4096])

    def call(n=128, G=64, scores=FAKE, ws=FAKE, wsb=1 << 40, d=128):
        return a(FAKE, FAKE, FAKE, FAKE, FAKE, _p(c4), 1, 8, 2, d, 0.0, 500000.0, n, G, FAKE,
                 scores, None, ws, ctypes.c_size_t(wsb), None)

    assert call(n=0) == UP_EINVAL
    assert call(G=48) == UP_EUNSUPPORTED
    assert call(d=80) == UP_EUNSUPPORTED
    assert call(scores=None) == UP_EINVAL
    assert call(wsb=16) == UP_EWORKSPACE
    assert call(ws=None) == UP_EWORKSPACE
