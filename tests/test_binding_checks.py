"""CPU: the Python binding refuses buffers too small for what the library would write
or read through them, before any library call.

The library is replaced by a stand-in whose workspace-size queries answer a fixed
size and whose compute entry points fail the test if reached; the device check is
relaxed to accept CPU tensors, so only the shape and size checks are exercised."""
import numpy as np
import pytest
import torch

from block_wise_token_amd import _binding as bd

WS = 4096


class _StubLib:
    def __getattr__(self, name):
        if name.endswith("_workspace"):
            return lambda *a: WS
        if name == "up_status_string":
            return lambda st: b"stub"

        def reached(*a):
            raise _Reached(name)
        return reached


class _Reached(Exception):
    pass


@pytest.fixture(autouse=True)
def stub(monkeypatch):
    def dev(t, dtype, name):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t
    monkeypatch.setattr(bd, "lib", lambda: _StubLib())
    monkeypatch.setattr(bd, "layer_lib", lambda: _StubLib())
    monkeypatch.setattr(bd, "_dev", dev)
    monkeypatch.setattr(bd, "_stream", lambda s=None: 0)


BF, F32, I32, U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8
CU = np.array([0, 1000, 1300], dtype=np.int32)      # T = 1300; W = 128 + 128
N, G, HQ, HKV, D = 128, 64, 8, 2, 64
NBT = 16 + 5                                         # ceil(1000/64) + ceil(300/64)


def _scores_args():
    return (torch.zeros(256, HQ, D, dtype=BF), torch.zeros(1300, HKV, D, dtype=BF),
            torch.tensor(CU), CU, N, G)


def test_block_scores_accepts_exact_sizes():
    qwin, k, cu, cu_h, n, g = _scores_args()
    with pytest.raises(_Reached, match="up_block_scores"):
        bd.block_scores(qwin, k, cu, cu_h, n, g, out=torch.zeros(NBT, dtype=F32),
                        workspace=torch.zeros(WS, dtype=U8),
                        row_lse=torch.zeros(256 * HQ, dtype=F32))


@pytest.mark.parametrize("bad", ["out", "workspace", "row_lse", "qwin_rows", "k_rows", "k_dim"])
def test_block_scores_rejects_short_buffers(bad):
    qwin, k, cu, cu_h, n, g = _scores_args()
    kw = dict(out=torch.zeros(NBT, dtype=F32), workspace=torch.zeros(WS, dtype=U8),
              row_lse=torch.zeros(256 * HQ, dtype=F32))
    if bad in kw:
        kw[bad] = kw[bad][:-1].contiguous()
    elif bad == "qwin_rows":
        qwin = qwin[:-1].contiguous()
    elif bad == "k_rows":
        k = k[:-1].contiguous()
    else:
        k = torch.zeros(1300, HKV, D * 2, dtype=BF)
    name = {"qwin_rows": "qwin has", "k_rows": "k has", "k_dim": "head dimension"}.get(bad, bad)
    with pytest.raises(ValueError, match=name):
        bd.block_scores(qwin, k, cu, cu_h, n, g, **kw)


def test_block_scores_lse_needs_row_lse_rows():
    qwin, k, cu, cu_h, n, g = _scores_args()
    with pytest.raises(ValueError, match="row_lse"):
        bd.block_scores_lse(qwin, k, torch.zeros(256 * HQ - 1, dtype=F32), cu, cu_h, n, g)


def test_block_scores_paged_checks_table_and_out():
    qwin, _, cu, cu_h, n, g = _scores_args()
    pages = torch.zeros(30, 64, HKV, D, dtype=BF)
    with pytest.raises(ValueError, match="block_table"):
        bd.block_scores_paged(qwin, pages, torch.zeros(1, 20, dtype=I32), cu, cu_h, n, g)
    with pytest.raises(ValueError, match="out"):
        bd.block_scores_paged(qwin, pages, torch.zeros(2, 20, dtype=I32), cu, cu_h, n, g,
                              out=torch.zeros(NBT - 1, dtype=F32))


@pytest.mark.parametrize("fn,arg", [(bd.topp_select, 0.9), (bd.topk_select, 3)])
def test_select_rejects_short_buffers(fn, arg):
    cu = torch.tensor(CU)
    s = torch.zeros(NBT, dtype=F32)
    with pytest.raises(ValueError, match="scores"):
        fn(s[:-1].contiguous(), cu, CU, N, G, arg)
    with pytest.raises(ValueError, match="keep"):
        fn(s, cu, CU, N, G, arg, keep=torch.zeros(NBT - 1, dtype=U8))
    with pytest.raises(ValueError, match="cu_seqlens_out"):
        fn(s, cu, CU, N, G, arg, cu_out=torch.zeros(2, dtype=I32))
    with pytest.raises(_Reached):
        fn(s, cu, CU, N, G, arg)


@pytest.mark.parametrize("bad", ["hidden", "keep", "pos", "idx_out", "hidden_out", "pos_out",
                                 "prev_orig", "orig_out", "workspace"])
def test_expand_compact_rejects_short_buffers(bad):
    T, H = 1300, 32
    t = dict(hidden=torch.zeros(T, H, dtype=BF), pos=torch.zeros(T, dtype=I32),
             keep=torch.zeros(NBT, dtype=U8), idx_out=torch.zeros(T, dtype=I32),
             hidden_out=torch.zeros(T, H, dtype=BF), pos_out=torch.zeros(T, dtype=I32),
             prev_orig=torch.zeros(T, dtype=I32), orig_out=torch.zeros(T, dtype=I32),
             workspace=torch.zeros(WS, dtype=U8))
    t[bad] = t[bad][:-1].contiguous()
    cu, cu_out = torch.tensor(CU), torch.zeros(3, dtype=I32)
    name = {"keep": "keep_blocks"}.get(bad, bad)
    with pytest.raises(ValueError, match=name):
        bd.expand_compact(t["hidden"], t["pos"], t["keep"], cu, cu_out, CU, G,
                          idx_out=t["idx_out"], hidden_out=t["hidden_out"], pos_out=t["pos_out"],
                          workspace=t["workspace"], prev_orig=t["prev_orig"],
                          orig_out=t["orig_out"])


def test_expand_compact_accepts_exact_sizes():
    T, H = 1300, 32
    with pytest.raises(_Reached, match="up_expand_compact"):
        bd.expand_compact(torch.zeros(T, H, dtype=BF), torch.zeros(T, dtype=I32),
                          torch.zeros(NBT, dtype=U8), torch.tensor(CU), torch.zeros(3, dtype=I32),
                          CU, G, prev_orig=torch.zeros(T, dtype=I32))


def test_compose_drops_checks_capacity():
    prev, cnt = torch.zeros(100, dtype=I32), torch.zeros(1, dtype=I32)
    with pytest.raises(ValueError, match="idx"):
        bd.compose_drops(prev, torch.zeros(50, dtype=I32), cnt, capacity=60)
    with pytest.raises(ValueError, match="out"):
        bd.compose_drops(prev, torch.zeros(50, dtype=I32), cnt, out=torch.zeros(49, dtype=I32))
    with pytest.raises(_Reached):
        bd.compose_drops(prev, torch.zeros(50, dtype=I32), cnt)


def test_layer_decision_checks_inputs():
    qwin, k, cu, cu_h, n, g = _scores_args()
    hid, pos = torch.zeros(1300, 16, dtype=BF), torch.zeros(1300, dtype=I32)
    with pytest.raises(ValueError, match="hidden"):
        bd.LayerDecision(qwin, k, cu, cu_h, hid[:-1].contiguous(), pos, n, g, 0.9)
    with pytest.raises(ValueError, match="prev_orig"):
        bd.LayerDecision(qwin, k, cu, cu_h, hid, pos, n, g, 0.9,
                         prev_orig=torch.zeros(1299, dtype=I32))
    with pytest.raises(ValueError, match="qwin"):
        bd.LayerDecision(qwin[:200].contiguous(), k, cu, cu_h, hid, pos, n, g, 0.9)


ATT_CU = np.array([0, 70, 200], dtype=np.int32)


@pytest.mark.parametrize("bad", ["q", "k", "v_shape", "pos", "out", "workspace"])
def test_rope_attention_rejects_mismatched_buffers(bad):
    R = 200
    t = dict(q=torch.zeros(R, 8, 64, dtype=BF), k=torch.zeros(R, 2, 64, dtype=BF),
             v=torch.zeros(R, 2, 64, dtype=BF), pos=torch.zeros(R, dtype=I32),
             out=torch.zeros(R, 8, 64, dtype=BF), workspace=torch.zeros(WS, dtype=U8))
    if bad == "v_shape":
        t["v"] = torch.zeros(R, 2, 128, dtype=BF)
    else:
        t[bad] = t[bad][:-1].contiguous()
    name = {"q": "q has", "k": "must both be", "v_shape": "must both be"}.get(bad, bad)
    with pytest.raises(ValueError, match=name):
        bd.rope_attention(t["q"], t["k"], t["v"], t["pos"], torch.tensor(ATT_CU), ATT_CU,
                          out=t["out"], workspace=t["workspace"])


def test_rope_attention_accepts_exact_sizes():
    R = 200
    with pytest.raises(_Reached, match="up_rope_attention"):
        bd.rope_attention(torch.zeros(R, 8, 64, dtype=BF), torch.zeros(R, 2, 64, dtype=BF),
                          torch.zeros(R, 2, 64, dtype=BF), torch.zeros(R, dtype=I32),
                          torch.tensor(ATT_CU), ATT_CU)


def test_linear_and_ffn_shape_checks():
    x = torch.zeros(10, 32, dtype=BF)
    with pytest.raises(ValueError, match="does not match"):
        bd.linear(x, torch.zeros(48, 31, dtype=BF))
    with pytest.raises(ValueError, match="out"):
        bd.linear(x, torch.zeros(48, 32, dtype=BF), out=torch.zeros(10, 47, dtype=BF))
    with pytest.raises(ValueError, match="residual"):
        bd.linear(x, torch.zeros(48, 32, dtype=BF), residual=torch.zeros(9, 48, dtype=BF))
    with pytest.raises(_Reached, match="up_linear"):
        bd.linear(x, torch.zeros(48, 32, dtype=BF))
    with pytest.raises(ValueError, match="gate"):
        bd.swiglu(torch.zeros(10, 33, dtype=BF))
    with pytest.raises(ValueError, match="out"):
        bd.swiglu(torch.zeros(10, 32, dtype=BF), out=torch.zeros(10, 15, dtype=BF))
    wgu, wd = torch.zeros(96, 32, dtype=BF), torch.zeros(32, 48, dtype=BF)
    with pytest.raises(ValueError, match="w_gu"):
        bd.swiglu_ffn(x, wgu, torch.zeros(32, 47, dtype=BF))
    with pytest.raises(ValueError, match="workspace"):
        bd.swiglu_ffn(x, wgu, wd, workspace=torch.zeros(WS - 1, dtype=U8))
    with pytest.raises(_Reached, match="up_swiglu_ffn"):
        bd.swiglu_ffn(x, wgu, wd)


def test_short_device_cu_seqlens_is_refused():
    """Every call reads B + 1 entries through the device cu_seqlens pointer."""
    qwin, k, _, cu_h, n, g = _scores_args()
    short = torch.tensor(CU[:-1])
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.block_scores(qwin, k, short, cu_h, n, g)
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.block_scores_lse(qwin, k, torch.zeros(256 * HQ, dtype=F32), short, cu_h, n, g)
    pages = torch.zeros(30, 64, HKV, D, dtype=BF)
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.block_scores_paged(qwin, pages, torch.zeros(2, 20, dtype=I32), short, cu_h, n, g)
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.block_scores_lse_paged(qwin, pages, torch.zeros(2, 20, dtype=I32),
                                  torch.zeros(256 * HQ, dtype=F32), short, cu_h, n, g)
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.topp_select(torch.zeros(NBT, dtype=F32), short, CU, N, G, 0.9)
    with pytest.raises(ValueError, match="cu_seqlens"):
        bd.expand_compact(torch.zeros(1300, 8, dtype=BF), None, torch.zeros(NBT, dtype=U8), short,
                          torch.zeros(3, dtype=I32), CU, G)
