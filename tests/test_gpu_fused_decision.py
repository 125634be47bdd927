"""GPU: up_layer_decision (the whole decision in one call) against the three separate
calls on the same inputs: every output must be bit-identical (scores, keep flags,
cu_seqlens_out, indices, rows, positions, composed original indices).  The one call
currently makes the three calls itself: its fused select path (normalisation and
block destinations inside the select kernel) is switched off, see
test_fused_select_path.  (The other GPU tests reach the one call through
LayerDecision and compare it with the oracle.)"""
import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from tests.gpu_helpers import GpuBatch, say
from workloads import synth

pytestmark = pytest.mark.gpu


def _batch(lengths, Hq, Hkv, d, n, G, seed, zero_q=False):
    reqs = [synth.gen_request(L, Hq, Hkv, d, n, G, 2,
                              np.random.default_rng([seed, synth.TAG_VARLEN_REQUEST, i]))
            for i, L in enumerate(lengths)]
    b = synth.pack(reqs, Hq, Hkv, d, n, G)
    if zero_q:
        b.qwin[:] = 0
    return b


def _both(gb, p, H_prev=None):
    b = gb.b
    T = b.T
    prev = torch.from_numpy(np.random.default_rng(1).permutation(T * 2)[:T].astype(np.int32)).cuda()
    outs = []
    for separate in (False, True):
        dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, p,
                               prev_orig=prev, separate=separate)
        assert dec.one_call == (not separate)
        dec.run()
        torch.cuda.synchronize()
        assert up.device_error() == 0
        outs.append(dec)
    return outs


def _assert_same(a, c):
    assert torch.equal(a.scores, c.scores)
    assert torch.equal(a.keep, c.keep)
    assert torch.equal(a.cu_out, c.cu_out)
    kept = int(a.cu_out[-1].item())
    for name in ("idx", "hidden_out", "pos_out", "orig"):
        assert torch.equal(getattr(a, name)[:kept], getattr(c, name)[:kept]), name
    return kept


CASES = [
    # lengths, Hq, Hkv, d, n, G, p, zero queries
    ([4096], 8, 2, 64, 128, 64, 0.99, False),
    ([1000], 4, 2, 64, 128, 64, 0.9, False),          # ragged last block
    ([50], 4, 2, 64, 128, 64, 0.5, False),            # L < n: all in the window
    ([3000], 8, 2, 128, 128, 64, 1.0, False),         # p = 1 keeps everything
    ([20000], 8, 2, 64, 128, 64, 0.97, True),         # exact ties at the cut
    ([5000], 16, 2, 128, 256, 32, 0.99, False),       # G = 32
    ([262144], 8, 2, 64, 128, 64, 0.95, False),       # exactly 4096 blocks: the fused limit
    ([262208], 8, 2, 64, 128, 64, 0.95, False),       # 4097 blocks: the separate calls
    ([129, 0, 3000, 64, 1], 8, 2, 128, 128, 64, 0.97, False),   # several requests
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_one_call_equals_the_separate_calls(case):
    lengths, Hq, Hkv, d, n, G, p, zq = case
    say(f"[case] one call vs separate {case}")
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=len(lengths) + G, zero_q=zq)
    gb = GpuBatch(b, H=64)
    a, c = _both(gb, p)
    kept = _assert_same(a, c)
    say(f"[ok] {case}: {kept} of {b.T} tokens kept")


@pytest.mark.timeout(600)
def test_one_call_equals_the_separate_calls_at_128k():
    cfg = synth.WORKLOADS["llama31_8b_128k"]
    say("[setup] generating llama31_8b_128k")
    b = synth.make_batch(cfg)
    gb = GpuBatch(b, H=cfg["H"])
    a, c = _both(gb, cfg["p"])
    kept = _assert_same(a, c)
    say(f"[ok] 128K: {kept} kept, identical outputs")


def test_one_call_with_inconsistent_device_cu_writes_nothing():
    """A valid decision, then one whose device cu_seqlens disagrees with the host copy:
    the second raises error bit 1, writes cu_seqlens_out = 0 and moves no row (the
    compaction header left by the first call is cleared)."""
    b = _batch([4096], 8, 2, 64, 128, 64, seed=3)
    gb = GpuBatch(b, H=64)
    dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, 0.9)
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0 and int(dec.cu_out[-1].item()) > 0
    dec.cu.copy_(torch.tensor([0, 4000], dtype=torch.int32))
    dec.hidden_out.fill_(3.0)
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() & 1
    assert dec.cu_out.cpu().numpy().tolist() == [0, 0]
    assert bool((dec.hidden_out == 3.0).all())


@pytest.mark.skip(reason="the fused select path of up_layer_decision is switched off "
                         "(kFusedSelect = false): a benchmark run that first used it, together "
                         "with the 8-wave attention kernel, left the GPU faulted and no cause "
                         "has been shown; the path stays off the GPU until one is")
def test_fused_select_path():
    """Would compare the fused select path (masses normalised and block destinations
    assigned inside the select kernel) with the separate calls, bit for bit."""
