"""GPU: up_layer_decision (the whole decision in one call) against the three separate
calls on the same inputs: every output must be bit-identical (scores, keep flags,
cu_seqlens_out, indices, rows, positions, composed original indices).  When no request
has more than 4096 blocks the one call normalises and assigns block destinations
inside the select kernel (the fused path; several requests also take a finalize
launch that scans the kept counts and makes the destinations absolute); otherwise it
makes the three calls.  (The other GPU tests reach the one call through LayerDecision
and compare it with the oracle.)"""
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
    ([50000], 8, 2, 64, 128, 64, 0.99, False),        # 782 blocks: four select slots per thread
    ([262144], 8, 2, 64, 128, 64, 0.95, False),       # exactly 4096 blocks: the fused limit
    ([262208], 8, 2, 64, 128, 64, 0.95, False),       # 4097 blocks: the separate calls
    ([129, 0, 3000, 64, 1], 8, 2, 128, 128, 64, 0.97, False),   # several requests
    ([262144, 700, 0, 9000], 8, 2, 64, 128, 64, 0.95, False),   # 4096 blocks beside others
    ([262208, 700, 9000], 8, 2, 64, 128, 64, 0.95, False),      # one of 4097: separate calls
    ([40000, 40000, 12345], 8, 2, 64, 128, 64, 0.99, True),     # ties, several requests
    ([0, 0, 5000, 0], 4, 2, 64, 128, 64, 0.9, False),           # empty requests around one
    (list(np.random.default_rng(77).integers(0, 400, 1500)), 4, 2, 64, 128, 64, 0.9,
     False),                                                    # 1500 requests: scan > 1024
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_one_call_equals_the_separate_calls(case):
    lengths, Hq, Hkv, d, n, G, p, zq = case
    lengths = [int(x) for x in lengths]
    shown = lengths if len(lengths) <= 8 else f"{len(lengths)} requests"
    say(f"[case] one call vs separate {shown} Hq={Hq} Hkv={Hkv} d={d} n={n} G={G} p={p}")
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=len(lengths) + G, zero_q=zq)
    gb = GpuBatch(b, H=64)
    a, c = _both(gb, p)
    kept = _assert_same(a, c)
    say(f"[ok] {shown}: {kept} of {b.T} tokens kept")


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


def test_one_call_with_inconsistent_device_cu_writes_nothing_several_requests():
    """As above for a pack of three requests (the fused finalize path): the second call's
    device cu_seqlens disagrees with the host copy, so it raises error bit 1, writes
    cu_seqlens_out = 0 and moves no row."""
    b = _batch([3000, 5000, 200], 8, 2, 64, 128, 64, seed=4)
    gb = GpuBatch(b, H=64)
    dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, 0.9)
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0 and int(dec.cu_out[-1].item()) > 0
    dec.cu.copy_(torch.tensor([0, 3000, 7900, 8200], dtype=torch.int32))
    dec.hidden_out.fill_(3.0)
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() & 1
    assert dec.cu_out.cpu().numpy().tolist() == [0, 0, 0, 0]
    assert bool((dec.hidden_out == 3.0).all())


def _fused_launches(gb, p):
    """Launches of the fused select kernel in one up_layer_decision call."""
    b = gb.b
    dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, p)
    up.profile_reset()
    up.profile_enable(True)
    dec.run()
    torch.cuda.synchronize()
    up.profile_enable(False)
    n, _ = up.profile_read("select_fused")
    up.profile_reset()
    assert up.device_error() == 0
    return n


def test_fused_select_path():
    """Requests of at most 4096 blocks each: up_layer_decision normalises the block
    masses and assigns the compaction's block destinations inside the select kernel
    (one launch instead of three for one request, two instead of four for several);
    every output is bit-identical to the separate calls (see
    test_one_call_equals_the_separate_calls for the case list)."""
    b = _batch([4096], 8, 2, 64, 128, 64, seed=5)
    gb = GpuBatch(b, H=64)
    assert _fused_launches(gb, 0.99) == 1
    big = _batch([262208], 8, 2, 64, 128, 64, seed=6)   # 4097 blocks: the separate calls
    assert _fused_launches(GpuBatch(big, H=64), 0.95) == 0
    a, c = _both(gb, 0.99)
    _assert_same(a, c)
    # several requests of at most 4096 blocks each: the fused path too
    many = GpuBatch(_batch([3000, 0, 262144, 64], 8, 2, 64, 128, 64, seed=7), H=64)
    assert _fused_launches(many, 0.95) == 1
    a, c = _both(many, 0.95)
    _assert_same(a, c)
    mixed = _batch([3000, 262208, 64], 8, 2, 64, 128, 64, seed=8)   # one of 4097 blocks
    assert _fused_launches(GpuBatch(mixed, H=64), 0.95) == 0


@pytest.mark.timeout(600)
def test_fused_select_beside_another_stream():
    """Regression test of the select kernel's pass loop: a wave must not read the
    shared winning-bin index after the pass's last barrier (the next pass resets it).
    Waves of one select workgroup drift apart most when they share SIMDs with another
    kernel's waves, so fused decisions run here while independent decisions on a
    second stream keep the CUs busy with score passes; every repetition's outputs must
    equal the separate calls' bit for bit."""
    cfg = synth.WORKLOADS["llama31_8b_128k"]
    say("[setup] generating llama31_8b_128k")
    b = synth.make_batch(cfg)
    gb = GpuBatch(b, H=cfg["H"])
    ref = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G,
                           cfg["p"], separate=True)
    ref.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    kept = int(ref.cu_out[-1].item())
    da = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, cfg["p"])
    db = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, cfg["p"])
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    say("[case] fused decisions on two streams, 40 repetitions")
    for rep in range(40):
        da.hidden_out.zero_()
        torch.cuda.synchronize()
        for j in range(3):
            db.run(stream=sb)
            da.run(stream=sa)
        torch.cuda.synchronize()
        assert up.device_error() == 0, f"device error at repetition {rep}"
        for name in ("scores", "keep", "cu_out"):
            assert torch.equal(getattr(da, name), getattr(ref, name)), (rep, name)
        for name in ("idx", "pos_out", "orig"):
            assert torch.equal(getattr(da, name)[:kept], getattr(ref, name)[:kept]), (rep, name)
        assert torch.equal(da.hidden_out[:kept].view(torch.int16),
                           ref.hidden_out[:kept].view(torch.int16)), rep
    say("[ok] 40 repetitions identical")
