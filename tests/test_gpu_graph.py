"""GPU: the library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed.

Every call is asynchronous on the caller's stream and allocates nothing once its
buffers exist, so a decision (or the rotary attention) can be captured once and
replayed.  Each test captures after an eager warm-up, then replays several times;
before every replay the outputs are overwritten with sentinels and an unrelated
eager decision runs and is synchronised, and after it every output must equal the
eager result bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from tests.gpu_helpers import GpuBatch, bf16_dev, i32_dev, say
from workloads import synth

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _batch(lengths, Hq, Hkv, d, n, G, seed):
    reqs = [synth.gen_request(L, Hq, Hkv, d, n, G, 2,
                              np.random.default_rng([seed, synth.TAG_VARLEN_REQUEST, i]))
            for i, L in enumerate(lengths)]
    return synth.pack(reqs, Hq, Hkv, d, n, G)


def _outputs(dec):
    kept = int(dec.cu_out[-1].item())
    return dict(scores=dec.scores.clone(), keep=dec.keep.clone(), cu_out=dec.cu_out.clone(),
                idx=dec.idx[:kept].clone(), hidden_out=dec.hidden_out[:kept].clone(),
                pos_out=dec.pos_out[:kept].clone(), orig=dec.orig[:kept].clone())


def _scribble(dec):
    dec.scores.fill_(-1.0)
    dec.keep.fill_(7)
    dec.cu_out.fill_(-5)
    dec.idx.fill_(-9)
    dec.hidden_out.fill_(3.0)
    dec.pos_out.fill_(-9)
    dec.orig.fill_(-9)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                       # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


CASES = [
    # lengths, Hq, Hkv, d, n, G, p, topk, label
    ([4096], 8, 2, 64, 128, 64, 0.99, None, "one call, single 4K request"),
    ([1000, 0, 3000, 64, 129], 8, 2, 128, 128, 64, 0.6, None, "one call, five requests"),
    ([5000], 8, 2, 128, 128, 32, 0.95, 20, "separate calls, Top-k"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[-1].replace(" ", "_").replace(",", "")
                                             for c in CASES])
def test_decision_replays_match_eager(case):
    lengths, Hq, Hkv, d, n, G, p, topk, label = case
    say(f"[case] graph replay: {label}")
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=len(lengths) + G)
    gb = GpuBatch(b, H=96)
    T = b.T
    prev = i32_dev(np.random.default_rng(2).permutation(2 * T)[:T].astype(np.int32))
    dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, n, G, p,
                           prev_orig=prev, topk=topk)
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    want = _outputs(dec)
    # an unrelated decision, run eagerly between the replays
    ob = _batch([3000], 8, 2, 64, 128, 64, seed=99)
    og = GpuBatch(ob, H=32)
    other = up.LayerDecision(og.qwin, og.k, og.cu, og.cu_h, og.hidden, og.pos, 128, 64, 0.9)
    g = _capture(dec.run)
    for r in range(REPLAYS):
        _scribble(dec)
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert up.device_error() == 0
        got = _outputs(dec)
        for name, w in want.items():
            assert torch.equal(got[name], w), f"replay {r}: {name} differs"
    say(f"[ok] {label}: {REPLAYS} replays equal the eager decision "
        f"({int(want['cu_out'][-1])} of {T} tokens kept)")


def test_rope_attention_replays_match_eager():
    lengths, Hq, Hkv, d = [300, 0, 65, 129], 8, 2, 128
    say("[case] graph replay: rotary attention")
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, 7)
    R = int(cu[-1])
    args = (bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d), bf16_dev(v).view(R, Hkv, d),
            i32_dev(pos), i32_dev(cu), cu)
    ws = torch.empty(up.rope_attention_workspace_bytes(cu, Hq, Hkv, d), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((R, Hq, d), dtype=torch.bfloat16, device="cuda")

    def run():
        up.rope_attention(*args, scale=1.0 / math.sqrt(d), out=out, workspace=ws)
    run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    want = out.clone()
    g = _capture(run)
    for r in range(REPLAYS):
        out.fill_(0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert up.device_error() == 0
        assert torch.equal(out, want), f"replay {r} differs"
    say(f"[ok] rotary attention: {REPLAYS} replays equal the eager call")


def test_rope_attention_scores_replays_match_eager():
    """The attention with the window rows' block scores: its window tiles run on the
    library's second stream, forked from and joined back into the captured stream with
    events, so the graph holds both branches."""
    lengths, Hq, Hkv, d, n, G = [300, 0, 65, 129], 8, 2, 128, 128, 64
    say("[case] graph replay: rotary attention with block scores")
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, 8)
    R = int(cu[-1])
    args = (bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d), bf16_dev(v).view(R, Hkv, d),
            i32_dev(pos), i32_dev(cu), cu, n, G)
    ws = torch.empty(up.rope_attention_scores_workspace_bytes(cu, Hq, Hkv, d, n, G),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((R, Hq, d), dtype=torch.bfloat16, device="cuda")
    nb = sum((L + G - 1) // G for L in lengths)
    sc = torch.empty(nb, dtype=torch.float32, device="cuda")

    def run():
        up.rope_attention_scores(*args, out=out, scores=sc, workspace=ws)
    run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    want_out, want_sc = out.clone(), sc.clone()
    g = _capture(run)
    for r in range(REPLAYS):
        out.fill_(0.5)
        sc.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert up.device_error() == 0
        assert torch.equal(out, want_out), f"replay {r}: out differs"
        assert torch.equal(sc, want_sc), f"replay {r}: scores differ"
    say(f"[ok] rotary attention with block scores: {REPLAYS} replays equal the eager call")


def test_paged_score_passes_replay_match_eager():
    """Both paged score passes (row statistics computed, and given) in one graph, as a
    serving loop over a paged cache would capture them."""
    from tests.test_gpu_paged import _bf16, _paginate
    say("[case] graph replay: paged score passes")
    b = _batch([3000, 0, 1234], 8, 2, 128, 128, 64, seed=17)
    gb = GpuBatch(b)
    pages, table = _paginate(b.k, b.cu_seqlens, 32, seed=5)
    pg, tb = _bf16(pages), i32_dev(table)
    nbt = int(sum((int(L) + 63) // 64 for L in np.diff(b.cu_seqlens)))
    lse = torch.empty((b.qwin.shape[0], 8), dtype=torch.float32, device="cuda")
    s_full = torch.empty(nbt, dtype=torch.float32, device="cuda")
    s_given = torch.empty_like(s_full)
    ws = torch.empty(up.block_scores_workspace_bytes(b.cu_seqlens, 8, 2, 128, 128, 64),
                     dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(max(1, up.block_scores_lse_workspace_bytes(b.cu_seqlens, 8, 2, 128, 128, 64)),
                      dtype=torch.uint8, device="cuda")

    def run():
        up.block_scores_paged(gb.qwin, pg, tb, gb.cu, gb.cu_h, 128, 64, out=s_full, workspace=ws,
                              row_lse=lse)
        up.block_scores_lse_paged(gb.qwin, pg, tb, lse, gb.cu, gb.cu_h, 128, 64, out=s_given,
                                  workspace=ws2)
    run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    want = (s_full.clone(), lse.clone(), s_given.clone())
    g = _capture(run)
    for r in range(REPLAYS):
        s_full.fill_(-1.0)
        lse.fill_(-1.0)
        s_given.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert up.device_error() == 0
        for got, w, name in zip((s_full, lse, s_given), want, ("scores", "row_lse", "given")):
            assert torch.equal(got, w), f"replay {r}: {name} differs"
    say(f"[ok] paged score passes: {REPLAYS} replays equal the eager calls")
