"""GPU parity at full workload sizes, through the same LayerDecision path bench.py times.

* Llama-3.1-8B shape at 128K tokens, p in {0.95, 0.99, 0.999};
* the 8-request continuous-batching pack (8K-64K tokens each);
* the Gemma-3-12B-like d=256 stack: 4 successive decisions with fresh Q/K over the
  survivors, drops composed back to original positions.

Scores, keep flags, indices, positions, composed indices and every compacted hidden
row are compared in full.
"""
import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from oracle import uniprefill_oracle as O
from workloads import synth
from tests.gpu_helpers import (GpuBatch, ambiguous_blocks, bf16_dev, check_compaction, check_keep,
                               check_packed_equals_alone, check_rows, check_scores, i32_dev,
                               run_decision, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def llama128k():
    cfg = synth.WORKLOADS["llama31_8b_128k"]
    say("[setup] generating llama31_8b_128k")
    b = synth.make_batch(cfg)
    gb = GpuBatch(b, H=cfg["H"], seed=cfg["seed"])
    s32, s64, _ = O.block_scores(b.qwin, b.k, b.cu_seqlens, b.Hq, b.Hkv, b.d, b.n, b.G)
    return cfg, b, gb, s32, s64


@pytest.mark.timeout(600)
@pytest.mark.parametrize("p", [0.95, 0.99, 0.999])
def test_llama_128k_full_size(llama128k, p):
    cfg, b, gb, s32, s64 = llama128k
    say(f"[case] llama31_8b_128k p={p}")
    res = run_decision(gb, p)
    worst = check_scores(res["scores"], s64)
    ref_keep, _, _ = O.topp_select(s32, b.cu_seqlens, b.n, b.G, p)
    amb = ambiguous_blocks(s32, b.cu_seqlens, b.n, b.G, p)
    ndiff = check_keep(res["keep"], ref_keep, amb)
    own_keep, own_cu, _ = O.topp_select(res["scores"], b.cu_seqlens, b.n, b.G, p)
    np.testing.assert_array_equal(res["keep"], own_keep)
    np.testing.assert_array_equal(res["cu_out"], own_cu)
    check_compaction(gb, res)
    # every planted needle block and the window survive
    kept = set(np.nonzero(res["keep"])[0].tolist())
    assert set(b.needles[0].tolist()) <= kept
    assert set(O.window_blocks(b.T, b.n, b.G)) <= kept
    say(f"[ok] 128K p={p}: worst rel err {worst:.2e}, ambiguous {len(amb)}, differing {ndiff}, "
        f"kept {res['count']}/{b.T}")


@pytest.mark.timeout(600)
def test_varlen_pack_full_size():
    cfg = synth.WORKLOADS["varlen8_8k_64k"]
    say("[setup] generating varlen8_8k_64k")
    b = synth.make_batch(cfg)
    gb = GpuBatch(b, H=cfg["H"], seed=cfg["seed"])
    say(f"[case] varlen lengths {np.diff(b.cu_seqlens).tolist()}")
    res = run_decision(gb, cfg["p"])
    s32, s64, _ = O.block_scores(b.qwin, b.k, b.cu_seqlens, b.Hq, b.Hkv, b.d, b.n, b.G)
    worst = check_scores(res["scores"], s64)
    ref_keep, _, _ = O.topp_select(s32, b.cu_seqlens, b.n, b.G, cfg["p"])
    amb = ambiguous_blocks(s32, b.cu_seqlens, b.n, b.G, cfg["p"])
    ndiff = check_keep(res["keep"], ref_keep, amb)
    own_keep, own_cu, _ = O.topp_select(res["scores"], b.cu_seqlens, b.n, b.G, cfg["p"])
    np.testing.assert_array_equal(res["keep"], own_keep)
    np.testing.assert_array_equal(res["cu_out"], own_cu)
    check_compaction(gb, res)
    # packed == each request alone, bitwise (scores, keep flags, kept rows): a request's
    # results do not depend on the rest of the batch
    n_alone = check_packed_equals_alone(gb, res, cfg["p"])
    assert n_alone == b.B
    say(f"[ok] varlen: worst rel err {worst:.2e}, ambiguous {len(amb)}, differing {ndiff}, "
        f"kept {res['count']}/{b.T}")


@pytest.mark.timeout(900)
def test_four_layer_stack_composes_drops():
    cfg = synth.WORKLOADS["gemma3_12b_like_128k_4layers"]
    Hq, Hkv, d, n, G, p = cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["n"], cfg["G"], cfg["p"]
    say("[setup] generating gemma3_12b_like_128k_4layers layer 0")
    b0 = synth.make_batch(cfg)
    L0 = b0.T
    needles = b0.needles[0]
    hidden0 = synth.gen_hidden(L0, cfg["H"], cfg["seed"])
    pos0 = synth.positions(b0.cu_seqlens)
    hid = bf16_dev(hidden0)
    pos = i32_dev(pos0)
    orig_np = np.arange(L0, dtype=np.int32)
    orig = i32_dev(orig_np)
    for layer in range(cfg["layers"]):
        L = int(orig_np.size)
        if layer == 0:
            b = b0
        else:
            req = synth.gen_layer(orig_np, L0, needles, Hq, Hkv, d, n, G, cfg["seed"], layer)
            b = synth.pack([req], Hq, Hkv, d, n, G)
        say(f"[case] layer {layer}: L={L}")
        cu_h = np.array([0, L], np.int32)
        dec = up.LayerDecision(bf16_dev(b.qwin), bf16_dev(b.k), i32_dev(cu_h), cu_h, hid, pos, n,
                               G, p, prev_orig=orig)
        dec.run()
        torch.cuda.synchronize()
        assert up.device_error() == 0
        s_gpu = dec.scores.cpu().numpy()
        keep = dec.keep.cpu().numpy()
        s32, s64, _ = O.block_scores(b.qwin, b.k, cu_h, Hq, Hkv, d, n, G)
        worst = check_scores(s_gpu, s64)
        ref_keep, _, _ = O.topp_select(s32, cu_h, n, G, p)
        amb = ambiguous_blocks(s32, cu_h, n, G, p)
        check_keep(keep, ref_keep, amb)
        own_keep, _, _ = O.topp_select(s_gpu, cu_h, n, G, p)
        np.testing.assert_array_equal(keep, own_keep)
        # the oracle composes the GPU's decision: idx, then original indices
        idx = O.expand(keep, cu_h, G)
        cnt = int(dec.cu_out[-1].item())
        assert cnt == idx.size
        np.testing.assert_array_equal(dec.idx[:cnt].cpu().numpy(), idx)
        orig_next = O.compose(orig_np, idx) if idx.size < 4096 else orig_np[idx]
        np.testing.assert_array_equal(dec.orig[:cnt].cpu().numpy(), orig_next)
        # positions and hidden rows are those of the original tokens
        np.testing.assert_array_equal(dec.pos_out[:cnt].cpu().numpy(), pos0[orig_next])
        check_rows(dec.hidden_out[:cnt], hidden0, orig_next)
        # the last n tokens of the original sequence survive every layer
        assert np.array_equal(orig_next[-n:], np.arange(L0 - n, L0, dtype=np.int32))
        say(f"[ok] layer {layer}: worst rel err {worst:.2e}, kept {cnt}/{L}")
        # next layer's inputs: the survivors, compacted on the GPU
        hid = dec.hidden_out[:cnt].clone()
        pos = dec.pos_out[:cnt].clone()
        orig = dec.orig[:cnt].clone()
        orig_np = orig_next


@pytest.mark.timeout(900)
def test_largest_supported_request():
    """One request of 16384 blocks of 64 tokens (1,048,576 tokens, the selection
    limit): the full decision against the oracle (Hq=4, Hkv=2, d=64 keeps the oracle
    to about half a minute)."""
    L, Hq, Hkv, d, n, G, p = 16384 * 64, 4, 2, 64, 128, 64, 0.99
    say(f"[setup] generating one request of {L} tokens")
    req = synth.gen_request(L, Hq, Hkv, d, n, G, 16,
                            np.random.default_rng([11, synth.TAG_VARLEN_REQUEST, 0]))
    b = synth.pack([req], Hq, Hkv, d, n, G)
    gb = GpuBatch(b, H=256, seed=11)
    say("[case] largest request: decision")
    res = run_decision(gb, p)
    say("[case] largest request: oracle scores")
    s32, s64, _ = O.block_scores(b.qwin, b.k, b.cu_seqlens, Hq, Hkv, d, n, G)
    worst = check_scores(res["scores"], s64)
    ref_keep, _, _ = O.topp_select(s32, b.cu_seqlens, n, G, p)
    amb = ambiguous_blocks(s32, b.cu_seqlens, n, G, p)
    ndiff = check_keep(res["keep"], ref_keep, amb)
    own_keep, own_cu, _ = O.topp_select(res["scores"], b.cu_seqlens, n, G, p)
    np.testing.assert_array_equal(res["keep"], own_keep)
    np.testing.assert_array_equal(res["cu_out"], own_cu)
    check_compaction(gb, res)
    say(f"[ok] {L} tokens: worst rel err {worst:.2e}, ambiguous {len(amb)}, differing {ndiff}, "
        f"kept {res['count']}/{b.T}")
