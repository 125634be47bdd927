"""GPU parity of the given-lse score pass and of the row log-sum-exp output.

* up_block_scores' row_lse output against the oracle's row_lse;
* up_block_scores_lse, fed the oracle's own log-sum-exp (rounded to float32),
  against the oracle's block_scores_given_lse on the same float32 values: scores to
  the score tolerance, the cut bit-exact on the GPU's scores, compaction bit-exact;
* at 128K tokens, fed the GPU's own row_lse: the two GPU passes agree closely and
  both meet the oracle.
"""
import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from oracle import uniprefill_oracle as O
from workloads import synth
from tests.gpu_helpers import (GpuBatch, ambiguous_blocks, bf16_dev, check_compaction, check_keep,
                               check_scores, i32_dev, say)

pytestmark = pytest.mark.gpu

CASES = [
    # lengths, Hq, Hkv, d, n, G, p
    ([4096], 8, 2, 64, 128, 64, 0.99),
    ([1000], 4, 2, 64, 128, 64, 0.9),             # ragged last block
    ([300], 8, 2, 128, 128, 32, 0.95),            # G = 32
    ([2000], 4, 2, 256, 128, 64, 0.99),           # d = 256
    ([1500], 8, 1, 64, 64, 96, 0.9),              # MQA, G = 96
    ([50], 4, 2, 64, 128, 64, 0.5),               # L < n
    ([129, 0, 3000, 64, 1], 8, 2, 128, 128, 64, 0.97),   # varlen with an empty request
    ([5000], 16, 2, 128, 256, 64, 0.99),          # two row tiles
]


def _batch(lengths, Hq, Hkv, d, n, G, seed):
    reqs = [synth.gen_request(L, Hq, Hkv, d, n, G, 2,
                              np.random.default_rng([seed, synth.TAG_VARLEN_REQUEST, i]))
            for i, L in enumerate(lengths)]
    return synth.pack(reqs, Hq, Hkv, d, n, G)


def _lse_f32(b):
    return O.row_lse(b.qwin, b.k, b.cu_seqlens, b.Hq, b.Hkv, b.d, b.n).astype(np.float32)


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_row_lse_output_matches_oracle(case):
    lengths, Hq, Hkv, d, n, G, p = case
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=len(lengths) + d)
    say(f"[case] row_lse output {case}")
    gb = GpuBatch(b)
    lse = torch.empty((b.qwin.shape[0], Hq), dtype=torch.float32, device="cuda")
    up.block_scores(gb.qwin, gb.k, gb.cu, gb.cu_h, n, G, row_lse=lse)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    ref = O.row_lse(b.qwin, b.k, b.cu_seqlens, Hq, Hkv, d, n)
    got = lse.cpu().numpy().astype(np.float64)
    # float32 logits (MFMA accumulation over d) and float32 statistics: a 1e-4 shift of
    # a row's log-sum-exp scales its probabilities by 1e-4, far inside the score bar
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_given_lse_pass_matches_oracle(case):
    lengths, Hq, Hkv, d, n, G, p = case
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=len(lengths) * 7 + d)
    say(f"[case] given-lse pass {case}")
    _check_given_lse(b, p, H=128, label=str(case))


def _check_given_lse(b, p, H, label):
    """The decision from the oracle's log-sum-exp (float32) against the oracle's
    given-lse scores, its cut and the compaction."""
    Hq, Hkv, d, n, G = b.Hq, b.Hkv, b.d, b.n, b.G
    lse32 = _lse_f32(b)
    gb = GpuBatch(b, H=H)
    dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, n, G, p,
                           row_lse=torch.from_numpy(lse32).cuda())
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    s_gpu = dec.scores.cpu().numpy()
    s32, s64, _ = O.block_scores_given_lse(b.qwin, b.k, lse32.astype(np.float64), b.cu_seqlens,
                                           Hq, Hkv, d, n, G)
    worst = check_scores(s_gpu, s64)
    ref_keep, _, _ = O.topp_select(s32, b.cu_seqlens, n, G, p)
    amb = ambiguous_blocks(s32, b.cu_seqlens, n, G, p)
    keep = dec.keep.cpu().numpy()
    ndiff = check_keep(keep, ref_keep, amb)
    own_keep, own_cu, _ = O.topp_select(s_gpu, b.cu_seqlens, n, G, p)
    np.testing.assert_array_equal(keep, own_keep)
    cnt = int(dec.cu_out[-1].item())
    res = dict(scores=s_gpu, keep=keep, cu_out=dec.cu_out.cpu().numpy(), count=cnt, dec=dec)
    np.testing.assert_array_equal(res["cu_out"], own_cu)
    check_compaction(gb, res)
    say(f"[ok] given-lse {label}: worst rel err {worst:.2e}, ambiguous {len(amb)}, "
        f"differing {ndiff}")


def test_given_lse_pass_is_deterministic():
    b = _batch([20000], 8, 2, 128, 128, 64, seed=3)
    gb = GpuBatch(b)
    lse = torch.from_numpy(_lse_f32(b)).cuda()
    say("[case] given-lse determinism")
    a = up.block_scores_lse(gb.qwin, gb.k, lse, gb.cu, gb.cu_h, 128, 64)
    c = up.block_scores_lse(gb.qwin, gb.k, lse, gb.cu, gb.cu_h, 128, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


@pytest.mark.timeout(600)
def test_given_lse_pass_at_128k():
    """The 128K Llama-3.1-8B shape: the given-lse pass on the GPU's own row statistics
    agrees with the full pass to 1e-4 and with the oracle to the score tolerance."""
    cfg = synth.WORKLOADS["llama31_8b_128k"]
    say("[setup] generating llama31_8b_128k")
    b = synth.make_batch(cfg)
    gb = GpuBatch(b)
    nbt = int(sum((int(L) + b.G - 1) // b.G for L in np.diff(b.cu_seqlens)))
    lse = torch.empty((b.qwin.shape[0], b.Hq), dtype=torch.float32, device="cuda")
    s_full = up.block_scores(gb.qwin, gb.k, gb.cu, gb.cu_h, b.n, b.G, row_lse=lse)
    s_lse = up.block_scores_lse(gb.qwin, gb.k, lse, gb.cu, gb.cu_h, b.n, b.G)
    torch.cuda.synchronize()
    assert up.device_error() == 0 and s_lse.numel() == nbt
    a, c = s_full.cpu().numpy().astype(np.float64), s_lse.cpu().numpy().astype(np.float64)
    big = a >= 1e-6
    rel = np.abs(c - a)[big] / a[big]
    say(f"[ok] 128K: given-lse vs full pass max rel {rel.max():.2e}")
    assert rel.max() <= 1e-4
    _, s64, _ = O.block_scores(b.qwin, b.k, b.cu_seqlens, b.Hq, b.Hkv, b.d, b.n, b.G)
    worst = check_scores(s_lse.cpu().numpy(), s64)
    say(f"[ok] 128K given-lse vs oracle: worst rel err {worst:.2e}")


def _random_lse_configs(count=12, seed=4242):
    """Seeded draws: 1-4 requests of 0-3000 tokens, GQA group sizes 1-8, every head
    dimension, windows of 1-260, block sizes 32-1024 and p in [0.3, 1]."""
    rng = np.random.default_rng(seed)
    heads = [(8, 2), (4, 1), (4, 4), (12, 4), (16, 2), (6, 3)]
    out = []
    while len(out) < count:
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(0, 3001, B)]
        Hq, Hkv = heads[int(rng.integers(len(heads)))]
        d = int(rng.choice([64, 128, 256]))
        n = int(rng.integers(1, 261))
        if sum(L * Hq * min(L, n) * d for L in lengths) > 1.0e9:
            continue
        out.append((lengths, Hq, Hkv, d, n, 32 * int(rng.integers(1, 33)),
                    float(np.float32(rng.uniform(0.3, 1.0))), int(rng.integers(1 << 30))))
    return out


RANDOM_LSE = _random_lse_configs()


@pytest.mark.parametrize("case", RANDOM_LSE, ids=[f"r{i}" for i in range(len(RANDOM_LSE))])
def test_random_configurations_row_lse_and_given_lse(case):
    """Per seeded draw: the full pass's row log-sum-exp output against the oracle's, and
    the decision from the oracle's log-sum-exp against the oracle's given-lse scores."""
    lengths, Hq, Hkv, d, n, G, p, seed = case
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=seed)
    say(f"[case] random lse {case}")
    gb = GpuBatch(b)
    lse = torch.empty((b.qwin.shape[0], Hq), dtype=torch.float32, device="cuda")
    up.block_scores(gb.qwin, gb.k, gb.cu, gb.cu_h, n, G, row_lse=lse)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    ref = O.row_lse(b.qwin, b.k, b.cu_seqlens, Hq, Hkv, d, n)
    np.testing.assert_allclose(lse.cpu().numpy().astype(np.float64), ref, rtol=1e-5, atol=1e-4)
    _check_given_lse(b, p, H=int(8 + seed % 41), label=f"random {case}")
