"""GPU: up_rope_attention_scores, the block scores of the window rows taken inside the
layer's own attention kernel.

Against the oracle: the rotated operands (rope of the bf16 inputs at the carried
positions, rounded to bf16) feed the decision oracle's block_scores and row_lse for
the last W = min(n, L) rows of every request; the GPU's scores meet the score
tolerance and its row log-sum-exp the row_lse bar.  The attention output is
bit-identical to up_rope_attention's.  Cases cover both attention kernels (8 waves at
d = 64, 128; 4 waves at d = 256), block sizes 32 to 1024 (a block of 32 whose last
half-step lies past the request's last key, blocks longer than the request), rebases
inside a block, one-hot rows, L < n, empty and ragged requests."""
import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from oracle import consumer_oracle as C
from oracle import uniprefill_oracle as O
from workloads import synth
from tests.gpu_helpers import bf16_dev, check_scores, i32_dev, say

pytestmark = pytest.mark.gpu

THETA = 500000.0

CASES = [
    # lengths, Hq, Hkv, d, n, G, q_sigma
    ([300, 0, 65, 129, 1], 8, 2, 128, 128, 64, 1.0),   # varlen, empty and ragged requests
    ([980], 8, 2, 64, 128, 32, 1.0),                   # G = 32: the last half-step is padding
    ([2000], 16, 8, 256, 128, 64, 1.0),                # d = 256: the 4-wave kernel
    ([1200, 77], 8, 8, 256, 100, 32, 4.0),             # d = 256, G = 32, n = 100
    ([700], 8, 2, 128, 128, 128, 12.0),                # large logits: rebases inside blocks
    ([513], 4, 2, 64, 100, 96, 30.0),                  # nearly one-hot rows, G = 96
    ([50], 4, 1, 64, 128, 64, 1.0),                    # L < n: every row is a window row
    ([257], 8, 8, 128, 64, 1024, 1.0),                 # a block longer than the request
    ([4096], 32, 8, 128, 128, 64, 1.0),                # the Llama-3.1-8B head layout
    ([150, 3000, 64], 12, 4, 128, 128, 64, 4.0),       # three query heads per kv head
]


def _oracle(q, k, pos, cu, Hq, Hkv, d, n, G):
    qr = C.bits_from_bf16_values(C.rotate_bf16(q, pos, THETA))
    kr = C.bits_from_bf16_values(C.rotate_bf16(k, pos, THETA))
    win = [qr[cu[i + 1] - min(n, cu[i + 1] - cu[i]):cu[i + 1]] for i in range(cu.size - 1)]
    qwin = np.concatenate(win) if win else qr[:0]
    _, s64, _ = O.block_scores(qwin, kr, cu, Hq, Hkv, d, n, G)
    lse = O.row_lse(qwin, kr, cu, Hq, Hkv, d, n)
    return s64, lse


def _run(lengths, Hq, Hkv, d, n, G, sigma, seed):
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, seed, q_sigma=sigma)
    R = int(cu[-1])
    W = int(sum(min(L, n) for L in lengths))
    qd, kd, vd = (bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d),
                  bf16_dev(v).view(R, Hkv, d))
    pd, cd = i32_dev(pos), i32_dev(cu)
    lse = torch.full((W, Hq), float("nan"), dtype=torch.float32, device="cuda")
    out, scores = up.rope_attention_scores(qd, kd, vd, pd, cd, cu, n, G, rope_theta=THETA,
                                           row_lse=lse)
    ref_out = up.rope_attention(qd, kd, vd, pd, cd, cu, rope_theta=THETA)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    return q, k, pos, cu, out, ref_out, scores.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_attention_scores_match_oracle(case):
    lengths, Hq, Hkv, d, n, G, sigma = case
    say(f"[case] attention scores {case}")
    q, k, pos, cu, out, ref_out, s_gpu, lse_gpu = _run(lengths, Hq, Hkv, d, n, G, sigma,
                                                        seed=len(lengths) * 7 + d + G)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    s64, lse_ref = _oracle(q, k, pos, cu, Hq, Hkv, d, n, G)
    worst = check_scores(s_gpu, s64)
    np.testing.assert_allclose(lse_gpu.astype(np.float64), lse_ref, rtol=1e-5, atol=1e-4)
    # each request's scores sum to one
    boff = 0
    for L in lengths:
        nb = O.n_blocks(L, G)
        if nb:
            assert abs(float(s_gpu[boff:boff + nb].astype(np.float64).sum()) - 1.0) < 1e-5
        boff += nb
    say(f"[ok] {case}: worst rel err {worst:.2e}")


@pytest.mark.timeout(600)
def test_attention_scores_at_32k():
    """32K rows of the Llama-3.1-8B head layout (Hq = 32, Hkv = 8, d = 128): 512 blocks,
    window rows spread over the last two 64-token tiles of every head."""
    lengths, Hq, Hkv, d, n, G = [32768], 32, 8, 128, 128, 64
    say("[case] attention scores at 32K")
    q, k, pos, cu, out, ref_out, s_gpu, lse_gpu = _run(lengths, Hq, Hkv, d, n, G, 1.0, seed=5)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    s64, lse_ref = _oracle(q, k, pos, cu, Hq, Hkv, d, n, G)
    worst = check_scores(s_gpu, s64)
    np.testing.assert_allclose(lse_gpu.astype(np.float64), lse_ref, rtol=1e-5, atol=1e-4)
    say(f"[ok] 32K: worst rel err {worst:.2e}")


def test_attention_scores_with_inconsistent_device_cu_write_nothing():
    """A device cu_seqlens that disagrees with the host copy: error bit 1, the scores
    are left as they were."""
    lengths, Hq, Hkv, d, n, G = [1000], 8, 2, 128, 128, 64
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, 3)
    R = int(cu[-1])
    qd, kd, vd = (bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d),
                  bf16_dev(v).view(R, Hkv, d))
    bad = i32_dev(np.array([0, 900], np.int32))
    scores = torch.full((O.n_blocks(1000, G),), 7.0, dtype=torch.float32, device="cuda")
    up.rope_attention_scores(qd, kd, vd, i32_dev(pos), bad, cu, n, G, rope_theta=THETA,
                             scores=scores)
    torch.cuda.synchronize()
    assert up.device_error() & 1
    assert bool((scores == 7.0).all())
