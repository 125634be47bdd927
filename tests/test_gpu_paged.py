"""GPU parity of the paged-key score pass (keys read through a block table).

Keys are scattered into shuffled pages (with unused pages in between); the paged
pass must give bit-identical scores and row statistics to the contiguous pass on
the same keys (the same arithmetic on the same values) and meet the oracle on the
keys it gathers from the pages; a page index outside the cache raises error bit 8
without touching memory outside it.
"""
import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from oracle import uniprefill_oracle as O
from workloads import synth
from tests.gpu_helpers import GpuBatch, check_scores, i32_dev, say

pytestmark = pytest.mark.gpu


def _batch(lengths, Hq, Hkv, d, n, G, seed):
    reqs = [synth.gen_request(L, Hq, Hkv, d, n, G, 2,
                              np.random.default_rng([seed, synth.TAG_VARLEN_REQUEST, i]))
            for i, L in enumerate(lengths)]
    return synth.pack(reqs, Hq, Hkv, d, n, G)


def _paginate(k_bits, cu, ps, seed, spare=7):
    """Scatter contiguous keys [T, Hkv, d] into shuffled pages; returns (pages, table)."""
    rng = np.random.default_rng(seed)
    lens = np.diff(np.asarray(cu, np.int64))
    need = [int((L + ps - 1) // ps) for L in lens]
    num_pages = sum(need) + spare
    perm = rng.permutation(num_pages)
    pages = rng.integers(0, 1 << 15, (num_pages, ps) + k_bits.shape[1:]).astype(np.uint16)
    table = np.full((len(lens), max(1, max(need))), -1, np.int32)
    nxt = 0
    for i, L in enumerate(lens):
        for pg in range(need[i]):
            table[i, pg] = perm[nxt]
            nxt += 1
            lo, hi = pg * ps, min((pg + 1) * ps, int(L))
            pages[table[i, pg], :hi - lo] = k_bits[cu[i] + lo:cu[i] + hi]
    return pages, table


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


CASES = [
    # lengths, Hq, Hkv, d, n, G, page size
    ([4096], 8, 2, 64, 128, 64, 16),
    ([1000], 4, 2, 64, 128, 64, 32),
    ([300], 8, 2, 128, 128, 32, 64),
    ([2000], 4, 2, 256, 128, 64, 16),
    ([1500], 8, 1, 64, 64, 96, 256),              # G = 96: stages straddle 64-key pages
    ([129, 0, 3000, 64, 1], 8, 2, 128, 128, 64, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_paged_pass_matches_contiguous_and_oracle(case):
    lengths, Hq, Hkv, d, n, G, ps = case
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=ps + d + len(lengths))
    say(f"[case] paged keys {case}")
    pages, table = _paginate(b.k, b.cu_seqlens, ps, seed=ps)
    gb = GpuBatch(b)
    lse_c = torch.empty((b.qwin.shape[0], Hq), dtype=torch.float32, device="cuda")
    lse_p = torch.empty_like(lse_c)
    s_c = up.block_scores(gb.qwin, gb.k, gb.cu, gb.cu_h, n, G, row_lse=lse_c)
    s_p = up.block_scores_paged(gb.qwin, _bf16(pages), i32_dev(table), gb.cu, gb.cu_h, n, G,
                                row_lse=lse_p)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    assert torch.equal(s_c, s_p)
    assert torch.equal(lse_c, lse_p)
    kk = O.gather_paged_keys(pages, table, b.cu_seqlens, ps)
    _, s64, _ = O.block_scores(b.qwin, kk, b.cu_seqlens, Hq, Hkv, d, n, G)
    worst = check_scores(s_p.cpu().numpy(), s64)
    say(f"[ok] paged {case}: bit-identical to contiguous, worst rel err {worst:.2e}")


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_paged_given_lse_pass_matches_contiguous_and_oracle(case):
    """The given-lse pass over paged keys: bit-identical to the same pass over the
    contiguous keys, and within the score bar of the oracle's given-lse scores on the
    keys gathered from the pages, fed the oracle's own log-sum-exp."""
    lengths, Hq, Hkv, d, n, G, ps = case
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=ps + d + len(lengths) + 11)
    say(f"[case] paged keys, given lse {case}")
    pages, table = _paginate(b.k, b.cu_seqlens, ps, seed=ps + 1)
    kk = O.gather_paged_keys(pages, table, b.cu_seqlens, ps)
    assert np.array_equal(kk, b.k)
    lse32 = O.row_lse(b.qwin, kk, b.cu_seqlens, Hq, Hkv, d, n).astype(np.float32)
    gb = GpuBatch(b)
    lse = torch.from_numpy(lse32).cuda()
    s_c = up.block_scores_lse(gb.qwin, gb.k, lse, gb.cu, gb.cu_h, n, G)
    s_p = up.block_scores_lse_paged(gb.qwin, _bf16(pages), i32_dev(table), lse, gb.cu, gb.cu_h,
                                    n, G)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    assert torch.equal(s_c, s_p)
    _, s64, _ = O.block_scores_given_lse(b.qwin, kk, lse32.astype(np.float64), b.cu_seqlens,
                                         Hq, Hkv, d, n, G)
    worst = check_scores(s_p.cpu().numpy(), s64)
    say(f"[ok] paged given-lse {case}: bit-identical to contiguous, worst rel err {worst:.2e}")


def test_page_index_outside_the_cache_raises_error_bit():
    b = _batch([1000], 8, 2, 64, 128, 64, seed=1)
    pages, table = _paginate(b.k, b.cu_seqlens, 16, seed=3)
    bad = table.copy()
    bad[0, 5] = pages.shape[0] + 1000     # past the cache
    bad[0, 9] = -3
    gb = GpuBatch(b)
    say("[case] paged keys with out-of-range page indices")
    up.device_error()
    up.block_scores_paged(gb.qwin, _bf16(pages), i32_dev(bad), gb.cu, gb.cu_h, 128, 64)
    torch.cuda.synchronize()
    assert up.device_error() & 8
    lse = torch.empty((b.qwin.shape[0], 8), dtype=torch.float32, device="cuda")
    up.block_scores(gb.qwin, gb.k, gb.cu, gb.cu_h, 128, 64, row_lse=lse)
    up.block_scores_lse_paged(gb.qwin, _bf16(pages), i32_dev(bad), lse, gb.cu, gb.cu_h, 128, 64)
    torch.cuda.synchronize()
    assert up.device_error() & 8
    s = up.block_scores_paged(gb.qwin, _bf16(pages), i32_dev(table), gb.cu, gb.cu_h, 128, 64)
    torch.cuda.synchronize()
    assert up.device_error() == 0 and torch.isfinite(s).all()


@pytest.mark.timeout(600)
def test_paged_pass_at_128k_is_bit_identical():
    cfg = synth.WORKLOADS["llama31_8b_128k"]
    say("[setup] generating llama31_8b_128k")
    b = synth.make_batch(cfg)
    pages, table = _paginate(b.k, b.cu_seqlens, 16, seed=16)
    gb = GpuBatch(b)
    say("[case] paged keys at 128K, 16-token pages")
    s_c = up.block_scores(gb.qwin, gb.k, gb.cu, gb.cu_h, b.n, b.G)
    s_p = up.block_scores_paged(gb.qwin, _bf16(pages), i32_dev(table), gb.cu, gb.cu_h, b.n, b.G)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    assert torch.equal(s_c, s_p)


def _random_paged_configs(count=12, seed=77):
    """Seeded draws: 1-4 requests of 0-5000 tokens, page sizes 16-1024, every head
    dimension, GQA group sizes 1-4 and block sizes 32-1024 (pages smaller and larger
    than a block, and a stage of 64 keys spanning up to four pages)."""
    rng = np.random.default_rng(seed)
    heads = [(8, 2), (4, 1), (4, 4), (6, 2), (8, 8)]
    out = []
    for _ in range(count):
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(0, 5001, B)]
        Hq, Hkv = heads[int(rng.integers(len(heads)))]
        out.append((lengths, Hq, Hkv, int(rng.choice([64, 128, 256])), int(rng.integers(1, 200)),
                    32 * int(rng.integers(1, 33)), int(1 << rng.integers(4, 11)),
                    int(rng.integers(1 << 30))))
    return out


RANDOM_PAGED = _random_paged_configs()


@pytest.mark.parametrize("case", RANDOM_PAGED, ids=[f"r{i}" for i in range(len(RANDOM_PAGED))])
def test_random_paged_configurations_are_bit_identical(case):
    """Both paged passes (row statistics computed, and given) equal the contiguous passes
    bit for bit on the same keys; the contiguous passes meet the oracle in the other
    tests."""
    lengths, Hq, Hkv, d, n, G, ps, seed = case
    b = _batch(lengths, Hq, Hkv, d, n, G, seed=seed)
    say(f"[case] random paged {case}")
    pages, table = _paginate(b.k, b.cu_seqlens, ps, seed=seed + 1, spare=int(seed % 5))
    gb = GpuBatch(b)
    pg, tb = _bf16(pages), i32_dev(table)
    lse_c = torch.empty((b.qwin.shape[0], Hq), dtype=torch.float32, device="cuda")
    lse_p = torch.empty_like(lse_c)
    s_c = up.block_scores(gb.qwin, gb.k, gb.cu, gb.cu_h, n, G, row_lse=lse_c)
    s_p = up.block_scores_paged(gb.qwin, pg, tb, gb.cu, gb.cu_h, n, G, row_lse=lse_p)
    g_c = up.block_scores_lse(gb.qwin, gb.k, lse_c, gb.cu, gb.cu_h, n, G)
    g_p = up.block_scores_lse_paged(gb.qwin, pg, tb, lse_c, gb.cu, gb.cu_h, n, G)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    assert torch.equal(s_c, s_p) and torch.equal(lse_c, lse_p)
    assert torch.equal(g_c, g_p)
    say(f"[ok] random paged {case}: both passes bit-identical to contiguous")
