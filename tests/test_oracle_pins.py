"""Pins for the CPU oracle: each check ties it to something other than itself.

* float64 brute force (pure-Python loops) on tiny inputs,
* the library routine torch.nn.functional.scaled_dot_product_attention with V = I,
  which returns the probability matrix itself,
* the printed result of the chunked-prefill example on the Ultralytics glossary
  page (tests/golden/chunked_prefill_demo.json),
* closed forms (all-zero queries; planted needles over all-zero keys),
* exhaustive subset enumeration for the Top-p cut,
* invariants stated by the UniPrefill pages (kept mass >= p, the window is kept,
  later layers see a subset in order, requests are independent, partial scores
  over head shards add up).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import uniprefill_oracle as O
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_request(rng, L, Hq, Hkv, d, n, scale_k=1.0):
    W = min(n, L)
    q = synth.f32_to_bf16_bits(rng.standard_normal((W, Hq, d), dtype=np.float32))
    k = synth.f32_to_bf16_bits(scale_k * rng.standard_normal((L, Hkv, d), dtype=np.float32))
    return q, k


def _brute_probs(qf, kf, scale):
    """Pure-Python float64 loops: P[h][j][key] for window row j at position L-W+j."""
    W, Hq, d = qf.shape
    L, Hkv, _ = kf.shape
    gs = Hq // Hkv
    P = [[[0.0] * L for _ in range(W)] for _ in range(Hq)]
    for h in range(Hq):
        for j in range(W):
            t = L - W + j
            logits = []
            for key in range(t + 1):
                acc = 0.0
                for x in range(d):
                    acc += float(qf[j, h, x]) * float(kf[key, h // gs, x])
                logits.append(acc * scale)
            m = max(logits)
            ex = [math.exp(v - m) for v in logits]
            z = math.fsum(ex)
            for key in range(t + 1):
                P[h][j][key] = ex[key] / z
    return P


@pytest.mark.parametrize("L,n,G,Hq,Hkv,d", [
    (37, 8, 16, 4, 2, 8),      # ragged last block, window inside one block
    (130, 40, 32, 4, 1, 16),   # window spanning two blocks, MQA
    (64, 128, 32, 2, 2, 4),    # L < n: the whole request is the window
    (1, 8, 16, 2, 1, 8),       # a single token
    (257, 16, 64, 4, 4, 8),    # one key past a block boundary
])
def test_block_mass_matches_brute_force(L, n, G, Hq, Hkv, d):
    rng = np.random.default_rng(L * 7 + n)
    qb, kb = _rand_request(rng, L, Hq, Hkv, d, n)
    qf, kf = O.bf16_bits_to_f64(qb), O.bf16_bits_to_f64(kb)
    scale = O.default_scale(d)
    P = _brute_probs(qf, kf, scale)
    W = min(n, L)
    nb = (L + G - 1) // G
    mass_bf = [0.0] * nb
    for h in range(Hq):
        for j in range(W):
            for key in range(L):
                mass_bf[key // G] += P[h][j][key]
    Po = O.window_probs(qf, kf, scale)
    np.testing.assert_allclose(Po, np.array(P), rtol=1e-12, atol=1e-15)
    mass = O.request_block_mass(qf, kf, G, scale)
    np.testing.assert_allclose(mass, mass_bf, rtol=1e-12, atol=1e-15)
    # through the packed entry point: scores are the masses normalised to one
    cu = np.array([0, L], np.int32)
    s32, s64, m64 = O.block_scores(qb, kb, cu, Hq, Hkv, d, n, G)
    np.testing.assert_allclose(s64, np.array(mass_bf) / math.fsum(mass_bf), rtol=1e-12, atol=1e-16)
    assert abs(math.fsum(s64) - 1.0) < 1e-12
    # every window row is a probability distribution: total mass = Hq * W
    assert abs(math.fsum(mass_bf) - Hq * W) < 1e-9


def test_probs_match_library_sdpa_with_identity_values():
    """SDPA(q, k, V=I) returns the attention matrix; pins scale, softmax and causal mask."""
    rng = np.random.default_rng(3)
    L, n, Hq, Hkv, d = 200, 48, 4, 2, 16
    qb, kb = _rand_request(rng, L, Hq, Hkv, d, n)
    qf, kf = O.bf16_bits_to_f64(qb), O.bf16_bits_to_f64(kb)
    W = min(n, L)
    start = L - W
    q = torch.from_numpy(qf).permute(1, 0, 2).unsqueeze(0)                    # [1, Hq, W, d]
    k = torch.from_numpy(kf).repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2).unsqueeze(0)
    v = torch.eye(L, dtype=torch.float64).expand(1, Hq, L, L)
    # the final "chunk" of the glossary example: causal over absolute positions
    mask = torch.ones(W, L, dtype=torch.bool).tril(diagonal=start)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)[0].numpy()
    P = O.window_probs(qf, kf, O.default_scale(d))
    np.testing.assert_allclose(P, ref, rtol=1e-6, atol=1e-9)
    # and the window rows equal the last W rows of a one-pass causal prefill
    qall = torch.from_numpy(rng.standard_normal((1, Hq, L, d))).to(torch.float64)
    qall[:, :, start:, :] = q[0]
    full = torch.nn.functional.scaled_dot_product_attention(qall, k, v, is_causal=True)[0].numpy()
    np.testing.assert_allclose(P, full[:, start:, :], rtol=1e-6, atol=1e-9)


def test_golden_chunked_prefill_example():
    """The glossary page prints: 4 chunks of 256, 256, 256, 232 equal one pass.

    The oracle's window (the last W queries of a request, attending to keys
    0..t) is exactly such a chunk: chunk [start, end) is the window of a request
    truncated to length ``end``.  Rebuilding the page's experiment from the
    oracle's window probabilities must reproduce the printed result."""
    g = json.load(open(os.path.join(GOLDEN, "chunked_prefill_demo.json")))
    L, C, H, d = g["prompt_len"], g["chunk"], g["heads"], g["head_dim"]
    rng = np.random.default_rng(0)
    q = rng.standard_normal((L, H, d))
    k = rng.standard_normal((L, H, d))
    v = rng.standard_normal((L, H, d))
    scale = 1.0 / math.sqrt(d)
    full = np.einsum("hjk,khd->hjd", O.window_probs(q, k, scale), v)       # W = L: one pass
    sizes, outs = [], []
    for start in range(0, L, C):
        end = min(start + C, L)
        P = O.window_probs(q[start:end], k[:end], scale)                  # window of length end-start
        outs.append(np.einsum("hjk,khd->hjd", P, v[:end]))
        sizes.append(end - start)
    chunked = np.concatenate(outs, axis=1)
    assert sizes == g["expected_chunk_sizes"]
    assert np.allclose(full, chunked, atol=g["atol"]) == g["expected_same_as_one_pass"]


def _zero_query_case(L, n, G, Hq=2, Hkv=1, d=8):
    W = min(n, L)
    qb = np.zeros((W, Hq, d), np.uint16)
    rng = np.random.default_rng(L)
    kb = synth.f32_to_bf16_bits(rng.standard_normal((L, Hkv, d), dtype=np.float32))
    return qb, kb


@pytest.mark.parametrize("L,n,G,p", [(1024, 128, 64, 0.5), (1000, 100, 32, 0.75), (4096, 128, 64, 0.95)])
def test_closed_form_zero_queries(L, n, G, p):
    """Q = 0: every visible logit is 0, so P[j, key] = 1/(t_j + 1) for key <= t_j.

    A block lying wholly at or before position L-W gets mass Hq*G*sum_j 1/(t_j+1);
    the scores are that over Hq*W.  All such blocks tie exactly and are taken
    lowest index first."""
    Hq = 2
    qb, kb = _zero_query_case(L, n, G, Hq=Hq)
    W = min(n, L)
    nb = (L + G - 1) // G
    t = [L - W + j for j in range(W)]
    exact = []
    for b in range(nb):
        lo, hi = b * G, min((b + 1) * G, L)
        m = sum(Fraction(sum(1 for key in range(lo, hi) if key <= tj), tj + 1) for tj in t)
        exact.append(m / W)                      # per-head mass over total per-head mass W
    assert sum(exact) == 1
    cu = np.array([0, L], np.int32)
    s32, s64, _ = O.block_scores(qb, kb, cu, Hq, 1, 8, n, G)
    np.testing.assert_allclose(s64, [float(x) for x in exact], rtol=1e-13)
    early = [b for b in range(nb) if min((b + 1) * G, L) - 1 <= L - W]
    assert len({float(s32[b]) for b in early}) == 1, "early blocks must tie exactly"
    s_early = Fraction(float(s32[early[0]]))
    p32 = Fraction(float(np.float32(p)))
    kstar = next(k for k in range(1, nb + 1) if k * s_early >= p32)
    assert kstar <= len(early)
    keep, _, det = O.topp_select(s32, cu, n, G, p)
    assert det[0]["kstar"] == kstar
    expected = set(early[:kstar]) | set(O.window_blocks(L, n, G))
    assert set(np.nonzero(keep)[0].tolist()) == expected


def test_closed_form_planted_needles_over_zero_keys():
    """Identical query rows, keys zero except two needle blocks with logits a and b.

    Row j sees (t_j+1-2G) zero logits plus G copies of a and G of b, so the needle
    masses are sums of G e^a / Z_j with Z_j = (t_j+1-2G) + G e^a + G e^b."""
    L, n, G, Hq, Hkv, d = 2048, 128, 64, 4, 2, 16
    W = n
    rng = np.random.default_rng(11)
    v = rng.standard_normal(d).astype(np.float32)
    v /= np.linalg.norm(v)
    qf32 = np.tile(4.0 * v, (W, Hq, 1)).astype(np.float32)
    kf32 = np.zeros((L, Hkv, d), np.float32)
    bA, bB = 5, 17
    kf32[bA * G:(bA + 1) * G] = 6.0 * v
    kf32[bB * G:(bB + 1) * G] = 5.2 * v
    qb, kb = synth.f32_to_bf16_bits(qf32), synth.f32_to_bf16_bits(kf32)
    qf, kf = O.bf16_bits_to_f64(qb), O.bf16_bits_to_f64(kb)
    scale = O.default_scale(d)
    a = float(qf[0, 0] @ kf[bA * G, 0]) * scale
    b = float(qf[0, 0] @ kf[bB * G, 0]) * scale
    tot = Hq * W
    mA = mB = 0.0
    for j in range(W):
        Z = (L - W + j + 1 - 2 * G) + G * math.exp(a) + G * math.exp(b)
        mA += Hq * G * math.exp(a) / Z
        mB += Hq * G * math.exp(b) / Z
    cu = np.array([0, L], np.int32)
    s32, s64, _ = O.block_scores(qb, kb, cu, Hq, Hkv, d, n, G, scale)
    assert s64[bA] == pytest.approx(mA / tot, rel=1e-12)
    assert s64[bB] == pytest.approx(mB / tot, rel=1e-12)
    win = set(O.window_blocks(L, n, G))
    sA, sB = mA / tot, mB / tot
    keep, _, _ = O.topp_select(s32, cu, n, G, sA * 0.999)
    assert set(np.nonzero(keep)[0].tolist()) == {bA} | win
    keep, _, _ = O.topp_select(s32, cu, n, G, (sA + 0.5 * sB))
    assert set(np.nonzero(keep)[0].tolist()) == {bA, bB} | win


def test_one_hot_block_dominates():
    """A block whose logits exceed all others by >= 30 takes all but ~e^-30 of the mass."""
    L, n, G, Hq, Hkv, d = 4096, 128, 64, 4, 2, 16
    rng = np.random.default_rng(5)
    v = rng.standard_normal(d).astype(np.float32)
    v /= np.linalg.norm(v)
    q = np.tile(8.0 * v, (n, Hq, 1)).astype(np.float32)
    k = (0.01 * rng.standard_normal((L, Hkv, d))).astype(np.float32)
    bstar = 23
    k[bstar * G:(bstar + 1) * G] += 16.0 * v      # logit ~ 8*16/4 = 32
    qb, kb = synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k)
    cu = np.array([0, L], np.int32)
    s32, s64, _ = O.block_scores(qb, kb, cu, Hq, Hkv, d, n, G)
    assert s64[bstar] > 1 - 1e-9
    for p in (0.5, 0.9, 0.99, 0.999):
        keep, _, det = O.topp_select(s32, cu, n, G, p)
        assert det[0]["kstar"] == 1
        assert set(np.nonzero(keep)[0].tolist()) == {bstar} | set(O.window_blocks(L, n, G))


@pytest.mark.parametrize("seed", range(12))
def test_topp_minimal_by_subset_enumeration(seed):
    """The prefix cut is the smallest block set reaching p, and no equal-size set has more mass.

    Sums are exact (Fractions), as the oracle's cut is."""
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(2, 13))
    s = rng.dirichlet(np.full(nb, 0.7)).astype(np.float32)
    p = float(rng.uniform(0.3, 0.999))
    L, G, n = nb * 16, 16, 1                      # window = last token only
    keep, det = O.topp_request(s, L, n, G, p)
    kstar = det["kstar"]
    pf = Fraction(float(np.float32(p)))
    sf = [Fraction(float(x)) for x in s]
    best_size = None
    for size in range(1, nb + 1):
        if any(sum(sf[i] for i in c) >= pf for c in itertools.combinations(range(nb), size)):
            best_size = size
            break
    if best_size is None:
        assert kstar == nb                        # every sum stays below p: keep all
    else:
        assert kstar == best_size
        pref = sum(sf[i] for i in det["order"][:kstar])
        assert pref >= pf
        assert all(pref >= sum(sf[i] for i in c) for c in itertools.combinations(range(nb), kstar))
        if kstar > 1:
            assert sum(sf[i] for i in det["order"][:kstar - 1]) < pf
    # the window block (the last one) is always kept
    assert keep[nb - 1]


def test_topp_cut_is_exact_at_the_boundary():
    """Scores whose float64 running sum rounds differently from the exact one.

    2**-30 added to 1 - 2**-30 ... : sequential float64 rounding is irrelevant to the
    exact comparison; a running sum that equals p exactly counts as reaching it."""
    s = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    for p, k in ((0.75, 2), (0.875, 3), (0.8750001, 4), (1.0, 4), (0.5, 1)):
        keep, det = O.topp_request(s, 4 * 16, 1, 16, p)
        assert det["kstar"] == k, (p, det["kstar"])
    # many tiny scores after a large one: the exact sum of the tail crosses p
    tiny = np.float32(2.0 ** -40)
    s = np.array([np.float32(1.0) - np.float32(2.0 ** -24)] + [tiny] * 2**4 + [np.float32(0)] * 3, np.float32)
    p = float(np.float32(1.0) - np.float32(2.0 ** -24))
    keep, det = O.topp_request(s, s.size * 16, 1, 16, p)
    assert det["kstar"] == 1


def test_topp_special_cases_and_nesting():
    rng = np.random.default_rng(9)
    nb = 40
    s = rng.dirichlet(np.full(nb, 0.5)).astype(np.float32)
    L, G, n = nb * 64, 64, 128
    win = set(O.window_blocks(L, n, G))
    assert win == {nb - 2, nb - 1}
    keep1, det1 = O.topp_request(s, L, n, G, 1.0)
    assert keep1.all() and det1["kstar"] == nb
    keep0, det0 = O.topp_request(s, L, n, G, 1e-9)
    assert det0["kstar"] == 1
    assert set(np.nonzero(keep0)[0].tolist()) == {int(np.argmax(s))} | win
    prev = None
    for p in np.linspace(0.05, 0.999, 40):
        keep, det = O.topp_request(s, L, n, G, float(p))
        kept = set(np.nonzero(keep)[0].tolist())
        dropped_mass = float(np.sum(s.astype(np.float64)[~keep]))
        assert dropped_mass <= 1 - float(np.float32(p)) + 1e-6
        if prev is not None:
            assert prev <= kept                   # kept sets nest as p grows
        prev = kept
    # ties are broken by the lower block index
    t = np.full(8, 0.125, np.float32)
    keep, det = O.topp_request(t, 8 * 64, 1, 64, 0.5)
    assert det["kstar"] == 4 and list(det["order"][:4]) == [0, 1, 2, 3]


def test_short_request_keeps_everything():
    rng = np.random.default_rng(1)
    for L in (1, 50, 127, 128):
        qb, kb = _rand_request(rng, L, 4, 2, 8, 128)
        cu = np.array([0, L], np.int32)
        s32, _, _ = O.block_scores(qb, kb, cu, 4, 2, 8, 128, 64)
        keep, cu_out, _ = O.topp_select(s32, cu, 128, 64, 0.5)
        assert keep.all() and cu_out[-1] == L


def test_expand_compact_compose_against_independent_routes():
    rng = np.random.default_rng(21)
    lens = [130, 64, 1, 500, 0, 77]
    G = 32
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    nbs = [(L + G - 1) // G for L in lens]
    keep = (rng.random(sum(nbs)) < 0.6).astype(np.uint8)
    idx = O.expand(keep, cu, G)
    # token-level route: a token survives iff its block does
    tok = []
    boff = 0
    for i, L in enumerate(lens):
        tok.append(np.repeat(keep[boff:boff + nbs[i]], G)[:L])
        boff += nbs[i]
    ref_idx = np.nonzero(np.concatenate(tok))[0].astype(np.int32)
    np.testing.assert_array_equal(idx, ref_idx)
    H = 24
    hidden = rng.integers(0, 2**16, size=(cu[-1], H), dtype=np.uint16)
    pos = synth.positions(cu)
    h_out, p_out = O.compact(hidden, pos, idx)
    np.testing.assert_array_equal(h_out, np.take(hidden, idx, axis=0))
    np.testing.assert_array_equal(p_out, np.take(pos, idx))
    # strictly increasing within each request, requests in order
    assert np.all(np.diff(idx) > 0)
    # composition of two decisions equals a direct gather of the originals
    orig0 = np.arange(cu[-1], dtype=np.int32)
    o1 = O.compose(orig0, idx)
    np.testing.assert_array_equal(o1, idx)
    sub = np.sort(rng.choice(idx.size, size=idx.size // 2, replace=False)).astype(np.int32)
    o2 = O.compose(o1, sub)
    np.testing.assert_array_equal(o2, idx[sub])
    # with pos = arange per request, compacted positions are original offsets in the request
    req_of = np.searchsorted(cu, idx, side="right") - 1
    np.testing.assert_array_equal(p_out, idx - cu[req_of])


def test_packed_requests_are_independent():
    rng = np.random.default_rng(4)
    Hq, Hkv, d, n, G = 4, 2, 8, 40, 32
    reqs = [synth.gen_request(L, Hq, Hkv, d, n, G, 2, np.random.default_rng([7, i]))
            for i, L in enumerate([300, 33, 129, 1000])]
    batch = synth.pack(reqs, Hq, Hkv, d, n, G)
    s_all, _, _ = O.block_scores(batch.qwin, batch.k, batch.cu_seqlens, Hq, Hkv, d, n, G)
    keep_all, cu_out, _ = O.topp_select(s_all, batch.cu_seqlens, n, G, 0.9)
    boff = 0
    kept_tokens = 0
    for r in reqs:
        one = synth.pack([r], Hq, Hkv, d, n, G)
        s1, _, _ = O.block_scores(one.qwin, one.k, one.cu_seqlens, Hq, Hkv, d, n, G)
        k1, c1, _ = O.topp_select(s1, one.cu_seqlens, n, G, 0.9)
        np.testing.assert_array_equal(s_all[boff:boff + s1.size], s1)
        np.testing.assert_array_equal(keep_all[boff:boff + s1.size], k1)
        boff += s1.size
        kept_tokens += int(c1[-1])
    assert cu_out[-1] == kept_tokens


def test_partial_scores_over_head_shards_add_up():
    """Masses over disjoint query-head subsets sum to the full mass (tensor-parallel sync)."""
    Hq, Hkv, d, n, G = 8, 2, 16, 64, 32
    r = synth.gen_request(700, Hq, Hkv, d, n, G, 3, np.random.default_rng(2))
    b = synth.pack([r], Hq, Hkv, d, n, G)
    _, _, full = O.block_scores(b.qwin, b.k, b.cu_seqlens, Hq, Hkv, d, n, G)
    parts = [O.block_scores(b.qwin, b.k, b.cu_seqlens, Hq, Hkv, d, n, G, heads=range(h0, h0 + 4))[2]
             for h0 in (0, 4)]
    np.testing.assert_allclose(parts[0] + parts[1], full, rtol=1e-12)


def test_generator_is_seeded():
    cfg = synth.WORKLOADS["single_4k_h8_d64"]
    a, b = synth.make_batch(cfg), synth.make_batch(cfg)
    np.testing.assert_array_equal(a.qwin, b.qwin)
    np.testing.assert_array_equal(a.k, b.k)
    c = synth.make_batch(dict(cfg, seed=1))
    assert not np.array_equal(a.k, c.k)
    # bf16 rounding: ties go to even, values round to nearest
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5], np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = O.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(back, [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5])


def test_topk_keeps_the_k_best_and_the_window():
    rng = np.random.default_rng(31)
    nb = 50
    s = rng.dirichlet(np.full(nb, 0.4)).astype(np.float32)
    L, G, n = nb * 64 - 10, 64, 128
    for k in (0, 1, 7, nb, nb + 5):
        keep = O.topk_request(s, L, n, G, k)
        top = set(np.argsort(-s.astype(np.float64), kind="stable")[:min(k, nb)].tolist())
        assert set(np.nonzero(keep)[0].tolist()) == top | set(O.window_blocks(L, n, G))
    cu = np.array([0, L, L + 100], np.int32)
    s2 = np.concatenate([s, np.array([0.5, 0.5], np.float32)])
    keep, cu_out = O.topk_select(s2, cu, n, G, 3)
    assert cu_out[-1] - cu_out[-2] == 100           # a short request keeps everything


# ---------------------------------------------------------------------------
# Block scores from given row statistics (the layer's own log-sum-exp)
# ---------------------------------------------------------------------------

def test_row_lse_matches_brute_force():
    """row_lse against pure-Python float64 loops: log of the softmax denominator."""
    rng = np.random.default_rng(31)
    L, n, Hq, Hkv, d = 37, 12, 4, 2, 8
    qb, kb = _rand_request(rng, L, Hq, Hkv, d, n)
    qf, kf = O.bf16_bits_to_f64(qb), O.bf16_bits_to_f64(kb)
    scale = O.default_scale(d)
    lse = O.row_lse(qb, kb, np.array([0, L], np.int32), Hq, Hkv, d, n)
    gs = Hq // Hkv
    W = min(n, L)
    for h in range(Hq):
        for j in range(W):
            t = L - W + j
            logits = [scale * math.fsum(float(qf[j, h, x]) * float(kf[key, h // gs, x])
                                        for x in range(d)) for key in range(t + 1)]
            m = max(logits)
            want = m + math.log(math.fsum(math.exp(v - m) for v in logits))
            assert abs(lse[j, h] - want) <= 1e-12 * max(1.0, abs(want))


def test_row_lse_closed_forms():
    """Zero queries: every visible logit is 0, lse = ln(t + 1) exactly; a single
    visible key (t = 0) has lse equal to its own logit."""
    L, n = 300, 40
    qb, kb = _zero_query_case(L, n, 64, Hq=2)
    lse = O.row_lse(qb, kb, np.array([0, L], np.int32), 2, 1, 8, n)
    t = np.arange(L - n, L)
    np.testing.assert_allclose(lse, np.log(t + 1.0)[:, None].repeat(2, axis=1), rtol=1e-14)
    rng = np.random.default_rng(2)
    qb1, kb1 = _rand_request(rng, 1, 2, 1, 8, 4)
    lse1 = O.row_lse(qb1, kb1, np.array([0, 1], np.int32), 2, 1, 8, 4)
    s = (O.bf16_bits_to_f64(qb1)[0] @ O.bf16_bits_to_f64(kb1)[0, 0]) * O.default_scale(8)
    np.testing.assert_allclose(lse1[0], s, rtol=1e-14)


def test_given_lse_closed_form_zero_queries():
    """Q = 0 with lse = ln(t + 1) written from the closed form (not from row_lse): the
    scores are the exact Fraction closed form of the zero-query case."""
    L, n, G, Hq = 1000, 100, 32, 2
    qb, kb = _zero_query_case(L, n, G, Hq=Hq)
    W = min(n, L)
    nb = (L + G - 1) // G
    t = [L - W + j for j in range(W)]
    exact = []
    for b in range(nb):
        lo, hi = b * G, min((b + 1) * G, L)
        exact.append(sum(Fraction(sum(1 for key in range(lo, hi) if key <= tj), tj + 1)
                         for tj in t) / W)
    lse = np.log(np.array(t, np.float64) + 1.0)[:, None].repeat(Hq, axis=1)
    _, s64, m64 = O.block_scores_given_lse(qb, kb, lse, np.array([0, L], np.int32), Hq, 1, 8,
                                           n, G)
    np.testing.assert_allclose(s64, [float(x) for x in exact], rtol=1e-13)
    np.testing.assert_allclose(m64.sum(), Hq * W, rtol=1e-13)   # every row's weights sum to 1


def test_given_exact_lse_reproduces_block_scores():
    """With each row's true log-sum-exp the weights are the softmax probabilities, so
    the scores equal block_scores' (a packed batch: ragged, L < n, empty, MQA)."""
    rng = np.random.default_rng(44)
    lens, Hq, Hkv, d, n, G = [200, 9, 0, 130], 4, 1, 16, 24, 16
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    reqs = [_rand_request(rng, L, Hq, Hkv, d, n) for L in lens]
    qb = np.concatenate([q for q, _ in reqs])
    kb = np.concatenate([k for _, k in reqs])
    lse = O.row_lse(qb, kb, cu, Hq, Hkv, d, n)
    assert lse.shape == (sum(min(n, L) for L in lens), Hq)
    _, s_ref, m_ref = O.block_scores(qb, kb, cu, Hq, Hkv, d, n, G)
    _, s_lse, m_lse = O.block_scores_given_lse(qb, kb, lse, cu, Hq, Hkv, d, n, G)
    np.testing.assert_allclose(s_lse, s_ref, rtol=1e-12)
    np.testing.assert_allclose(m_lse, m_ref, rtol=1e-12)


def test_given_lse_is_linear_in_each_rows_weight():
    """Masses are sum over rows of exp(-lse_row) * (row's unnormalised block sums):
    shifting one row's lse by delta changes the masses by (e^-delta - 1) times that
    row's contribution, which is the difference made by removing the row
    (lse = +inf)."""
    rng = np.random.default_rng(5)
    L, Hq, Hkv, d, n, G = 150, 2, 1, 8, 20, 16
    qb, kb = _rand_request(rng, L, Hq, Hkv, d, n)
    cu = np.array([0, L], np.int32)
    lse = O.row_lse(qb, kb, cu, Hq, Hkv, d, n)
    _, _, m0 = O.block_scores_given_lse(qb, kb, lse, cu, Hq, Hkv, d, n, G)
    j, h, delta = 7, 1, 0.75
    gone = lse.copy()
    gone[j, h] = np.inf
    _, _, m_gone = O.block_scores_given_lse(qb, kb, gone, cu, Hq, Hkv, d, n, G)
    shifted = lse.copy()
    shifted[j, h] += delta
    _, _, m_shift = O.block_scores_given_lse(qb, kb, shifted, cu, Hq, Hkv, d, n, G)
    np.testing.assert_allclose(m_shift - m0, (math.exp(-delta) - 1.0) * (m0 - m_gone),
                               rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose((m0 - m_gone).sum(), 1.0, rtol=1e-12)   # one row's weights sum to 1


# ---------------------------------------------------------------------------
# Paged key cache
# ---------------------------------------------------------------------------

def test_gather_paged_keys_inverts_a_scatter():
    """Pages built by scattering a contiguous K through a shuffled page table (pages
    of 16 tokens, partial last pages, an empty request, unused pages) gather back to
    that K exactly, and the scores computed on it are those of the contiguous K."""
    rng = np.random.default_rng(12)
    lens, ps, Hkv, d = [70, 0, 33, 16], 16, 2, 8
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    k = synth.f32_to_bf16_bits(rng.standard_normal((T, Hkv, d), dtype=np.float32))
    need = [(L + ps - 1) // ps for L in lens]
    num_pages = sum(need) + 5
    perm = rng.permutation(num_pages)
    pages = np.zeros((num_pages, ps, Hkv, d), np.uint16)
    table = np.full((len(lens), max(need)), -1, np.int64)
    nxt = 0
    for i, L in enumerate(lens):
        for pg in range(need[i]):
            table[i, pg] = perm[nxt]
            nxt += 1
            lo, hi = pg * ps, min((pg + 1) * ps, L)
            pages[table[i, pg], :hi - lo] = k[cu[i] + lo:cu[i] + hi]
    got = O.gather_paged_keys(pages, table, cu, ps)
    np.testing.assert_array_equal(got, k)
    q = synth.f32_to_bf16_bits(rng.standard_normal((sum(min(8, L) for L in lens), 4, d),
                                                   dtype=np.float32))
    a = O.block_scores(q, k, cu, 4, Hkv, d, 8, 16)[1]
    b = O.block_scores(q, got, cu, 4, Hkv, d, 8, 16)[1]
    np.testing.assert_array_equal(a, b)
