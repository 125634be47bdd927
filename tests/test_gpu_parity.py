"""GPU parity: the HIP path through the C ABI against the CPU oracle on seeded inputs.

Every test prints the case it is about to run (config, seed, shape) before its GPU
step.  Tolerances: see tests/gpu_helpers.py.
"""
import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from oracle import uniprefill_oracle as O
from workloads import synth
from tests.gpu_helpers import (GpuBatch, ambiguous_blocks, bf16_dev, check_compaction, check_keep,
                               check_packed_equals_alone, check_scores, i32_dev, run_decision,
                               say)

pytestmark = pytest.mark.gpu


def _batch(lengths, Hq, Hkv, d, n, G, needles=2, seed=0, recency=0):
    reqs = [synth.gen_request(L, Hq, Hkv, d, n, G, needles,
                              np.random.default_rng([seed, synth.TAG_VARLEN_REQUEST, i]),
                              recency=recency)
            for i, L in enumerate(lengths)]
    return synth.pack(reqs, Hq, Hkv, d, n, G)


def _full_check(batch, p, H=None, topk=None, label=""):
    say(f"[case] {label} B={batch.B} T={batch.T} Hq={batch.Hq} Hkv={batch.Hkv} d={batch.d} "
        f"n={batch.n} G={batch.G} p={p} topk={topk} H={H}")
    gb = GpuBatch(batch, H=H)
    res = run_decision(gb, p, topk=topk)
    s32, s64, _ = O.block_scores(batch.qwin, batch.k, batch.cu_seqlens, batch.Hq, batch.Hkv,
                                 batch.d, batch.n, batch.G)
    worst = check_scores(res["scores"], s64)
    if topk is None:
        ref_keep, ref_cu, _ = O.topp_select(s32, batch.cu_seqlens, batch.n, batch.G, p)
        amb = ambiguous_blocks(s32, batch.cu_seqlens, batch.n, batch.G, p)
        ndiff = check_keep(res["keep"], ref_keep, amb)
        # the GPU's cut is exactly the oracle's cut applied to the GPU's own scores
        own_keep, own_cu, _ = O.topp_select(res["scores"], batch.cu_seqlens, batch.n, batch.G, p)
    else:
        ref_keep, ref_cu = O.topk_select(s32, batch.cu_seqlens, batch.n, batch.G, topk)
        amb = set()
        ndiff = int(np.sum(res["keep"] != ref_keep))
        own_keep, own_cu = O.topk_select(res["scores"], batch.cu_seqlens, batch.n, batch.G, topk)
    np.testing.assert_array_equal(res["keep"], own_keep)
    np.testing.assert_array_equal(res["cu_out"], own_cu)
    check_compaction(gb, res)
    say(f"[ok] {label} worst score rel err {worst:.2e}; ambiguous {len(amb)}, differing {ndiff}; "
        f"kept {res['count']}/{batch.T}")
    return res, gb


SMALL_CASES = [
    # lengths, Hq, Hkv, d, n, G, p
    ([4096], 8, 2, 64, 128, 64, 0.99),            # the small single-request workload's shape
    ([1000], 4, 2, 64, 128, 64, 0.9),             # ragged last block
    ([300], 8, 2, 128, 128, 32, 0.95),            # G = 32: one 32-key stage per block
    ([2000], 4, 2, 256, 128, 64, 0.99),           # d = 256
    ([777], 4, 4, 128, 128, 128, 0.8),            # MHA (Hq = Hkv), G = 128
    ([1500], 8, 1, 64, 64, 96, 0.9),              # MQA, G = 96 (multiple of 32, not of 64)
    ([50], 4, 2, 64, 128, 64, 0.5),               # L < n: everything kept
    ([1], 4, 2, 128, 128, 64, 0.99),              # a single token
    ([129, 0, 3000, 64, 1], 8, 2, 128, 128, 64, 0.97),   # varlen with an empty request
    ([5000], 16, 2, 128, 256, 64, 0.99),          # 8-query groups, n = 256: two row tiles
    ([8192], 4, 1, 128, 128, 64, 0.99),           # one rank's heads of the Llama shape, TP = 8
    ([20000], 8, 2, 128, 100, 1024, 0.7),         # G = 1024 (largest block), window not 32-aligned
    ([7777], 4, 1, 64, 33, 512, 0.9),             # G = 512, n = 33
    ([3000], 8, 2, 256, 128, 32, 0.9),            # d = 256 with G = 32
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[f"c{i}" for i in range(len(SMALL_CASES))])
def test_small_cases_match_oracle(case):
    lengths, Hq, Hkv, d, n, G, p = case
    batch = _batch(lengths, Hq, Hkv, d, n, G, needles=2, seed=len(lengths) * 131 + d)
    _full_check(batch, p, H=256, label=f"small {case}")


def test_many_requests_full_decision():
    """150 requests of 0-700 tokens (some empty) through the whole decision: more than
    two 64-request rounds of the score pass's request lookup, the row-statistics and
    block-mass searches over many requests, the per-request select with its
    finalising scan."""
    rng = np.random.default_rng(33)
    lengths = rng.integers(0, 701, 150)
    lengths[rng.integers(0, 150, 12)] = 0
    batch = _batch([int(x) for x in lengths], 4, 2, 64, 64, 32, needles=1, seed=33)
    res, gb = _full_check(batch, 0.9, H=64, label="150 requests")
    # every request decided alone: bit-identical scores, keep flags and rows
    n = check_packed_equals_alone(gb, res, 0.9)
    say(f"[ok] 150 requests: {n} non-empty requests alone == packed, bitwise")


def test_single_4k_workload():
    cfg = synth.WORKLOADS["single_4k_h8_d64"]
    _full_check(synth.make_batch(cfg), cfg["p"], H=cfg["H"], label="single_4k_h8_d64")


@pytest.mark.parametrize("p", [0.95, 0.99, 0.999, 1.0])
def test_llama_32k_workload(p):
    cfg = synth.WORKLOADS["llama31_8b_32k"]
    _full_check(synth.make_batch(cfg), p, H=cfg["H"],
                label=f"llama31_8b_32k p={p}")


def test_topk_matches_oracle():
    cfg = synth.WORKLOADS["llama31_8b_32k"]
    for k in (1, 100, 511, 4096):
        _full_check(synth.make_batch(cfg), 0.99, H=64, topk=k, label=f"topk k={k}")


def test_select_is_bit_exact_on_oracle_scores():
    """Given identical float32 scores the GPU cut equals the oracle's exactly,
    including exact ties (zero queries) and p = 1."""
    rng = np.random.default_rng(8)
    cases = []
    lens = [4096, 700, 1, 0, 12000]
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    nbt = sum(O.n_blocks(L, 64) for L in lens)
    s = np.concatenate([rng.dirichlet(np.full(O.n_blocks(L, 64), 0.3)).astype(np.float32)
                        for L in lens if L > 0])
    cases.append((s, cu, "dirichlet"))
    # exact ties everywhere: the zero-query closed form
    qb = np.zeros((128, 2, 8), np.uint16)
    kb = synth.f32_to_bf16_bits(rng.standard_normal((4096, 1, 8), dtype=np.float32))
    cu1 = np.array([0, 4096], np.int32)
    s1, _, _ = O.block_scores(qb, kb, cu1, 2, 1, 8, 128, 64)
    cases.append((s1, cu1, "ties"))
    # large requests, up to the 16384-block limit (every slot of every thread in use)
    big = [131072, 3000 * 64, 8192 * 64 - 5, 64 * 1500, 16384 * 64]
    cub = np.zeros(len(big) + 1, np.int32)
    cub[1:] = np.cumsum(big)
    sb = np.concatenate([rng.dirichlet(np.full(O.n_blocks(L, 64), 0.5)).astype(np.float32)
                         for L in big])
    cases.append((sb, cub, "large"))
    # few distinct values: long tie runs at the cut, zeros, denormals, mixed exponents
    vals = np.array([0.0, 2e-45, 1e-40, 3e-20, 0.125 / 4096, 0.25 / 4096, 0.5 / 4096], np.float32)
    lens = [16384 * 64 - 17, 777 * 64, 64]
    cut = np.zeros(len(lens) + 1, np.int32)
    cut[1:] = np.cumsum(lens)
    st = np.concatenate([rng.choice(vals, O.n_blocks(L, 64)) for L in lens]).astype(np.float32)
    cases.append((st, cut, "tie runs"))
    # one request per slot count of the 256-thread select (2, 4, 8 and 16 per thread)
    for nb in (300, 777, 1500, 4096):
        sm = rng.dirichlet(np.full(nb, 0.4)).astype(np.float32)
        cases.append((sm, np.array([0, nb * 64 - 9], np.int32), f"one request of {nb} blocks"))
    # a single block holding all the mass (score exactly 1.0) among zeros
    s1b = np.zeros(9000, np.float32)
    s1b[4321] = 1.0
    cases.append((s1b, np.array([0, 9000 * 64], np.int32), "one-hot"))
    for s, c, name in cases:
        for p in (1e-6, 0.3, 0.9, 0.95, 0.99, 0.999, 1.0):
            say(f"[case] select {name} p={p} nb={s.size}")
            keep, cu_out = up.topp_select(torch.from_numpy(s).cuda(), i32_dev(c), c, 128, 64, p)
            torch.cuda.synchronize()
            ref_keep, ref_cu, _ = O.topp_select(s, c, 128, 64, p)
            np.testing.assert_array_equal(keep.cpu().numpy(), ref_keep)
            np.testing.assert_array_equal(cu_out.cpu().numpy(), ref_cu)
        nbs = np.diff(np.array([0] + [O.n_blocks(int(L), 64) for L in np.diff(c)]).cumsum())
        for k in (0, 1, 7, int(nbs.max()) // 3, int(nbs.max()) - 1, int(nbs.max()) + 5):
            say(f"[case] topk select {name} k={k} nb={s.size}")
            keep, cu_out = up.topk_select(torch.from_numpy(s).cuda(), i32_dev(c), c, 128, 64, k)
            torch.cuda.synchronize()
            ref_keep, ref_cu = O.topk_select(s, c, 128, 64, k)
            np.testing.assert_array_equal(keep.cpu().numpy(), ref_keep)
            np.testing.assert_array_equal(cu_out.cpu().numpy(), ref_cu)
    # exact boundaries: a running sum equal to p counts as reaching it
    s = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    c = np.array([0, 4 * 64], np.int32)
    for p in (0.5, 0.75, 0.875, 0.8750001):
        keep, _ = up.topp_select(torch.from_numpy(s).cuda(), i32_dev(c), c, 1, 64, p)
        ref_keep, _, _ = O.topp_select(s, c, 1, 64, p)
        np.testing.assert_array_equal(keep.cpu().numpy(), ref_keep)
    assert up.device_error() == 0


def test_zero_queries_give_exact_ties_on_gpu():
    """Q = 0: early blocks must get bit-identical scores and the cut the closed form's k*."""
    L, n, G, Hq, p = 4096, 128, 64, 2, 0.95
    qb = np.zeros((n, Hq, 128), np.uint16)
    rng = np.random.default_rng(3)
    kb = synth.f32_to_bf16_bits(rng.standard_normal((L, 1, 128), dtype=np.float32))
    batch = synth.Batch(cu_seqlens=np.array([0, L], np.int32), qwin=qb, k=kb, Hq=Hq, Hkv=1,
                        d=128, n=n, G=G)
    say("[case] zero queries L=4096 d=128")
    gb = GpuBatch(batch, H=64)
    res = run_decision(gb, p)
    s = res["scores"]
    early = [b for b in range(L // G) if (b + 1) * G - 1 <= L - n]
    assert len({float(s[b]) for b in early}) == 1
    s32, s64, _ = O.block_scores(qb, kb, batch.cu_seqlens, Hq, 1, 128, n, G)
    check_scores(s, s64)
    ref_keep, _, _ = O.topp_select(s32, batch.cu_seqlens, n, G, p)
    np.testing.assert_array_equal(res["keep"], ref_keep)
    check_compaction(gb, res)


@pytest.mark.parametrize("lengths", [[0], [0, 0, 0]])
@pytest.mark.parametrize("separate", [False, True])
def test_all_empty_batch_decides_nothing(lengths, separate):
    """Every request empty (T = 0): the decision writes cu_seqlens_out = 0 and nothing
    else, through the one-call entry and through the three separate calls (the
    zero-length buffers are passed as whatever torch gives for empty tensors)."""
    say(f"[case] all-empty batch {lengths} separate={separate}")
    batch = _batch(lengths, 8, 2, 128, 128, 64, seed=11)
    assert batch.T == 0
    gb = GpuBatch(batch, H=64)
    b = gb.b
    dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, 0.9,
                           separate=separate)
    dec.cu_out.fill_(-7)
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    assert dec.cu_out.cpu().tolist() == [0] * (len(lengths) + 1)


def test_runs_are_bitwise_reproducible():
    cfg = synth.WORKLOADS["single_4k_h8_d64"]
    batch = synth.make_batch(cfg)
    say("[case] determinism single_4k_h8_d64")
    gb = GpuBatch(batch, H=cfg["H"])
    a = run_decision(gb, cfg["p"])
    b = run_decision(gb, cfg["p"])
    assert np.array_equal(a["scores"].view(np.uint32), b["scores"].view(np.uint32))
    assert np.array_equal(a["keep"], b["keep"])
    assert torch.equal(a["dec"].hidden_out, b["dec"].hidden_out)


def test_inconsistent_device_cu_seqlens_raises_error_word():
    """Device cu_seqlens disagreeing with the host copy: kernels do nothing, error bit 1."""
    cfg = synth.WORKLOADS["single_4k_h8_d64"]
    batch = synth.make_batch(cfg)
    gb = GpuBatch(batch, H=cfg["H"])
    say("[case] inconsistent cu_seqlens")
    up.device_error()
    bad_cu = i32_dev(np.array([0, 4000], np.int32))
    scores = torch.full((64,), -7.0, device="cuda")
    up.block_scores(gb.qwin, gb.k, bad_cu, gb.cu_h, batch.n, batch.G, out=scores)
    torch.cuda.synchronize()
    assert up.device_error() & 1
    assert torch.all(scores == -7.0)
    # compose: out-of-range indices give -1 and raise bit 2
    prev = i32_dev(np.arange(10, dtype=np.int32))
    idx = i32_dev(np.array([0, 9, 10, -1], np.int32))
    cnt = i32_dev(np.array([4], np.int32))
    out = up.compose_drops(prev, idx, cnt)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tolist() == [0, 9, -1, -1]
    assert up.device_error() & 2


def test_inconsistent_compaction_inputs_write_nothing():
    """expand_compact and select on device inputs that disagree with the host copy or
    with each other: nothing is written and error bit 1 is raised."""
    G, T, H = 64, 4096, 64
    cu_h = np.array([0, T], np.int32)
    rng = np.random.default_rng(5)
    hid = bf16_dev(rng.integers(0, 1 << 15, (T, H)).astype(np.uint16))
    pos = i32_dev(np.arange(T, dtype=np.int32))
    keep = torch.ones(T // G, dtype=torch.uint8, device="cuda")
    keep[3] = 0
    good_out = i32_dev(np.array([0, T - G], np.int32))
    cases = {
        "cu_out disagrees with keep": (i32_dev(cu_h), i32_dev(np.array([0, T], np.int32))),
        "device cu disagrees with host": (i32_dev(np.array([0, T - 5], np.int32)), good_out),
        "cu_out[0] not zero": (i32_dev(cu_h), i32_dev(np.array([G, T], np.int32))),
    }
    up.device_error()
    for name, (cu_d, cu_out_d) in cases.items():
        say(f"[case] compaction: {name}")
        idx_out = torch.full((T,), -9, dtype=torch.int32, device="cuda")
        hid_out = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
        pos_out = torch.full((T,), -9, dtype=torch.int32, device="cuda")
        up.expand_compact(hid, pos, keep, cu_d, cu_out_d, cu_h, G, idx_out=idx_out,
                          hidden_out=hid_out, pos_out=pos_out)
        torch.cuda.synchronize()
        assert up.device_error() & 1, name
        assert torch.all(idx_out == -9) and torch.all(pos_out == -9), name
        assert torch.all(hid_out.view(torch.int16) == 0), name
    # the consistent call on the same buffers compacts (one dropped block)
    idx_out, hid_out, pos_out = up.expand_compact(hid, pos, keep, i32_dev(cu_h), good_out, cu_h,
                                                  G)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    want = np.concatenate([np.arange(3 * G), np.arange(4 * G, T)]).astype(np.int32)
    np.testing.assert_array_equal(idx_out[:T - G].cpu().numpy(), want)
    np.testing.assert_array_equal(pos_out[:T - G].cpu().numpy(), want)
    # select with a device cu_seqlens that disagrees with the host copy
    say("[case] select: device cu disagrees with host")
    sc = torch.full((T // G,), 1.0 / (T // G), device="cuda")
    keep2 = torch.full((T // G,), 7, dtype=torch.uint8, device="cuda")
    for fn, arg in ((up.topp_select, 0.9), (up.topk_select, 5)):
        fn(sc, i32_dev(np.array([0, T - 5], np.int32)), cu_h, 128, G, arg, keep=keep2)
        torch.cuda.synchronize()
        assert up.device_error() & 1
        assert torch.all(keep2 == 7)


@pytest.mark.parametrize("dtype,H", [(torch.uint8, 33), (torch.float32, 3), (torch.bfloat16, 6),
                                     (torch.float64, 5), (torch.int16, 4096)])
def test_compaction_of_rows_of_any_width(dtype, H):
    """Rows whose byte width is not a multiple of 16 (or of 4) take the gather's 4-byte
    and 1-byte paths; every width must give the rows the oracle's expansion names, bit
    for bit, with positions and composed indices."""
    G, lens = 64, [1000, 0, 777, 64, 3000]
    cu_h = np.zeros(len(lens) + 1, np.int32)
    cu_h[1:] = np.cumsum(lens)
    T = int(cu_h[-1])
    nbs = [O.n_blocks(L, G) for L in lens]
    rng = np.random.default_rng(H)
    keep = (rng.random(sum(nbs)) < 0.6).astype(np.uint8)
    cnt = [0] + [int(sum(min(G, L - b * G) for b in range(nb) if keep[sum(nbs[:i]) + b]))
                 for i, (L, nb) in enumerate(zip(lens, nbs))]
    cu_out = np.cumsum(cnt).astype(np.int32)
    raw = rng.integers(0, 256, (T, H * torch.tensor([], dtype=dtype).element_size()),
                       dtype=np.uint8)
    hid = torch.from_numpy(raw).cuda().view(dtype).view(T, H)
    pos = rng.integers(0, 1 << 30, T).astype(np.int32)
    prev = rng.integers(0, 1 << 30, T).astype(np.int32)
    say(f"[case] compaction of {H} x {dtype} rows ({hid.element_size() * H} bytes)")
    orig = torch.empty(T, dtype=torch.int32, device="cuda")
    idx_out, hid_out, pos_out = up.expand_compact(
        hid, i32_dev(pos), torch.from_numpy(keep).cuda(), i32_dev(cu_h), i32_dev(cu_out), cu_h, G,
        prev_orig=i32_dev(prev), orig_out=orig)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    idx_ref = O.expand(keep, cu_h, G)
    n = int(cu_out[-1])
    assert idx_ref.size == n
    np.testing.assert_array_equal(idx_out[:n].cpu().numpy(), idx_ref)
    got = hid_out[:n].contiguous().view(torch.uint8).view(n, -1).cpu().numpy()
    np.testing.assert_array_equal(got, raw[idx_ref])
    np.testing.assert_array_equal(pos_out[:n].cpu().numpy(), pos[idx_ref])
    np.testing.assert_array_equal(orig[:n].cpu().numpy(), prev[idx_ref])


def test_many_short_requests_select_and_compact():
    """2500 requests (more than one 1024-request chunk of the compaction scan), lengths
    0..300 with empty ones, G = 32: select and compaction against the oracle."""
    rng = np.random.default_rng(21)
    B, G, n, H = 2500, 32, 64, 32
    lens = rng.integers(0, 301, B)
    lens[rng.integers(0, B, 200)] = 0
    cu_h = np.zeros(B + 1, np.int32)
    cu_h[1:] = np.cumsum(lens)
    T = int(cu_h[-1])
    nbs = [O.n_blocks(int(L), G) for L in lens]
    s = np.concatenate([rng.dirichlet(np.full(k, 0.4)).astype(np.float32) if k else
                        np.zeros(0, np.float32) for k in nbs])
    say(f"[case] many short requests: B={B} T={T} blocks={s.size}")
    cu_d = i32_dev(cu_h)
    keep, cu_out = up.topp_select(torch.from_numpy(s).cuda(), cu_d, cu_h, n, G, 0.7)
    torch.cuda.synchronize()
    ref_keep, ref_cu, _ = O.topp_select(s, cu_h, n, G, 0.7)
    np.testing.assert_array_equal(keep.cpu().numpy(), ref_keep)
    np.testing.assert_array_equal(cu_out.cpu().numpy(), ref_cu)
    hid_np = rng.integers(0, 1 << 15, (T, H)).astype(np.uint16)
    pos_np = rng.integers(0, 1 << 30, T).astype(np.int32)
    idx_out, hid_out, pos_out = up.expand_compact(bf16_dev(hid_np), i32_dev(pos_np), keep, cu_d,
                                                  cu_out, cu_h, G)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    idx_ref = O.expand(ref_keep.astype(np.uint8), cu_h, G)
    cnt = int(ref_cu[-1])
    assert cnt == idx_ref.size
    np.testing.assert_array_equal(idx_out[:cnt].cpu().numpy(), idx_ref)
    h_ref, p_ref = O.compact_fast(hid_np, pos_np, idx_ref)
    np.testing.assert_array_equal(hid_out[:cnt].view(torch.int16).cpu().numpy().view(np.uint16),
                                  h_ref)
    np.testing.assert_array_equal(pos_out[:cnt].cpu().numpy(), p_ref)


def test_compose_drops_standalone_matches_oracle():
    """up_compose_drops on its own (the decision fuses it into the compaction pass):
    30000 survivors of 50000 rows through a scrambled original-index table."""
    rng = np.random.default_rng(9)
    prev_len, cnt, cap = 50000, 30000, 40000
    prev = rng.permutation(1_000_000)[:prev_len].astype(np.int32)
    idx = np.sort(rng.choice(prev_len, cnt, replace=False)).astype(np.int32)
    idx_full = np.full(cap, -5, np.int32)
    idx_full[:cnt] = idx
    say("[case] compose_drops standalone")
    up.device_error()
    out = up.compose_drops(i32_dev(prev), i32_dev(idx_full), i32_dev(np.array([cnt], np.int32)),
                           capacity=cap)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    np.testing.assert_array_equal(out[:cnt].cpu().numpy(), O.compose(prev, idx))


def _random_configs(count=24, seed=2026):
    """Seeded draws over the supported argument space: 1-5 requests of 0-4000 tokens
    (empty and one-token requests included), GQA group sizes 1, 2, 3, 4 and 8, every
    head dimension, window sizes 1-300, every block size 32-1024 in steps of 32, p in
    [0.3, 1] and, for a quarter of the cases, a Top-k cut with k anywhere from 0 to past
    the longest request's block count."""
    rng = np.random.default_rng(seed)
    heads = [(8, 2), (4, 1), (4, 4), (12, 4), (6, 2), (16, 2), (2, 1), (3, 3)]
    out = []
    while len(out) < count:
        B = int(rng.integers(1, 6))
        lengths = [int(x) for x in rng.integers(0, 4001, B)]
        for j in range(B):
            r = rng.random()
            if r < 0.1:
                lengths[j] = 0
            elif r < 0.2:
                lengths[j] = int(rng.integers(1, 40))
        Hq, Hkv = heads[int(rng.integers(len(heads)))]
        d = int(rng.choice([64, 128, 256]))
        n = int(rng.integers(1, 301))
        G = 32 * int(rng.integers(1, 33))
        p = 1.0 if rng.random() < 0.1 else float(np.float32(rng.uniform(0.3, 0.999)))
        nb_max = max((L + G - 1) // G for L in lengths)
        topk = int(rng.integers(0, nb_max + 4)) if rng.random() < 0.25 else None
        # keep the float64 oracle to about a second per case
        if sum(L * Hq * min(L, n) * d for L in lengths) > 1.2e9:
            continue
        out.append((lengths, Hq, Hkv, d, n, G, p, topk, int(rng.integers(1 << 30))))
    return out


RANDOM_CASES = _random_configs()


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"r{i}" for i in range(len(RANDOM_CASES))])
def test_random_configurations_match_oracle(case):
    lengths, Hq, Hkv, d, n, G, p, topk, seed = case
    batch = _batch(lengths, Hq, Hkv, d, n, G, needles=int(seed % 4), seed=seed,
                   recency=int(seed % 3) * 16)
    _full_check(batch, p, H=int(8 + seed % 57), topk=topk, label=f"random {case}")
