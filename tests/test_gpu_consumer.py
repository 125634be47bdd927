"""GPU parity of the layer on the surviving tokens against the consumer oracle.

Tolerances, derived from the arithmetic:
  * attention: the rotated q and k are the same bfloat16 values on both sides; the
    GPU rounds each probability to bfloat16 for the P.V product (relative error
    <= 2^-9, so an output row moves by <= 2^-9 max|v|) and rounds the output to
    bfloat16 (<= 2^-9 relative); logits and statistics in float32 add ~1e-5.  Bar:
    |gpu - oracle| <= 2^-8 |oracle| + 2^-8 max|v| (per request and kv head);
  * GEMM: float32 accumulation and one bfloat16 rounding of the result:
    |gpu - oracle| <= 2^-8 |oracle| + 1e-5 sum_k |x_k w_k|;
  * SwiGLU gate: float32 math and one bfloat16 rounding: <= 2^-8 relative to the
    exact value (plus 1e-30);
  * FFN: as the GEMM, with the gated activation allowed to move by 2^-7 relative
    per element (its bfloat16 rounding and that of x.w_gu^T before it):
    |gpu - oracle| <= 2^-8 |oracle| + 2^-7 sum_j |a_j w_j|.
"""
import math

import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from oracle import consumer_oracle as C
from tests.gpu_helpers import bf16_dev, i32_dev, say
from workloads import synth

pytestmark = pytest.mark.gpu


def _to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


CASES = [
    # lengths, Hq, Hkv, d, q_sigma
    ([200], 8, 2, 128, 1.0),
    ([64], 4, 1, 64, 1.0),                     # Hq / Hkv = 4, d = 64
    ([1], 8, 2, 128, 1.0),                     # one row
    ([300, 0, 65, 129, 1], 8, 2, 128, 1.0),    # varlen, empty and ragged requests
    ([257], 8, 8, 128, 1.0),                   # one query head per kv head: 4 tiles per workgroup
    ([190], 8, 4, 64, 1.0),                    # two query heads per kv head: 2 tiles per workgroup
    ([150], 16, 2, 128, 1.0),                  # eight per kv head: two workgroups per kv head
    ([700], 8, 2, 128, 12.0),                  # large logits: the reference rebases often
    ([513], 4, 2, 64, 30.0),                   # very large logits, nearly one-hot rows
    ([200], 16, 8, 256, 1.0),                  # d = 256, Gemma-like GQA: 32-token tiles
    ([300, 0, 65, 129, 1], 8, 2, 256, 1.0),    # d = 256, varlen with empty and ragged requests
    ([130], 8, 8, 256, 1.0),                   # d = 256, one query head per kv head
    ([190], 16, 4, 256, 1.0),                  # d = 256, four query heads per kv head
    ([700], 4, 2, 256, 12.0),                  # d = 256, large logits: many rebases
]


def _attention_case(lengths, Hq, Hkv, d, sigma, seed, theta=500000.0):
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, seed, q_sigma=sigma)
    R = int(cu[-1])
    scale = 1.0 / math.sqrt(d)
    out = up.rope_attention(bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d),
                            bf16_dev(v).view(R, Hkv, d), i32_dev(pos), i32_dev(cu), cu,
                            scale=scale, rope_theta=theta)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    return q, k, v, pos, cu, scale, _to_f64(out)


def _check_attention(got, ref, vmax_rows, Hq, Hkv):
    g = Hq // Hkv
    vm = np.repeat(vmax_rows, g, axis=1)[:, :, None]          # [R, Hq, 1]
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -8 * vm
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{int(bad.sum())} elements over the bar; worst excess "
                           f"{float((err - tol).max()):.3e}")
    return float((err / np.maximum(tol, 1e-30)).max())


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_rope_attention_matches_oracle(case):
    lengths, Hq, Hkv, d, sigma = case
    say(f"[case] rope_attention {case}")
    q, k, v, pos, cu, scale, got = _attention_case(lengths, Hq, Hkv, d, sigma, seed=len(lengths) + d)
    ref = C.rope_attention(q, k, v, pos, cu, Hq, Hkv, d, scale, 500000.0)
    worst = _check_attention(got, ref, C.attention_vmax(v, cu, Hkv, d), Hq, Hkv)
    say(f"[ok] {case}: worst error / bar {worst:.3f}")


def _random_attention_configs(count=16, seed=909):
    """Seeded draws: 1-4 requests of 0-900 survivors, GQA group sizes 1, 2, 3, 4, 6 and
    8 (3 and 6 take one query head per tile row group), every head dimension, logit
    scales from plain to nearly one-hot, and rotary bases 1e4, 5e5 and 1e6."""
    rng = np.random.default_rng(seed)
    heads = [(8, 2), (4, 1), (8, 8), (16, 2), (12, 4), (12, 2), (6, 2), (4, 2)]
    out = []
    while len(out) < count:
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(0, 901, B)]
        Hq, Hkv = heads[int(rng.integers(len(heads)))]
        d = int(rng.choice([64, 128, 256]))
        if sum(L * L for L in lengths) * Hq * d > 1.5e9:   # keeps the oracle near a second
            continue
        out.append((lengths, Hq, Hkv, d, float(rng.choice([1.0, 4.0, 15.0])),
                    float(rng.choice([1e4, 5e5, 1e6])), int(rng.integers(1 << 30))))
    return out


RANDOM_ATTENTION = _random_attention_configs()


@pytest.mark.parametrize("case", RANDOM_ATTENTION,
                         ids=[f"r{i}" for i in range(len(RANDOM_ATTENTION))])
def test_random_attention_configurations_match_oracle(case):
    lengths, Hq, Hkv, d, sigma, theta, seed = case
    say(f"[case] random rope_attention {case}")
    q, k, v, pos, cu, scale, got = _attention_case(lengths, Hq, Hkv, d, sigma, seed=seed,
                                                   theta=theta)
    ref = C.rope_attention(q, k, v, pos, cu, Hq, Hkv, d, scale, theta)
    worst = _check_attention(got, ref, C.attention_vmax(v, cu, Hkv, d), Hq, Hkv)
    say(f"[ok] random {case}: worst error / bar {worst:.3f}")


def test_rope_attention_over_many_requests():
    """120 short requests (0-150 survivors, some empty): the plan's padded offsets and
    tile offsets over many requests and the tile-to-request search."""
    rng = np.random.default_rng(44)
    lengths = [int(x) for x in rng.integers(0, 151, 120)]
    for j in rng.integers(0, 120, 10):
        lengths[int(j)] = 0
    Hq, Hkv, d = 8, 2, 64
    say(f"[case] rope_attention over {len(lengths)} requests, {sum(lengths)} rows")
    q, k, v, pos, cu, scale, got = _attention_case(lengths, Hq, Hkv, d, 1.0, seed=44)
    ref = C.rope_attention(q, k, v, pos, cu, Hq, Hkv, d, scale, 500000.0)
    worst = _check_attention(got, ref, C.attention_vmax(v, cu, Hkv, d), Hq, Hkv)
    say(f"[ok] many requests: worst error / bar {worst:.3f}")


def test_rope_attention_uses_the_carried_positions():
    """Renumbering the survivors 0..R-1 changes the output; the GPU follows the carried
    positions (checked against the oracle at both)."""
    lengths, Hq, Hkv, d = [256], 8, 2, 128
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, 5)
    assert np.any(np.diff(pos) > 1)
    R = int(cu[-1])
    outs = {}
    for name, p in (("carried", pos), ("renumbered", np.arange(R, dtype=np.int32))):
        o = up.rope_attention(bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d),
                              bf16_dev(v).view(R, Hkv, d), i32_dev(p), i32_dev(cu), cu)
        torch.cuda.synchronize()
        ref = C.rope_attention(q, k, v, p, cu, Hq, Hkv, d, 1 / math.sqrt(d), 500000.0)
        _check_attention(_to_f64(o), ref, C.attention_vmax(v, cu, Hkv, d), Hq, Hkv)
        outs[name] = _to_f64(o)
    assert np.abs(outs["carried"] - outs["renumbered"]).max() > 1e-2


def test_rope_attention_is_deterministic_and_rejects_bad_cu():
    lengths, Hq, Hkv, d = [1000, 37], 8, 2, 128
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, 9)
    R = int(cu[-1])
    args = (bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d), bf16_dev(v).view(R, Hkv, d),
            i32_dev(pos))
    a = up.rope_attention(*args, i32_dev(cu), cu)
    b = up.rope_attention(*args, i32_dev(cu), cu)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # a device cu_seqlens whose totals disagree with the host copy (18 workgroup tiles
    # and 1152 padded rows instead of 17 and 1088): nothing written, bit 1 raised
    bad = cu.copy()
    bad[1] = 970
    pad = lambda c: sum(-(-int(L) // 64) * 64 for L in np.diff(c))
    assert pad(bad) != pad(cu)
    out = torch.full_like(a, 7.0)
    up.rope_attention(*args, i32_dev(bad), cu, out=out)
    torch.cuda.synchronize()
    assert up.device_error() == 1
    assert bool((out == 7.0).all())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("R,Hq,Hkv,d", [(129600, 32, 8, 128), (129344, 16, 8, 256)],
                         ids=["llama_d128", "gemma_like_d256"])
def test_rope_attention_at_128k_sampled_rows(R, Hq, Hkv, d):
    """The Llama-3.1-8B shape at 129600 survivors and the Gemma-like d = 256 shape at
    129344 (what p = 0.99 keeps of 128K in each): sampled rows of the GPU output against
    the oracle computed for those rows alone."""
    say(f"[setup] generating {R} survivors, Hq={Hq}, Hkv={Hkv}, d={d}")
    q, k, v, pos, cu = synth.gen_consumer_attention([R], Hq, Hkv, d, 2026)
    out = up.rope_attention(bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d),
                            bf16_dev(v).view(R, Hkv, d), i32_dev(pos), i32_dev(cu), cu)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    rows = [0, 1, 31, 32, 63, 64, 4095, 65536, 100003, R - 65, R - 33, R - 2, R - 1]
    got = out[rows].float().cpu().numpy().astype(np.float64)
    say("[setup] oracle on sampled rows")
    ref = C.rope_attention_rows(q, k, v, pos, cu, Hq, Hkv, d, 1 / math.sqrt(d), 500000.0, rows)
    vmax = np.abs(C.bits_to_f64(v).reshape(R, Hkv, d)).max(axis=(0, 2))[None, :]
    worst = _check_attention(got, ref, np.repeat(vmax, len(rows), axis=0), Hq, Hkv)
    say(f"[ok] 128K sampled rows: worst error / bar {worst:.3f}")


@pytest.mark.timeout(900)
def test_rope_attention_varlen_sampled_rows():
    """Eight requests of 8K-64K survivors (the continuous-batching shape), Hq=8, Hkv=2,
    d=128: sampled rows at the start, middle and end of every request against the
    oracle computed for those rows."""
    lengths = synth.varlen_lengths(11, 8, 8192, 65536)
    Hq, Hkv, d = 8, 2, 128
    say(f"[setup] varlen survivors {lengths}")
    q, k, v, pos, cu = synth.gen_consumer_attention(lengths, Hq, Hkv, d, 77)
    R = int(cu[-1])
    out = up.rope_attention(bf16_dev(q).view(R, Hq, d), bf16_dev(k).view(R, Hkv, d),
                            bf16_dev(v).view(R, Hkv, d), i32_dev(pos), i32_dev(cu), cu)
    torch.cuda.synchronize()
    assert up.device_error() == 0
    rows = []
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        rows += [a, a + 63, (a + b) // 2, b - 1]
    got = out[rows].float().cpu().numpy().astype(np.float64)
    ref = C.rope_attention_rows(q, k, v, pos, cu, Hq, Hkv, d, 1 / math.sqrt(d), 500000.0, rows)
    vmax = C.attention_vmax(v, cu, Hkv, d)[rows]
    worst = _check_attention(got, ref, vmax, Hq, Hkv)
    say(f"[ok] varlen {R} rows: worst error / bar {worst:.3f}")


@pytest.mark.parametrize("R,K,N,res", [(300, 256, 512, False), (1, 128, 64, True),
                                       (4099, 4096, 1024, True)])
def test_linear_matches_oracle(R, K, N, res):
    say(f"[case] linear R={R} K={K} N={N} residual={res}")
    rng = np.random.default_rng(R + K)
    x = synth.f32_to_bf16_bits(rng.standard_normal((R, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    r = synth.f32_to_bf16_bits(rng.standard_normal((R, N)).astype(np.float32)) if res else None
    y = up.linear(bf16_dev(x).view(R, K), bf16_dev(w).view(N, K),
                  residual=None if r is None else bf16_dev(r).view(R, N))
    torch.cuda.synchronize()
    ref = C.linear(x, w) + (0 if r is None else C.bits_to_f64(r))
    mag = np.abs(C.bits_to_f64(x)) @ np.abs(C.bits_to_f64(w)).T
    err = np.abs(_to_f64(y) - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-5 * mag + 1e-30).all()


def test_swiglu_matches_oracle():
    rng = np.random.default_rng(3)
    R, F = 517, 1032
    gu = synth.f32_to_bf16_bits((rng.standard_normal((R, 2 * F)) * 3).astype(np.float32))
    a = up.swiglu(bf16_dev(gu).view(R, 2 * F))
    torch.cuda.synchronize()
    g = C.bits_to_f64(gu)
    exact = C.silu(g[:, :F]) * g[:, F:]
    assert (np.abs(_to_f64(a) - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30).all()


@pytest.mark.parametrize("R,H,F", [(300, 256, 512), (64, 4096, 14336)])
def test_swiglu_ffn_matches_oracle(R, H, F):
    say(f"[case] swiglu_ffn R={R} H={H} F={F}")
    x, wgu, wd, res = synth.gen_ffn(R, H, F, seed=R)
    y = up.swiglu_ffn(bf16_dev(x).view(R, H), bf16_dev(wgu).view(2 * F, H), bf16_dev(wd).view(H, F),
                      residual=bf16_dev(res).view(R, H))
    torch.cuda.synchronize()
    ref, _, a = C.ffn(x, wgu, wd, F, residual_bits=res)
    mag = np.abs(a) @ np.abs(C.bits_to_f64(wd)).T
    err = np.abs(_to_f64(y) - ref)
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -7 * mag + 1e-30
    assert (err <= tol).all(), f"worst excess {float((err - tol).max()):.3e}"


def _random_dense_shapes(seed=515):
    """Seeded draws for the dense calls: GEMMs of 1-3000 rows with K and N multiples of 8
    up to 2048 (half with a residual), gates of 1-2000 rows with F a multiple of 8 up to
    3000, and FFNs of 1-700 rows with H a multiple of 64 and F a multiple of 8."""
    rng = np.random.default_rng(seed)
    lin = [(int(rng.integers(1, 3001)), 8 * int(rng.integers(1, 257)), 8 * int(rng.integers(1, 257)),
            bool(rng.random() < 0.5)) for _ in range(8)]
    gate = [(int(rng.integers(1, 2001)), 8 * int(rng.integers(1, 376))) for _ in range(6)]
    ffn = [(int(rng.integers(1, 701)), 64 * int(rng.integers(1, 17)), 8 * int(rng.integers(1, 257)))
           for _ in range(4)]
    return lin, gate, ffn


RANDOM_LIN, RANDOM_GATE, RANDOM_FFN = _random_dense_shapes()


@pytest.mark.parametrize("R,K,N,res", RANDOM_LIN, ids=[f"r{i}" for i in range(len(RANDOM_LIN))])
def test_random_linear_shapes(R, K, N, res):
    test_linear_matches_oracle(R, K, N, res)


@pytest.mark.parametrize("R,F", RANDOM_GATE, ids=[f"r{i}" for i in range(len(RANDOM_GATE))])
def test_random_swiglu_shapes(R, F):
    say(f"[case] swiglu R={R} F={F}")
    rng = np.random.default_rng(R * 7 + F)
    gu = synth.f32_to_bf16_bits((rng.standard_normal((R, 2 * F)) * 3).astype(np.float32))
    a = up.swiglu(bf16_dev(gu).view(R, 2 * F))
    torch.cuda.synchronize()
    g = C.bits_to_f64(gu)
    exact = C.silu(g[:, :F]) * g[:, F:]
    assert (np.abs(_to_f64(a) - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30).all()


@pytest.mark.parametrize("R,H,F", RANDOM_FFN, ids=[f"r{i}" for i in range(len(RANDOM_FFN))])
def test_random_swiglu_ffn_shapes(R, H, F):
    test_swiglu_ffn_matches_oracle(R, H, F)
