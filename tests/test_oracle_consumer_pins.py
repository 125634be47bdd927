"""Pins of the consumer oracle (oracle/consumer_oracle.py) to facts outside itself:
closed forms, a library routine, brute force on tiny inputs and invariants of the
rotary embedding.  CPU only."""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import consumer_oracle as C


def _bf16_bits(rng, shape, sigma=1.0):
    f = (rng.standard_normal(shape) * sigma).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# --- bfloat16 rounding (reading C4) -------------------------------------------

def test_round_bf16_ties_go_to_even():
    one = 1.0
    ulp = 2.0 ** -7                      # bfloat16 spacing in [1, 2)
    cases = {
        one: one,
        one + ulp / 2: one,              # tie, 1.0 has an even mantissa
        one + 3 * ulp / 2: one + 2 * ulp,  # tie, rounds up to the even neighbour
        one + ulp / 2 + 2.0 ** -30: one + ulp,   # just above the tie
        one + ulp / 2 - 2.0 ** -30: one,          # just below the tie
        -(one + ulp / 2): -one,
        2.0 ** -130: 2.0 ** -130,        # a bfloat16 subnormal, exact
        2.0 ** -134: 0.0,                # half of the subnormal step: tie to even (0)
        3 * 2.0 ** -134: 2.0 ** -132,    # 1.5 steps: tie, rounds to the even 2 steps
        0.0: 0.0,
    }
    got = C.round_bf16(np.array(list(cases)))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))


def test_round_bf16_matches_float32_bit_rounding():
    """For float32 inputs the result must equal the usual float32 -> bfloat16 rounding
    done on the 32-bit pattern (add 0x7FFF plus the kept LSB, drop 16 bits)."""
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    ref = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(C.round_bf16(f.astype(np.float64)), ref.astype(np.float64))


# --- rotary embedding (reading C2) ---------------------------------------------

def test_rope_d2_is_a_complex_rotation_by_pos_radians():
    """d = 2: one pair with frequency theta^0 = 1, so the pair turns by pos radians."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 3, 2))
    pos = rng.integers(0, 200000, 50)
    z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos.astype(np.float64))[:, None]
    got = C.rope(x, pos, theta=10000.0)
    np.testing.assert_allclose(got[..., 0], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., 1], z.imag, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d,theta", [(8, 10000.0), (64, 500000.0), (128, 500000.0)])
def test_rope_pairs_i_with_i_plus_half_d(d, theta):
    """Pair (x_i, x_{i+d/2}) as the complex number x_i + j x_{i+d/2}; the rotation is
    multiplication by exp(j pos w_i) with w_i = exp(-(2i/d) ln theta)."""
    rng = np.random.default_rng(d)
    x = rng.standard_normal((40, 2, d))
    pos = rng.integers(0, 131072, 40)
    w = np.exp(-(2.0 * np.arange(d // 2) / d) * math.log(theta))
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * np.outer(pos, w))[:, None, :]
    got = C.rope(x, pos, theta)
    np.testing.assert_allclose(got[..., : d // 2], z.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(got[..., d // 2:], z.imag, rtol=0, atol=1e-9)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    d = 128
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    # identity at position 0; norms preserved
    np.testing.assert_array_equal(C.rope(q, np.array([0]), 500000.0), q)
    r = C.rope(q, np.array([123457]), 500000.0)
    assert abs(np.linalg.norm(r) - np.linalg.norm(q)) < 1e-12
    # the product of a rotated query and key depends only on their distance
    for p1, p2, delta in [(1000, 10, 77777), (5, 5, 131000), (65536, 0, 1)]:
        a = float(np.sum(C.rope(q, np.array([p1]), 500000.0) * C.rope(k, np.array([p2]), 500000.0)))
        b = float(np.sum(C.rope(q, np.array([p1 + delta]), 500000.0)
                         * C.rope(k, np.array([p2 + delta]), 500000.0)))
        assert abs(a - b) <= 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)


# --- attention over the survivors (readings C2, C3) -----------------------------

def _packed(rng, lengths, Hq, Hkv, d, gaps=True):
    R = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    q = _bf16_bits(rng, (R, Hq, d))
    k = _bf16_bits(rng, (R, Hkv, d))
    v = _bf16_bits(rng, (R, Hkv, d))
    pos = np.zeros(R, dtype=np.int64)
    for i, L in enumerate(lengths):
        if L == 0:
            continue
        step = rng.integers(1, 5, L) if gaps else np.ones(L, dtype=np.int64)
        pos[cu[i]:cu[i + 1]] = np.cumsum(step) - step[0]
    return q, k, v, pos, cu


def test_zero_queries_give_the_running_mean_of_values():
    """q = 0: every causal logit is 0, so row t is the plain mean of v over keys 0..t."""
    rng = np.random.default_rng(3)
    L, Hq, Hkv, d = 37, 4, 2, 16
    q, k, v, pos, cu = _packed(rng, [L], Hq, Hkv, d)
    q[:] = 0
    out = C.rope_attention(q, k, v, pos, cu, Hq, Hkv, d, 1 / math.sqrt(d), 10000.0)
    vf = C.bits_to_f64(v).reshape(L, Hkv, d)
    mean = np.cumsum(vf, axis=0) / np.arange(1, L + 1)[:, None, None]
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], mean[:, h // 2], rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_on_the_rotated_operands():
    """Library routine: torch's CPU scaled_dot_product_attention in float64 with a
    causal mask, given the same rotated and rounded q and k, per request."""
    rng = np.random.default_rng(4)
    lengths, Hq, Hkv, d = [50, 1, 130], 8, 2, 32
    q, k, v, pos, cu = _packed(rng, lengths, Hq, Hkv, d)
    scale, theta = 0.17, 500000.0
    out = C.rope_attention(q, k, v, pos, cu, Hq, Hkv, d, scale, theta)
    qr = C.rotate_bf16(q, pos, theta)
    kr = C.rotate_bf16(k, pos, theta)
    vf = C.bits_to_f64(v).reshape(-1, Hkv, d)
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        tq = torch.from_numpy(qr[a:b]).permute(1, 0, 2)                 # [Hq, L, d]
        tk = torch.from_numpy(kr[a:b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        tv = torch.from_numpy(vf[a:b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                               scale=scale)
        np.testing.assert_allclose(out[a:b], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_rotated_operands_are_bf16_values_of_the_rotation():
    rng = np.random.default_rng(6)
    q, k, v, pos, cu = _packed(rng, [20], 2, 1, 64)
    r = C.rotate_bf16(q, pos, 500000.0)
    exact = C.rope(C.bits_to_f64(q).reshape(20, 2, 64), pos, 500000.0)
    # every value is a bfloat16 (round trip through its bit pattern) within half an ulp
    np.testing.assert_array_equal(C.bits_to_f64(C.bits_from_bf16_values(r)).reshape(r.shape), r)
    assert np.all(np.abs(r - exact) <= np.abs(exact) * 2.0 ** -8 + 2.0 ** -133)


def test_packed_requests_equal_each_request_alone():
    rng = np.random.default_rng(7)
    lengths, Hq, Hkv, d = [9, 0, 64, 3], 4, 1, 16
    q, k, v, pos, cu = _packed(rng, lengths, Hq, Hkv, d)
    out = C.rope_attention(q, k, v, pos, cu, Hq, Hkv, d, 0.25, 10000.0)
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        one = C.rope_attention(q[a:b], k[a:b], v[a:b], pos[a:b], np.array([0, b - a]),
                               Hq, Hkv, d, 0.25, 10000.0)
        np.testing.assert_array_equal(out[a:b], one)


def test_original_positions_change_the_result():
    """Carrying the original positions (with gaps) is not the same as renumbering the
    survivors 0..R-1; with no gaps the two agree exactly."""
    rng = np.random.default_rng(8)
    q, k, v, pos, cu = _packed(rng, [40], 4, 2, 32, gaps=True)
    a = C.rope_attention(q, k, v, pos, cu, 4, 2, 32, 0.2, 10000.0)
    b = C.rope_attention(q, k, v, np.arange(40), cu, 4, 2, 32, 0.2, 10000.0)
    assert np.abs(a - b).max() > 1e-3
    q, k, v, pos, cu = _packed(rng, [40], 4, 2, 32, gaps=False)
    np.testing.assert_array_equal(pos, np.arange(40))


# --- SwiGLU FFN (reading C5) --------------------------------------------------

def test_silu_matches_the_logistic_function():
    x = np.linspace(-40, 40, 10001)
    np.testing.assert_allclose(C.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)


def test_ffn_brute_force_on_tiny_inputs():
    rng = np.random.default_rng(9)
    R, H, F = 3, 4, 5
    x = _bf16_bits(rng, (R, H))
    wgu = _bf16_bits(rng, (2 * F, H), 0.5)
    wd = _bf16_bits(rng, (H, F), 0.5)
    res = _bf16_bits(rng, (R, H))
    y, gu, a = C.ffn(x, wgu, wd, F, residual_bits=res)
    xf, wguf, wdf, rf = (C.bits_to_f64(t) for t in (x, wgu, wd, res))
    for r in range(R):
        g = [sum(xf[r, c] * wguf[j, c] for c in range(H)) for j in range(2 * F)]
        g = [float(C.round_bf16(np.array([t]))[0]) for t in g]
        act = [float(C.round_bf16(np.array([g[j] / (1 + math.exp(-g[j])) * g[F + j]]))[0])
               for j in range(F)]
        for o in range(H):
            want = sum(act[j] * wdf[o, j] for j in range(F)) + rf[r, o]
            assert abs(y[r, o] - want) <= 1e-12 * (1 + abs(want))
        np.testing.assert_allclose(gu[r], g, rtol=1e-15, atol=0)
        np.testing.assert_allclose(a[r], act, rtol=1e-15, atol=0)


def test_ffn_with_zero_gate_returns_the_residual():
    rng = np.random.default_rng(10)
    R, H, F = 6, 16, 24
    x = _bf16_bits(rng, (R, H))
    wgu = _bf16_bits(rng, (2 * F, H))
    wgu[:F] = 0
    wd = _bf16_bits(rng, (H, F))
    res = _bf16_bits(rng, (R, H))
    y, _, a = C.ffn(x, wgu, wd, F, residual_bits=res)
    assert np.all(a == 0)
    np.testing.assert_array_equal(y, C.bits_to_f64(res))


def test_sampled_rows_equal_the_full_attention():
    rng = np.random.default_rng(11)
    lengths, Hq, Hkv, d = [70, 33], 4, 2, 16
    q, k, v, pos, cu = _packed(rng, lengths, Hq, Hkv, d)
    full = C.rope_attention(q, k, v, pos, cu, Hq, Hkv, d, 0.3, 10000.0)
    rows = [0, 1, 69, 70, 71, 102]
    part = C.rope_attention_rows(q, k, v, pos, cu, Hq, Hkv, d, 0.3, 10000.0, rows)
    np.testing.assert_allclose(part, full[rows], rtol=1e-12, atol=1e-14)
