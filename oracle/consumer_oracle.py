"""Plain CPU oracle for the layer that consumes the surviving tokens.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite and the bench's CPU baseline use it.  It
shares no code with the HIP library; the only common dependency is the seeded
input generator (``workloads.synth``), which holds none of the method's arithmetic.

What it follows:
  [UP] "UniPrefill: 블록 단위 동적 희소화를 통한 범용적 롱 컨텍스트 프리필 가속화"
       (AI Trends article):
         - "propagation" paragraph: after a drop, every later layer computes on
           the surviving tokens only, which shrinks the GEMMs as well as attention;
         - "Sparsity Propagation" paragraph: FFN and other sub-layers take only the
           kept tokens, so FFN work falls from O(N) to O(rho N) and attention
           work shrinks with the kept fraction as well;
         - "scheduler" paragraph: the positions of the survivors are tracked, so
           later steps address the right places.

Readings where the pages are silent (each repeated next to its code):
  C1  The consumer is one decoder layer's attention and SwiGLU FFN, run on the
      compacted rows; normalisations and the output projection are plain GEMMs
      or elementwise work and are not part of this oracle.
  C2  Survivors keep their original positions, so the rotary embedding is applied
      at ``pos_out`` (not at 0..R-1).  Rotary embedding: element i pairs with
      element i + d/2 and turns by the angle pos * theta^(-2i/d); theta is an
      argument (500000 for the Llama-3.1 shape, without frequency rescaling).
  C3  Compacted order is ascending original order, so a survivor attends to the
      survivors at or before it in compacted order, within its own request.
  C4  Precision: q, k, v arrive as bfloat16; the rotated q and k are rounded to
      bfloat16 (they are the matrix-core operands); everything else here is
      float64.  The rounding is the exact round-to-nearest-even of the float64
      rotation.
  C5  FFN: y = (silu(x Wg^T) * (x Wu^T)) Wd^T with Wg and Wu stored as one
      [2F, H] matrix (gate rows first).  The two products x Wg^T and x Wu^T and
      the gated activation are stored as bfloat16 (they are GEMM outputs and the
      next GEMM's operand), so the oracle rounds at those two points.
"""
from __future__ import annotations

import numpy as np


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even (reading C4).

    Works on the float64 bit pattern: a bfloat16 keeps 7 of the 52 stored mantissa
    bits.  Values below the bfloat16 normal range are rounded on the fixed grid of
    bfloat16 subnormals, 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    tiny = np.abs(x) < 2.0 ** -126
    # subnormal grid: np.rint rounds half to even
    out[tiny] = np.rint(x[tiny] * 2.0 ** 133) * 2.0 ** -133
    bits = x[~tiny].view(np.uint64)
    drop = np.uint64(45)
    lsb = (bits >> drop) & np.uint64(1)
    bias = np.uint64((1 << 44) - 1) + lsb
    r = ((bits + bias) >> drop) << drop
    out[~tiny] = r.view(np.float64)
    return out


def bits_from_bf16_values(x: np.ndarray) -> np.ndarray:
    """float64 values that are exact bfloat16 values -> their uint16 bit patterns."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Rotary embedding at the carried positions (reading C2)
# ---------------------------------------------------------------------------

def rope_angles(pos: np.ndarray, d: int, theta: float) -> np.ndarray:
    """[R, d/2] angles pos * theta^(-2i/d) in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate x [R, H, d] (float64) at positions pos [R]; no rounding.

    Element i and element i + d/2 form a pair turned by the pair's angle."""
    R, H, d = x.shape
    ang = rope_angles(pos, d, theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rotate_bf16(bits: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """The rotated matrix-core operand: rope of the bf16 input, rounded to bf16 (C4)."""
    return round_bf16(rope(bits_to_f64(bits), pos, theta))


# ---------------------------------------------------------------------------
# Causal attention over the survivors (readings C2, C3)
# ---------------------------------------------------------------------------

def rope_attention(q_bits, k_bits, v_bits, pos, cu_seqlens, Hq: int, Hkv: int, d: int,
                   scale: float, theta: float) -> np.ndarray:
    """out [R, Hq, d] float64: per request and query head, softmax over the causal
    keys of the rotated logits, times v.  Query head h reads kv head h // (Hq / Hkv)."""
    q = rotate_bf16(q_bits.reshape(-1, Hq, d), pos, theta)
    k = rotate_bf16(k_bits.reshape(-1, Hkv, d), pos, theta)
    v = bits_to_f64(v_bits).reshape(-1, Hkv, d)
    g = Hq // Hkv
    out = np.zeros((q.shape[0], Hq, d))
    for i in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        L = b - a
        if L == 0:
            continue
        mask = np.tril(np.ones((L, L), dtype=bool))
        for h in range(Hq):
            kv = h // g
            s = (q[a:b, h, :] @ k[a:b, kv, :].T) * float(scale)
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[a:b, h, :] = p @ v[a:b, kv, :]
    return out


def attention_vmax(v_bits, cu_seqlens, Hkv: int, d: int) -> np.ndarray:
    """max |v| per (token's request, kv head), broadcast to [R, Hkv]: the scale of the
    error that rounding probabilities to bfloat16 can cause in an output row."""
    v = np.abs(bits_to_f64(v_bits).reshape(-1, Hkv, d)).max(axis=2)
    out = np.zeros_like(v)
    for i in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        if b > a:
            out[a:b] = v[a:b].max(axis=0)[None, :]
    return out


# ---------------------------------------------------------------------------
# SwiGLU FFN on the survivors (reading C5)
# ---------------------------------------------------------------------------

def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def linear(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """x [R, K] times w [N, K] transposed, in float64 (no rounding)."""
    return bits_to_f64(x_bits) @ bits_to_f64(w_bits).T


def swiglu(gu: np.ndarray, F: int) -> np.ndarray:
    """silu(gate) * up for gu [R, 2F] (gate columns first), rounded to bf16 (C5)."""
    return round_bf16(silu(gu[:, :F]) * gu[:, F:])


def ffn(x_bits, w_gu_bits, w_down_bits, F: int, residual_bits=None):
    """y [R, H] float64 = swiglu(round_bf16(x Wgu^T)) Wd^T (+ residual)."""
    gu = round_bf16(linear(x_bits, w_gu_bits))
    a = swiglu(gu, F)
    y = a @ bits_to_f64(w_down_bits).T
    if residual_bits is not None:
        y = y + bits_to_f64(residual_bits)
    return y, gu, a


def rope_attention_rows(q_bits, k_bits, v_bits, pos, cu_seqlens, Hq: int, Hkv: int, d: int,
                        scale: float, theta: float, rows) -> np.ndarray:
    """The same attention as ``rope_attention`` for the listed rows only
    (out [len(rows), Hq, d] float64): each row reads its request's keys up to itself.
    Keys are rotated once per request, up to its last listed row."""
    rows = np.asarray(rows, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    g = Hq // Hkv
    out = np.zeros((len(rows), Hq, d))
    q = q_bits.reshape(-1, Hq, d)
    k = k_bits.reshape(-1, Hkv, d)
    v = v_bits.reshape(-1, Hkv, d)
    req = np.searchsorted(cu, rows, side="right") - 1
    for i in np.unique(req):
        a = int(cu[i])
        sel = np.nonzero(req == i)[0]
        last = int(rows[sel].max())
        kr = rotate_bf16(k[a:last + 1], pos[a:last + 1], theta)      # [n_keys, Hkv, d]
        vf = bits_to_f64(v[a:last + 1])
        for n in sel:
            r = int(rows[n])
            qr = rotate_bf16(q[r:r + 1], pos[r:r + 1], theta)[0]       # [Hq, d]
            nk = r - a + 1
            for h in range(Hq):
                s_ = (kr[:nk, h // g, :] @ qr[h]) * float(scale)
                s_ = s_ - s_.max()
                p = np.exp(s_)
                p /= p.sum()
                out[n, h] = p @ vf[:nk, h // g, :]
    return out
