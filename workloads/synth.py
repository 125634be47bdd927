"""Seeded synthetic inputs for block-wise token dropping.

This module is shared by the CPU oracle and the GPU path.  It holds only the
input recipe (random draws, the planted sink / needle / recency structure and
the float32 -> bfloat16 storage rounding); none of the method's arithmetic
(scores, softmax, selection, compaction) lives here.

Arrays are returned in their storage form:
  * bfloat16 tensors as ``uint16`` bit patterns,
  * positions and offsets as ``int32``.

The recipe stands in for the long-context needle-retrieval workloads that the
UniPrefill write-up evaluates on (Llama-3.1-8B at 128K tokens, the RULER
benchmark).  Nothing from that benchmark is reproduced; only the shape
(a strong sink token, a few high-attention "needle" blocks, mild recency)
is imitated with Gaussian vectors.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Seed-sequence tags: they keep the streams of different workload kinds apart.
TAG_VARLEN_REQUEST = 1
TAG_LAYER = 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 to bfloat16 (round to nearest, ties to even); return bits.

    For finite inputs the rounding add cannot overflow 32 bits (the largest
    finite pattern is 0xFF7FFFFF), so uint32 arithmetic is exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("bf16 rounding expects finite values")
    u = x.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def _unit_query_direction(q: np.ndarray, Hkv: int) -> np.ndarray:
    """Per kv head: unit vector along the sum of its group's window queries."""
    W, Hq, d = q.shape
    gs = Hq // Hkv
    s = q.reshape(W, Hkv, gs, d).sum(axis=(0, 2), dtype=np.float64)
    s /= np.linalg.norm(s, axis=1, keepdims=True)
    return s.astype(np.float32)  # [Hkv, d]


def needle_candidates(L: int, n: int, G: int) -> np.ndarray:
    """Blocks eligible for a needle: not block 0 (the sink) and clear of the window."""
    hi = (L - n) // G - 1
    return np.arange(1, hi + 1, dtype=np.int64) if hi >= 1 else np.zeros(0, np.int64)


@dataclass
class Request:
    """One request's attention inputs at a full-attention layer."""
    L: int
    qwin: np.ndarray          # uint16 [W, Hq, d] bfloat16 bits: the last W query rows
    k: np.ndarray             # uint16 [L, Hkv, d] bfloat16 bits
    needles: np.ndarray       # int64 block ids that received the needle bias
    sink: bool = True


CHUNK_ELEMS = 1 << 20   # values drawn, biased and rounded per step (keeps temporaries small)


def gen_request(L: int, Hq: int, Hkv: int, d: int, n: int, G: int,
                n_needles: int, rng: np.random.Generator,
                recency: int = 0) -> Request:
    """Sink/needle generator.

    Draw order: window queries [W, Hq, d], the needle blocks, then the keys
    [L, Hkv, d] in row order.  With u_g the unit direction of kv head g's window
    queries:
      * key 0 (the sink) gets + 4 sqrt(d) u_g,
      * every key of each needle block gets + 2 sqrt(d) u_g,
      * when ``recency`` > 0, the last ``recency`` keys get + 0.5 sqrt(d) u_g,
    and only then are the keys rounded to bfloat16.  Keys are drawn in chunks of
    rows; the stream of draws is the same as one draw of the whole array.
    """
    W = min(n, L)
    q = rng.standard_normal((W, Hq, d), dtype=np.float32)
    u = _unit_query_direction(q, Hkv) if W > 0 else np.zeros((Hkv, d), np.float32)
    sd = np.float32(np.sqrt(d))
    cand = needle_candidates(L, n, G)
    m = min(n_needles, cand.size)
    needles = np.sort(rng.choice(cand, size=m, replace=False)) if m else cand[:0]
    is_needle = np.zeros((L + G - 1) // G, dtype=bool)
    is_needle[needles] = True
    kb = np.empty((L, Hkv, d), dtype=np.uint16)
    rows_per = max(1, CHUNK_ELEMS // (Hkv * d))
    for r0 in range(0, L, rows_per):
        r1 = min(L, r0 + rows_per)
        kc = rng.standard_normal((r1 - r0, Hkv, d), dtype=np.float32)
        if r0 == 0:
            kc[0] += np.float32(4.0) * sd * u
        rows = np.arange(r0, r1)
        nrow = is_needle[rows // G]
        if nrow.any():
            kc[nrow] += np.float32(2.0) * sd * u
        if recency > 0:
            rec = rows >= L - recency
            if rec.any():
                kc[rec] += np.float32(0.5) * sd * u
        kb[r0:r1] = f32_to_bf16_bits(kc)
    return Request(L=L, qwin=f32_to_bf16_bits(q), k=kb, needles=needles)


def gen_hidden(T: int, H: int, seed: int) -> np.ndarray:
    """Hidden states [T, H] as bfloat16 bits, drawn N(0,1) from default_rng(seed + 1)."""
    rng = np.random.default_rng(seed + 1)
    out = np.empty((T, H), dtype=np.uint16)
    rows_per = max(1, CHUNK_ELEMS // max(1, H))
    for r0 in range(0, T, rows_per):
        r1 = min(T, r0 + rows_per)
        out[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, H), dtype=np.float32))
    return out


def positions(cu_seqlens: np.ndarray) -> np.ndarray:
    """Per-request token positions 0..L_i-1, packed."""
    lens = np.diff(cu_seqlens)
    return np.concatenate([np.arange(L, dtype=np.int32) for L in lens]) if lens.size else np.zeros(0, np.int32)


@dataclass
class Batch:
    """A packed (varlen) batch for one layer decision."""
    cu_seqlens: np.ndarray    # int32 [B+1]
    qwin: np.ndarray          # uint16 [sum W_i, Hq, d]
    k: np.ndarray             # uint16 [T, Hkv, d]
    Hq: int
    Hkv: int
    d: int
    n: int
    G: int
    needles: list = field(default_factory=list)

    @property
    def B(self) -> int:
        return int(self.cu_seqlens.size - 1)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])


def pack(reqs: list, Hq: int, Hkv: int, d: int, n: int, G: int) -> Batch:
    lens = [r.L for r in reqs]
    cu = np.zeros(len(reqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    if reqs:
        qwin = np.concatenate([r.qwin for r in reqs], axis=0)
        k = np.concatenate([r.k for r in reqs], axis=0)
    else:
        qwin = np.zeros((0, Hq, d), np.uint16)
        k = np.zeros((0, Hkv, d), np.uint16)
    return Batch(cu_seqlens=cu, qwin=qwin, k=k, Hq=Hq, Hkv=Hkv, d=d, n=n, G=G,
                 needles=[r.needles for r in reqs])


# ---------------------------------------------------------------------------
# Named workloads.  Shapes follow the model families named in the UniPrefill
# write-up (Llama-3.1-8B full attention: 32 query heads, 8 kv heads, head dim
# 128, hidden 4096; a Gemma-3-12B-like GQA stack: 16/8 heads, head dim 256,
# hidden 3840) with the ablation's defaults G=64, n=128, p=0.99.
# ---------------------------------------------------------------------------

WORKLOADS = {
    "single_4k_h8_d64": dict(lengths=[4096], Hq=8, Hkv=2, d=64, n=128, G=64, p=0.99,
                             needles=3, recency=0, H=1024, seed=0),
    "llama31_8b_32k": dict(lengths=[32768], Hq=32, Hkv=8, d=128, n=128, G=64, p=0.99,
                           needles=16, recency=0, H=4096, seed=0),
    "llama31_8b_128k": dict(lengths=[131072], Hq=32, Hkv=8, d=128, n=128, G=64, p=0.99,
                            needles=64, recency=2048, H=4096, seed=0),
    "varlen8_8k_64k": dict(lengths=None, B=8, lmin=8192, lmax=65536, Hq=32, Hkv=8, d=128,
                           n=128, G=64, p=0.99, needles=8, recency=0, H=4096, seed=0),
    "gemma3_12b_like_128k_4layers": dict(lengths=[131072], Hq=16, Hkv=8, d=256, n=128, G=64,
                                         p=0.99, needles=64, recency=0, H=3840, seed=0,
                                         layers=4),
}


def varlen_lengths(seed: int, B: int, lmin: int, lmax: int) -> list:
    """Request lengths drawn uniformly from [lmin, lmax] (first draw of default_rng(seed))."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lmin, lmax + 1, size=B)]


def make_batch(cfg: dict) -> Batch:
    """Build the layer-0 batch of a named workload configuration."""
    Hq, Hkv, d, n, G = cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["n"], cfg["G"]
    seed = cfg["seed"]
    if cfg.get("lengths") is None:
        lens = varlen_lengths(seed, cfg["B"], cfg["lmin"], cfg["lmax"])
        reqs = [gen_request(L, Hq, Hkv, d, n, G, cfg["needles"],
                            np.random.default_rng([seed, TAG_VARLEN_REQUEST, i]),
                            recency=cfg.get("recency", 0))
                for i, L in enumerate(lens)]
    else:
        lens = cfg["lengths"]
        if len(lens) == 1:
            reqs = [gen_request(lens[0], Hq, Hkv, d, n, G, cfg["needles"],
                                np.random.default_rng(seed), recency=cfg.get("recency", 0))]
        else:
            reqs = [gen_request(L, Hq, Hkv, d, n, G, cfg["needles"],
                                np.random.default_rng([seed, TAG_VARLEN_REQUEST, i]),
                                recency=cfg.get("recency", 0))
                    for i, L in enumerate(lens)]
    return pack(reqs, Hq, Hkv, d, n, G)


def gen_layer(orig: np.ndarray, L0: int, needles: np.ndarray, Hq: int, Hkv: int, d: int,
              n: int, G: int, seed: int, layer: int) -> Request:
    """Fresh inputs for a later full-attention layer over the surviving tokens.

    ``orig`` holds the original positions of the survivors (ascending).  Q/K are
    redrawn from default_rng([seed, TAG_LAYER, layer]); the sink and needle biases
    follow each survivor's *original* position, so structure planted at layer 0
    persists across layers.
    """
    rng = np.random.default_rng([seed, TAG_LAYER, layer])
    L = int(orig.size)
    W = min(n, L)
    q = rng.standard_normal((W, Hq, d), dtype=np.float32)
    u = _unit_query_direction(q, Hkv) if W > 0 else np.zeros((Hkv, d), np.float32)
    sd = np.float32(np.sqrt(d))
    is_needle = np.zeros((L0 + G - 1) // G, dtype=bool)
    is_needle[needles] = True
    kb = np.empty((L, Hkv, d), dtype=np.uint16)
    rows_per = max(1, CHUNK_ELEMS // (Hkv * d))
    for r0 in range(0, L, rows_per):
        r1 = min(L, r0 + rows_per)
        kc = rng.standard_normal((r1 - r0, Hkv, d), dtype=np.float32)
        o = orig[r0:r1]
        kc[o == 0] += np.float32(4.0) * sd * u
        nrow = is_needle[o // G]
        if nrow.any():
            kc[nrow] += np.float32(2.0) * sd * u
        kb[r0:r1] = f32_to_bf16_bits(kc)
    return Request(L=L, qwin=f32_to_bf16_bits(q), k=kb, needles=needles)


# ---------------------------------------------------------------------------
# Planted large logits: keys that stand far above everything a subset of the window
# rows has seen so far, at chosen token positions (inputs that make a running
# softmax reference move by a large step in the middle of the keys)
# ---------------------------------------------------------------------------
TAG_PLANTED = 4


def gen_planted_request(L: int, Hq: int, Hkv: int, d: int, n: int, plants, seed: int,
                        beta: float = 8.0, gap: float = 62.0) -> Request:
    """Gaussian queries and keys, with m = len(plants) orthonormal directions v_s
    removed from every query.  Window rows [s * r, (s + 1) * r) (r = W // (m + 1)) then
    get beta * v_s added in every head, and the key at token plants[s] is replaced, in
    every kv head, by alpha * v_s with alpha = gap * sqrt(d) / beta: its scaled logit
    against those rows is about ``gap`` (natural units, at scale 1/sqrt(d)) while
    every other key gives them a logit of order one, and every other row gets about
    0 from it.  Rows outside every subset see plain Gaussian keys.  Draws from
    default_rng([seed, TAG_PLANTED]); positions must lie before the window."""
    rng = np.random.default_rng([seed, TAG_PLANTED])
    W = min(n, L)
    m = len(plants)
    q = rng.standard_normal((W, Hq, d), dtype=np.float32)
    k = rng.standard_normal((L, Hkv, d), dtype=np.float32)
    V = np.linalg.qr(rng.standard_normal((d, m)))[0].T.astype(np.float32)   # [m, d]
    q -= np.einsum("whm,md->whd", np.einsum("whd,md->whm", q, V), V)
    r = max(1, W // (m + 1))
    alpha = np.float32(gap * np.sqrt(d) / beta)
    for s_, t in enumerate(plants):
        if not 0 <= t < L - W:
            raise ValueError(f"plant {t} is not before the window of a {L}-token request")
        q[s_ * r:(s_ + 1) * r] += np.float32(beta) * V[s_]
        k[t] = alpha * V[s_]
    return Request(L=L, qwin=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k),
                   needles=np.zeros(0, np.int64), sink=False)


# ---------------------------------------------------------------------------
# Inputs of the layer on the surviving tokens
# ---------------------------------------------------------------------------
TAG_CONSUMER = 3


def survivor_positions(lengths, rng, G: int = 64, drop_rate: float = 0.25) -> np.ndarray:
    """Original positions of survivors: per request, ascending, in runs of G tokens
    with whole dropped blocks (a drop_rate share of them) between the runs, the way a
    block-wise drop leaves them.  int32 [sum(lengths)]."""
    out = []
    for L in lengths:
        if L == 0:
            continue
        runs = (L + G - 1) // G
        gaps = rng.binomial(3, drop_rate, size=runs) * G   # dropped tokens before each run
        start = np.cumsum(gaps) + np.arange(runs) * G
        p = (start[:, None] + np.arange(G)[None, :]).reshape(-1)[:L]
        out.append(p)
    return (np.concatenate(out) if out else np.zeros(0, np.int64)).astype(np.int32)


def _normal_bits(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """Standard normal float32 draws times sigma, rounded to bfloat16 bits, drawn in
    chunks of rows (the stream equals one draw of the whole array)."""
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1)
    per_row = flat.shape[1]
    rows_per = max(1, CHUNK_ELEMS // max(per_row, 1))
    for r0 in range(0, shape[0], rows_per):
        r1 = min(shape[0], r0 + rows_per)
        x = rng.standard_normal((r1 - r0, per_row), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        flat[r0:r1] = f32_to_bf16_bits(x)
    return out


def gen_consumer_attention(lengths, Hq: int, Hkv: int, d: int, seed: int,
                           q_sigma: float = 1.0, G: int = 64):
    """q [R, Hq, d], k, v [R, Hkv, d] (bf16 bits, standard normal, q scaled by q_sigma),
    carried positions pos [R] and row offsets cu [B+1] for the attention on the
    survivors."""
    rng = np.random.default_rng([seed, TAG_CONSUMER])
    R = int(sum(lengths))
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    q = _normal_bits(rng, (R, Hq, d), q_sigma)
    k = _normal_bits(rng, (R, Hkv, d))
    v = _normal_bits(rng, (R, Hkv, d))
    pos = survivor_positions(lengths, rng, G)
    return q, k, v, pos, cu


def gen_ffn(R: int, H: int, F: int, seed: int):
    """x [R, H], w_gu [2F, H], w_down [H, F], residual [R, H] as bf16 bits; the weights
    are scaled by 1/sqrt(fan-in) so activations stay of order one."""
    rng = np.random.default_rng([seed, TAG_CONSUMER, 1])
    x = _normal_bits(rng, (R, H))
    wgu = _normal_bits(rng, (2 * F, H), 1.0 / np.sqrt(H))
    wd = _normal_bits(rng, (H, F), 1.0 / np.sqrt(F))
    res = _normal_bits(rng, (R, H))
    return x, wgu, wd, res
