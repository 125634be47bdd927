"""Plain CPU oracle for UniPrefill-style block-wise token dropping.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the only common dependency is the seeded input generator
(``workloads.synth``), which holds none of the method's arithmetic.

It is deliberately slow and literal: NumPy in float64, one query head at a
time, the full probability matrix materialised, a stable sort and a sequential
cumulative sum.

Pages followed (cited by title and paragraph/section, the pages carry no
numbered equations):
  [UP]  "UniPrefill: 블록 단위 동적 희소화를 통한 범용적 롱 컨텍스트 프리필 가속화"
        (AI Trends article on UniPrefill).  Paragraphs used:
          - "drop" paragraph: a full-attention layer measures each token's
            contribution from query-key similarity; tokens whose softmax
            probability is near zero are dropped;
          - "propagation" paragraph: the drop carries into all later layers;
          - "block-wise estimation" paragraph: fixed blocks of G tokens, the
            last n query tokens, per-block average attention, normalised into
            per-block importance scores;
          - "Top-p selection" paragraph: sort blocks by descending score, keep
            them until the running sum reaches p (example 0.99), output the
            token indices to keep;
          - "scheduler" paragraph: positions of dropped tokens are tracked so
            later steps address the right KV-cache slots;
          - "ablation" paragraph: G=64 and n=128 are the chosen defaults;
          - "Sparsity Propagation" paragraph: every later sub-layer receives only
            the surviving tokens.
  [UPA] "UniPrefill: Universal Long-Context Prefill Acceleration via Block-wise
        Dynamic Sparsification" (ChatPaper abstract page): the operator works
        under continuous batching.
  [CP]  "Chunked Prefill" (Ultralytics glossary), section "how chunked prefill
        works": a chunk of queries at absolute positions attends causally to all
        earlier keys plus itself, giving the same result as one pass.

Readings where the pages are silent are listed next to the code that takes them.
Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


# ---------------------------------------------------------------------------
# Storage decoding
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def default_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d), represented in float32 (the pages state no scale;
    reading: the layer's own attention scale, carried as a float32 argument)."""
    return float(np.float32(1.0 / math.sqrt(d)))


def n_blocks(L: int, G: int) -> int:
    """Blocks of G tokens from the request's token 0; the last one may be partial."""
    return (L + G - 1) // G


def window_size(L: int, n: int) -> int:
    """The observation window: the last n query tokens, or all L if the request is shorter."""
    return min(n, L)


# ---------------------------------------------------------------------------
# Step 1: attention probabilities of the window rows  ([UP] drop paragraph,
# [UP] block-wise estimation paragraph, [CP] causal mask over absolute positions)
# ---------------------------------------------------------------------------

def window_probs(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Softmax probabilities of the W window queries over the L causal keys.

    q: float64 [W, Hq, d], the last W query tokens of a request of length L.
    k: float64 [L, Hkv, d].
    Returns P float64 [Hq, W, L].  Window row j sits at absolute position
    t_j = L - W + j and sees keys 0..t_j (the causal mask of [CP]).  Query head
    h reads kv head floor(h / (Hq/Hkv)) (reading: contiguous GQA groups).
    """
    W, Hq, d = q.shape
    L, Hkv, _ = k.shape
    gs = Hq // Hkv
    t = np.arange(L - W, L)
    visible = np.arange(L)[None, :] <= t[:, None]        # [W, L]
    P = np.empty((Hq, W, L), dtype=np.float64)
    for h in range(Hq):
        s = (q[:, h, :] @ k[:, h // gs, :].T) * scale     # logits [W, L]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        P[h] = e / e.sum(axis=1, keepdims=True)
    return P


def request_block_mass(q: np.ndarray, k: np.ndarray, G: int, scale: float) -> np.ndarray:
    """Attention mass of each G-block: sum over heads, window rows and the block's keys.

    Same inputs as ``window_probs``; processes one head at a time so that long
    requests fit in memory.  Returns float64 [ceil(L/G)].
    Reading: every query head and every window row weighs the same; block b
    covers keys [bG, min((b+1)G, L)).
    """
    W, Hq, d = q.shape
    L, Hkv, _ = k.shape
    gs = Hq // Hkv
    nb = n_blocks(L, G)
    t = np.arange(L - W, L)
    visible = np.arange(L)[None, :] <= t[:, None]
    mass = np.zeros(nb, dtype=np.float64)
    pad = nb * G - L
    for h in range(Hq):
        s = (q[:, h, :] @ k[:, h // gs, :].T) * scale
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        P = e / e.sum(axis=1, keepdims=True)
        if pad:
            P = np.concatenate([P, np.zeros((W, pad))], axis=1)
        mass += P.reshape(W, nb, G).sum(axis=(0, 2))
    return mass


def block_scores(qwin_bits: np.ndarray, k_bits: np.ndarray, cu_seqlens: np.ndarray,
                 Hq: int, Hkv: int, d: int, n: int, G: int, scale: float | None = None,
                 heads: range | None = None):
    """Per-block importance scores of a packed batch ([UP] block-wise estimation).

    Each request is independent ([UPA] continuous batching).  For request i the
    block masses are divided by their sum, so its scores sum to 1 (reading of the
    page's "softmax normalisation" step: the softmax is taken per query row over
    tokens, then block masses are normalised).  Equivalently each score is the
    block's mean probability (divisor W*Hq*G for every block, a partial last block
    included) rescaled to sum to one.

    ``heads`` restricts the sum to a subset of query heads (used to pin the
    additivity of partial scores across head shards) and then returns the
    un-normalised masses only.

    Returns (scores_f32 [NB_tot], scores_f64 [NB_tot], masses_f64 [NB_tot]).
    """
    if scale is None or scale <= 0:
        scale = default_scale(d)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = cu.size - 1
    out64, mass_all = [], []
    qoff = 0
    for i in range(B):
        L = int(cu[i + 1] - cu[i])
        W = window_size(L, n)
        q = bf16_bits_to_f64(qwin_bits[qoff:qoff + W])
        kk = bf16_bits_to_f64(k_bits[cu[i]:cu[i + 1]])
        qoff += W
        if L == 0:
            continue
        if heads is not None:
            gs = Hq // Hkv
            mass = np.zeros(n_blocks(L, G))
            for h in heads:
                mass += request_block_mass(q[:, h:h + 1, :], kk[:, h // gs:h // gs + 1, :], G, scale)
            mass_all.append(mass)
            out64.append(mass)
            continue
        mass = request_block_mass(q, kk, G, scale)
        mass_all.append(mass)
        out64.append(mass / mass.sum())
    s64 = np.concatenate(out64) if out64 else np.zeros(0)
    m64 = np.concatenate(mass_all) if mass_all else np.zeros(0)
    return s64.astype(np.float32), s64, m64


# ---------------------------------------------------------------------------
# Step 1b: block scores from the layer's own softmax statistics
# ([UP] Triton kernels paragraph: the full-attention layer already runs an online
# softmax over these rows, so its row statistics can be reused)
# ---------------------------------------------------------------------------

def row_lse(qwin_bits: np.ndarray, k_bits: np.ndarray, cu_seqlens: np.ndarray, Hq: int,
            Hkv: int, d: int, n: int, scale: float | None = None) -> np.ndarray:
    """Natural-log log-sum-exp of every window row's scaled logits over its causal
    keys: lse = m + log(sum exp(s - m)), m the row maximum.  Float64 [sum W_i, Hq],
    window rows in qwin order; these are the statistics a FlashAttention-style forward
    keeps per query row.  Same masks and head map as ``window_probs``."""
    if scale is None or scale <= 0:
        scale = default_scale(d)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    gs = Hq // Hkv
    out, qoff = [], 0
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        W = window_size(L, n)
        q = bf16_bits_to_f64(qwin_bits[qoff:qoff + W])
        kk = bf16_bits_to_f64(k_bits[cu[i]:cu[i + 1]])
        qoff += W
        if W == 0:
            continue
        t = np.arange(L - W, L)
        visible = np.arange(L)[None, :] <= t[:, None]
        lse = np.empty((W, Hq), dtype=np.float64)
        for h in range(Hq):
            s_ = (q[:, h, :] @ kk[:, h // gs, :].T) * scale
            s_ = np.where(visible, s_, -np.inf)
            m = s_.max(axis=1)
            lse[:, h] = m + np.log(np.exp(s_ - m[:, None]).sum(axis=1))
        out.append(lse)
    return np.concatenate(out) if out else np.zeros((0, Hq))


def block_scores_given_lse(qwin_bits: np.ndarray, k_bits: np.ndarray, lse: np.ndarray,
                           cu_seqlens: np.ndarray, Hq: int, Hkv: int, d: int, n: int, G: int,
                           scale: float | None = None):
    """Block scores when each window row's log-sum-exp is given rather than computed.

    lse: [sum W_i, Hq] (window rows in qwin order, natural log).  A row's weights are
    exp(s - lse_row) over its causal keys; block masses sum them over heads, rows and
    the block's keys; each request's masses are divided by their sum.  With
    lse = row_lse(...) the weights are the softmax probabilities and the result is
    ``block_scores``'s.  A row with lse = +inf contributes nothing.

    Returns (scores_f32 [NB_tot], scores_f64 [NB_tot], masses_f64 [NB_tot]).
    """
    if scale is None or scale <= 0:
        scale = default_scale(d)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lse = np.asarray(lse, dtype=np.float64)
    gs = Hq // Hkv
    out64, mass_all, qoff = [], [], 0
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        W = window_size(L, n)
        q = bf16_bits_to_f64(qwin_bits[qoff:qoff + W])
        kk = bf16_bits_to_f64(k_bits[cu[i]:cu[i + 1]])
        lrow = lse[qoff:qoff + W]
        qoff += W
        if L == 0:
            continue
        nb = n_blocks(L, G)
        t = np.arange(L - W, L)
        visible = np.arange(L)[None, :] <= t[:, None]
        mass = np.zeros(nb, dtype=np.float64)
        pad = nb * G - L
        for h in range(Hq):
            s_ = (q[:, h, :] @ kk[:, h // gs, :].T) * scale
            P = np.where(visible, np.exp(s_ - lrow[:, h:h + 1]), 0.0)
            if pad:
                P = np.concatenate([P, np.zeros((W, pad))], axis=1)
            mass += P.reshape(W, nb, G).sum(axis=(0, 2))
        mass_all.append(mass)
        out64.append(mass / mass.sum())
    s64 = np.concatenate(out64) if out64 else np.zeros(0)
    m64 = np.concatenate(mass_all) if mass_all else np.zeros(0)
    return s64.astype(np.float32), s64, m64


# ---------------------------------------------------------------------------
# Paged key cache (scope: next; [UPA] continuous-batching operator, [CP] chunked
# prefill reads earlier chunks' keys from the cache)
# ---------------------------------------------------------------------------

def gather_paged_keys(k_pages: np.ndarray, block_table: np.ndarray, cu_seqlens: np.ndarray,
                      page_size: int) -> np.ndarray:
    """Contiguous keys [T, Hkv, d] of a packed batch from a paged cache.

    k_pages: [num_pages, page_size, Hkv, d] (any dtype, copied as is).
    block_table: int [B, max_pages]; token t of request i lives in page
    block_table[i, t // page_size], slot t % page_size (reading: the layout of a
    paged KV cache with one page table per request, pages of page_size tokens).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = []
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        for t in range(L):
            out.append(k_pages[int(block_table[i, t // page_size]), t % page_size])
    if not out:
        return np.zeros((0,) + k_pages.shape[2:], dtype=k_pages.dtype)
    return np.stack(out)


# ---------------------------------------------------------------------------
# Step 2: Top-p selection  ([UP] Top-p selection paragraph)
# ---------------------------------------------------------------------------

def window_blocks(L: int, n: int, G: int) -> list:
    """Blocks that hold at least one window token: b with (b+1)G > L - W.

    Reading: the observation window is always kept, whole blocks only (a block is
    never split), so its tokens stay visible to later layers."""
    W = window_size(L, n)
    nb = n_blocks(L, G)
    return [b for b in range(nb) if (b + 1) * G > L - W]


EXACT_SHIFT = 149   # every float32 in [0, 1] is an integer multiple of 2**-149


def exact_units(x: float) -> int:
    """A float32 value in [0, 1] as an exact integer count of 2**-149."""
    f = Fraction(float(np.float32(x))) * (1 << EXACT_SHIFT)
    assert f.denominator == 1
    return int(f)


def topp_request(scores: np.ndarray, L: int, n: int, G: int, p: float):
    """Top-p cut for one request.

    scores: float32 [nb].  Blocks are ordered by descending score, ties by lower
    block index (reading: a stable sort).  The running sum of the sorted scores is
    compared with p, both as float32 values, and the sum is taken exactly, with no
    rounding (reading: the plain meaning of "the cumulative sum reaches p"; it also
    makes the cut independent of summation order).  The cut keeps the shortest
    prefix whose running sum reaches p ("reaches" read as >=).  With p >= 1, or if
    every running sum stays below p, all blocks are kept.  The window blocks are
    added afterwards.

    Returns (keep bool [nb], detail dict with order, the float64 running sums for
    reports, and the cut size).
    """
    nb = n_blocks(L, G)
    s = np.asarray(scores, dtype=np.float32)
    assert s.size == nb
    order = sorted(range(nb), key=lambda b: (-float(s[b]), b))
    p64 = float(np.float32(p))
    p_units = exact_units(p64) if p64 <= 1.0 else None
    csum = []
    acc = 0.0
    exact = 0
    kstar = nb
    found = False
    for r, b in enumerate(order):
        acc = acc + float(s[b])
        csum.append(acc)
        exact += exact_units(float(s[b]))
        if not found and p64 < 1.0 and exact >= p_units:
            kstar = r + 1
            found = True
    keep = np.zeros(nb, dtype=bool)
    for b in order[:kstar]:
        keep[b] = True
    for b in window_blocks(L, n, G):
        keep[b] = True
    return keep, dict(order=np.array(order, dtype=np.int64), cumsum=np.array(csum),
                      kstar=kstar, p64=p64)


def topk_request(scores: np.ndarray, L: int, n: int, G: int, k: int):
    """Fixed-count alternative from the [UP] ablation paragraph: the k highest-scoring
    blocks (same order and tie rule as Top-p), plus the window blocks."""
    nb = n_blocks(L, G)
    s = np.asarray(scores, dtype=np.float32)
    order = sorted(range(nb), key=lambda b: (-float(s[b]), b))
    keep = np.zeros(nb, dtype=bool)
    for b in order[:min(k, nb)]:
        keep[b] = True
    for b in window_blocks(L, n, G):
        keep[b] = True
    return keep


def topk_select(scores: np.ndarray, cu_seqlens: np.ndarray, n: int, G: int, k: int):
    """Top-k over a packed batch: (keep uint8 [NB_tot], cu_seqlens_out int32 [B+1])."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    keeps, out, boff = [], np.zeros(cu.size, dtype=np.int32), 0
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        nb = n_blocks(L, G)
        keep = topk_request(scores[boff:boff + nb], L, n, G, k)
        boff += nb
        out[i + 1] = out[i] + sum(min((b + 1) * G, L) - b * G for b in range(nb) if keep[b])
        keeps.append(keep)
    keep_all = np.concatenate(keeps).astype(np.uint8) if keeps else np.zeros(0, np.uint8)
    return keep_all, out


def topp_select(scores: np.ndarray, cu_seqlens: np.ndarray, n: int, G: int, p: float):
    """Top-p over a packed batch; each request independently ([UPA]).

    Returns (keep uint8 [NB_tot], cu_seqlens_out int32 [B+1], details per request).
    cu_seqlens_out holds the packed offsets of the kept tokens.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = cu.size - 1
    keeps, details = [], []
    out = np.zeros(B + 1, dtype=np.int32)
    boff = 0
    for i in range(B):
        L = int(cu[i + 1] - cu[i])
        nb = n_blocks(L, G)
        keep, det = topp_request(scores[boff:boff + nb], L, n, G, p)
        boff += nb
        kept_tokens = sum(min((b + 1) * G, L) - b * G for b in range(nb) if keep[b])
        out[i + 1] = out[i] + kept_tokens
        keeps.append(keep)
        details.append(det)
    keep_all = np.concatenate(keeps).astype(np.uint8) if keeps else np.zeros(0, np.uint8)
    return keep_all, out, details


# ---------------------------------------------------------------------------
# Step 3: expand kept blocks to token indices ([UP] Top-p selection paragraph:
# the output is the set of token indices to keep)
# ---------------------------------------------------------------------------

def expand(keep: np.ndarray, cu_seqlens: np.ndarray, G: int) -> np.ndarray:
    """Packed row indices of the kept tokens, ascending within each request,
    requests in input order (reading: original order is preserved, which keeps
    later layers causal)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = []
    boff = 0
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        nb = n_blocks(L, G)
        for b in range(nb):
            if keep[boff + b]:
                idx.extend(range(int(cu[i]) + b * G, int(cu[i]) + min((b + 1) * G, L)))
        boff += nb
    return np.array(idx, dtype=np.int32)


# ---------------------------------------------------------------------------
# Step 4: compaction and drop composition ([UP] propagation and Sparsity
# Propagation paragraphs; [UP] scheduler paragraph for positions)
# ---------------------------------------------------------------------------

def compact(hidden: np.ndarray, pos: np.ndarray, idx: np.ndarray):
    """Rows of the surviving tokens, in order; original positions carried, never renumbered."""
    hidden_out = np.empty((idx.size,) + hidden.shape[1:], dtype=hidden.dtype)
    pos_out = np.empty(idx.size, dtype=pos.dtype)
    for r, j in enumerate(idx):
        hidden_out[r] = hidden[j]
        pos_out[r] = pos[j]
    return hidden_out, pos_out


def compact_fast(hidden: np.ndarray, pos: np.ndarray, idx: np.ndarray):
    """The same gather as ``compact`` through NumPy fancy indexing (large inputs)."""
    return hidden[idx], pos[idx]


def compose(prev_orig: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Original index of every survivor after another decision: orig[r] = prev_orig[idx[r]]."""
    return np.array([prev_orig[j] for j in idx], dtype=np.int32)


# ---------------------------------------------------------------------------
# One full layer decision
# ---------------------------------------------------------------------------

def decide(qwin_bits, k_bits, cu_seqlens, hidden, pos, Hq, Hkv, d, n, G, p,
           scale=None, prev_orig=None, fast=True):
    """Scores -> Top-p -> expand -> compact -> compose for one full-attention layer."""
    s32, s64, mass = block_scores(qwin_bits, k_bits, cu_seqlens, Hq, Hkv, d, n, G, scale)
    keep, cu_out, details = topp_select(s32, cu_seqlens, n, G, p)
    idx = expand(keep, cu_seqlens, G)
    if hidden is not None:
        hidden_out, pos_out = (compact_fast if fast else compact)(hidden, pos, idx)
    else:
        hidden_out, pos_out = None, None
    if prev_orig is None:
        prev_orig = np.arange(int(cu_seqlens[-1]), dtype=np.int32)
    orig = prev_orig[idx] if fast else compose(prev_orig, idx)
    return dict(scores=s32, scores64=s64, mass=mass, keep=keep, cu_seqlens_out=cu_out,
                idx=idx, hidden_out=hidden_out, pos_out=pos_out, orig=orig, details=details)
