"""Shared helpers of the GPU parity tests: moving seeded inputs to the device, running
the HIP path through the C ABI, and comparing with the oracle under the parity rules.

Parity rules (tolerances stated where they are used):
  * block scores: within 2e-3 relative where the oracle's score is >= 1e-6, within
    2e-9 absolute below that;
  * kept blocks: bit-exact, except "ambiguous" blocks -- a block whose running sum
    (just before or at it, in the oracle's sorted order) lies within 1e-5 of p, or
    whose score is within 1e-6 relative of a score at the cut -- which are counted
    and reported;
  * token indices, compacted rows, positions and composed indices: bit-exact given
    the same kept set.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_wise_token_amd as up
from oracle import uniprefill_oracle as O

SCORE_RTOL = 2e-3
SCORE_FLOOR = 1e-6
SCORE_ATOL_TINY = 2e-9
CUT_BAND = 1e-5
TIE_BAND = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def i32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def check_scores(gpu: np.ndarray, ref64: np.ndarray) -> float:
    """Assert the score tolerance; return the largest relative error on scores >= 1e-6."""
    assert gpu.shape == ref64.shape
    assert np.isfinite(gpu).all()
    big = ref64 >= SCORE_FLOOR
    err = np.abs(gpu.astype(np.float64) - ref64)
    rel = err[big] / ref64[big]
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= SCORE_RTOL, f"score relative error {worst:.3e} > {SCORE_RTOL}"
    if (~big).any():
        assert float(err[~big].max()) <= SCORE_ATOL_TINY
    return worst


def ambiguous_blocks(s32: np.ndarray, cu: np.ndarray, n: int, G: int, p: float) -> set:
    """Global ids of blocks whose keep decision may legitimately differ (see module doc)."""
    amb = set()
    p64 = float(np.float32(p))
    boff = 0
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        nb = O.n_blocks(L, G)
        if nb == 0:
            continue
        s = s32[boff:boff + nb]
        keep, det = O.topp_request(s, L, n, G, p)
        order, c, k = det["order"], det["cumsum"], det["kstar"]
        for r in range(nb):
            before = c[r - 1] if r > 0 else 0.0
            if abs(before - p64) <= CUT_BAND or abs(c[r] - p64) <= CUT_BAND:
                amb.add(boff + int(order[r]))
        cut_scores = [float(s[order[k - 1]])] + ([float(s[order[k]])] if k < nb else [])
        for cs in cut_scores:
            for b in range(nb):
                if abs(float(s[b]) - cs) <= TIE_BAND * max(cs, 1e-30):
                    amb.add(boff + b)
        boff += nb
    return amb


def check_keep(gpu_keep: np.ndarray, ref_keep: np.ndarray, amb: set) -> int:
    """Bit-exact outside the ambiguous blocks; returns how many ambiguous blocks differ."""
    diff = np.nonzero(gpu_keep.astype(bool) != ref_keep.astype(bool))[0]
    bad = [int(b) for b in diff if int(b) not in amb]
    assert not bad, f"kept-set mismatch outside the ambiguity bands at blocks {bad[:10]}"
    return int(diff.size)


class GpuBatch:
    """A synth.Batch (plus hidden states and positions) resident on the device."""

    def __init__(self, batch, H: int | None = None, hidden: np.ndarray | None = None, seed=0):
        from workloads import synth
        self.b = batch
        self.cu_h = batch.cu_seqlens.astype(np.int32)
        self.qwin = bf16_dev(batch.qwin)
        self.k = bf16_dev(batch.k)
        self.cu = i32_dev(self.cu_h)
        self.hidden_np = hidden if hidden is not None else (
            synth.gen_hidden(batch.T, H, seed) if H else None)
        self.hidden = bf16_dev(self.hidden_np) if self.hidden_np is not None else None
        self.pos_np = synth.positions(batch.cu_seqlens)
        self.pos = i32_dev(self.pos_np)


def run_decision(gb: GpuBatch, p: float, topk=None, prev_orig=None) -> dict:
    b = gb.b
    dec = up.LayerDecision(gb.qwin, gb.k, gb.cu, gb.cu_h, gb.hidden, gb.pos, b.n, b.G, p,
                           prev_orig=prev_orig, topk=topk)
    dec.run()
    torch.cuda.synchronize()
    assert up.device_error() == 0
    cnt = int(dec.cu_out[-1].item())
    return dict(scores=dec.scores.cpu().numpy(), keep=dec.keep.cpu().numpy(),
                cu_out=dec.cu_out.cpu().numpy(), count=cnt, dec=dec)


def check_rows(hidden_out: torch.Tensor, src_np: np.ndarray, idx: np.ndarray, chunk=16384):
    """Every compacted row bit-exact: hidden_out[r] == src_np[idx[r]] for all r, copied
    back and compared chunk by chunk (bounded host memory at full size)."""
    cnt = int(idx.size)
    flat = hidden_out.view(torch.int16)
    for r0 in range(0, cnt, chunk):
        r1 = min(cnt, r0 + chunk)
        got = flat[r0:r1].cpu().numpy().view(np.uint16)
        want = src_np[idx[r0:r1]]
        if not np.array_equal(got, want):
            bad = np.nonzero((got != want).any(axis=1))[0]
            raise AssertionError(f"compacted rows differ at {(bad[:8] + r0).tolist()} "
                                 f"({bad.size} rows in [{r0}, {r1}))")


def check_compaction(gb: GpuBatch, res: dict):
    """idx/hidden/pos/orig bit-exact against the oracle given the GPU's kept set; every
    compacted row is compared."""
    b = gb.b
    dec = res["dec"]
    keep = res["keep"]
    idx_ref = O.expand(keep, b.cu_seqlens, b.G)
    _, cu_out_ref, _ = _counts(keep, b.cu_seqlens, b.G)
    np.testing.assert_array_equal(res["cu_out"], cu_out_ref)
    cnt = res["count"]
    assert cnt == idx_ref.size
    idx = dec.idx[:cnt].cpu().numpy()
    np.testing.assert_array_equal(idx, idx_ref)
    pos_out = dec.pos_out[:cnt].cpu().numpy()
    np.testing.assert_array_equal(pos_out, gb.pos_np[idx_ref])
    orig = dec.orig[:cnt].cpu().numpy()
    prev = dec.prev_orig.cpu().numpy()
    np.testing.assert_array_equal(orig, prev[idx_ref])
    if gb.hidden is None:
        return
    check_rows(dec.hidden_out[:cnt], gb.hidden_np, idx_ref)


def _counts(keep, cu, G):
    cu = np.asarray(cu, dtype=np.int64)
    out = np.zeros(cu.size, dtype=np.int32)
    boff = 0
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        nb = O.n_blocks(L, G)
        out[i + 1] = out[i] + sum(min((b + 1) * G, L) - b * G for b in range(nb) if keep[boff + b])
        boff += nb
    return None, out, None


def check_packed_equals_alone(gb: GpuBatch, res: dict, p: float, requests=None):
    """Requests are independent ([UPA]: a continuous-batching operator): each request
    decided alone gives bit-identical scores and keep flags to its slice of the packed
    decision, the same kept-token count, and the same compacted rows.  Returns the
    number of requests checked."""
    b = gb.b
    cu = b.cu_seqlens.astype(np.int64)
    boff = 0
    checked = 0
    dec = res["dec"]
    for i in range(b.B):
        L = int(cu[i + 1] - cu[i])
        nb = O.n_blocks(L, b.G)
        if (requests is None or i in requests) and L > 0:
            from workloads import synth
            wo = int(sum(min(b.n, int(cu[r + 1] - cu[r])) for r in range(i)))
            W = min(b.n, L)
            one = synth.Batch(cu_seqlens=np.array([0, L], np.int32), qwin=b.qwin[wo:wo + W],
                              k=b.k[cu[i]:cu[i + 1]], Hq=b.Hq, Hkv=b.Hkv, d=b.d, n=b.n, G=b.G)
            hid = gb.hidden_np[cu[i]:cu[i + 1]] if gb.hidden_np is not None else None
            r1 = run_decision(GpuBatch(one, H=None, hidden=hid), p)
            assert np.array_equal(r1["scores"].view(np.uint32),
                                  res["scores"][boff:boff + nb].view(np.uint32)), \
                f"request {i} (L={L}): scores differ between alone and packed"
            assert np.array_equal(r1["keep"], res["keep"][boff:boff + nb]), \
                f"request {i} (L={L}): keep flags differ between alone and packed"
            o0, o1 = int(res["cu_out"][i]), int(res["cu_out"][i + 1])
            assert r1["count"] == o1 - o0
            if hid is not None and r1["count"]:
                a = r1["dec"].hidden_out[:r1["count"]]
                c = dec.hidden_out[o0:o1]
                assert torch.equal(a.view(torch.int16), c.view(torch.int16)), \
                    f"request {i}: compacted rows differ between alone and packed"
            checked += 1
        boff += nb
    return checked
