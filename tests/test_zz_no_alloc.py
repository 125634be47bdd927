"""GPU: up_expand_compact_noalloc (the compaction with its run table in the library's
own device array, for callers that cannot allocate) against up_expand_compact (run
table in a caller workspace), through the C ABI: two calls in a row, the second with a
smaller input, every output bit-identical; the block limit is refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

import block_wise_token_amd as up
from oracle import uniprefill_oracle as O
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _case(lengths, G, H, seed, p_keep=0.7):
    rng = np.random.default_rng(seed)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    nbt = sum(O.n_blocks(L, G) for L in lengths)
    keep = (rng.random(nbt) < p_keep).astype(np.uint8)
    # cu_seqlens_out from the keep flags (the selection's output format)
    counts = []
    b0 = 0
    for L in lengths:
        nb = O.n_blocks(L, G)
        counts.append(sum(min((b + 1) * G, L) - b * G for b in range(nb) if keep[b0 + b]))
        b0 += nb
    cu_out = np.zeros(len(lengths) + 1, np.int32)
    cu_out[1:] = np.cumsum(counts)
    hidden = torch.from_numpy(rng.integers(-2**15, 2**15, (T, H), dtype=np.int16)).cuda()
    pos = torch.from_numpy(rng.permutation(T).astype(np.int32)).cuda()
    prev = torch.from_numpy(rng.permutation(2 * T)[:T].astype(np.int32)).cuda()
    return dict(cu_h=cu, cu=torch.from_numpy(cu).cuda(), keep=torch.from_numpy(keep).cuda(),
                cu_out=torch.from_numpy(cu_out).cuda(), hidden=hidden, pos=pos, prev=prev,
                T=T, kept=int(cu_out[-1]))


def _run(c, G, noalloc):
    T, H = c["T"], int(c["hidden"].shape[1])
    dev = c["hidden"].device
    outs = dict(idx=torch.full((T,), -7, dtype=torch.int32, device=dev),
                hid=torch.full((T, H), 5, dtype=torch.int16, device=dev),
                pos=torch.full((T,), -7, dtype=torch.int32, device=dev),
                orig=torch.full((T,), -7, dtype=torch.int32, device=dev))
    if noalloc:
        up.expand_compact_noalloc(c["hidden"], c["pos"], c["keep"], c["cu"], c["cu_out"], c["cu_h"],
                                  G, outs["idx"], outs["hid"], pos_out=outs["pos"],
                                  prev_orig=c["prev"], orig_out=outs["orig"])
    else:
        up.expand_compact(c["hidden"], c["pos"], c["keep"], c["cu"], c["cu_out"], c["cu_h"], G,
                          idx_out=outs["idx"], hidden_out=outs["hid"], pos_out=outs["pos"],
                          prev_orig=c["prev"], orig_out=outs["orig"])
    torch.cuda.synchronize()
    assert up.device_error() == 0
    return outs


def test_noalloc_compaction_matches_the_workspace_call_twice():
    G, H = 64, 512
    first = _case([70000, 0, 3000, 65, 1, 129000], G, H, seed=1)     # 3163 blocks
    second = _case([5000, 130], G, H, seed=2)                        # fewer blocks, rows
    for label, c in (("first", first), ("second (smaller)", second)):
        say(f"[case] no-alloc compaction, {label}: T={c['T']}, kept {c['kept']}")
        a = _run(c, G, noalloc=True)
        b = _run(c, G, noalloc=False)
        for name in ("idx", "hid", "pos", "orig"):
            assert torch.equal(a[name], b[name]), (label, name)
        # the rows past the kept count are untouched
        assert bool((a["idx"][c["kept"]:] == -7).all())
        idx = a["idx"][:c["kept"]].cpu().numpy()
        assert np.array_equal(idx, O.expand(c["keep"].cpu().numpy(), c["cu_h"], G))
        say(f"[ok] {label}: identical to the workspace call")


def test_noalloc_compaction_refuses_more_than_its_table():
    G = 32
    lengths = [65537 * G]
    cu = np.array([0, lengths[0]], np.int32)
    L = up.lib()
    st = L.up_expand_compact_noalloc(None, 8, 2, None, None, None, None,
                                     cu.ctypes.data_as(ctypes.c_void_p), 1, G,
                                     None, None, None, None, None, None)
    assert st == -2   # UP_EUNSUPPORTED, before any pointer is looked at
