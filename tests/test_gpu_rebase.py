"""GPU: the score pass when a key's logit jumps far above a row's running softmax
reference in the middle of a statistics chunk.

The score kernel keeps one reference per query and rescales the sums it has
accumulated (of the current block and of the current statistics chunk) only when a
32-key half would push a sum past 2^64, i.e. when a key's logit exceeds the reference
by more than about 64 log2 units.  The generator (workloads.synth.gen_planted_request)
gives chosen window rows one key each whose logit stands about 62 natural units
(about 90 log2 units) above everything else they see; the key sits after the row's
reference was set at its chunk's first half, so the rescale must be right for the
scores to match the oracle: a skipped or wrong rescale would leave the earlier sums
at the old reference, about 2^90 too large.  Keys are planted, relative to the
statistics chunks the library reports (up_block_scores_chunks), in the middle of a
half, on a half boundary that is not a block boundary, on a block boundary, in the
chunk's last stage and in the chunk's second half (where long chunks leave the
unrolled loop), over head dimensions 64, 128 and 256 and block sizes 32 and 64, and
in a packed batch whose work items span several statistics chunks.
"""
import numpy as np
import pytest

import block_wise_token_amd as up
from oracle import uniprefill_oracle as O
from workloads import synth
from tests.gpu_helpers import (GpuBatch, ambiguous_blocks, check_compaction, check_keep,
                               check_packed_equals_alone, check_scores, run_decision, say)

pytestmark = pytest.mark.gpu


def _plants(CL: int, G: int, L: int, n: int):
    """Token positions: one per statistics chunk 1..5, each at a chosen offset."""
    offsets = [
        5 * 32 + 13,            # middle of a half (the unrolled loop for long chunks)
        7 * 32,                 # first key of a half that does not start a block (G = 64)
        (256 // G) * G,         # first key of a block
        CL - 40,                # the chunk's last 64-key stage
        CL // 2 + 7,            # second half of the chunk
    ]
    out = []
    for c, off in enumerate(offsets, start=1):
        t = c * CL + off % CL
        if t < L - n:
            out.append(t)
    return out


CASES = [
    # L, Hq, Hkv, d, G
    (32768, 32, 8, 64, 64),
    (32768, 32, 8, 128, 64),
    (32768, 32, 8, 128, 32),
    (32768, 16, 8, 256, 64),
    (32768, 16, 8, 256, 32),
    (32768, 32, 8, 64, 32),
]


def _check(batch, p, label):
    gb = GpuBatch(batch, H=128)
    res = run_decision(gb, p)
    s32, s64, _ = O.block_scores(batch.qwin, batch.k, batch.cu_seqlens, batch.Hq, batch.Hkv,
                                 batch.d, batch.n, batch.G)
    worst = check_scores(res["scores"], s64)
    ref_keep, _, _ = O.topp_select(s32, batch.cu_seqlens, batch.n, batch.G, p)
    amb = ambiguous_blocks(s32, batch.cu_seqlens, batch.n, batch.G, p)
    ndiff = check_keep(res["keep"], ref_keep, amb)
    check_compaction(gb, res)
    say(f"[ok] {label}: worst score rel err {worst:.2e}, ambiguous {len(amb)}, "
        f"differing {ndiff}, kept {res['count']}/{batch.T}")
    return res, gb


@pytest.mark.parametrize("case", CASES, ids=[f"L{c[0]}_h{c[1]}_{c[2]}_d{c[3]}_G{c[4]}" for c in CASES])
def test_rebase_at_planted_keys(case):
    L, Hq, Hkv, d, G = case
    n, p = 128, 0.9
    CL = int(up.block_scores_chunks([0, L], Hq, Hkv, d, n, G)[0]) * G
    plants = _plants(CL, G, L, n)
    assert len(plants) == 5, (CL, plants)
    say(f"[case] rebase {case}: chunk {CL} keys, plants {plants}")
    req = synth.gen_planted_request(L, Hq, Hkv, d, n, plants, seed=L + d + G)
    batch = synth.pack([req], Hq, Hkv, d, n, G)
    res, _ = _check(batch, p, f"rebase {case}")
    # each planted key's block carries its rows' mass: it is kept
    for t in plants:
        assert res["keep"][t // G] == 1


def test_rebase_in_packed_work_items():
    """Four 32K requests: the planner packs several statistics chunks into one work
    item, so the reference restarts inside workgroups; planted keys in every request,
    and each request alone must give bit-identical scores and keep flags."""
    Hq, Hkv, d, n, G, p = 32, 8, 64, 128, 64, 0.9
    lens = [32768, 30000, 32768, 28000]
    chunks = up.block_scores_chunks(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                                    Hq, Hkv, d, n, G)
    reqs = []
    for i, L in enumerate(lens):
        plants = _plants(int(chunks[i]) * G, G, L, n)
        reqs.append(synth.gen_planted_request(L, Hq, Hkv, d, n, plants, seed=100 + i))
    batch = synth.pack(reqs, Hq, Hkv, d, n, G)
    say(f"[case] rebase packed: lengths {lens}, chunks {chunks.tolist()}")
    res, gb = _check(batch, p, "rebase packed")
    assert check_packed_equals_alone(gb, res, p) == len(lens)
