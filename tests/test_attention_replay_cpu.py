"""CPU: host replay of the attention kernels' addressing (tests/attn_replay.cpp, built
here with g++ against the index functions the kernels themselves call,
block_wise_token_amd/csrc/attn_geom.h): the 8-wave kernel (d = 64 and 128, up to 256 kv
heads) and the 4-wave kernel (d = 256, and more kv heads).

For every launch shape below -- the layer-on-the-survivors shapes of the 128K Llama
decision (129,600 survivors and all 131,072 rows, Hq = 32, Hkv = 8, d = 128) and of the
Gemma-like d = 256 layer (129,344 and 131,072 rows, Hq = 16, Hkv = 8), every shape the
GPU attention tests launch, and edge shapes -- the replay
checks every copy, operand read, key-norm read and output store against its buffer,
the ring's stage hand-over against the waits and barriers, the causal mask and the
operand layouts, and that every output element is written once (the program's own
header lists the checks)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "attn_replay.cpp")
INC = os.path.join(ROOT, "block_wise_token_amd", "csrc")


@pytest.fixture(scope="module")
def replay(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("replay") / "attn_replay")
    subprocess.run([gxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-I", INC, SRC, "-o", exe],
                   check=True)
    return exe


def _run(exe, d, Hq, Hkv, lengths, n=None, G=None):
    args = [exe, str(d), str(Hq), str(Hkv), ",".join(str(x) for x in lengths)]
    if n is not None:
        args += [str(n), str(G)]
    r = subprocess.run(args, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def _gpu_test_shapes():
    """(lengths, Hq, Hkv, d) of every GPU attention test launch (either kernel)."""
    from tests import test_gpu_consumer as T
    shapes = [(c[0], c[1], c[2], c[3]) for c in T.CASES]
    shapes += [(c[0], c[1], c[2], c[3]) for c in T.RANDOM_ATTENTION]
    shapes += [([256], 8, 2, 128), ([1000, 37], 8, 2, 128)]
    return [s for s in shapes if sum(s[0]) > 0]


@pytest.mark.parametrize("rows", [129600, 131072])
def test_replay_at_the_128k_layer_shapes(replay, rows):
    _run(replay, 128, 32, 8, [rows])


@pytest.mark.parametrize("rows", [129344, 131072])
def test_replay_at_the_gemma_like_d256_layer_shapes(replay, rows):
    """The 4-wave kernel at the Gemma-like layer's shapes (d = 256, Hq = 16, Hkv = 8)."""
    _run(replay, 256, 16, 8, [rows])


def test_replay_of_the_gpu_test_shapes(replay):
    shapes = _gpu_test_shapes()
    assert len(shapes) >= 10 and any(s[3] == 256 for s in shapes)
    for lengths, Hq, Hkv, d in shapes:
        _run(replay, d, Hq, Hkv, lengths)


@pytest.mark.parametrize("shape", [
    ([1], 8, 2, 64),                                 # one row
    ([63, 64, 65, 127, 128, 129], 8, 8, 128),        # tile edges, 4 tiles per workgroup
    ([0, 0, 5, 0], 6, 2, 64),                        # empty requests around one row
    ([8192, 16384, 65536, 24576, 49152, 32768, 12288, 12244], 32, 8, 128),   # varlen pack
    ([700, 1], 256, 256, 128),                       # the largest kv-head count served
    ([20000], 8, 1, 128),                            # MQA
    ([1], 4, 2, 256),                                # the 4-wave kernel: one row
    ([31, 32, 33, 95, 96, 97], 8, 8, 256),           # 32-token tile edges, 4 tiles per workgroup
    ([0, 0, 5, 0], 12, 2, 256),                      # empty requests around one row, HQ = 2
    ([700, 1], 512, 512, 128),                       # more kv heads than the 8-wave kernel serves
    ([3000], 2048, 512, 64),                         # four query heads per kv head, 512 kv heads
])
def test_replay_edge_shapes(replay, shape):
    lengths, Hq, Hkv, d = shape
    _run(replay, d, Hq, Hkv, lengths)


def test_replay_of_many_small_requests(replay):
    rng = np.random.default_rng(44)
    lengths = [int(x) for x in rng.integers(0, 151, 120)]
    for j in rng.integers(0, 120, 10):
        lengths[int(j)] = 0
    _run(replay, 64, 8, 2, lengths)
    _run(replay, 128, 12, 4, lengths)


def test_replay_of_the_window_statistics(replay):
    """The block statistics of up_rope_attention_scores: every (window row, block) pair
    written once, inside the request's pairs, for both kernels' tilings and every block
    size the GPU tests use (and the 128K decision's shape)."""
    from tests import test_gpu_attention_scores as T
    for lengths, Hq, Hkv, d, n, G, _ in T.CASES:
        _run(replay, d, Hq, Hkv, lengths, n, G)
    _run(replay, 128, 32, 8, [32768], 128, 64)
    _run(replay, 128, 32, 8, [131072], 128, 64)
    for G in (32, 96, 160, 1024):
        _run(replay, 64, 8, 2, [980, 1, 63, 64, 65, 4000], 128, G)
        _run(replay, 256, 16, 8, [980, 1, 63, 64, 65, 4000], 100, G)
