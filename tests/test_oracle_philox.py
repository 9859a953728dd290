"""Pin of the oracle's Philox4x32-10 generator and its dropout-mask rule.

The pages fix only that each FC6/FC7 unit is dropped with probability 0.5
during training (paper-graph-ui "Dropout"); the counter-based generator is how
the masks are made reproducible, and the oracle implements Philox4x32-10 from
its published definition (Salmon, Moraes, Dror, Shaw, SC'11).  This test pins
that implementation to a second, independent one: PyTorch's source-level
engine in ATen/core/PhiloxRNGEngine.h, compiled here with g++ into a tiny
wrapper (tests/philox_torch_ref.cpp).  A swapped output word, a wrong Weyl key
increment, a wrong round count or multiplier, or a mask that indexes the
counter by element instead of by block of four all fail it.

Counter mapping: the oracle's counter (block, layer, step mod 2^32, step / 2^32)
is the engine's (offset lo, offset hi, subsequence lo, subsequence hi) with
offset = layer * 2^32 + block and subsequence = step; both keys are
(seed mod 2^32, seed / 2^32).
"""
import ctypes as C
import math
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    torch = pytest.importorskip("torch")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    hdr = os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")
    if not os.path.exists(hdr):
        pytest.skip("torch's PhiloxRNGEngine.h source header is not installed")
    out = str(tmp_path_factory.mktemp("philox") / "libphilox_torch_ref.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-I" + inc,
                    os.path.join(HERE, "philox_torch_ref.cpp"), "-o", out], check=True)
    lib = C.CDLL(out)
    lib.ref_philox_block.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.POINTER(C.c_uint32)]
    lib.ref_philox_block.restype = None

    def block(seed, step, layer, blk):
        w = (C.c_uint32 * 4)()
        lib.ref_philox_block(seed, step, (layer << 32) | blk, w)
        return np.array(list(w), np.uint32)
    return block


def _tuples():
    rng = np.random.default_rng(20121203)
    edge = [0, 1, 2**31, 2**32 - 1, 2**32, 2**32 + 7, 2**63 + 12345, 2**64 - 1]
    out = [(0, 0, 0, 0), (3, 0, 0, 0), (3, 0, 1, 0), (2**64 - 1, 2**64 - 1, 2**32 - 1, 2**32 - 1)]
    for s in edge:
        for t in edge[::2]:
            out.append((s, t, int(rng.integers(0, 2)), int(rng.integers(0, 2**32))))
    for _ in range(300):
        out.append((int(rng.integers(0, 2**64, dtype=np.uint64)),
                    int(rng.integers(0, 2**64, dtype=np.uint64)),
                    int(rng.integers(0, 2**32)) if rng.random() < 0.2 else int(rng.integers(0, 2)),
                    int(rng.integers(0, 2**32))))
    return out


def test_philox_block_matches_torch_engine(orc, torch_philox):
    """Every output word of the oracle's Philox4x32-10 equals the torch
    engine's, over 340 (seed, step, layer, block) tuples including seeds and
    steps at and above 2^32 and both FC layers."""
    bad = []
    for seed, step, layer, blk in _tuples():
        ctr = [blk, layer, step & 0xFFFFFFFF, step >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        got = np.asarray(orc.philox4x32_10(ctr, key), np.uint32)
        ref = torch_philox(seed, step, layer, blk)
        if not np.array_equal(got, ref):
            bad.append((seed, step, layer, blk, got.tolist(), ref.tolist()))
    assert not bad, f"{len(bad)} Philox blocks differ from the torch engine, first: {bad[0]}"


@pytest.mark.parametrize("seed,step,layer,rows,cols", [
    (3, 0, 0, 5, 4096),              # the training workload's key, FC6, step 0
    (3, 0, 1, 3, 4096),              # FC7
    (2**40 + 9, 2**33 + 5, 0, 2, 4096),   # key and step above 2^32
    (11, 7, 1, 3, 1001),             # ragged: the last block of four is partial
])
def test_dropout_mask_rule_matches_torch_engine(orc, torch_philox, seed, step, layer, rows, cols):
    """Element e = row*cols + col draws word (e mod 4) of the block at counter
    e / 4 and is dropped iff that word is below floor(p * 2^32); checked
    element by element against the torch engine's words for p = 0.5, 0.3, 0.75."""
    total = rows * cols
    words = np.concatenate([torch_philox(seed, step, layer, b) for b in range((total + 3) // 4)])[:total]
    for p in (0.5, 0.3, 0.75):
        thresh = math.floor(p * 2.0**32)
        want = (words >= np.uint32(thresh)).astype(np.uint8).reshape(rows, cols)
        got = np.asarray(orc.dropout_mask(seed, step, layer, rows, cols, p))
        assert got.shape == (rows, cols)
        np.testing.assert_array_equal(got, want, err_msg=f"p={p}")
