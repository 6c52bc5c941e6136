"""The seeded rotation draws (CPU): the library's tq_make_rotation and the oracle's
make_rotation are two independent implementations of one stated definition (SplitMix64
draws, a sign per draw's top bit, fp64 Box-Muller pairs rounded to fp32).  The oracle's
generator is pinned to the published SplitMix64 reference outputs and its draws to the
laws they must follow; the library's tables must then equal the oracle's bit for bit."""
import ctypes
import math
import os

import numpy as np
import pytest
from scipy import stats

import compressed_attention_rotate_amd as tq
from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [int(line) for line in f if line.strip() and not line.startswith("#")]


def test_splitmix64_matches_published_reference_outputs():
    assert O.splitmix64(1234567, 5) == _golden_ints("splitmix64_seed1234567.txt")


@pytest.mark.parametrize("d", [8, 128, 256])
@pytest.mark.parametrize("seed", [0, 1, 1_500_002, 2**63 + 7, 2**64 - 1])
def test_library_rotation_equals_oracle_bit_for_bit(d, seed):
    s_o, S_o = O.make_rotation(d, seed)
    s_l, S_l = tq.make_rotation(d, seed)
    assert np.array_equal(s_o, s_l)
    assert np.array_equal(S_o.view(np.uint32), S_l.view(np.uint32))


def test_rotation_draws_follow_their_laws():
    """Signs are fair coins, S entries standard normal (Kolmogorov-Smirnov over 65536
    values), and distinct seeds give unrelated tables."""
    signs, S = O.make_rotation(256, 4242)
    assert set(np.unique(signs).tolist()) == {-1, 1}
    assert abs(int(np.sum(signs))) < 4 * math.sqrt(256)
    ks = stats.kstest(S.astype(np.float64).ravel(), "norm")
    assert ks.pvalue > 1e-3, ks
    assert abs(float(np.mean(S))) < 4 / 256 and abs(float(np.var(S)) - 1.0) < 0.03
    _, S2 = O.make_rotation(256, 4243)
    assert abs(np.corrcoef(S.ravel(), S2.ravel())[0, 1]) < 0.02


def test_make_rotation_argument_errors():
    lib = tq.load()
    signs = np.zeros(64, np.int8)
    S = np.zeros((64, 64), np.float32)
    for d in (0, 4, 100, 8192):
        assert lib.tq_make_rotation(d, 1, signs.ctypes.data, S.ctypes.data) == -2
    assert lib.tq_make_rotation(64, 1, None, S.ctypes.data) == -1
    assert lib.tq_make_rotation(64, 1, signs.ctypes.data, None) == -1
    assert lib.tq_make_rotation(64, ctypes.c_uint64(7), signs.ctypes.data, S.ctypes.data) == 0
    assert np.array_equal(S, O.make_rotation(64, 7)[1])
