"""GPU parity of small-row calls whose activations come prepared (slices above the 8 KB LDS
staging budget per wave) with packed zero points on 64-column tiles: the instance that streams a
3-step ring of weight and activation fragments. Each wave's K piece takes 9 to 16 steps, so every
remainder of the ring's whole rounds (0, 1 and 2 steps left over) occurs, also within one launch
where the pieces differ by a step; 11 to 16 rows; a ragged last tile. Outputs are checked element
by element against the oracle, and repeats are bit-identical.
"""
import numpy as np
import pytest

import oracle
from tests import parity
from verify_matmul_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import verify_matmul_amd as vm
    from tests import gpu_util
    vm.load()
    return gpu_util


# (M, K, N, g, splits, waves_k): steps per wave = K / 32 / (splits * waves_k), rounded both ways
CASES = [
    (16, 576, 264, 32, 1, 2),     # 9 steps a wave (3 whole rounds)
    (13, 640, 264, 64, 1, 2),     # 10 (one step left)
    (12, 704, 264, 32, 1, 2),     # 11 (two left)
    (14, 800, 136, 32, 1, 2),     # 12 and 13 in one launch
    (11, 864, 520, 32, 1, 2),     # 13 and 14
    (16, 2048, 264, 128, 2, 2),   # 16, two K slices
    (15, 3072, 200, 64, 2, 4),    # 12, two slices of four waves
]


@pytest.mark.parametrize("M,K,N,g,splits,wk", CASES)
def test_prepared_ring_parity(gu, M, K, N, g, splits, wk):
    steps = K // 32
    longest = -(-steps // (splits * wk))
    assert M * longest * 4 * 16 > 8 * 1024   # the slice exceeds the staging budget: prepared
    inp = synth.make_random(7000 + M + K // 32 + N, M, K, N, g, symmetric=False)
    d = gu.DevInputs(inp)
    gu.say(f"[prepared ring] M={M} K={K} N={N} g={g} splits={splits} waves_k={wk}")
    y = d.run(M, splits=splits, waves_k=wk, tile_cols=64)
    y_ref, bound = oracle.gemm(inp.act, inp.qweight, inp.scales, inp.qzeros, g)
    frac = parity.check_close(y, y_ref, bound, f"prepared ring M={M} K={K} N={N}")
    gu.say(f"  worst err/tol {frac:.3e}")
    assert np.array_equal(d.run(M, splits=splits, waves_k=wk, tile_cols=64), y)
