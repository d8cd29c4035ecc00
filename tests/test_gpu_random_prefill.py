"""Seeded random tail-Q prefill problems through the C ABI against the fp64
oracle (needs an MI355X).

Each seed draws the number of new queries Q (1 to 600), the cached length L
(Q to Q + 4000), a page size (1 token up to 1024, not only multiples of 16),
the key-split count (left to the library, or forced from 1 to 64, which can
leave splits with only masked or no keys) and the softmax scale. Every query
row is checked with the bounds of the prefill tests (bf16 elementwise, fp32
within 2^-8 max|v| of the row's visible keys), and a second call must give
the same bits.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_36_amd as pkv
from paged_kv_cache_36_amd import synth
from tests.parity_util import bits
from tests.test_gpu_prefill import check, run_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    pkv.load()


def draw_problem(seed):
    rng = np.random.default_rng(3000 + seed)
    if rng.random() < 0.3:
        nq = int(rng.choice([1, 2, 128, 129]))
    else:
        nq = int(rng.integers(3, 601))
    length = nq + int(rng.choice([0, 1, int(rng.integers(2, 4001))]))
    bsz = int(rng.choice([1, 5, 16, 48, 64, 100, 784, 832, int(rng.integers(1, 1025))]))
    splits = int(rng.choice([0, 0, 1, 2, 3, 7, 16, 64]))
    scale = float(rng.choice([1.0 / 16.0, 0.05, 0.125]))
    return nq, length, bsz, splits, scale


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_problem(seed):
    nq, length, bsz, splits, scale = draw_problem(seed)
    print(f"[gpu] random prefill seed={seed}: Q={nq} L={length} B={bsz} splits={splits} "
          f"scale={scale}", flush=True)
    case, q_new = synth.build_prefill_case(f"rpf{seed}", nq, length, bsz, seed=4000 + seed,
                                           device="cuda")
    case.scale = scale
    out, out32 = run_prefill(case, q_new, key_splits=splits)
    again, _ = run_prefill(case, q_new, key_splits=splits)
    assert np.array_equal(bits(out), bits(again)), "repeat call differs"
    check(case, q_new, out, out32)
