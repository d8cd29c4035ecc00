"""Seeded random window-compression problems through the C ABI (needs an
MI355X).

Each seed draws 1 to 4 requests of 1 to 3000 tokens, a window length C (1 to
512), a state block size (1 to 32 rows), the boundary tokens (every token,
the window ends, or a random subset) and a part count (the library's, or a
forced one the limits allow). Every compressed row is checked against the
fp64 oracle within the compression tests' bound; the one-call operator
(pkv_compress_pack) must write exactly the bytes of pkv_compress followed by
pkv_compress_finalize, and a repeat call the same rows.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_36_amd as pkv
from paged_kv_cache_36_amd import synth
from tests.test_gpu_compress import check, run, to_dev
from tests.test_gpu_compress_pack import check_equal_to_two_calls

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    pkv.load()


def draw_problem(seed):
    rng = np.random.default_rng(5000 + seed)
    nreq = int(rng.integers(1, 5))
    lens = [int(rng.choice([1, int(rng.integers(2, 3001))])) for _ in range(nreq)]
    c = int(rng.choice([1, 2, 3, 16, 64, 100, 128, 256, 512]))
    bsz = int(rng.choice([1, 3, 8, 8, 16, 32]))
    kind = str(rng.choice(["all", "chunk_ends", "subset"]))
    total = sum(lens)
    if kind == "subset":
        bnd = sorted(int(x) for x in rng.choice(total, size=min(total, 50), replace=False))
    else:
        bnd = kind
    splits = int(rng.choice([0, 0, 1, 2, 3, 5, 8, 64]))
    return lens, c, bsz, bnd, splits


@pytest.mark.parametrize("seed", range(12))
def test_random_compress_problem(seed):
    lens, c, bsz, bnd, splits = draw_problem(seed)
    case = to_dev(synth.build_compress_case(f"rc{seed}", len(lens), sum(lens), c, block_size=bsz,
                                            seed=6000 + seed, lens=lens, boundaries=bnd))
    prm = pkv.compress_params(case.state_cache, case.token_to_req, case.boundaries,
                              case.block_table, c, splits)
    if pkv.compress_splits(prm) < 0:   # a forced count outside the limits: the library's own
        splits = 0
    print(f"[gpu] random compress seed={seed}: lens={lens} C={c} B={bsz} "
          f"boundaries={bnd if isinstance(bnd, str) else len(bnd)} splits={splits}", flush=True)
    if case.num_outputs == 0:
        return
    out = run(case, splits)
    assert torch.equal(out.view(torch.int32), run(case, splits).view(torch.int32)), "repeat"
    check(case, out, what=f"seed {seed}")
    check_equal_to_two_calls(case, splits, seed=seed)
