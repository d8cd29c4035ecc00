"""Seeded random decode problems across the plan space, through the C ABI,
against the fp64 oracle (needs an MI355X).

Each seed draws a batch (1 to 40 sequences), a page size (any multiple of 16
up to 1024), a partition size (left to the library, which picks the balanced
split for a batch, or fixed from 64 to 4096 tokens), lengths mixing empty
sequences, single tokens, lengths one off a page or partition boundary and
long ones, the K/V layout (separate caches or the unbind view of one joint
cache) and the softmax scale. The plan the library reports must match the
documented rule; the bf16 output must be within the elementwise tolerance,
the fp32 output within the per-row bound, empty sequences must give zero rows,
and a second call must give the same bits.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_36_amd as pkv
from paged_kv_cache_36_amd import synth
from tests.parity_util import (assert_bf16_close, assert_rows_rel, bits, f64,
                               oracle_case_parallel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    pkv.load()


def draw_problem(seed):
    rng = np.random.default_rng(1000 + seed)
    nseq = int(rng.choice([1, 2, 3, 7, 17, 40]))
    bsz = 16 * int(rng.integers(1, 65))
    ptok = int(rng.choice([0, 64, 128, 192, 256, 512, 1024, 4096]))
    edge = ptok if ptok else 64
    lens = []
    for _ in range(nseq):
        kind = rng.random()
        if kind < 0.1:
            lens.append(0)
        elif kind < 0.15:
            lens.append(1)
        elif kind < 0.35:
            lens.append(max(1, bsz * int(rng.integers(1, 8)) + int(rng.integers(-1, 2))))
        elif kind < 0.55:
            lens.append(max(1, edge * int(rng.integers(1, 6)) + int(rng.integers(-1, 2))))
        else:
            lens.append(int(rng.integers(2, 12001)))
    if nseq == 1 and lens[0] == 0:
        lens[0] = 5000
    joint = bool(rng.random() < 0.3)
    scale = float(rng.choice([1.0 / 16.0, 0.05, 0.125]))
    return lens, bsz, ptok, joint, scale


@pytest.mark.parametrize("seed", range(48))
def test_random_decode_problem(seed):
    lens, bsz, ptok, joint, scale = draw_problem(seed)
    print(f"[gpu] random seed={seed}: S={len(lens)} B={bsz} P={ptok} joint={joint} "
          f"scale={scale} max_len={max(lens)}", flush=True)
    case = synth.build_case(f"rnd{seed}", lens=lens, block_size=bsz, seed=2000 + seed,
                            scale=scale, device="cuda", joint_kv=joint)
    max_len = max(max(lens), 1)
    prm = pkv.make_params(case.q, case.k_cache, case.v_cache, case.block_table, bsz, scale,
                          max_len, ptok)
    info = pkv.plan(prm)
    multi = len(lens) > 1
    assert info["balanced"] == (1 if ptok == 0 and multi else 0)
    assert info["k_rows"] == (1 if multi else 0)
    assert info["ordered"] == (1 if not info["balanced"] and multi and
                               info["num_partitions"] > 1 else 0)
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    out = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens, bsz,
                     scale, max_seq_len=max_len, partition_tokens=ptok, out_f32=out32)
    again = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens, bsz,
                       scale, max_seq_len=max_len, partition_tokens=ptok)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(again)), "repeat call differs"
    live = [s for s, n in enumerate(lens) if n > 0]
    ref, _ = oracle_case_parallel(case, seqs=live)
    assert_bf16_close(out, ref, rows=live, what=f"seed {seed}")
    assert_rows_rel(f64(out32)[live], ref[live], what=f"seed {seed} fp32")
    for s, n in enumerate(lens):
        if n == 0:
            assert np.all(f64(out)[s] == 0) and np.all(f64(out32)[s] == 0)
