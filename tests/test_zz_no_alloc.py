"""pkv_decode_noalloc through the C ABI against pkv_decode (needs an MI355X).

The allocation-free entry point runs pkv_decode's plan and kernels with the
library's static scratch array as the workspace, so its outputs must equal
pkv_decode's bit for bit. Three calls in a row on one GPU, each smaller than
the last, check that the array's earlier contents never leak into a later
call: the wide batch (fixed 4096-token partitions, the largest workspace of
the decode workloads), then the batched workload (balanced split), then a
small ragged batch, and the largest batched workload once more at the end.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_36_amd as pkv
from paged_kv_cache_36_amd import synth
from tests.parity_util import assert_bf16_close, bits, oracle_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    pkv.load()


def both(case, partition_tokens):
    """(pkv_decode bits, fp32) and (pkv_decode_noalloc bits, fp32) for a case."""
    kw = dict(max_seq_len=max(case.max_seq_len, 1), partition_tokens=partition_tokens)
    ref32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    ref = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                     case.block_size, case.scale, out_f32=ref32, **kw)
    out = torch.empty_like(case.q)
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    pkv.decode_noalloc(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                       case.block_size, case.scale, out, out_f32=out32, **kw)
    torch.cuda.synchronize()
    return (bits(ref), ref32), (bits(out), out32), out


def test_noalloc_matches_decode_on_shrinking_calls():
    prm_sizes = []
    for name in ("wide_64seq_b832_p4096", "batched_8seq_t131072_b832"):
        case = synth.make_case(name, device="cuda")
        prm = pkv.make_params(case.q, case.k_cache, case.v_cache, case.block_table,
                              case.block_size, case.scale, case.max_seq_len,
                              case.partition_tokens)
        need = pkv.workspace_bytes(prm)
        prm_sizes.append(need)
        assert 0 < need <= pkv.noalloc_scratch_bytes(), (name, need)
        print(f"[gpu] noalloc {name}: workspace {need} bytes", flush=True)
        (rb, r32), (ob, o32), out = both(case, case.partition_tokens)
        assert np.array_equal(ob, rb), name
        assert torch.equal(o32, r32), name
        if name.startswith("batched"):
            assert_bf16_close(out, oracle_case(case)[0], what=f"noalloc {name}")
        del case
        torch.cuda.empty_cache()
    assert prm_sizes[1] < prm_sizes[0]
    # a smaller ragged batch with an empty sequence, fixed partitions, then the
    # same batch balanced
    small = synth.build_case("na_small", lens=[3000, 0, 65, 1, 777], block_size=784, seed=71,
                             device="cuda")
    ref_o = oracle_case(small, seqs=[0, 2, 3, 4])[0]
    for ptok in (512, 0):
        print(f"[gpu] noalloc small P={ptok}", flush=True)
        (rb, r32), (ob, o32), out = both(small, ptok)
        assert np.array_equal(ob, rb), ptok
        assert torch.equal(o32, r32), ptok
        assert np.all(bits(out)[1] == 0)
        assert_bf16_close(out, ref_o, rows=[0, 2, 3, 4], what=f"noalloc small P={ptok}")


def test_noalloc_rejects_a_plan_beyond_the_array():
    # 4096 sequences of up to 65536 tokens with 64-token partitions need far
    # more than the array: refused on the host, before any launch
    case = synth.build_case("na_big", lens=[64, 64], block_size=64, seed=72, device="cuda")
    q = torch.zeros((4096, 24, 256), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((4096, 1024), dtype=torch.int32, device="cuda")
    lens = torch.full((4096,), 64, dtype=torch.int32, device="cuda")
    prm = pkv.make_params(q, case.k_cache, case.v_cache, table, 64, 1 / 16, 65536, 64)
    assert pkv.workspace_bytes(prm) > pkv.noalloc_scratch_bytes()
    out = torch.empty_like(q)
    with pytest.raises(pkv.PkvError, match="status -9"):
        pkv.decode_noalloc(q, case.k_cache, case.v_cache, table, lens, 64, 1 / 16, out,
                           max_seq_len=65536, partition_tokens=64)
