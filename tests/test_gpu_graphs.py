"""Every entry point the bench times (and the allocation-free decode) under HIP
graphs, replayed: each replay
must reproduce the eager result bit for bit, with unrelated eager work and
synchronisations between the replays (the library records no memsets and
allocates nothing, so a captured call is the same launches as an eager one).
"""

from __future__ import annotations

import pytest
import torch

import paged_kv_cache_36_amd as pkv
from paged_kv_cache_36_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    pkv.load()


def replay_matches(fn, outputs, replays=3, reset=None):
    """Run fn eagerly, capture it, then replay and compare every output.
    Between replays the outputs are overwritten (reset() restores the state
    the call starts from for outputs it only partly writes)."""
    stream = torch.cuda.Stream()
    if reset:
        reset()
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    noise = torch.randn(1 << 20, device="cuda")
    for r in range(replays):
        for o in outputs:
            o.fill_(7)                          # eager work between replays
        if reset:
            reset()
        noise.mul_(1.0001)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):   # raw bytes: random bit patterns include NaNs
            assert torch.equal(o.contiguous().view(torch.uint8), w.view(torch.uint8)), \
                f"replay {r} differs from the eager result"


@pytest.mark.parametrize("name", ["long_l8192_b832", "batched_8seq_t131072_b832",
                                  "wide_64seq_b832_p4096"])
def test_decode_graph_replays(name):
    print(f"[gpu] graph decode {name}", flush=True)
    case = synth.make_case(name, device="cuda")
    prm = pkv.make_params(case.q, case.k_cache, case.v_cache, case.block_table, case.block_size,
                          case.scale, case.max_seq_len, case.partition_tokens)
    ws = torch.empty(max(pkv.workspace_bytes(prm), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(case.q)
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")

    def fn():
        pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                   case.block_size, case.scale, max_seq_len=case.max_seq_len,
                   partition_tokens=case.partition_tokens, out=out, out_f32=out32, workspace=ws)

    replay_matches(fn, [out, out32])


def test_decode_noalloc_graph_replays():
    # the allocation-free entry point is meant for callers that capture
    # graphs: captured after one eager call, each replay gives its bits
    print("[gpu] graph decode_noalloc", flush=True)
    case = synth.build_case("gna", lens=[3000, 65, 1, 777], block_size=784, seed=33,
                            device="cuda")
    out = torch.empty_like(case.q)
    out32 = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")

    def fn():
        pkv.decode_noalloc(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                           case.block_size, case.scale, out, max_seq_len=case.max_seq_len,
                           out_f32=out32)

    replay_matches(fn, [out, out32])


def test_prefill_graph_replays():
    print("[gpu] graph prefill", flush=True)
    case, q_new = synth.build_prefill_case("gp", 700, 3000, 832, seed=31, device="cuda")
    out = torch.empty_like(q_new)

    def fn():
        pkv.prefill(q_new, case.k_cache, case.v_cache, case.block_table[0], case.lens[0],
                    case.block_size, case.scale, out=out)

    replay_matches(fn, [out])


def test_append_graph_replays():
    print("[gpu] graph append", flush=True)
    pool, rows, slots = synth.append_inputs(3000, 832, 8, seed=5, pad_every=9, device="cuda")
    kc = pool.clone()
    vc = pool.clone()

    def reset():
        kc.copy_(pool)
        vc.copy_(pool)

    def fn():
        pkv.append(rows, rows, slots, kc, vc)

    replay_matches(fn, [kc, vc], reset=reset)


@pytest.mark.parametrize("name", ["compress_r1_t8192_c512", "compress_r8_t65536_c128"])
def test_compress_and_finalize_graph_replays(name):
    print(f"[gpu] graph compress {name}", flush=True)
    case = synth.make_compress_case(name, device="cuda")
    n = case.num_outputs
    prm = pkv.compress_params(case.state_cache, case.token_to_req, case.boundaries,
                              case.block_table, case.compress_ratio)
    ws = torch.empty(max(pkv.compress_workspace_bytes(prm), 256), dtype=torch.uint8,
                     device="cuda")
    comp = torch.empty((n, 512), dtype=torch.float32, device="cuda")
    gen = torch.Generator().manual_seed(3)
    weight = (torch.rand(512, generator=gen) + 0.5).cuda()
    th = torch.rand((int(case.positions.max()) + 1, 32), generator=gen) * 6.283
    cos_sin = torch.cat([torch.cos(th), torch.sin(th)], 1).cuda()
    pages = (n + 63) // 64 + 1
    slots = torch.full((case.positions.shape[0],), -1, dtype=torch.int64)
    slots[case.boundaries.cpu()] = torch.randperm(pages * 64, generator=gen)[:n]
    slots = slots.cuda()
    kv = torch.zeros((pages, pkv.KV_PAGE_BYTES), dtype=torch.uint8, device="cuda")

    def fn():
        pkv.compress(case.state_cache, case.token_to_req, case.positions, case.boundaries,
                     case.block_table, case.compress_ratio, out=comp, workspace=ws)
        pkv.compress_finalize(comp, case.positions, case.boundaries, weight, cos_sin, slots, kv,
                              case.compress_ratio)

    replay_matches(fn, [comp, kv], reset=kv.zero_)
