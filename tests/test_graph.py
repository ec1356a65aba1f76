"""A decode step, and a chunked-prefill step, captured in a HIP graph and replayed.

The step is what a serving loop issues per generated token: write each
sequence's new K / V into its slot (pa_append_kv, from the lengths and the
tables), then attend over the grown context (pa_decode, split plan with a
caller-owned workspace).  Neither call allocates, synchronises or clears
memory, so the pair can be captured once and replayed while the caller
updates the lengths, the new token's K / V and the query in place.

The chunked-prefill step writes each prompt's next chunk of K / V by a slot
mapping (pa_write_kv), then runs the causal multi-token call over the chunk
(pa_prefill): the caller moves the slots, queries, K / V and lengths one
chunk further between replays.

Every replay is checked bit for bit against the same two calls issued
eagerly on a second copy of the state (same kernels, same plan), with eager
work and synchronisations between replays; the last replay is also checked
against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_check import check
from paged_kv_cache_301_amd import binding, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def _step(knew, vnew, q, tables, lens, kc, vc, out, ws, scale, kernel, part, tw):
    binding.append_kv(knew, vnew, tables, lens, kc, vc)
    binding.decode(q, kc, vc, tables, lens, scale, out, kernel=kernel, partition_tokens=part,
                   workspace=ws, token_waves=tw)


@pytest.mark.parametrize("kernel,Hq,Hkv,B,part,tw", [
    ("valu", 8, 8, 16, 128, 0), ("mfma", 16, 4, 16, 128, 0), ("mfma", 64, 1, 8, 96, 0),
    ("generic", 4, 2, 16, 0, 0), ("valu", 8, 8, 16, 512, 4), ("mfma", 32, 8, 1, 512, 2)])
def test_append_and_decode_graph_replays(kernel, Hq, Hkv, B, part, tw):
    print(f"case: graph append+decode {kernel} Hq={Hq} Hkv={Hkv} B={B} part={part} tw={tw}",
          flush=True)
    final = (40, 300, 17, 1000, 513, 64)
    spec = workloads.WorkloadSpec("graph", S=len(final), Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                                  lens=("fixed", final), max_len=1024, pool=("free", 0.3), seed=9)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    S, D = w.S, w.D
    tables = w.block_tables
    # the tables already hold the blocks of the final lengths; start REPLAYS
    # tokens short of them, so every replay appends into an allocated slot
    lens = (w.seq_lens - REPLAYS).contiguous()
    ref_lens = lens.clone()
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    ref_kc, ref_vc = w.key_cache.clone(), w.value_cache.clone()
    q = torch.empty_like(w.query)
    knew = torch.empty((S, Hkv, D), dtype=w.dtype, device=DEV)
    vnew = torch.empty_like(knew)
    plan = binding.plan(S, Hq, Hkv, D, B, w.NB, w.max_blocks, w.dtype, torch.float32,
                        kernel=kernel, partition_tokens=part, token_waves=tw)
    assert tw == 0 or plan["token_waves"] == tw
    nbytes = max(plan["workspace_bytes"], 256)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ref_ws = torch.empty_like(ws)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=DEV)
    ref_out = torch.empty_like(out)
    args = dict(scale=w.scale, kernel=kernel, part=part, tw=tw)

    # load the kernels' code once, eagerly, on throw-away copies of the state
    q.zero_(); knew.zero_(); vnew.zero_()
    _step(knew, vnew, q, tables, lens.clone(), kc.clone(), vc.clone(), out.clone(), ws.clone(),
          **args)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(DEV)
    stream.wait_stream(torch.cuda.current_stream(DEV))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        _step(knew, vnew, q, tables, lens, kc, vc, out, ws, **args)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(1234)
    for r in range(REPLAYS):
        # the caller's per-token updates, eager and in place
        q.copy_(torch.randn(q.shape, generator=gen).to(w.dtype))
        knew.copy_(torch.randn(knew.shape, generator=gen).to(w.dtype))
        vnew.copy_(torch.randn(vnew.shape, generator=gen).to(w.dtype))
        lens += 1
        graph.replay()
        torch.cuda.synchronize()
        ref_lens += 1
        _step(knew, vnew, q, tables, ref_lens, ref_kc, ref_vc, ref_out, ref_ws, **args)
        torch.cuda.synchronize()
        assert torch.equal(lens, ref_lens)
        assert torch.equal(out, ref_out), f"replay {r}: output differs from the eager step"
        assert torch.equal(kc.view(torch.int16), ref_kc.view(torch.int16)), f"replay {r}: key cache"
        assert torch.equal(vc.view(torch.int16), ref_vc.view(torch.int16)), f"replay {r}: value cache"
    assert torch.equal(lens.cpu(), torch.tensor(final, dtype=torch.int32))
    ref = oracle.decode(q, kc, vc, tables, lens, w.scale)
    check(out, ref, w.dtype, f"graph/{kernel}")


def _chunk(knew, vnew, q, slots, tables, lens, qstart, kc, vc, out, ws, scale, kernel, chunk):
    binding.write_kv(knew, vnew, slots, kc, vc)
    binding.prefill(q, kc, vc, tables, lens, qstart, scale, out, max_query_len=chunk,
                    kernel=kernel, workspace=ws)


@pytest.mark.parametrize("kernel,Hq,Hkv,B,chunk", [("mfma", 32, 8, 16, 32), ("mfma", 8, 8, 1, 64),
                                                   ("mfma", 64, 1, 8, 4), ("generic", 8, 2, 16, 32)])
def test_chunked_prefill_graph_replays(kernel, Hq, Hkv, B, chunk):
    """A chunked-prefill step captured once: the slot-mapped write of each
    sequence's next chunk of prompt K / V, then causal attention of the
    chunk's queries over everything before them.  Every replay moves each
    sequence one chunk further, the caller updating slots, queries, K / V
    and lengths in place; each replay equals the same calls issued eagerly
    on a second copy of the state, bit for bit, and the last one the oracle."""
    print(f"case: graph chunked prefill {kernel} Hq={Hq} Hkv={Hkv} B={B} chunk={chunk}",
          flush=True)
    final = (4 * chunk + 40, 4 * chunk + 300, 4 * chunk, 4 * chunk + 700)
    spec = workloads.WorkloadSpec("graph_prefill", S=len(final), Hq=Hq, Hkv=Hkv, D=128, B=B,
                                  dtype="bf16", lens=("fixed", final), max_len=max(final),
                                  pool=("free", 0.3), seed=19)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    S, D, T = w.S, w.D, w.S * chunk
    tables = w.block_tables
    lens = (w.seq_lens - REPLAYS * chunk).contiguous()
    ref_lens = lens.clone()
    kc, vc = w.key_cache.clone(), w.value_cache.clone()
    ref_kc, ref_vc = w.key_cache.clone(), w.value_cache.clone()
    q = torch.zeros((T, Hq, D), dtype=w.dtype, device=DEV)
    knew = torch.zeros((T, Hkv, D), dtype=w.dtype, device=DEV)
    vnew = torch.zeros_like(knew)
    slots = torch.full((T,), -1, dtype=torch.int32, device=DEV)
    qstart = torch.arange(0, T + 1, chunk, dtype=torch.int32, device=DEV)
    plan = binding.plan_prefill(S, T, Hq, Hkv, D, B, w.NB, w.max_blocks, chunk, w.dtype,
                                torch.float32, kernel=kernel)
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device=DEV)
    ref_ws = torch.empty_like(ws)
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=DEV)
    ref_out = torch.empty_like(out)
    args = dict(scale=w.scale, kernel=kernel, chunk=chunk)

    # load the kernels' code once, eagerly, on throw-away copies of the state
    _chunk(knew, vnew, q, slots, tables, lens.clone() + chunk, qstart, kc.clone(), vc.clone(),
           out.clone(), ws.clone(), **args)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(DEV)
    stream.wait_stream(torch.cuda.current_stream(DEV))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        _chunk(knew, vnew, q, slots, tables, lens, qstart, kc, vc, out, ws, **args)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(4321)
    tab = w.tables_host
    for r in range(REPLAYS):
        # the next chunk of every prompt: its slots by the table, then the
        # grown lengths (they count the chunk)
        start = lens.cpu().numpy()
        sl = [int(tab[s, t // B]) * B + t % B for s in range(S)
              for t in range(int(start[s]), int(start[s]) + chunk)]
        slots.copy_(torch.tensor(sl, dtype=torch.int32))
        q.copy_(torch.randn(q.shape, generator=gen).to(w.dtype))
        knew.copy_(torch.randn(knew.shape, generator=gen).to(w.dtype))
        vnew.copy_(torch.randn(vnew.shape, generator=gen).to(w.dtype))
        lens += chunk
        graph.replay()
        torch.cuda.synchronize()
        ref_lens += chunk
        _chunk(knew, vnew, q, slots, tables, ref_lens, qstart, ref_kc, ref_vc, ref_out, ref_ws,
               **args)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: output differs from the eager step"
        assert torch.equal(kc.view(torch.int16), ref_kc.view(torch.int16)), f"replay {r}: key cache"
        assert torch.equal(vc.view(torch.int16), ref_vc.view(torch.int16)), f"replay {r}: value cache"
    assert torch.equal(lens.cpu(), torch.tensor(final, dtype=torch.int32))
    ref = oracle.prefill(q, kc, vc, tables, lens, qstart, w.scale)
    check(out, ref, w.dtype, f"graph prefill/{kernel}")
