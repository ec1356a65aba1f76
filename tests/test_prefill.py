"""Several new tokens per sequence, causal (chunked prefill).

CPU: the oracle's causal rows pinned to the pages' worked example read as a
five-token prefill (each row's closed form; the last row is the printed
4.1256), to unpaged attention with an explicit causal mask computed by
torch's SDPA routine, and to causality itself (NaN in every later token
leaves a row unchanged).  Host validation of the C ABI.
GPU: the library against the oracle on identical inputs (both kernels, every
group size, block sizes 1..32, forced partitions, ragged chunks, and a seeded
sweep of random shapes over all of these), an exact
needle check of positions, staged calls, and the benchmark-sized workload on
every (query row, head).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_build import random_logical, scatter_paged
from paged_kv_cache_301_amd import binding as b
from paged_kv_cache_301_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda:0"


def causal_reference(q_rows, Ks, Vs, n_new, scale):
    """torch SDPA in fp64 with an explicit mask: row k of sequence s (position
    L - n + k) may see logical tokens 0 .. L - n + k."""
    S = len(Ks)
    T, Hq, D = q_rows.shape
    out = torch.zeros((T, Hq, D), dtype=torch.float64)
    r0 = 0
    for s in range(S):
        L, n = Ks[s].shape[0], int(n_new[s])
        if n == 0:
            continue
        Hkv = Ks[s].shape[1]
        G = Hq // Hkv
        q = q_rows[r0:r0 + n].double().permute(1, 0, 2)                  # [Hq, n, D]
        k = Ks[s].double().permute(1, 0, 2).repeat_interleave(G, 0)      # [Hq, L, D]
        v = Vs[s].double().permute(1, 0, 2).repeat_interleave(G, 0)
        pos = torch.arange(L - n, L)
        mask = torch.arange(L)[None, :] <= pos[:, None]                   # [n, L]
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=mask[None, None], scale=scale)[0]
        out[r0:r0 + n] = o.permute(1, 0, 2)
        r0 += n
    return out


def _worked_pool():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    kc = torch.full((9, 1, 2, 2), float("nan"))
    vc = torch.full((9, 1, 2, 2), float("nan"))
    for pid, blk in ex["blocks"].items():
        kc[int(pid), 0] = torch.tensor(blk["K"])
        vc[int(pid), 0] = torch.tensor(blk["V"])
    kc[1, 0, 1] = float("nan")
    vc[1, 0, 1] = float("nan")
    return ex, kc, vc


def test_worked_example_as_prefill():
    """All five tokens new, each with the example's query: row k attends the
    first k+1 (score, value) pairs of the page's Step 2 / Setup."""
    ex, kc, vc = _worked_pool()
    q = torch.tensor(ex["query"]).repeat(5, 1).reshape(5, 1, 2)
    out = oracle.prefill(q, kc, vc, torch.tensor([ex["block_table"]], dtype=torch.int32),
                         torch.tensor([5], dtype=torch.int32),
                         torch.tensor([0, 5], dtype=torch.int32), 1.0)
    scores = [1.0, 2.0, 3.0, 2.0, 4.0]
    values = [1.0, 2.0, 3.0, 4.0, 5.0]
    for k in range(5):
        m = max(scores[:k + 1])
        w = [math.exp(x - m) for x in scores[:k + 1]]
        expect = math.fsum(a * v for a, v in zip(w, values)) / math.fsum(w)
        assert abs(out[k, 0, 0] - expect) < 1e-14 and out[k, 0, 0] == out[k, 0, 1]
    assert out[0, 0, 0] == 1.0                                  # one token: its V exactly
    assert round(out[4, 0, 0], 4) == ex["printed"]["output_code"][0]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_oracle_matches_masked_sdpa(dtype):
    gen = torch.Generator().manual_seed(11)
    rng = np.random.default_rng(11)
    lens = [1, 7, 16, 40, 33, 9]
    n_new = [1, 7, 5, 17, 0, 3]                                 # full prefill, chunk, empty
    Hkv, Hq, D, B = 2, 6, 8, 4
    Ks, Vs = random_logical(len(lens), Hkv, D, lens, gen=gen, dtype=dtype)
    pk = scatter_paged(Ks, Vs, B, rng=rng, dtype=dtype)
    T = sum(n_new)
    q = torch.randn((T, Hq, D), generator=gen).to(dtype)
    qs = torch.tensor(np.concatenate([[0], np.cumsum(n_new)]), dtype=torch.int32)
    got = oracle.prefill(q, pk["key_cache"], pk["value_cache"], pk["block_tables"],
                         pk["seq_lens"], qs, 0.37)
    ref = causal_reference(q, Ks, Vs, n_new, 0.37).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def test_oracle_is_causal():
    """Every token after a row's position set to NaN: that row is unchanged."""
    gen = torch.Generator().manual_seed(12)
    L, n, D, B = 30, 12, 8, 4
    Ks, Vs = random_logical(1, 1, D, [L], gen=gen)
    pk = scatter_paged(Ks, Vs, B, rng=np.random.default_rng(12))
    q = torch.randn((n, 2, D), generator=gen)
    qs = torch.tensor([0, n], dtype=torch.int32)
    args = (pk["block_tables"], pk["seq_lens"], qs, 0.5)
    full = oracle.prefill(q, pk["key_cache"], pk["value_cache"], *args)
    for k in (0, 5, n - 1):
        pos = L - n + k
        K2, V2 = Ks[0].clone(), Vs[0].clone()
        K2[pos + 1:] = float("nan")
        V2[pos + 1:] = float("nan")
        p2 = scatter_paged([K2], [V2], B, rng=np.random.default_rng(12))
        cut = oracle.prefill(q, p2["key_cache"], p2["value_cache"], *args)
        assert np.array_equal(cut[k], full[k])
        if k < n - 1:
            assert np.isnan(cut[n - 1]).all()                   # a later row does see them


def test_oracle_single_new_token_is_decode():
    gen = torch.Generator().manual_seed(13)
    lens = [3, 17, 8]
    Ks, Vs = random_logical(3, 2, 8, lens, gen=gen, dtype=torch.bfloat16)
    pk = scatter_paged(Ks, Vs, 4, rng=np.random.default_rng(13), dtype=torch.bfloat16)
    q = torch.randn((3, 4, 8), generator=gen).to(torch.bfloat16)
    a = oracle.prefill(q, pk["key_cache"], pk["value_cache"], pk["block_tables"], pk["seq_lens"],
                       torch.tensor([0, 1, 2, 3], dtype=torch.int32), 0.3)
    d = oracle.decode(q, pk["key_cache"], pk["value_cache"], pk["block_tables"], pk["seq_lens"], 0.3)
    assert np.array_equal(a, d)


# ------------------------------------------------------------------ C ABI (host)

def test_prefill_validation():
    lib = b.load()
    fake = 1 << 20

    def call(S=2, T=4, Hq=4, Hkv=2, D=128, B=16, NB=8, mb=4, mq=2, dt=b.PA_BF16, odt=b.PA_BF16,
             null=(), cfg=None, ws=None, ws_bytes=0):
        ptrs = [None if i in null else fake for i in range(7)]
        import ctypes
        return lib.pa_prefill(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], ptrs[5], 0.1, ptrs[6],
                              S, T, Hq, Hkv, D, B, NB, mb, mq, dt, odt,
                              ctypes.byref(cfg) if cfg else None, ws, ws_bytes, None)
    assert call(T=-1) == b.PA_ERR_SHAPE
    assert call(T=70000) == b.PA_ERR_SHAPE
    assert call(mq=0) == b.PA_ERR_SHAPE
    assert call(Hq=6, Hkv=4) == b.PA_ERR_SHAPE
    assert call(dt=7) == b.PA_ERR_UNSUPPORTED
    for i in range(7):
        assert call(null=(i,)) == b.PA_ERR_NULL
    assert call(T=0, null=tuple(range(7))) == b.PA_OK
    assert call(cfg=b.PaConfig(b.KERNEL_VALU, 0, 0)) == b.PA_ERR_UNSUPPORTED
    assert call(cfg=b.PaConfig(b.KERNEL_MFMA, 0, 0), D=64) == b.PA_ERR_UNSUPPORTED
    assert call(cfg=b.PaConfig(b.KERNEL_AUTO, 48, 0)) == b.PA_ERR_SHAPE
    assert call(cfg=b.PaConfig(b.KERNEL_AUTO, 32, 0)) == b.PA_ERR_WORKSPACE


def test_prefill_plans():
    p = b.plan_prefill(16, 8192, 32, 8, 128, 16, 20000, 512, 512, torch.bfloat16)
    assert p["kernel"] == b.KERNEL_MFMA and p["split"] == 0
    p = b.plan_prefill(2, 100, 32, 8, 128, 16, 20000, 512, 64, torch.bfloat16)
    assert p["kernel"] == b.KERNEL_MFMA and p["split"] == 1
    assert p["workspace_bytes"] >= 100 * 32 * p["max_partitions"] * 130 * 4
    for G in (1, 2, 4, 8, 16, 32, 64):
        assert b.plan_prefill(2, 10, 64, 64 // G, 128, 16, 100, 8, 5, torch.float16)["kernel"] == b.KERNEL_MFMA
    assert b.plan_prefill(2, 10, 8, 8, 96, 16, 100, 8, 5, torch.bfloat16)["kernel"] == b.KERNEL_GENERIC
    assert b.plan_prefill(2, 10, 8, 8, 128, 16, 100, 8, 5, torch.float32)["kernel"] == b.KERNEL_GENERIC
    assert b.plan_prefill(2, 10, 8, 8, 128, 3, 100, 8, 5, torch.bfloat16)["kernel"] == b.KERNEL_GENERIC


# ------------------------------------------------------------------ GPU

def _small(dt, Hq, Hkv, B, lens, n_new, seed, D=128):
    spec = workloads.WorkloadSpec("mq", S=len(lens), Hq=Hq, Hkv=Hkv, D=D, B=B, dtype=dt,
                                  lens=("fixed", tuple(lens)), max_len=max(lens) + B,
                                  pool=("free", 0.3), seed=seed)
    return workloads.make_prefill_workload(spec, n_new, device=DEV, poison=True)


def _oracle_full(pw):
    w = pw.base
    return oracle.prefill(pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                          pw.query_start, w.scale)


SMALL = [
    # (kernel, dtype, Hq, Hkv, B, partition)
    ("mfma", "bf16", 8, 8, 16, 0),
    ("mfma", "f16", 8, 8, 16, 64),
    ("mfma", "bf16", 16, 8, 16, 128),
    ("mfma", "bf16", 16, 4, 8, 0),
    ("mfma", "bf16", 32, 4, 1, 96),
    ("mfma", "f16", 32, 2, 32, 0),
    ("mfma", "bf16", 32, 1, 16, 256),
    ("mfma", "bf16", 64, 1, 2, 0),
    ("mfma", "bf16", 64, 2, 16, 64),
    ("generic", "bf16", 8, 2, 16, 0),
    ("generic", "f32", 4, 2, 3, 0),
]
LENS = (1, 30, 300, 700, 129, 64)
NEW = (1, 30, 77, 200, 0, 64)


@pytest.mark.gpu
@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("kernel,dt,Hq,Hkv,B,part", SMALL)
def test_prefill_matches_oracle(kernel, dt, Hq, Hkv, B, part, out_f32):
    from gpu_check import check
    D = 128 if kernel == "mfma" else 64
    print(f"case: prefill {kernel} {dt} Hq={Hq} Hkv={Hkv} B={B} part={part} out_f32={out_f32}", flush=True)
    pw = _small(dt, Hq, Hkv, B, LENS, NEW, seed=500 + Hq + B, D=D)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    od = torch.float32 if out_f32 else tdt
    out = b.prefill_workload(pw, out_dtype=od, kernel=kernel, partition_tokens=part)
    torch.cuda.synchronize()
    check(out, _oracle_full(pw), tdt, f"prefill/{kernel}/{dt}/G{Hq // Hkv}/B{B}")


# A few new tokens per sequence (G * max_query_len <= 64): two-wave,
# 64-column work-groups
FEW = [
    # (dtype, Hq, Hkv, B, partition, new tokens per sequence)
    ("bf16", 32, 8, 16, 0, (1, 4, 16, 2, 0, 16)),
    ("f16", 8, 8, 1, 0, (1, 30, 64, 2, 0, 64)),
    ("bf16", 64, 1, 16, 0, (1, 1, 1, 1, 0, 1)),
    ("bf16", 16, 1, 2, 96, (1, 4, 3, 4, 0, 2)),
    ("bf16", 64, 2, 8, 64, (1, 2, 2, 1, 0, 2)),
    ("f16", 16, 8, 32, 0, (1, 30, 32, 17, 0, 32)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("dt,Hq,Hkv,B,part,new", FEW)
def test_prefill_few_tokens_matches_oracle(dt, Hq, Hkv, B, part, new, out_f32):
    from gpu_check import check
    assert (Hq // Hkv) * max(new) <= 64
    print(f"case: prefill few tokens {dt} Hq={Hq} Hkv={Hkv} B={B} part={part} new={new} "
          f"out_f32={out_f32}", flush=True)
    pw = _small(dt, Hq, Hkv, B, LENS, new, seed=600 + Hq + B)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    out = b.prefill_workload(pw, out_dtype=torch.float32 if out_f32 else tdt,
                             partition_tokens=part)
    torch.cuda.synchronize()
    check(out, _oracle_full(pw), tdt, f"prefill few/{dt}/G{Hq // Hkv}/B{B}")


@pytest.mark.gpu
@pytest.mark.parametrize("Hq,Hkv,part,new", [(8, 8, 0, (40, 100, 64)), (32, 4, 64, (40, 100, 64)),
                                             (64, 1, 0, (40, 100, 64)),
                                             (32, 8, 0, (8, 16, 4)), (64, 1, 0, (1, 1, 1)),
                                             (8, 8, 64, (40, 64, 33))])
def test_prefill_needle_positions_exact(Hq, Hkv, part, new):
    """q = e_0, K[0] = 2048 at one token per sequence: every row at or after
    that position outputs exactly its V (which encodes block, slot and kv
    head); rows before it never see it."""
    print(f"case: prefill needle Hq={Hq} Hkv={Hkv} part={part} new={new}", flush=True)
    B = 16
    lens, new = [40, 300, 129], list(new)
    pw = _small("bf16", Hq, Hkv, B, lens, new, seed=77)
    w = pw.base
    kc = torch.zeros_like(w.key_cache)
    vc = torch.zeros_like(w.value_cache)
    ids = torch.arange(w.NB, dtype=torch.float32, device=DEV)
    vc[:, :, :, 0] = (ids % 256)[:, None, None]
    vc[:, :, :, 1] = torch.div(ids, 256, rounding_mode="floor")[:, None, None]
    vc[:, :, :, 2] = torch.arange(B, dtype=torch.float32, device=DEV)[None, None, :]
    vc[:, :, :, 3] = torch.arange(Hkv, dtype=torch.float32, device=DEV)[None, :, None]
    q = torch.zeros_like(pw.query)
    q[:, :, 0] = 1.0
    needles = []
    for s, L in enumerate(lens):
        t = L - new[s] + new[s] // 2                              # inside the chunk
        needles.append(t)
        p = int(w.tables_host[s, t // B])
        kc[p, :, t % B, 0] = 2048.0
    out = b.prefill(q, kc, vc, w.block_tables, w.seq_lens, pw.query_start, w.scale,
                    out_dtype=torch.float32, partition_tokens=part).cpu()
    torch.cuda.synchronize()
    qs = pw.query_start.cpu().tolist()
    G = Hq // Hkv
    for s, t in enumerate(needles):
        p = int(w.tables_host[s, t // B])
        for k in range(new[s]):
            pos = lens[s] - new[s] + k
            for h in range(0, Hq, max(1, Hq // 8)):
                row = out[qs[s] + k, h]
                expect = vc[p, h // G, t % B, :].float().cpu()
                if pos >= t:
                    assert torch.equal(row, expect), (s, k, h)
                else:
                    assert not torch.equal(row, expect), (s, k, h)


@pytest.mark.gpu
def test_prefill_stages_and_determinism():
    print("case: prefill staged = one call, deterministic", flush=True)
    pw = _small("bf16", 32, 8, 16, LENS, NEW, seed=3)
    p = b.plan_prefill(pw.base.S, pw.T, 32, 8, 128, 16, pw.base.NB, pw.base.max_blocks,
                       pw.max_query_len, torch.bfloat16, partition_tokens=64)
    ws = torch.empty(p["workspace_bytes"], dtype=torch.uint8, device=DEV)
    a = b.prefill_workload(pw, partition_tokens=64, workspace=ws)
    a2 = b.prefill_workload(pw, partition_tokens=64, workspace=ws)
    o1 = torch.empty_like(a)
    w = pw.base
    for st in (b.STAGE_PARTITIONS, b.STAGE_COMBINE):
        b.prefill(pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                  pw.query_start, w.scale, o1, max_query_len=pw.max_query_len,
                  partition_tokens=64, workspace=ws, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(a, a2) and torch.equal(a, o1)
    assert torch.isfinite(a).all()


@pytest.mark.gpu
def test_prefill_many_sequences_longest_first():
    """A launch of several rounds of work-groups takes its (sequence, kv
    head) pairs in decreasing context length: 300 ragged sequences (the
    length search then spans five chunks of 64 lanes), every row against the
    oracle, the output NaN-filled so that a sequence the order skipped or
    repeated shows."""
    from gpu_check import check
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 600, size=300)]
    lens[5], lens[70], lens[299] = 600, 1, 600     # ties at the top, a one-token context
    print(f"case: prefill 300 sequences, longest first (lens {min(lens)}..{max(lens)})", flush=True)
    pw = _small("bf16", 32, 8, 16, lens, 16, seed=31)
    w = pw.base
    p = b.plan_prefill(w.S, pw.T, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, pw.max_query_len,
                       w.dtype)
    # 64-column work-groups of two waves, four per CU: 2400 of them are
    # more than the 1024 resident ones
    assert (w.S * w.Hkv + 7) // 8 * 8 > 1024 and pw.max_query_len * (w.Hq // w.Hkv) <= 64
    out = torch.full((pw.T, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    b.prefill(pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, pw.query_start,
              w.scale, out, max_query_len=pw.max_query_len)
    torch.cuda.synchronize()
    ref = oracle.prefill(pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                         pw.query_start, w.scale)
    check(out, ref, w.dtype, "prefill 300 sequences")
    assert p["split"] == 0


@pytest.mark.gpu
@pytest.mark.parametrize("over", [{}, {"Hq": 8, "Hkv": 8}, {"Hq": 64, "Hkv": 1}])
def test_prefill_full_size_every_row(over):
    """The benchmark's chunked-prefill workload at full size, automatic plan:
    every (query row, head) pair against the oracle, with a NaN-filled
    workspace so that a partial result the kernels fail to rewrite shows."""
    from gpu_check import check
    print(f"case: prefill full size {over}", flush=True)
    pw = workloads.make_prefill_workload("prefill", device=DEV, poison=True, **over)
    w = pw.base
    p = b.plan_prefill(w.S, pw.T, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, pw.max_query_len,
                       w.dtype)
    ws = (torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
          if p["workspace_bytes"] else None)
    out = b.prefill_workload(pw, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    print(f"  plan {p}; T={pw.T} rows x {w.Hq} heads, running the oracle", flush=True)
    ref = oracle.prefill(pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                         pw.query_start, w.scale)
    check(out, ref, w.dtype, "prefill full")


def _prefill_sweep_case(i):
    """A seeded random shape for the multi-token sweep: kernel, group, kv
    heads, block size, type, partition, a ragged length mix and new-token
    counts that reach each work-group width (64, 128 or 256 columns), with
    sequences that take no new token.  The oracle's work (rows x heads x
    attended tokens) is kept to about a second."""
    rng = np.random.default_rng(9500 + i)
    kernel = "generic" if i % 8 == 7 else "mfma"
    dt = ("bf16", "f16")[(i // 2) % 2]
    G = int(rng.choice((1, 2, 4, 8, 16, 32, 64)))
    Hkv = int(rng.choice((1, 2) if G >= 32 else (1, 2, 4)))
    B = int(rng.choice((1, 2, 4, 8, 16, 32)))
    if kernel == "generic" and B == 1:
        B = 3                                  # the generic kernel takes any block size
    part = 0 if rng.random() < 0.4 else 32 * int(rng.integers(2, 33))
    S = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(1, 2001, size=S)]
    for k in range(min(S, 2)):
        lens[int(rng.integers(0, S))] = int(rng.choice((1, 32, 33, max(part, 64), 2000)))
    cap = int(rng.choice((2, 8, 64, 300)))     # longest chunk: 64, 128 or 256 columns
    new = [int(rng.integers(0, min(L, cap) + 1)) for L in lens]
    j = int(rng.integers(0, S))
    new[j] = min(lens[j], cap)                 # one chunk reaches the cap
    if sum(new) == 0:
        new[0] = 1
    budget = 2.5e8 / (G * Hkv)                 # attended (row, token) pairs per head
    while sum(n * L for n, L in zip(new, lens)) > budget:
        new = [n // 2 for n in new]
        if sum(new) == 0:
            new[0] = 1
            break
    return kernel, dt, G * Hkv, Hkv, B, part, tuple(lens), tuple(new)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(32))
def test_prefill_sweep(i):
    """Random shapes through the multi-token path: every row against the
    oracle, in fp32 and in the native type, the workspace NaN-filled."""
    from gpu_check import check
    kernel, dt, Hq, Hkv, B, part, lens, new = _prefill_sweep_case(i)
    print(f"case: prefill sweep {i}: {kernel} {dt} Hq={Hq} Hkv={Hkv} B={B} part={part} "
          f"lens={lens} new={new}", flush=True)
    D = 128 if kernel == "mfma" else 64
    pw = _small(dt, Hq, Hkv, B, lens, new, seed=9600 + i, D=D)
    w = pw.base
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    p = b.plan_prefill(w.S, pw.T, Hq, Hkv, D, B, w.NB, w.max_blocks, pw.max_query_len, tdt,
                       kernel=kernel, partition_tokens=part)
    assert p["kernel"] == b.KERNELS[kernel]
    ws = (torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
          if p["workspace_bytes"] else None)
    ref = _oracle_full(pw)
    for od in (torch.float32, tdt):
        out = b.prefill_workload(pw, out_dtype=od, kernel=kernel, partition_tokens=part,
                                 workspace=ws)
        torch.cuda.synchronize()
        check(out, ref, tdt, f"prefill sweep {i}/{od}")
