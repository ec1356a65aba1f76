"""Edge cases at the limits of the C ABI, against the oracle.

* the largest batch the launch grid allows (65535 sequences), short and
  empty contexts, every kernel family;
* contexts that fill their block table exactly (the last used entry is the
  table's last column), with single-pass and split plans;
* the generic kernel at the smallest, an odd and the largest head size;
* contexts of 300k and 512k tokens, at blocks of 16 tokens and of one.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_check import check
from paged_kv_cache_301_amd import binding, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("kernel,Hq,Hkv", [("valu", 2, 1), ("mfma", 4, 1), ("generic", 1, 1)])
def test_largest_batch(kernel, Hq, Hkv):
    S = 65535
    say(f"case: largest batch S={S} {kernel} Hq={Hq} Hkv={Hkv}")
    spec = workloads.WorkloadSpec("maxS", S=S, Hq=Hq, Hkv=Hkv, D=128, B=16, dtype="bf16",
                                  lens=("uniform", 0, 48), max_len=48, pool=("free", 0.1),
                                  seed=65535 + Hq)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    out = binding.decode_workload(w, out_dtype=torch.float32, kernel=kernel)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    empty = torch.nonzero(w.seq_lens == 0).flatten()
    assert empty.numel() > 0 and torch.count_nonzero(out[empty]) == 0
    rng = np.random.default_rng(7)
    seqs = sorted(set(rng.choice(S, size=40, replace=False).tolist()) | {0, S - 1})
    rows = [s * Hq + h for s in seqs for h in range(Hq)]
    ref = oracle.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                        w.scale, rows=rows)
    got = out.reshape(S * Hq, w.D)[torch.as_tensor(rows, device=DEV)]
    check(got, ref, w.dtype, f"maxS/{kernel}")


@pytest.mark.parametrize("kernel,Hq,Hkv,B,part", [("valu", 8, 8, 16, 0), ("valu", 8, 8, 16, 96),
                                                  ("mfma", 16, 2, 16, 0), ("mfma", 16, 2, 8, 64),
                                                  ("mfma", 64, 1, 16, 128), ("generic", 8, 2, 16, 0)])
def test_full_tables(kernel, Hq, Hkv, B, part):
    """Every sequence but one uses its whole table; one sequence is one token
    short of it."""
    say(f"case: full tables {kernel} Hq={Hq} Hkv={Hkv} B={B} part={part}")
    max_len = 40 * B
    lens = (max_len, max_len, max_len - 1, max_len)
    spec = workloads.WorkloadSpec("full", S=len(lens), Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                                  lens=("fixed", lens), max_len=max_len, pool=("free", 0.2),
                                  seed=97 + B)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    assert w.max_blocks * w.B == max_len
    out = binding.decode_workload(w, out_dtype=torch.float32, kernel=kernel, partition_tokens=part)
    torch.cuda.synchronize()
    ref = oracle.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale)
    check(out, ref, w.dtype, f"full/{kernel}")


@pytest.mark.parametrize("D,dt", [(1, "f32"), (1, "bf16"), (257, "f16"), (512, "bf16"), (512, "f32")])
def test_generic_head_sizes(D, dt):
    say(f"case: generic head size D={D} {dt}")
    dtype = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt]
    spec = workloads.WorkloadSpec("heads", S=5, Hq=6, Hkv=3, D=D, B=8, dtype=dt,
                                  lens=("fixed", (1, 9, 64, 300, 0)), max_len=304,
                                  pool=("free", 0.3), seed=D)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    for out_dtype in (torch.float32, dtype):
        out = binding.decode_workload(w, out_dtype=out_dtype, kernel="generic")
        torch.cuda.synchronize()
        ref = oracle.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                            w.scale)
        check(out, ref, dtype, f"generic/D{D}/{dt}")


@pytest.mark.parametrize("B", [16, 1])
def test_long_contexts(B):
    """A 512k-token context beside a 300k-token and a one-token one: the
    automatic plan (hundreds of partitions for this small batch, merged by the
    wide combine), forced 1024-token partitions (513 per row), the VALU kernel,
    and four waves per item; every row against the oracle, the workspace
    NaN-filled."""
    lens = (524288, 300001, 1)
    say(f"case: long contexts B={B} lens={lens}")
    spec = workloads.WorkloadSpec("long_context", S=len(lens), Hq=32, Hkv=8, D=128, B=B,
                                  dtype="bf16", lens=("fixed", lens), max_len=max(lens) + B,
                                  pool=("free", 0.1), seed=31 + B)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    ref = oracle.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale)
    for kw in (dict(), dict(kernel="mfma", partition_tokens=1024), dict(kernel="valu"),
               dict(kernel="mfma", partition_tokens=1024 if B < 4 else 8192, token_waves=4)):
        p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype, **kw)
        say(f"  plan {kw}: {p}")
        assert p["split"] == 1 and p["max_partitions"] > 32
        ws = torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
        out = binding.decode_workload(w, out_dtype=torch.float32, workspace=ws, **kw)
        torch.cuda.synchronize()
        check(out, ref, w.dtype, f"long/B{B}/{kw}")
