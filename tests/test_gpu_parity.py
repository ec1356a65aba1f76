"""GPU parity: the HIP library against the CPU oracle on identical seeded inputs.

Every test compares every output element: small cases, and the
benchmark-sized workloads at full size in the launch configuration the
benchmark times.  Indexing is checked bit-exactly (needle, physical
relabelling, NaN poison, run-to-run determinism, block ids repeated within a
table).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_check import check
from paged_kv_cache_301_amd import binding, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(msg, flush=True)


def run(w, **kw):
    out = binding.decode_workload(w, **kw)
    torch.cuda.synchronize()
    return out


def oracle_full(w):
    return oracle.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale)


# ------------------------------------------------------------------ tiny cases

def test_tiny_fp32():
    say("case: tiny fp32 (1 seq, D=2, B=2, 5 tokens, pool 8)")
    w = workloads.make_workload("tiny", device=DEV, poison=True)
    out = run(w)
    check(out, oracle_full(w), torch.float32, "tiny")


def test_worked_example_on_gpu():
    say("case: worked example, generic kernel, fp32")
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    kc = torch.full((9, 1, 2, 2), float("nan"))
    vc = torch.full((9, 1, 2, 2), float("nan"))
    for pid, blk in ex["blocks"].items():
        kc[int(pid), 0] = torch.tensor(blk["K"])
        vc[int(pid), 0] = torch.tensor(blk["V"])
    kc[1, 0, 1] = float("nan")
    vc[1, 0, 1] = float("nan")
    q = torch.tensor(ex["query"]).reshape(1, 1, 2)
    bt = torch.tensor([ex["block_table"]], dtype=torch.int32)
    sl = torch.tensor([ex["context_length"]], dtype=torch.int32)
    out = binding.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), sl.to(DEV), 1.0)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()[0, 0]
    assert np.round(got, 4).tolist() == ex["printed"]["output_code"]
    ref = oracle.decode(q, kc, vc, bt, sl, 1.0)[0, 0]
    assert np.abs(got - ref).max() <= 1e-5


# ------------------------------------------------------------- small parity

SMALL = [
    # (kernel, dtype, Hq, Hkv, B, partition_tokens)
    ("generic", "f32", 8, 2, 16, 0),
    ("generic", "f16", 4, 4, 3, 0),
    ("generic", "bf16", 8, 1, 16, 0),
    ("valu", "f16", 8, 8, 16, 0),
    ("valu", "bf16", 8, 8, 16, 64),
    ("valu", "bf16", 8, 8, 1, 96),
    ("valu", "bf16", 8, 8, 2, 0),
    ("valu", "f16", 8, 8, 8, 128),
    ("valu", "bf16", 8, 8, 32, 32),
    ("valu", "bf16", 8, 8, 64, 0),
    ("valu", "bf16", 8, 4, 16, 64),
    ("valu", "f16", 16, 4, 4, 0),
    ("valu", "bf16", 16, 2, 16, 128),
    ("mfma", "bf16", 16, 4, 16, 0),
    ("mfma", "bf16", 16, 4, 16, 64),
    ("mfma", "f16", 16, 2, 16, 96),
    ("mfma", "bf16", 16, 2, 1, 64),
    ("mfma", "bf16", 16, 4, 8, 128),
    ("mfma", "f16", 16, 4, 4, 0),
    ("mfma", "bf16", 16, 4, 2, 32),
    ("mfma", "bf16", 32, 2, 32, 64),
    ("mfma", "bf16", 16, 1, 64, 0),
    # one or two heads per kv head, padded to 16 columns
    ("mfma", "bf16", 8, 8, 16, 0),
    ("mfma", "f16", 8, 8, 16, 64),
    ("mfma", "bf16", 8, 8, 1, 96),
    ("mfma", "bf16", 8, 4, 8, 0),
    ("mfma", "f16", 4, 2, 32, 32),
    # groups wider than 16: several waves per work-group (MQA when Hkv = 1)
    ("mfma", "bf16", 32, 1, 16, 0),
    ("mfma", "f16", 64, 1, 16, 64),
    ("mfma", "bf16", 64, 2, 8, 96),
    ("mfma", "bf16", 64, 1, 1, 64),
    ("mfma", "f16", 32, 1, 2, 32),
]


@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("kernel,dt,Hq,Hkv,B,part", SMALL)
def test_small_parity(kernel, dt, Hq, Hkv, B, part, out_f32):
    D = 128 if kernel != "generic" else (96 if dt != "f32" else 64)
    spec = workloads.WorkloadSpec(
        "small", S=6, Hq=Hq, Hkv=Hkv, D=D, B=B, dtype=dt,
        lens=("fixed", (1, 31, 32, 33, 700, 257)), max_len=704,
        pool=("free", 0.3), seed=1000 + Hq + B)
    say(f"case: small {kernel} {dt} Hq={Hq} Hkv={Hkv} B={B} part={part} out_f32={out_f32}")
    w = workloads.make_workload(spec, device=DEV, poison=True)
    od = torch.float32 if out_f32 else DT[dt]
    out = run(w, out_dtype=od, kernel=kernel, partition_tokens=part)
    check(out, oracle_full(w), DT[dt], f"{kernel}/{dt}/B{B}")


@pytest.mark.parametrize("kernel", ["generic", "valu", "mfma"])
def test_zero_length_rows_are_zero(kernel):
    say(f"case: zero-length sequences, {kernel}")
    spec = workloads.WorkloadSpec("zeros", S=5, Hq=8, Hkv=2, D=128, B=16, dtype="bf16",
                                  lens=("fixed", (0, 5, 0, 300, 0)), max_len=320,
                                  pool=("free", 0.5), seed=77)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    out = run(w, out_dtype=torch.float32, kernel=kernel, partition_tokens=64 if kernel != "generic" else 0)
    got = out.cpu()
    for s in (0, 2, 4):
        assert torch.equal(got[s], torch.zeros_like(got[s]))
    check(out, oracle_full(w), torch.bfloat16, kernel)


# ------------------------------------------------------------ exact indexing

NEEDLE_KERNELS = [("generic", 8, 2, 16, 0), ("valu", 8, 8, 16, 64), ("valu", 8, 8, 1, 64),
                  ("valu", 8, 4, 8, 0), ("mfma", 16, 2, 16, 64), ("mfma", 16, 4, 1, 96),
                  ("mfma", 32, 4, 8, 0), ("mfma", 64, 1, 16, 64), ("mfma", 64, 2, 1, 0),
                  ("mfma", 8, 8, 16, 64), ("mfma", 8, 4, 1, 0)]


@pytest.mark.parametrize("kernel,Hq,Hkv,B,part", NEEDLE_KERNELS)
def test_needle_bit_exact(kernel, Hq, Hkv, B, part):
    """q = e_0 and one token per sequence with K[0] = 2048: its score beats every
    other by more than exp can represent, so the output must be exactly that
    token's V, which encodes (physical block, slot, kv head) in small integers."""
    say(f"case: needle {kernel} Hq={Hq} Hkv={Hkv} B={B} part={part}")
    dt = torch.bfloat16
    lens = [1, 17, 64, 129, 400, 511]
    spec = workloads.WorkloadSpec("needle", S=len(lens), Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                                  lens=("fixed", tuple(lens)), max_len=512, pool=("free", 0.2),
                                  seed=5)
    w = workloads.make_workload(spec, device="cpu", poison=False)
    NB = w.NB
    vc = torch.zeros_like(w.value_cache)
    ids = torch.arange(NB, dtype=torch.float32)
    vc[:, :, :, 0] = (ids % 256)[:, None, None]
    vc[:, :, :, 1] = torch.div(ids, 256, rounding_mode="floor")[:, None, None]
    vc[:, :, :, 2] = torch.arange(B, dtype=torch.float32)[None, None, :]
    vc[:, :, :, 3] = torch.arange(Hkv, dtype=torch.float32)[None, :, None]
    q = torch.zeros_like(w.query)
    q[:, :, 0] = 1.0
    rng = np.random.default_rng(3)
    for trial in range(3):
        kc = torch.zeros_like(w.key_cache)
        pos = []
        for s, L in enumerate(lens):
            t = [0, L - 1, int(rng.integers(0, L))][trial]
            pos.append(t)
            p = int(w.tables_host[s, t // B])
            kc[p, :, t % B, 0] = 2048.0
        out = binding.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), w.block_tables.to(DEV),
                             w.seq_lens.to(DEV), w.scale, out_dtype=torch.float32,
                             kernel=kernel, partition_tokens=part)
        torch.cuda.synchronize()
        got = out.cpu()
        G = Hq // Hkv
        for s, t in enumerate(pos):
            p = int(w.tables_host[s, t // B])
            for h in range(Hq):
                expect = vc[p, h // G, t % B, :].float()
                assert torch.equal(got[s, h], expect), (kernel, s, h, t)


@pytest.mark.parametrize("kernel,Hq,Hkv,B,part", [("valu", 8, 8, 16, 64), ("mfma", 16, 2, 16, 64),
                                                  ("mfma", 16, 4, 1, 64), ("generic", 4, 2, 16, 0),
                                                  ("mfma", 64, 1, 16, 64), ("mfma", 8, 8, 16, 64)])
def test_relabel_poison_determinism(kernel, Hq, Hkv, B, part):
    say(f"case: relabel/poison/determinism {kernel} B={B}")
    spec = workloads.WorkloadSpec("perm", S=4, Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                                  lens=("fixed", (3, 100, 257, 640)), max_len=640,
                                  pool=("free", 0.3), seed=9)
    clean = workloads.make_workload(spec, device=DEV, poison=False)
    dirty = workloads.make_workload(spec, device=DEV, poison=True)
    kw = dict(out_dtype=torch.float32, kernel=kernel, partition_tokens=part)
    a = run(clean, **kw)
    b2 = run(clean, **kw)
    assert torch.equal(a, b2), "two runs differ"
    c = run(dirty, **kw)
    assert torch.isfinite(c).all()
    assert torch.equal(a, c), "NaN in unreferenced slots changed the output"
    # physical relabelling
    pi = torch.as_tensor(np.random.default_rng(4).permutation(clean.NB), device=DEV)
    kc2 = torch.empty_like(clean.key_cache)
    vc2 = torch.empty_like(clean.value_cache)
    kc2[pi] = clean.key_cache
    vc2[pi] = clean.value_cache
    bt2 = pi[clean.block_tables.long()].to(torch.int32)
    d = binding.decode(clean.query, kc2, vc2, bt2, clean.seq_lens, clean.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, d), "relabelling physical blocks changed the output"


@pytest.mark.parametrize("kernel", ["valu", "mfma", "mfma64"])
def test_stages_equal_one_call(kernel):
    say(f"case: staged partitions+combine vs one call, {kernel}")
    Hq, Hkv = {"valu": (8, 8), "mfma": (16, 2), "mfma64": (64, 1)}[kernel]
    kernel = kernel[:4] if kernel == "mfma64" else kernel
    spec = workloads.WorkloadSpec("stages", S=3, Hq=Hq, Hkv=Hkv, D=128, B=16, dtype="bf16",
                                  lens=("fixed", (33, 300, 900)), max_len=960,
                                  pool=("free", 0.3), seed=12)
    w = workloads.make_workload(spec, device=DEV)
    p = binding.plan(3, Hq, Hkv, 128, 16, w.NB, w.max_blocks, torch.bfloat16, kernel=kernel,
                     partition_tokens=64)
    ws = torch.empty(p["workspace_bytes"], dtype=torch.uint8, device=DEV)
    a = run(w, kernel=kernel, partition_tokens=64, workspace=ws)
    o1 = torch.empty_like(a)
    for stage in (binding.STAGE_PARTITIONS, binding.STAGE_COMBINE):
        binding.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                       w.scale, o1, kernel=kernel, partition_tokens=64, workspace=ws,
                       stages=stage)
    torch.cuda.synchronize()
    assert torch.equal(a, o1)


# --------------------------------------------------- benchmark-sized workloads

FULL = [("mha_small", {}), ("mha_7b", {}), ("gqa_70b", {}), ("gqa_long", {"B": 16}),
        ("gqa_long", {"B": 1}), ("gqa_long", {"B": 8}), ("gqa_long", {"B": 32}),
        ("mqa", {}), ("mqa", {"Hq": 32}), ("mha_7b", {"kernel": "mfma"}),
        ("mha_small", {"kernel": "mfma"})]


@pytest.mark.parametrize("name,over", FULL)
def test_full_size_every_row(name, over):
    """Full-size workload, automatic plan (what the benchmark times): every
    (sequence, head) row against the oracle, with fp32 and with native
    outputs.  The live-item grid decides which work-group computes which
    (sequence, kv head, partition) item; a dropped or doubled item would
    leave a row built from stale partial results, which only an all-row
    comparison is sure to catch."""
    say(f"case: full-size {name} {over}")
    over = dict(over)
    kernel = over.pop("kernel", "auto")
    w = workloads.make_workload(name, device=DEV, poison=True, **over)
    p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype, kernel=kernel)
    # workspace filled with NaN: any partial result the kernels do not
    # rewrite poisons its row
    ws = (torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
          if p["workspace_bytes"] else None)
    out = run(w, out_dtype=torch.float32, kernel=kernel, workspace=ws)
    ref = oracle_full(w)
    say(f"  plan {p}; oracle done")
    check(out, ref, w.dtype, name)
    check(run(w, kernel=kernel, workspace=ws), ref, w.dtype, name + "/native")


@pytest.mark.parametrize("kernel,Hq,Hkv,B", [("valu", 8, 8, 16), ("valu", 8, 8, 1), ("mfma", 16, 2, 16),
                                             ("mfma", 16, 4, 8), ("mfma", 32, 1, 16)])
def test_kv_reuse_hint_is_bit_identical(kernel, Hq, Hkv, B):
    """Streamed and cached K/V loads differ only in cache policy."""
    say(f"case: kv_reuse on/off {kernel} B={B}")
    spec = workloads.WorkloadSpec("hint", S=4, Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                                  lens=("fixed", (7, 100, 513, 1000)), max_len=1024,
                                  pool=("free", 0.3), seed=31)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    a = run(w, out_dtype=torch.float32, kernel=kernel, partition_tokens=256, kv_reuse=False)
    b2 = run(w, out_dtype=torch.float32, kernel=kernel, partition_tokens=256, kv_reuse=True)
    assert torch.equal(a, b2)
    check(a, oracle_full(w), torch.bfloat16, kernel)


@pytest.mark.parametrize("kernel,Hq,Hkv,S", [("valu", 4, 4, 700), ("mfma", 16, 2, 700),
                                             ("valu", 2, 2, 1100), ("mfma", 8, 2, 1100),
                                             ("mfma", 64, 1, 700), ("mfma", 32, 1, 1100)])
def test_many_sequences(kernel, Hq, Hkv, S):
    """Batches beyond one wave's worth of lengths (live-item decode over
    several register chunks) and beyond 1024 sequences (rectangular grid)."""
    say(f"case: many sequences {kernel} S={S}")
    spec = workloads.WorkloadSpec("many", S=S, Hq=Hq, Hkv=Hkv, D=128, B=16, dtype="bf16",
                                  lens=("uniform", 0, 200), max_len=200, pool=("free", 0.2),
                                  seed=S + Hq)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    out = run(w, out_dtype=torch.float32, kernel=kernel, partition_tokens=64)
    check(out, oracle_full(w), torch.bfloat16, f"{kernel}/S{S}")


# ------------------------------------------------------- precondition check

def _spare_pools(w, spare=16):
    """The workload's pools copied into allocations with `spare` extra blocks
    before and after the NB the calls see, returned as views of the middle NB
    blocks: ids from -spare to NB + spare - 1 then stay inside the allocation
    (the checked mode must reject them before any attention kernel reads
    them)."""
    big_k = torch.zeros((w.NB + 2 * spare,) + tuple(w.key_cache.shape[1:]), dtype=w.dtype,
                        device=DEV)
    big_v = torch.zeros_like(big_k)
    big_k[spare:spare + w.NB] = w.key_cache
    big_v[spare:spare + w.NB] = w.value_cache
    return big_k[spare:spare + w.NB], big_v[spare:spare + w.NB]


def test_check_inputs_reports_bad_tables_and_lengths(monkeypatch):
    """The device check counts exactly the sequences whose length or used
    table entries break the preconditions.  In the checked mode the library
    itself refuses to launch on them (PA_ERR_DEVICE_CHECK, raised as
    InputCheckError), leaves the output untouched and reports the first bad
    sequence once through pa_get_device_error."""
    say("case: device check of lengths and block tables")
    spec = workloads.WorkloadSpec("chk", S=6, Hq=8, Hkv=2, D=128, B=16, dtype="bf16",
                                  lens=("fixed", (0, 1, 16, 17, 100, 160)), max_len=160,
                                  pool=("free", 0.2), seed=41)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    kc, vc = _spare_pools(w)
    assert binding.check_inputs(w.block_tables, w.seq_lens, w.NB, w.B) == (0, None)
    bt = w.block_tables.clone()
    sl = w.seq_lens.clone()
    bt[3, 1] = w.NB                # used entry (17 tokens: blocks 0, 1) out of range
    bt[4, 0] = -1                  # negative id
    bt[5, 9] = w.NB + 7            # last used entry of a full 160-token context
    bt[2, 5] = -5                  # past ceil(16 / 16) = 1: never read, not an error
    sl[1] = w.max_blocks * w.B + 1 # longer than the table
    assert binding.check_inputs(bt, sl, w.NB, w.B) == (4, 1)
    sl2 = w.seq_lens.clone()
    sl2[0] = -3
    assert binding.check_inputs(w.block_tables, sl2, w.NB, w.B) == (1, 0)
    assert binding.device_error() == (binding.PA_OK, None)
    sentinel = torch.full(w.query.shape, 7.0, device=DEV)
    out = sentinel.clone()
    with pytest.raises(binding.InputCheckError):
        binding.decode(w.query, kc, vc, bt, sl, w.scale, out, check=True)
    torch.cuda.synchronize()
    assert torch.equal(out, sentinel), "an attention kernel ran on rejected inputs"
    assert binding.device_error() == (binding.PA_ERR_DEVICE_CHECK, 1)
    assert binding.device_error() == (binding.PA_OK, None)
    # the environment switch, read by the library at each call
    monkeypatch.setenv("PA_CHECK", "1")
    with pytest.raises(binding.InputCheckError):
        binding.decode(w.query, kc, vc, w.block_tables, sl2, w.scale, out)
    assert torch.equal(out, sentinel)
    assert binding.device_error() == (binding.PA_ERR_DEVICE_CHECK, 0)
    out = binding.decode(w.query, kc, vc, w.block_tables, w.seq_lens, w.scale,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert binding.device_error() == (binding.PA_OK, None)
    check(out, oracle_full(w), torch.bfloat16, "checked decode")
    # an explicit check=False wins over the environment (good inputs only)
    out = binding.decode(w.query, kc, vc, w.block_tables, w.seq_lens, w.scale,
                         out_dtype=torch.float32, check=False)
    torch.cuda.synchronize()
    check(out, oracle_full(w), torch.bfloat16, "unchecked decode")


def test_checked_prefill_rejects_bad_query_start():
    """Multi-token calls in the checked mode also verify query_start (ordered,
    0 .. T, each chunk within its sequence's length and max_query_len)."""
    say("case: checked multi-token call, bad query_start / table")
    spec = workloads.WorkloadSpec("chkq", S=3, Hq=8, Hkv=2, D=128, B=16, dtype="bf16",
                                  lens=("fixed", (40, 100, 300)), max_len=320,
                                  pool=("free", 0.2), seed=42)
    pw = workloads.make_prefill_workload(spec, (5, 20, 7), device=DEV, poison=True)
    w = pw.base
    kc, vc = _spare_pools(w)
    a = (pw.query, kc, vc, w.block_tables, w.seq_lens)
    good = binding.prefill(*a, pw.query_start, w.scale, max_query_len=pw.max_query_len,
                           out_dtype=torch.float32, check=True)
    torch.cuda.synchronize()
    ref = oracle.prefill(pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                         pw.query_start, w.scale)
    check(good, ref, torch.bfloat16, "checked prefill")
    qs = pw.query_start.clone()
    qs[1] = qs[2] + 1                              # sequence 1 gets a negative row count
    with pytest.raises(binding.InputCheckError):
        binding.prefill(*a, qs, w.scale, max_query_len=pw.max_query_len, check=True)
    assert binding.device_error() == (binding.PA_ERR_DEVICE_CHECK, 0)
    with pytest.raises(binding.InputCheckError):   # a chunk longer than max_query_len
        binding.prefill(*a, pw.query_start, w.scale, max_query_len=10, check=True)
    assert binding.device_error()[0] == binding.PA_ERR_DEVICE_CHECK
    bt = w.block_tables.clone()
    bt[2, 3] = w.NB + 2                            # 300 tokens use entries 0 .. 18
    with pytest.raises(binding.InputCheckError):
        binding.prefill(pw.query, kc, vc, bt, w.seq_lens, pw.query_start, w.scale,
                        max_query_len=pw.max_query_len, check=True)
    assert binding.device_error() == (binding.PA_ERR_DEVICE_CHECK, 2)


# ---------------------------------------------------- allocation and streams

def test_side_stream_without_workspace():
    """decode() on a side stream, with no workspace or output passed: both
    are allocated on that stream, so memory freed afterwards and reused on
    the current stream cannot be overwritten while the kernels still run."""
    say("case: side stream, library-allocated workspace")
    w = workloads.make_workload("mha_7b", device=DEV, poison=True, S=8,
                                lens=("uniform", 2048, 4096), max_len=4096)
    ref = oracle_full(w)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    results = []
    for trial in range(3):
        out = binding.decode_workload(w, out_dtype=torch.float32, partition_tokens=256,
                                      stream=side)
        with torch.cuda.stream(side):
            results.append(out.clone())
        del out
        # the current stream allocates and scribbles while the side stream runs
        junk = [torch.full((1 << 20,), float("nan"), device=DEV) for _ in range(16)]
        del junk
    torch.cuda.synchronize()
    for r in results:
        check(r, ref, torch.bfloat16, "side stream")


# ------------------------------------------------------ repeated block ids

@pytest.mark.parametrize("kernel,Hq,Hkv,B", [("generic", 8, 2, 16), ("valu", 8, 8, 16),
                                             ("valu", 8, 8, 1), ("mfma", 16, 2, 16),
                                             ("mfma", 16, 4, 2), ("mfma", 64, 1, 16)])
def test_repeated_block_ids_within_a_table(kernel, Hq, Hkv, B):
    """One sequence's table names the same physical block at several logical
    positions (the pages are silent on this; the oracle and the kernels read
    tables without assuming distinct ids).  Every row against the oracle."""
    say(f"case: repeated ids within a table {kernel} B={B}")
    spec = workloads.WorkloadSpec("rep", S=4, Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                                  lens=("fixed", (37, 200, 513, 900)), max_len=900,
                                  pool=("free", 0.3), seed=51)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    bt = w.block_tables.cpu().clone()
    rng = np.random.default_rng(52)
    for s, L in enumerate(w.lens):
        n = (int(L) + B - 1) // B
        n_full = int(L) // B     # blocks whose every slot holds a token (the last one's
        if n_full == 0:          # tail is NaN in this poisoned pool)
            continue
        own = bt[s, :n_full].clone()
        # every used entry drawn from a few of the sequence's own full blocks
        pick = rng.choice(n_full, size=min(3, n_full), replace=False)
        bt[s, :n] = own[torch.as_tensor(rng.choice(pick, size=n))]
        assert len(set(bt[s, :n].tolist())) < n
    bt = bt.to(DEV)
    out = binding.decode(w.query, w.key_cache, w.value_cache, bt, w.seq_lens, w.scale,
                         out_dtype=torch.float32, kernel=kernel,
                         partition_tokens=64 if kernel != "generic" else 0)
    torch.cuda.synchronize()
    ref = oracle.decode(w.query, w.key_cache, w.value_cache, bt, w.seq_lens, w.scale)
    check(out, ref, torch.bfloat16, f"repeated ids {kernel}")


# ------------------------------------------------ the small config, every row

@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_small_config_every_row(dt):
    """The 8-sequence, 32/32-head, B = 16 configuration (lengths U[1, 2048])
    compared on every output row: in fp32 (the plain kernel; max-abs 1e-5)
    and in its own fp16 (automatic plan, split contexts; rel 2e-3 with fp32
    output, plus the final rounding in fp16)."""
    say(f"case: small config every row, {dt}")
    w = workloads.make_workload("mha_small", device=DEV, poison=True, dtype=dt)
    ref = oracle_full(w)
    out = run(w, out_dtype=torch.float32)
    check(out, ref, DT[dt], f"mha_small/{dt}")
    if dt != "f32":
        check(run(w), ref, DT[dt], f"mha_small/{dt}/native")


# ------------------------------------------- pools beyond 4 GiB, small blocks

@pytest.mark.parametrize("kernel,Hq,Hkv,B", [("mfma", 16, 2, 1), ("mfma", 64, 8, 2),
                                             ("valu", 8, 8, 1)])
def test_pool_beyond_4gib_small_blocks(kernel, Hq, Hkv, B):
    """Row addresses past 4 GiB: a small workload's blocks are moved to ids
    near the top of a pool of more than 4 GiB per cache (and just below
    4 GiB), where block id times block size overflows 32 bits.  Small blocks
    take the most distinct ids for a given size.  The output must be
    bit-identical to the small pool's, which is compared with the oracle on
    every row."""
    say(f"case: pool > 4 GiB {kernel} Hq={Hq} Hkv={Hkv} B={B}")
    spec = workloads.WorkloadSpec("big", S=4, Hq=Hq, Hkv=Hkv, D=128, B=B, dtype="bf16",
                                  lens=("fixed", (5, 100, 513, 900)), max_len=900,
                                  pool=("free", 0.3), seed=61)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    kw = dict(out_dtype=torch.float32, kernel=kernel, partition_tokens=64)
    a = run(w, **kw)
    check(a, oracle_full(w), torch.bfloat16, f"small pool {kernel} B={B}")
    block_bytes = Hkv * B * 128 * 2
    NB = (1 << 32) // block_bytes + 4096
    assert w.NB < 4096      # the two id ranges below do not meet
    assert NB * block_bytes > (1 << 32) and NB < (1 << 24)
    # half the blocks at the very top of the pool, half just below 4 GiB
    pi = torch.as_tensor(np.random.default_rng(62).permutation(w.NB), device=DEV)
    top = torch.where(pi % 2 == 0, NB - 1 - pi, (1 << 32) // block_bytes - 1 - pi)
    big_k = torch.empty((NB, Hkv, B, 128), dtype=torch.bfloat16, device=DEV)
    big_v = torch.empty_like(big_k)
    big_k[top] = w.key_cache
    big_v[top] = w.value_cache
    bt = top[w.block_tables.long()].to(torch.int32)
    b = binding.decode(w.query, big_k, big_v, bt, w.seq_lens, w.scale, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "moving blocks beyond 4 GiB changed the output"
    del big_k, big_v
    torch.cuda.empty_cache()


# ------------------------------------------------- token-waves per item

@pytest.mark.parametrize("kernel,Hq,Hkv,B,part,tw", [
    ("valu", 8, 8, 16, 2048, 2), ("valu", 8, 8, 16, 4096, 4), ("valu", 16, 8, 4, 4096, 4),
    ("valu", 8, 8, 16, 8192, 4), ("valu", 16, 8, 16, 2048, 2), ("valu", 8, 8, 32, 4096, 4),
    ("valu", 8, 8, 16, 1024, 4),
    ("mfma", 32, 8, 16, 2048, 2), ("mfma", 32, 8, 16, 4096, 4), ("mfma", 64, 8, 4, 8192, 4),
    ("mfma", 128, 8, 16, 4096, 4), ("mfma", 8, 8, 32, 2048, 2), ("mfma", 16, 2, 16, 4096, 4),
    ("mfma", 32, 8, 16, 512, 4)])
def test_waves_per_item(kernel, Hq, Hkv, B, part, tw):
    """Items run on two or four waves of one work-group (pa_config
    token_waves), each streaming every second or fourth 32-token tile of the
    partition, their softmax states merged in LDS (the VALU kernel, and the
    matrix-core kernel's groups of at most 16 heads); a partition covering
    the context is one pass, and a short one leaves some waves without a
    tile.  Every row against the oracle, the workspace NaN-filled, with
    empty, one-tile and ragged contexts."""
    say(f"case: waves per item {kernel} Hq={Hq} Hkv={Hkv} B={B} part={part} tw={tw}")
    lens = (1, 33, 1000, 4096, 5000, 2047, 0, 8191)
    spec = workloads.WorkloadSpec("token_waves", S=len(lens), Hq=Hq, Hkv=Hkv, D=128, B=B,
                                  dtype="bf16", lens=("fixed", lens), max_len=8192,
                                  pool=("free", 0.2), seed=700 + part // 1024 + B)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    kw = dict(kernel=kernel, partition_tokens=part, token_waves=tw)
    p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype, **kw)
    assert p["kernel"] == binding.KERNELS[kernel] and p["partition_tokens"] == part
    assert p["token_waves"] == tw
    ws = (torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
          if p["workspace_bytes"] else None)
    ref = oracle_full(w)
    out = run(w, out_dtype=torch.float32, workspace=ws, **kw)
    check(out, ref, torch.bfloat16, f"{kernel} waves part={part} tw={tw}")
    assert torch.equal(out[6], torch.zeros_like(out[6]))
    check(run(w, workspace=ws, **kw), ref, torch.bfloat16,
          f"{kernel} waves part={part} tw={tw}/native")


@pytest.mark.parametrize("name,S,L,kernel,tw", [
    ("gqa_70b", 128, 1500, binding.KERNEL_MFMA, 2), ("mha_7b", 64, 3000, binding.KERNEL_VALU, 4)])
def test_short_context_waves_automatic(name, S, L, kernel, tw):
    """Batches of at least 512 (sequence, kv head) pairs whose partition the
    small-batch rule would halve run one pass on token-waves instead, with at
    most 1024 tokens a wave: the automatic plan, every row against the
    oracle, the output NaN-filled."""
    say(f"case: short-context waves {name} S={S} L={L}")
    w = workloads.make_workload(name, device=DEV, poison=True, S=S,
                                lens=("fixed", (L,) * S), max_len=L)
    p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype)
    assert p["kernel"] == kernel and p["split"] == 0 and p["token_waves"] == tw
    out = torch.full((w.S, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
    binding.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale, out)
    torch.cuda.synchronize()
    check(out, oracle_full(w), w.dtype, f"short-context waves {name}")


def _wave_sweep_case(i):
    """A seeded random shape for the token-wave sweep: kernel family, group,
    kv heads, block size, type, waves, partition and a ragged length mix
    with empty, one-token and partition-multiple contexts."""
    rng = np.random.default_rng(9100 + i)
    kernel = ("valu", "mfma")[i % 2]
    G = int(rng.choice((1, 2, 4, 8) if kernel == "valu" else (1, 2, 4, 8, 16)))
    Hkv = int(rng.choice((1, 2, 4)))
    B = int(rng.choice((4, 8, 16, 32, 64)))
    dtype = ("bf16", "f16")[(i // 2) % 2]
    tw = int(rng.choice((2, 4)))
    part = 32 * int(rng.integers(1, 65))
    S = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(0, 3000, size=S)]
    special = (0, 1, part, 2 * part + 1, 31, 33)
    for k in range(min(S, 2)):
        lens[int(rng.integers(0, S))] = int(rng.choice(special))
    max_len = max(max(lens), 1) + int(rng.integers(0, 2 * B))
    return kernel, G, Hkv, B, dtype, tw, part, lens, max_len


@pytest.mark.parametrize("i", range(40))
def test_token_wave_sweep(i):
    """Random shapes through explicit 2- and 4-wave items on both kernel
    families: every row against the oracle (fp32 output and the native
    type), empty contexts exactly zero, the workspace NaN-filled."""
    kernel, G, Hkv, B, dtype, tw, part, lens, max_len = _wave_sweep_case(i)
    say(f"case: wave sweep {i}: {kernel} G={G} Hkv={Hkv} B={B} {dtype} tw={tw} part={part} "
        f"lens={lens} max_len={max_len}")
    spec = workloads.WorkloadSpec("wave_sweep", S=len(lens), Hq=G * Hkv, Hkv=Hkv, D=128, B=B,
                                  dtype=dtype, lens=("fixed", tuple(lens)), max_len=max_len,
                                  pool=("free", 0.2), seed=9200 + i)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    kw = dict(kernel=kernel, partition_tokens=part, token_waves=tw)
    p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype, **kw)
    assert p["token_waves"] == tw
    ws = (torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
          if p["workspace_bytes"] else None)
    ref = oracle_full(w)
    out = run(w, out_dtype=torch.float32, workspace=ws, **kw)
    check(out, ref, DT[dtype], f"wave sweep {i}")
    for s, L in enumerate(lens):
        if L == 0:
            assert torch.equal(out[s], torch.zeros_like(out[s]))
    check(run(w, workspace=ws, **kw), ref, DT[dtype], f"wave sweep {i}/native")


@pytest.mark.parametrize("Hq,Hkv,B,part,tw", [
    (8, 8, 1, 1024, 2), (8, 8, 1, 1024, 4), (32, 8, 2, 2048, 4), (16, 2, 1, 512, 4),
    (128, 8, 1, 1024, 2), (64, 8, 2, 256, 4), (8, 1, 2, 1024, 2)])
def test_token_waves_small_blocks(Hq, Hkv, B, part, tw):
    """Matrix-core items on two or four waves with blocks of one or two
    tokens, where every lane looks its block up in the partition's slice of
    the table staged in LDS by all the work-group's waves: every row against
    the oracle, the workspace NaN-filled, with empty, one-token, ragged and
    partition-multiple contexts."""
    say(f"case: small-block waves Hq={Hq} Hkv={Hkv} B={B} part={part} tw={tw}")
    lens = (1, 33, 1000, 4096, 5000, 2047, 0, 8191, part, 2 * part + 1)
    spec = workloads.WorkloadSpec("token_waves_small_blocks", S=len(lens), Hq=Hq, Hkv=Hkv, D=128,
                                  B=B, dtype="bf16", lens=("fixed", lens), max_len=8192,
                                  pool=("free", 0.2), seed=7300 + part // 256 + B + tw)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    kw = dict(kernel="mfma", partition_tokens=part, token_waves=tw)
    p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype, **kw)
    assert p["kernel"] == binding.KERNEL_MFMA and p["partition_tokens"] == part
    assert p["token_waves"] == tw
    ws = (torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
          if p["workspace_bytes"] else None)
    ref = oracle_full(w)
    out = run(w, out_dtype=torch.float32, workspace=ws, **kw)
    check(out, ref, torch.bfloat16, f"small-block waves B={B} part={part} tw={tw}")
    assert torch.equal(out[6], torch.zeros_like(out[6]))
    check(run(w, workspace=ws, **kw), ref, torch.bfloat16,
          f"small-block waves B={B} part={part} tw={tw}/native")


def _decode_sweep_case(i):
    """A seeded random decode call: kernel family (or the automatic choice),
    a shape that family supports (the generic kernel: any head size up to
    256, block size and type), partition (automatic or forced), a ragged
    length mix with empty, one-token, tile-edge and partition-multiple
    contexts, and a table a little wider than the longest context."""
    rng = np.random.default_rng(9800 + i)
    kernel = ("auto", "generic", "valu", "mfma")[i % 4]
    if kernel == "generic" or (kernel == "auto" and rng.random() < 0.25):
        D = int(rng.choice((8, 64, 80, 96, 128, 192, 256)))
        dtype = str(rng.choice(("f32", "f16", "bf16")))
        B = int(rng.choice((1, 2, 3, 5, 8, 16, 24, 32)))
        G = int(rng.choice((1, 2, 3, 4, 6, 8, 16)))
        Hkv = int(rng.choice((1, 2, 4)))
    else:
        D = 128
        dtype = str(rng.choice(("f16", "bf16")))
        B = int(rng.choice((1, 2, 4, 8, 16, 32, 64)))
        G = int(rng.choice((1, 2, 4, 8) if kernel == "valu" else (1, 2, 4, 8, 16, 32, 64)))
        Hkv = int(rng.choice((1, 2, 4) if G >= 16 else (1, 2, 4, 8)))
    part = 0 if kernel == "generic" or rng.random() < 0.5 else 32 * int(rng.integers(1, 65))
    S = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.integers(0, 3001, size=S)]
    special = (0, 1, 31, 32, 33, max(part, 32), 2 * max(part, 32) + 1, 3000)
    for k in range(min(S, 3)):
        lens[int(rng.integers(0, S))] = int(rng.choice(special))
    max_len = max(max(lens), 1) + int(rng.integers(0, 2 * B + 1))
    return kernel, D, dtype, B, G * Hkv, Hkv, part, lens, max_len


@pytest.mark.parametrize("i", range(48))
def test_decode_sweep(i):
    """Random decode calls through every kernel family and the automatic
    plan: every row against the oracle in fp32 and in the native type, the
    workspace NaN-filled, empty contexts exactly zero."""
    kernel, D, dtype, B, Hq, Hkv, part, lens, max_len = _decode_sweep_case(i)
    say(f"case: decode sweep {i}: {kernel} D={D} {dtype} B={B} Hq={Hq} Hkv={Hkv} part={part} "
        f"lens={lens} max_len={max_len}")
    spec = workloads.WorkloadSpec("decode_sweep", S=len(lens), Hq=Hq, Hkv=Hkv, D=D, B=B,
                                  dtype=dtype, lens=("fixed", tuple(lens)), max_len=max_len,
                                  pool=("free", 0.2), seed=9900 + i)
    w = workloads.make_workload(spec, device=DEV, poison=True)
    kw = dict(kernel=kernel, partition_tokens=part)
    p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype, **kw)
    if kernel != "auto":
        assert p["kernel"] == binding.KERNELS[kernel]
    ws = (torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV)
          if p["workspace_bytes"] else None)
    ref = oracle_full(w)
    for od in (torch.float32, DT[dtype]):
        out = run(w, out_dtype=od, workspace=ws, **kw)
        check(out, ref, DT[dtype], f"decode sweep {i}/{od}")
        for s, L in enumerate(lens):
            if L == 0:
                assert torch.equal(out[s], torch.zeros_like(out[s]))


def test_concurrent_streams():
    """Calls in flight at once on three streams, each with its own workspace
    and output (the library keeps no per-call state outside them): decode on
    both kernel families and a multi-token call, issued back to back with no
    synchronisation between them, every row against the oracle afterwards."""
    say("case: concurrent streams")
    specs = [workloads.WorkloadSpec("conc_a", S=12, Hq=32, Hkv=32, D=128, B=16, dtype="bf16",
                                    lens=("uniform", 1, 3000), max_len=3008, pool=("free", 0.2),
                                    seed=501),
             workloads.WorkloadSpec("conc_b", S=20, Hq=64, Hkv=8, D=128, B=8, dtype="f16",
                                    lens=("uniform", 1, 5000), max_len=5008, pool=("free", 0.2),
                                    seed=502)]
    ws_ = [workloads.make_workload(sp, device=DEV, poison=True) for sp in specs]
    pspec = workloads.WorkloadSpec("conc_c", S=6, Hq=32, Hkv=8, D=128, B=16, dtype="bf16",
                                   lens=("fixed", (700, 1, 2000, 129, 64, 1500)), max_len=2016,
                                   pool=("free", 0.2), seed=503)
    pw = workloads.make_prefill_workload(pspec, (300, 1, 64, 0, 64, 7), device=DEV, poison=True)
    outs, wss = [], []
    for w, part in zip(ws_, (256, 512)):
        p = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype, torch.float32,
                         partition_tokens=part)
        assert p["split"] == 1
        wss.append(torch.full((p["workspace_bytes"] // 4,), float("nan"), device=DEV))
        outs.append(torch.full((w.S, w.Hq, w.D), float("nan"), device=DEV))
    pb = pw.base
    pp = binding.plan_prefill(pb.S, pw.T, pb.Hq, pb.Hkv, pb.D, pb.B, pb.NB, pb.max_blocks,
                              pw.max_query_len, pb.dtype, torch.float32, partition_tokens=256)
    pws = torch.full((max(pp["workspace_bytes"], 256) // 4,), float("nan"), device=DEV)
    pout = torch.full((pw.T, pb.Hq, pb.D), float("nan"), device=DEV)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(DEV) for _ in range(3)]
    for rep in range(3):
        for w, out, ws, part, st in zip(ws_, outs, wss, (256, 512), streams):
            binding.decode(w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens,
                           w.scale, out, partition_tokens=part, workspace=ws, stream=st)
        binding.prefill(pw.query, pb.key_cache, pb.value_cache, pb.block_tables, pb.seq_lens,
                        pw.query_start, pb.scale, pout, max_query_len=pw.max_query_len,
                        partition_tokens=256, workspace=pws, stream=streams[2])
    torch.cuda.synchronize()
    for w, out in zip(ws_, outs):
        check(out, oracle_full(w), w.dtype, f"concurrent {w.spec.name}")
    ref = oracle.prefill(pw.query, pb.key_cache, pb.value_cache, pb.block_tables, pb.seq_lens,
                         pw.query_start, pb.scale)
    check(pout, ref, pb.dtype, "concurrent prefill")
