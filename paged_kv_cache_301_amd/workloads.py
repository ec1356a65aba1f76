"""Seeded synthetic workloads for paged decode attention.

This module only draws random numbers and hands out physical blocks: it builds
the query, the paged K / V pools, the per-sequence block tables and the context
lengths.  It computes no attention, so both the HIP library's tests and the CPU
oracle can take their inputs from it.

Recipe (shared by every workload):

* ``rng = numpy.random.default_rng(seed)``; context lengths are drawn first,
  then ``perm = rng.permutation(NB)`` hands physical block ids out in order:
  first the shared-prefix blocks (if any), then each sequence's own blocks, so
  logically adjacent blocks land on unrelated physical ids.
* q, K and V are N(0, 1) draws in fp32 from a ``torch.Generator`` seeded with
  ``seed`` on the target device, rounded to the workload's element type.  The
  whole pool is filled, free blocks included.
* ``poison=True`` (correctness runs) fills every free block and every slot past
  a sequence's length in its last block with NaN, and pads the unused tail of
  each block table with the id of a NaN-filled free block.  ``poison=False``
  (timing runs) pads with 0, a valid id.

The five named workloads follow the benchmark's configurations; sizes can be
overridden for cut-down tests.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class WorkloadSpec:
    """Shape and distribution of one synthetic decode batch."""
    name: str
    S: int                      # sequences in the batch
    Hq: int                     # query heads
    Hkv: int                    # kv heads (Hq % Hkv == 0)
    D: int                      # head dimension
    B: int                      # tokens per physical block
    dtype: str                  # "f32" | "f16" | "bf16"
    lens: Tuple                 # ("fixed", (L0, ...)) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    max_len: int                # table width is ceil(max_len / B)
    pool: Tuple                 # ("fixed", NB) | ("free", frac) | ("fill", frac)
    seed: int
    prefix_tokens: int = 0      # tokens shared by every sequence (multiple of B)
    scale: Optional[float] = None   # None -> 1 / sqrt(D)

    def replace(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


SPECS = {
    # 1 seq, 1 head, D=2, B=2, 5 tokens in a pool of 8, fp32, scale 1/sqrt(2).
    "tiny": WorkloadSpec("tiny", S=1, Hq=1, Hkv=1, D=2, B=2, dtype="f32",
                         lens=("fixed", (5,)), max_len=5, pool=("fixed", 8),
                         seed=1),
    # 8 seqs, 32/32 heads, D=128, B=16, fp16, L ~ U[1, 2048], pool = need + 25 %.
    "mha_small": WorkloadSpec("mha_small", S=8, Hq=32, Hkv=32, D=128, B=16,
                              dtype="f16", lens=("uniform", 1, 2048),
                              max_len=2048, pool=("free", 0.25), seed=2),
    # 64 seqs, 32/32 heads, D=128, B=16, bf16, L ~ U[512, 4096], needed blocks
    # fill 60 % of the pool.
    "mha_7b": WorkloadSpec("mha_7b", S=64, Hq=32, Hkv=32, D=128, B=16,
                           dtype="bf16", lens=("uniform", 512, 4096),
                           max_len=4096, pool=("fill", 0.60), seed=3),
    # 128 seqs, 64 q / 8 kv heads, D=128, B=16, bf16, L log-uniform [128, 8192].
    "gqa_70b": WorkloadSpec("gqa_70b", S=128, Hq=64, Hkv=8, D=128, B=16,
                            dtype="bf16", lens=("loguniform", 128, 8192),
                            max_len=8192, pool=("free", 0.25), seed=4),
    # 16 seqs, 32 q / 8 kv heads, D=128, bf16, L ~ U[16384, 32768], the first
    # 4096 tokens one shared prefix; block size swept over {1, 8, 16, 32}.
    "gqa_long": WorkloadSpec("gqa_long", S=16, Hq=32, Hkv=8, D=128, B=16,
                             dtype="bf16", lens=("uniform", 16384, 32768),
                             max_len=32768, pool=("free", 0.25), seed=5,
                             prefix_tokens=4096),
    # chunked prefill: 16 seqs, 32 q / 8 kv heads, D=128, B=16, bf16, contexts
    # L ~ U[1024, 8192] of which the last 512 tokens are new (the chunk).
    "prefill": WorkloadSpec("prefill", S=16, Hq=32, Hkv=8, D=128, B=16, dtype="bf16",
                            lens=("uniform", 1024, 8192), max_len=8192, pool=("free", 0.25),
                            seed=7),
    # multi-query: 256 seqs, 64 q heads on one kv head, D=128, B=16, bf16,
    # L ~ U[512, 4096], pool = need + 25 %.
    "mqa": WorkloadSpec("mqa", S=256, Hq=64, Hkv=1, D=128, B=16, dtype="bf16",
                        lens=("uniform", 512, 4096), max_len=4096, pool=("free", 0.25),
                        seed=6),
}


@dataclass
class Workload:
    """One batch of decode-attention inputs, resident on ``device``."""
    spec: WorkloadSpec
    query: torch.Tensor          # [S, Hq, D]
    key_cache: torch.Tensor      # [NB, Hkv, B, D]
    value_cache: torch.Tensor    # [NB, Hkv, B, D]
    block_tables: torch.Tensor   # [S, max_blocks] int32
    seq_lens: torch.Tensor       # [S] int32
    scale: float
    NB: int
    max_blocks: int
    lens: np.ndarray             # host copy of seq_lens (int64)
    refcount: np.ndarray         # sequences referencing each physical block
    poison_block: int            # id of a NaN-filled free block, or -1
    tables_host: np.ndarray = field(repr=False, default=None)

    @property
    def S(self): return self.spec.S

    @property
    def Hq(self): return self.spec.Hq

    @property
    def Hkv(self): return self.spec.Hkv

    @property
    def D(self): return self.spec.D

    @property
    def B(self): return self.spec.B

    @property
    def dtype(self): return _DTYPES[self.spec.dtype]

    @property
    def esz(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    def kv_bytes(self) -> int:
        """K+V bytes of every logical token, once per (sequence, kv head)."""
        return int(self.lens.sum()) * self.Hkv * self.D * 2 * self.esz

    def unique_kv_bytes(self) -> int:
        """K+V bytes of the distinct physical slots the batch references."""
        B = self.B
        slots = 0
        seen = set()
        for s in range(self.S):
            L = int(self.lens[s])
            for j in range((L + B - 1) // B):
                p = int(self.tables_host[s, j])
                used = min(B, L - j * B)
                if p in seen:
                    continue
                seen.add(p)
                slots += used
        return slots * self.Hkv * self.D * 2 * self.esz


def _draw_lens(spec: WorkloadSpec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lens[0]
    if kind == "fixed":
        lens = np.asarray(spec.lens[1], dtype=np.int64)
        if lens.size != spec.S:
            raise ValueError("fixed lens must list one length per sequence")
    elif kind == "uniform":
        lo, hi = spec.lens[1], spec.lens[2]
        lens = rng.integers(lo, hi, size=spec.S, endpoint=True).astype(np.int64)
    elif kind == "loguniform":
        lo, hi = spec.lens[1], spec.lens[2]
        u = rng.uniform(math.log(lo), math.log(hi), size=spec.S)
        lens = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)
    else:
        raise ValueError(f"unknown length distribution {kind!r}")
    if lens.max(initial=0) > spec.max_len:
        raise ValueError("a drawn length exceeds max_len")
    return lens


def _normal_fill(t: torch.Tensor, gen: torch.Generator) -> None:
    """Fill ``t`` with N(0,1) fp32 draws rounded to its dtype, in chunks."""
    flat = t.view(-1)
    chunk = 1 << 26
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=gen, device=t.device,
                                    dtype=torch.float32).to(t.dtype)


def make_workload(name_or_spec, *, device="cpu", poison: bool = False,
                  **overrides) -> Workload:
    """Build the named workload (or a spec) on ``device``.

    ``overrides`` replace spec fields (e.g. ``S=4`` or ``B=8``) for cut-down
    or swept variants.
    """
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    if overrides:
        spec = spec.replace(**overrides)
    if spec.Hq % spec.Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if spec.prefix_tokens % spec.B:
        raise ValueError("the shared prefix must end on a block boundary")

    rng = np.random.default_rng(spec.seed)
    lens = _draw_lens(spec, rng)
    if spec.prefix_tokens and lens.min(initial=spec.prefix_tokens) < spec.prefix_tokens:
        raise ValueError("every sequence must contain the shared prefix")
    B = spec.B
    max_blocks = (spec.max_len + B - 1) // B
    nblk = (lens + B - 1) // B
    n_pre = spec.prefix_tokens // B
    unique = n_pre + int((nblk - n_pre).sum()) if spec.S else 0

    kind = spec.pool[0]
    if kind == "fixed":
        NB = int(spec.pool[1])
    elif kind == "free":
        NB = int(math.ceil((1.0 + spec.pool[1]) * unique))
    elif kind == "fill":
        NB = int(math.ceil(unique / spec.pool[1]))
    else:
        raise ValueError(f"unknown pool rule {kind!r}")
    if poison and NB == unique:
        NB += 1                          # keep one free block to poison
    NB = max(NB, 1)
    if NB < unique:
        raise ValueError("pool smaller than the blocks the batch needs")

    perm = rng.permutation(NB)
    tables = np.zeros((spec.S, max_blocks), dtype=np.int32)
    refcount = np.zeros(NB, dtype=np.int64)
    nxt = 0
    prefix_ids = perm[nxt:nxt + n_pre]
    nxt += n_pre
    for s in range(spec.S):
        own = int(nblk[s]) - n_pre
        ids = np.concatenate([prefix_ids, perm[nxt:nxt + own]])
        nxt += own
        tables[s, :ids.size] = ids
        refcount[ids] += 1
    free_ids = perm[nxt:]
    poison_block = int(free_ids[0]) if (poison and free_ids.size) else -1
    if poison:
        for s in range(spec.S):
            tables[s, int(nblk[s]):] = poison_block

    dt = _DTYPES[spec.dtype]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed)
    kc = torch.empty((NB, spec.Hkv, B, spec.D), dtype=dt, device=dev)
    vc = torch.empty_like(kc)
    _normal_fill(kc, gen)
    _normal_fill(vc, gen)
    q = torch.empty((spec.S, spec.Hq, spec.D), dtype=dt, device=dev)
    _normal_fill(q, gen)

    if poison:
        nan = float("nan")
        if free_ids.size:
            idx = torch.as_tensor(free_ids, dtype=torch.long, device=dev)
            kc[idx] = nan
            vc[idx] = nan
        for s in range(spec.S):
            L = int(lens[s])
            if L % B:
                p = int(tables[s, L // B])
                kc[p, :, L % B:, :] = nan
                vc[p, :, L % B:, :] = nan

    scale = spec.scale if spec.scale is not None else 1.0 / math.sqrt(spec.D)
    return Workload(
        spec=spec, query=q, key_cache=kc, value_cache=vc,
        block_tables=torch.as_tensor(tables).to(dev),
        seq_lens=torch.as_tensor(lens.astype(np.int32)).to(dev),
        scale=scale, NB=NB, max_blocks=max_blocks, lens=lens,
        refcount=refcount, poison_block=poison_block, tables_host=tables)


# New tokens per sequence of the multi-token (causal) workloads.
PREFILL_NEW = {"prefill": 512}


@dataclass
class PrefillWorkload:
    """A decode workload plus the new tokens' query rows of a causal call:
    sequence s owns rows query_start[s] .. query_start[s+1]-1, its last n_s
    tokens (already in the cache)."""
    base: Workload
    query: torch.Tensor          # [T, Hq, D]
    query_start: torch.Tensor    # [S+1] int32
    n_new: np.ndarray            # [S] int64
    max_query_len: int

    @property
    def T(self) -> int:
        return int(self.n_new.sum())

    def flops(self) -> int:
        """Algorithmic flops: 4 D per (query row, head, attended token)."""
        total = 0
        for L, n in zip(self.base.lens.tolist(), self.n_new.tolist()):
            # rows attend L-n+1 .. L tokens
            total += n * (L - n) + n * (n + 1) // 2
        return 4 * self.base.D * self.base.Hq * total


def make_prefill_workload(name_or_spec, n_new=None, *, device="cpu", poison: bool = False,
                          **overrides) -> PrefillWorkload:
    """The named workload with n_new new tokens per sequence (an int, capped
    at each length, or one count per sequence); query rows are N(0,1) draws
    from a generator seeded with the spec's seed + 1."""
    w = make_workload(name_or_spec, device=device, poison=poison, **overrides)
    if n_new is None:
        n_new = PREFILL_NEW[w.spec.name]
    if isinstance(n_new, (int, np.integer)):
        n = np.minimum(w.lens, int(n_new)).astype(np.int64)
    else:
        n = np.asarray(n_new, dtype=np.int64)
        if n.shape != w.lens.shape or (n > w.lens).any() or (n < 0).any():
            raise ValueError("n_new must give 0 <= n_s <= L_s per sequence")
    qs = np.zeros(w.S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(n)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.spec.seed + 1)
    q = torch.empty((int(n.sum()), w.Hq, w.D), dtype=w.dtype, device=dev)
    _normal_fill(q, gen)
    return PrefillWorkload(base=w, query=q, query_start=torch.as_tensor(qs).to(dev), n_new=n,
                           max_query_len=int(n.max(initial=0)))
