"""Test helper: build a paged KV pool from logical (contiguous) K / V.

The oracle reads a pool by gathering through block tables.  To pin it
against something other than itself, tests start from logical per-sequence
K / V matrices, *scatter* them into a shuffled pool here, and compute the
expected result from the logical matrices directly (closed forms, or a
library attention routine).  This module only moves data; it computes no
attention.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def scatter_paged(K_logical, V_logical, B, *, rng, dtype=torch.float32,
                  extra_blocks=2, max_blocks=None, fill=float("nan"),
                  pad_id=None):
    """Scatter logical K/V into a paged pool with shuffled physical ids.

    K_logical / V_logical: lists (one per sequence) of [L_s, Hkv, D] tensors.
    Returns dict(key_cache [NB,Hkv,B,D], value_cache, block_tables [S,maxb]
    int32, seq_lens [S] int32, NB, perm) with every unused slot and free block
    set to ``fill`` and unused table entries set to ``pad_id`` (default: a
    free block, or 0 if none).
    """
    S = len(K_logical)
    Hkv, D = K_logical[0].shape[1], K_logical[0].shape[2]
    lens = [int(k.shape[0]) for k in K_logical]
    nblk = [(L + B - 1) // B for L in lens]
    need = sum(nblk)
    NB = need + extra_blocks
    if max_blocks is None:
        max_blocks = max(max(nblk), 1)
    perm = rng.permutation(NB)
    kc = torch.full((NB, Hkv, B, D), fill, dtype=torch.float64)
    vc = torch.full((NB, Hkv, B, D), fill, dtype=torch.float64)
    free = perm[need:]
    if pad_id is None:
        pad_id = int(free[0]) if free.size else 0
    tables = np.full((S, max_blocks), pad_id, dtype=np.int32)
    nxt = 0
    for s in range(S):
        for j in range(nblk[s]):
            p = int(perm[nxt])
            nxt += 1
            tables[s, j] = p
            lo, hi = j * B, min(j * B + B, lens[s])
            # logical token t sits at physical block table[t // B], slot t % B
            kc[p, :, :hi - lo, :] = K_logical[s][lo:hi].permute(1, 0, 2).double()
            vc[p, :, :hi - lo, :] = V_logical[s][lo:hi].permute(1, 0, 2).double()
    return dict(key_cache=kc.to(dtype), value_cache=vc.to(dtype),
                block_tables=torch.as_tensor(tables),
                seq_lens=torch.as_tensor(np.asarray(lens, dtype=np.int32)),
                NB=NB, perm=perm)


def sdpa_reference(q, K_logical, V_logical, scale):
    """Unpaged attention with torch's library routine, in fp64 on the CPU.

    q [S,Hq,D]; K_logical / V_logical lists of [L_s,Hkv,D].  Query head h
    reads kv head h // (Hq // Hkv).  Zero-length sequences give zero rows.
    """
    S, Hq, D = q.shape
    out = torch.zeros((S, Hq, D), dtype=torch.float64)
    for s in range(S):
        K = K_logical[s].double()
        V = V_logical[s].double()
        L, Hkv = K.shape[0], K.shape[1]
        if L == 0:
            continue
        G = Hq // Hkv
        Kh = K.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        Vh = V.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        qs = q[s].double().unsqueeze(0).unsqueeze(2)          # [1,Hq,1,D]
        o = torch.nn.functional.scaled_dot_product_attention(qs, Kh, Vh, scale=scale)
        out[s] = o[0, :, 0, :]
    return out


def random_logical(S, Hkv, D, lens, *, gen, dtype=torch.float32, std=1.0):
    """Random logical K / V lists (values rounded to ``dtype``)."""
    Ks = [(torch.randn((L, Hkv, D), generator=gen, dtype=torch.float64) * std).to(dtype)
          for L in lens]
    Vs = [torch.randn((L, Hkv, D), generator=gen, dtype=torch.float64).to(dtype)
          for L in lens]
    return Ks, Vs


def default_scale(D):
    return 1.0 / math.sqrt(D)
