"""Pins for the CPU oracle (runs without a GPU).

Each test ties the oracle to something other than itself: values printed on
the pages, closed forms, invariants the pages state, or unpaged attention
computed by torch's library routine on the logical (contiguous) K / V.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_build import default_scale, random_logical, scatter_paged, sdpa_reference

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked_example_pool(dtype=torch.float32, poison=False):
    """The pages' worked example as a [9,1,2,2] pool (one kv head)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    NB, B, D = ex["num_physical_blocks"], ex["block_size"], ex["head_dim"]
    fill = float("nan") if poison else 0.0
    kc = torch.full((NB, 1, B, D), fill, dtype=torch.float64)
    vc = torch.full((NB, 1, B, D), fill, dtype=torch.float64)
    for pid, blk in ex["blocks"].items():
        kc[int(pid), 0] = torch.tensor(blk["K"], dtype=torch.float64)
        vc[int(pid), 0] = torch.tensor(blk["V"], dtype=torch.float64)
    if poison:
        # the empty slot of the last block holds whatever an evicted sequence left
        kc[1, 0, 1] = float("nan")
        vc[1, 0, 1] = float("nan")
    q = torch.tensor(ex["query"], dtype=torch.float64).reshape(1, 1, D)
    bt = torch.tensor([ex["block_table"]], dtype=torch.int32)
    sl = torch.tensor([ex["context_length"]], dtype=torch.int32)
    return ex, q.to(dtype), kc.to(dtype), vc.to(dtype), bt, sl


def _closed_form(scale):
    """Worked-example output from its five (score, value) pairs, by hand."""
    scores = [1.0, 2.0, 3.0, 2.0, 4.0]
    values = [1.0, 2.0, 3.0, 4.0, 5.0]
    m = max(scores)
    w = [math.exp(scale * (s - m)) for s in scores]
    return math.fsum(wi * v for wi, v in zip(w, values)) / math.fsum(w)


# ---------------------------------------------------------------- conversions

def test_half_decode_exhaustive():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.float16).double().numpy()
    got = np.array([oracle.half_to_double(i) for i in range(1 << 16)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decode_exhaustive():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(i) for i in range(1 << 16)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------ worked example

def test_worked_example_printed_output():
    ex, q, kc, vc, bt, sl = _worked_example_pool()
    out = oracle.decode(q, kc, vc, bt, sl, ex["scale"])
    printed = ex["printed"]["output_code"]
    assert np.round(out[0, 0], ex["printed"]["decimals"]).tolist() == printed
    # The page's hand value is rounded step by step and is not a pin.
    assert abs(out[0, 0, 0] - _closed_form(1.0)) < 1e-14
    assert abs(out[0, 0, 0] - 4.125619931153) < 1e-12
    assert out[0, 0, 0] == out[0, 0, 1]


def test_worked_example_printed_probs_and_scores():
    """Recover the per-token weights through the output: give token t the
    value (1, 0) and every other slot (0, 0); the output is then p_t."""
    ex, q, kc, vc, bt, sl = _worked_example_pool()
    probs = []
    slots = [(2, 0), (2, 1), (0, 0), (0, 1), (1, 0)]     # logical tokens 1..5
    for blk, slot in slots:
        v = torch.zeros_like(vc)
        v[blk, 0, slot] = torch.tensor([1.0, 0.0])
        probs.append(oracle.decode(q, kc, v, bt, sl, 1.0)[0, 0, 0])
    dec = ex["printed"]["decimals"]
    assert np.round(probs, dec).tolist() == ex["printed"]["probs"][:5]
    assert abs(math.fsum(probs) - 1.0) < 1e-15
    # log-ratios give the scores up to the shared max (printed scores minus 4)
    scores = np.log(np.asarray(probs) / max(probs))
    expect = np.asarray(ex["printed"]["scores"][:5], dtype=float) - 4.0
    assert np.allclose(scores, expect, atol=1e-13)
    e = np.round(np.exp(expect), dec)
    assert e.tolist() == ex["printed"]["exp_after_max_subtraction"][:5]
    assert round(float(np.exp(expect).sum()), dec) == ex["printed"]["sum_exp"]


def test_worked_example_scaled():
    ex, q, kc, vc, bt, sl = _worked_example_pool()
    s = 1.0 / math.sqrt(2.0)
    out = oracle.decode(q, kc, vc, bt, sl, s)
    assert abs(out[0, 0, 0] - _closed_form(s)) < 1e-14
    assert abs(out[0, 0, 0] - 3.838545216898) < 1e-11


def test_worked_example_unfilled_slot_is_ignored():
    """NaN in the unfilled slot and in every free block changes nothing."""
    ex, q, kc, vc, bt, sl = _worked_example_pool()
    _, q2, kc2, vc2, bt2, sl2 = _worked_example_pool(poison=True)
    bt2 = torch.tensor([ex["block_table"]], dtype=torch.int32)
    a = oracle.decode(q, kc, vc, bt, sl, 1.0)
    b = oracle.decode(q2, kc2, vc2, bt2, sl2, 1.0)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------- closed forms

def test_single_token_returns_its_value_exactly():
    gen = torch.Generator().manual_seed(11)
    for dtype in (torch.float32, torch.float16, torch.bfloat16):
        Ks, Vs = random_logical(3, 2, 16, [1, 1, 1], gen=gen, dtype=dtype)
        q = torch.randn((3, 4, 16), generator=gen).to(dtype)
        pk = scatter_paged(Ks, Vs, 4, rng=np.random.default_rng(3), dtype=dtype)
        out = oracle.decode(q, pk["key_cache"], pk["value_cache"],
                            pk["block_tables"], pk["seq_lens"], 0.25)
        for s in range(3):
            for h in range(4):
                assert np.array_equal(out[s, h], Vs[s][0, h // 2].double().numpy())


def test_zero_query_gives_mean_of_values():
    gen = torch.Generator().manual_seed(12)
    lens = [7, 19, 33]
    Ks, Vs = random_logical(3, 1, 8, lens, gen=gen)
    q = torch.zeros((3, 1, 8))
    pk = scatter_paged(Ks, Vs, 4, rng=np.random.default_rng(4))
    out = oracle.decode(q, pk["key_cache"], pk["value_cache"],
                        pk["block_tables"], pk["seq_lens"], 0.3)
    for s, L in enumerate(lens):
        for d in range(8):
            mean = math.fsum(float(Vs[s][t, 0, d]) for t in range(L)) / L
            assert abs(out[s, 0, d] - mean) < 1e-14


def test_needle_selects_one_token():
    """K is zero except one token whose key is 64 q/|q|^2: its score is 64
    above every other, so the output is that token's value to fp64 precision."""
    gen = torch.Generator().manual_seed(13)
    L, D, B = 37, 8, 4
    q = torch.randn((1, 1, D), generator=gen, dtype=torch.float64)
    for needle in (0, 5, 17, 36):
        K = torch.zeros((L, 1, D), dtype=torch.float64)
        K[needle, 0] = 64.0 * q[0, 0] / (q[0, 0] @ q[0, 0])
        V = torch.randn((L, 1, D), generator=gen, dtype=torch.float64)
        pk = scatter_paged([K.float()], [V.float()], B, rng=np.random.default_rng(needle))
        Kf = pk["key_cache"]
        out = oracle.decode(q.float(), Kf, pk["value_cache"], pk["block_tables"],
                            pk["seq_lens"], 1.0)
        expect = V[needle, 0].float().double().numpy()
        # others weigh <= L * e^-64 relative to the needle (score error from
        # rounding K to fp32 stays far below 1)
        assert np.allclose(out[0, 0], expect, rtol=0, atol=1e-12)


def test_zero_length_sequence_gives_zeros():
    gen = torch.Generator().manual_seed(14)
    Ks, Vs = random_logical(3, 1, 4, [5, 0, 3], gen=gen)
    q = torch.randn((3, 2, 4), generator=gen)
    pk = scatter_paged(Ks, Vs, 2, rng=np.random.default_rng(5))
    out = oracle.decode(q, pk["key_cache"], pk["value_cache"],
                        pk["block_tables"], pk["seq_lens"], 0.5)
    assert np.array_equal(out[1], np.zeros((2, 4)))
    assert np.all(np.isfinite(out[[0, 2]]))


# ----------------------------------------------------------------- invariants

def test_weights_sum_to_one():
    """With every value row equal to 1 the output is the sum of the weights."""
    gen = torch.Generator().manual_seed(15)
    lens = [1, 2, 9, 64, 300]
    Ks, _ = random_logical(5, 2, 16, lens, gen=gen, std=3.0)
    Vs = [torch.ones_like(k) for k in Ks]
    q = torch.randn((5, 4, 16), generator=gen)
    pk = scatter_paged(Ks, Vs, 8, rng=np.random.default_rng(6))
    out = oracle.decode(q, pk["key_cache"], pk["value_cache"],
                        pk["block_tables"], pk["seq_lens"], 0.25)
    assert np.max(np.abs(out - 1.0)) < 1e-15 * 4


def test_physical_relabelling_is_bit_identical():
    gen = torch.Generator().manual_seed(16)
    lens = [13, 40, 7]
    Ks, Vs = random_logical(3, 2, 8, lens, gen=gen, dtype=torch.bfloat16)
    q = torch.randn((3, 4, 8), generator=gen).to(torch.bfloat16)
    pk = scatter_paged(Ks, Vs, 4, rng=np.random.default_rng(7), dtype=torch.bfloat16)
    ref = oracle.decode(q, pk["key_cache"], pk["value_cache"],
                        pk["block_tables"], pk["seq_lens"], 0.3)
    NB = pk["NB"]
    for seed in range(5):
        pi = np.random.default_rng(100 + seed).permutation(NB)
        kc2 = torch.empty_like(pk["key_cache"])
        vc2 = torch.empty_like(pk["value_cache"])
        kc2[torch.as_tensor(pi)] = pk["key_cache"]
        vc2[torch.as_tensor(pi)] = pk["value_cache"]
        bt2 = torch.as_tensor(pi[pk["block_tables"].numpy()].astype(np.int32))
        out = oracle.decode(q, kc2, vc2, bt2, pk["seq_lens"], 0.3)
        assert np.array_equal(out, ref)


def test_large_scores_do_not_overflow():
    """Scores near 1e4 overflow exp() unless the maximum is subtracted first."""
    L = 9
    K = torch.zeros((L, 1, 2))
    K[:, 0, 0] = torch.arange(L, dtype=torch.float32) * 1000.0 + 5000.0
    V = torch.arange(2 * L, dtype=torch.float32).reshape(L, 1, 2)
    pk = scatter_paged([K], [V], 2, rng=np.random.default_rng(8), fill=0.0)
    q = torch.tensor([[[1.0, 0.0]]])
    out = oracle.decode(q, pk["key_cache"], pk["value_cache"], pk["block_tables"],
                        pk["seq_lens"], 1.0)
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0, 0], V[L - 1, 0].double().numpy(), atol=1e-12)


# ------------------------------------------------- unpaged attention (library)

@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("B,Hq,Hkv,D", [(1, 2, 2, 8), (2, 4, 1, 4), (3, 6, 3, 5),
                                        (4, 8, 2, 16), (16, 4, 4, 32), (32, 8, 1, 64)])
def test_equals_unpaged_attention(dtype, B, Hq, Hkv, D):
    gen = torch.Generator().manual_seed(B * 1000 + Hq * 10 + D)
    rng = np.random.default_rng(B + D)
    lens = [int(x) for x in rng.integers(1, 5 * B + 3, size=4)] + [1, B, B + 1]
    S = len(lens)
    Ks, Vs = random_logical(S, Hkv, D, lens, gen=gen, dtype=dtype)
    q = torch.randn((S, Hq, D), generator=gen).to(dtype)
    pk = scatter_paged(Ks, Vs, B, rng=rng, dtype=dtype, max_blocks=None)
    scale = default_scale(D)
    got = oracle.decode(q, pk["key_cache"], pk["value_cache"],
                        pk["block_tables"], pk["seq_lens"], scale)
    ref = sdpa_reference(q, Ks, Vs, scale).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def test_row_subset_matches_full():
    gen = torch.Generator().manual_seed(17)
    lens = [5, 12, 30]
    Ks, Vs = random_logical(3, 2, 8, lens, gen=gen)
    q = torch.randn((3, 4, 8), generator=gen)
    pk = scatter_paged(Ks, Vs, 4, rng=np.random.default_rng(9))
    args = (q, pk["key_cache"], pk["value_cache"], pk["block_tables"], pk["seq_lens"], 0.2)
    full = oracle.decode(*args)
    rows = [11, 0, 5, 7]
    sub = oracle.decode(*args, rows=rows)
    for i, r in enumerate(rows):
        assert np.array_equal(sub[i], full[r // 4, r % 4])


def test_first_page_demo_layout():
    """The first page's demonstration: seed 42, 8 blocks of 4 tokens, 2 heads,
    head_dim 8, tables [0,3,5] and [1,7] padded with 0, lengths 10 and 7.  Its
    pool is [blocks, block_size, heads, dim]; permuting to [blocks, heads,
    block_size, dim] gives the oracle's layout.  Only the output shape is
    printed there; the values are pinned by unpaged attention."""
    torch.manual_seed(42)
    kc_p1 = torch.randn(8, 4, 2, 8)
    vc_p1 = torch.randn(8, 4, 2, 8)
    bt = torch.tensor([[0, 3, 5, 0, 0, 0, 0, 0], [1, 7, 0, 0, 0, 0, 0, 0]], dtype=torch.int32)
    sl = torch.tensor([10, 7], dtype=torch.int32)
    q = torch.randn(2, 2, 1, 8)
    scale = 1.0 / 8 ** 0.5
    out = oracle.decode(q[:, :, 0, :], kc_p1.permute(0, 2, 1, 3).contiguous(),
                        vc_p1.permute(0, 2, 1, 3).contiguous(), bt, sl, scale)
    assert tuple(out[:, :, None, :].shape) == (2, 2, 1, 8)
    Ks, Vs = [], []
    for s, blocks in enumerate([[0, 3, 5], [1, 7]]):
        Ks.append(torch.cat([kc_p1[b] for b in blocks])[: int(sl[s])])
        Vs.append(torch.cat([vc_p1[b] for b in blocks])[: int(sl[s])])
    ref = sdpa_reference(q[:, :, 0, :], Ks, Vs, scale).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_exhaustive_tiny_tables():
    """Every assignment of a 3-token / B=2 sequence to an ordered pair of
    blocks from a 4-block pool gives the unpaged result, bit-identically."""
    gen = torch.Generator().manual_seed(18)
    for D in (1, 2, 3):
        K = torch.randn((3, 1, D), generator=gen)
        V = torch.randn((3, 1, D), generator=gen)
        q = torch.randn((1, 2, D), generator=gen)
        ref = sdpa_reference(q, [K], [V], 0.7).numpy()
        outs = []
        for a, b in itertools.permutations(range(4), 2):
            kc = torch.full((4, 1, 2, D), float("nan"))
            vc = torch.full((4, 1, 2, D), float("nan"))
            kc[a, 0] = K[0:2, 0]
            vc[a, 0] = V[0:2, 0]
            kc[b, 0, 0] = K[2, 0]
            vc[b, 0, 0] = V[2, 0]
            bt = torch.tensor([[a, b]], dtype=torch.int32)
            outs.append(oracle.decode(q, kc, vc, bt, torch.tensor([3], dtype=torch.int32), 0.7))
        for o in outs:
            assert np.array_equal(o, outs[0])
        assert np.max(np.abs(outs[0] - ref)) < 1e-14


def _brute_force_row(q, Kl, Vl, scale):
    """Attention of one query over logical rows, in plain Python with fsum."""
    x = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in Kl]
    m = max(x)
    w = [math.exp(v - m) for v in x]
    z = math.fsum(w)
    return [math.fsum(wi * v[d] for wi, v in zip(w, Vl)) / z for d in range(len(q))]


def test_brute_force_small_cases():
    """B in 1..4, L in 1..9, D in 1..3, group 1 or 2, tables drawn from a
    shuffled pool (at least 6 blocks): the oracle equals nested-loop Python."""
    rnd = np.random.default_rng(77)
    for B in (1, 2, 3, 4):
        for L in range(1, 10):
            for D in (1, 2, 3):
                for G in (1, 2):
                    nb = -(-L // B)
                    NB = max(6, nb)
                    Kl = rnd.standard_normal((L, D))
                    Vl = rnd.standard_normal((L, D))
                    q = rnd.standard_normal((G, D))
                    table = rnd.permutation(NB)[:nb]
                    kc = torch.full((NB, 1, B, D), float("nan"), dtype=torch.float32)
                    vc = kc.clone()
                    for t in range(L):
                        kc[table[t // B], 0, t % B] = torch.from_numpy(Kl[t]).float()
                        vc[table[t // B], 0, t % B] = torch.from_numpy(Vl[t]).float()
                    Kf = kc.double()
                    Vf = vc.double()
                    K32 = [[float(Kf[table[t // B], 0, t % B, d]) for d in range(D)] for t in range(L)]
                    V32 = [[float(Vf[table[t // B], 0, t % B, d]) for d in range(D)] for t in range(L)]
                    qt = torch.from_numpy(q).float().reshape(1, G, D)
                    out = oracle.decode(qt, kc, vc, torch.from_numpy(table[None].astype(np.int32)),
                                        torch.tensor([L], dtype=torch.int32), 0.6)
                    for h in range(G):
                        ref = _brute_force_row([float(v) for v in qt[0, h].double()], K32, V32, 0.6)
                        assert np.max(np.abs(out[0, h] - np.array(ref))) < 1e-14, (B, L, D, G)


def test_rejects_out_of_range_inputs():
    q = torch.zeros((1, 1, 2))
    kc = torch.zeros((2, 1, 2, 2))
    with pytest.raises(ValueError):
        oracle.decode(q, kc, kc, torch.tensor([[5]], dtype=torch.int32),
                      torch.tensor([2], dtype=torch.int32), 1.0)
    with pytest.raises(ValueError):
        oracle.decode(q, kc, kc, torch.tensor([[0]], dtype=torch.int32),
                      torch.tensor([3], dtype=torch.int32), 1.0)
