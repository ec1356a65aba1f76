"""Plant plausible mistakes in the oracle (on the CPU) and check the pins see them.

Each mutant is the oracle's C source with one edit: a dropped term, a wrong
index, a swapped operand.  It is compiled into a temporary library and run
through a short battery of the same pins ``test_oracle.py`` uses; every mutant
must fail at least one of them.
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from paged_build import random_logical, scatter_paged, sdpa_reference

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

MUTANTS = {
    "kv_head_mod": ("int g = h / G;", "int g = h % Hkv;"),
    "no_length_bound": ("int last = first + B < n ? first + B : n;", "int last = first + B;"),
    "slot_dropped": ("* Hkv + g) * B + slot)", "* Hkv + g) * B + 0)"),
    "page1_layout": ("(((size_t)phys * Hkv + g) * B + slot)", "(((size_t)phys * B + slot) * Hkv + g)"),
    "block_order_reversed": ("int phys = block_tables[(size_t)s * max_blocks + j];",
                             "int phys = block_tables[(size_t)s * max_blocks + (nblocks - 1 - j)];"),
    "scale_dropped": ("x[tt] = scale * acc;", "x[tt] = acc;"),
    "min_not_max": ("if (x[tt] > m) m = x[tt];", "if (x[tt] < m) m = x[tt];"),
    "no_normalise": ("for (int tt = 0; tt < n; ++tt) x[tt] /= Z;", ""),
    "k_for_v": ("o[d] += x[tt] * V[", "o[d] += x[tt] * K["),
    "last_token_dropped": ("for (int tt = 0; tt < n; ++tt)\n        for (int d = 0; d < D; ++d) o[d]",
                           "for (int tt = 0; tt < n - 1; ++tt)\n        for (int d = 0; d < D; ++d) o[d]"),
    "half_bias": ("e - 25", "e - 24"),
    "bf16_shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "query_index": ("((size_t)qrow * Hq + h) * D + d", "((size_t)h * 1 + qrow) * D + d"),
    "prefill_excludes_self": ("t, pos + 1, scale, out", "t, pos, scale, out"),
    "prefill_no_offset": ("int pos = seq_lens[s] - n + (t - query_start[s]);",
                          "int pos = t - query_start[s];"),
    "prefill_sequence_row": ("t, pos + 1, scale, out", "s, pos + 1, scale, out"),
    "prefill_future_visible": ("t, pos + 1, scale, out", "t, seq_lens[s], scale, out"),
    "score_sign": ("acc += qv[d] * K", "acc -= qv[d] * K"),
    "write_offset_dropped": ("* B + offset) * (size_t)D * esz;", "* B + 0) * (size_t)D * esz;"),
    "write_page_layout": ("(((size_t)block * Hkv + h) * B + offset)",
                          "(((size_t)block * B + offset) * Hkv + h)"),
    "write_key_into_values": ("memcpy((char *)value_cache + dst, (const char *)value + src",
                              "memcpy((char *)value_cache + dst, (const char *)key + src"),
    "write_block_zero": ("long long block = slot / B, offset", "long long block = 0 * slot / B, offset"),
}


def _build_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} is not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    str(path), "-o", str(so), "-lm"], check=True)
    return str(so)


def _battery():
    """Return the names of the pins that fail under the current oracle."""
    failed = []
    # worked example (printed output, scale 1)
    from test_oracle import _closed_form, _worked_example_pool
    ex, q, kc, vc, bt, sl = _worked_example_pool(poison=True)
    try:
        out = oracle.decode(q, kc, vc, bt, sl, 1.0)
        if not abs(out[0, 0, 0] - _closed_form(1.0)) < 1e-12:
            failed.append("worked_example")
        out = oracle.decode(q, kc, vc, bt, sl, 1.0 / math.sqrt(2))
        if not abs(out[0, 0, 0] - _closed_form(1.0 / math.sqrt(2))) < 1e-12:
            failed.append("worked_example_scaled")
    except ValueError:
        failed.append("worked_example_raised")
    # unpaged attention: GQA, several sequences, every dtype, NaN-poisoned pool
    for dtype in (torch.float16, torch.bfloat16):
        gen = torch.Generator().manual_seed(5)
        rng = np.random.default_rng(5)
        lens = [1, 3, 8, 13]
        Ks, Vs = random_logical(4, 2, 6, lens, gen=gen, dtype=dtype)
        qq = torch.randn((4, 4, 6), generator=gen).to(dtype)
        pk = scatter_paged(Ks, Vs, 4, rng=rng, dtype=dtype)
        got = oracle.decode(qq, pk["key_cache"], pk["value_cache"],
                            pk["block_tables"], pk["seq_lens"], 0.4)
        ref = sdpa_reference(qq, Ks, Vs, 0.4).numpy()
        if not np.max(np.abs(got - ref)) < 1e-12:
            failed.append(f"sdpa_{dtype}")
    # several new tokens per sequence against masked unpaged attention
    from test_prefill import causal_reference
    gen = torch.Generator().manual_seed(6)
    lens, n_new = [1, 9, 14, 6], [1, 4, 14, 2]
    Ks, Vs = random_logical(4, 2, 6, lens, gen=gen)
    qq = torch.randn((sum(n_new), 4, 6), generator=gen)
    pk = scatter_paged(Ks, Vs, 4, rng=np.random.default_rng(6))
    qs = torch.tensor(np.concatenate([[0], np.cumsum(n_new)]), dtype=torch.int32)
    try:
        got = oracle.prefill(qq, pk["key_cache"], pk["value_cache"], pk["block_tables"],
                             pk["seq_lens"], qs, 0.4)
        ref = causal_reference(qq, Ks, Vs, n_new, 0.4).numpy()
        if not np.max(np.abs(got - ref)) < 1e-12:
            failed.append("prefill_sdpa")
    except ValueError:
        failed.append("prefill_raised")
    # large scores
    L = 9
    K = torch.zeros((L, 1, 2))
    K[:, 0, 0] = torch.arange(L, dtype=torch.float32) * 1000.0 + 5000.0
    V = torch.arange(2 * L, dtype=torch.float32).reshape(L, 1, 2)
    pk = scatter_paged([K], [V], 2, rng=np.random.default_rng(8), fill=0.0)
    out = oracle.decode(torch.tensor([[[1.0, 0.0]]]), pk["key_cache"], pk["value_cache"],
                        pk["block_tables"], pk["seq_lens"], 1.0)
    if not np.allclose(out[0, 0], V[L - 1, 0].double().numpy(), atol=1e-12):
        failed.append("large_scores")
    # a decode-step write, then attention over the grown contexts
    from test_kv_write import append_then_attend_error
    try:
        if not append_then_attend_error(torch.float32) < 1e-12:
            failed.append("append_then_attend")
    except ValueError:
        failed.append("append_raised")
    # conversions (a sample of bit patterns)
    for bits in (0x3C00, 0x0001, 0x7BFF, 0xC000, 0x3555):
        ref = torch.tensor([bits], dtype=torch.int32).to(torch.int16).view(torch.float16).item()
        if oracle.half_to_double(bits) != ref:
            failed.append("half")
            break
    for bits in (0x3F80, 0x0001, 0x7F7F, 0xC000, 0x3EAB):
        ref = torch.tensor([bits], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).item()
        if oracle.bf16_to_double(bits) != ref:
            failed.append("bf16")
            break
    return failed


def test_unmutated_oracle_passes_battery():
    assert _battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    """Run the battery in a child process: a mutant may also crash (reading
    outside its buffers), which counts as caught."""
    so = _build_mutant(name, tmp_path)
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import sys, oracle\n"
        f"oracle.LIB_PATH = {so!r}\n"
        f"oracle._SRC = {so!r}\n"
        "import test_oracle_mutants as m\n"
        "failed = m._battery()\n"
        "print('FAILED:' + ','.join(failed))\n"
        "sys.exit(0 if failed else 3)\n")
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([here, os.path.dirname(here)]),
               OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 3, f"mutant {name} passed every pin:\n{r.stdout}{r.stderr}"
