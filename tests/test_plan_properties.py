"""Property tests of the host planner (no GPU): random shapes and
configurations through pa_decode_plan and pa_prefill_plan.  Whatever the
planner accepts must satisfy what the kernels assume of it:

* the chosen kernel family runs this head size, dtype, block size and group;
* partitions are positive multiples of the 32-token tile and cover the
  longest context with at most 65535 of them (a grid dimension);
* with blocks of fewer than 4 tokens the tiled kernels copy a partition's
  block-table slice to LDS, which holds 1024 ids: a partition is at most
  1024 blocks;
* one of the two decode grids (the 1-D live-item grid for at most 1024
  sequences, else the rectangular one) stays under the launch limit of 2^32
  threads, and the multi-token grid likewise (64-, 128- or 256-column
  work-groups by the longest chunk);
* a split plan's workspace holds every partial result (o, m, l in fp32);
* an explicit partition is honoured unless it is not needed (one pass),
  too small for the grid or too large for the table slice;
* items run on 1, 2 or 4 token-waves: the count asked for, else more than
  one only in batches of at least 512 (sequence, kv head) pairs whose
  partition the planner lengthened for them (more than 512 tokens a wave),
  and only on the kernels that run them.

and everything it refuses carries the documented status."""
import ctypes

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from paged_kv_cache_301_amd import binding as b  # noqa: E402

TILE = 32
MAX_PARTS = 65535
TABLE_LDS = 1024
SCHED_MAX_SEQS = 1024
LAUNCH_LIMIT = 1 << 32
PREFILL_COLUMNS = 128
PREFILL_NARROW = 64
PREFILL_WIDE = 256
KERNELS = {"auto": b.KERNEL_AUTO, "generic": b.KERNEL_GENERIC, "valu": b.KERNEL_VALU,
           "mfma": b.KERNEL_MFMA}
DTYPES = (b.PA_F32, b.PA_F16, b.PA_BF16)


def pow2(x):
    return x > 0 and x & (x - 1) == 0


def ceil_div(a, c):
    return (a + c - 1) // c


def supports(kernel, Hq, Hkv, D, B, dt):
    G = Hq // Hkv
    tiled = D == 128 and dt in (b.PA_F16, b.PA_BF16) and pow2(B)
    if kernel == b.KERNEL_VALU:
        return tiled and G in (1, 2, 4, 8)
    if kernel == b.KERNEL_MFMA:
        return tiled and G in (1, 2, 4, 8, 16, 32, 64)
    return D <= 512


# sizes at the planner's boundaries as well as random ones: the live-item
# decode's 1024 sequences, the 65535 grid rows, the int32 token index
EDGE_S = [1023, 1024, 1025, 4096, 16383, 16384, 65535, 65536]
EDGE_BLOCKS = [(1 << 31) // B - d for B in (1, 2, 16) for d in (0, 1)] + [1 << 21, 2097152 + 1]

shapes = st.fixed_dictionaries({
    "S": st.one_of(st.integers(0, 64), st.integers(0, 70000), st.sampled_from(EDGE_S)),
    "Hkv": st.sampled_from([1, 2, 4, 8, 16, 32, 64, 1024]),
    "G": st.sampled_from([1, 2, 3, 4, 8, 16, 32, 64, 128]),
    "D": st.one_of(st.just(128), st.integers(1, 600)),
    "B": st.one_of(st.sampled_from([1, 2, 4, 8, 16, 32, 64, 128]), st.integers(1, 300)),
    "NB": st.integers(1, 1 << 22),
    "max_blocks": st.one_of(st.integers(0, 64), st.integers(0, 1 << 20),
                            st.sampled_from(EDGE_BLOCKS)),
    "dt": st.sampled_from(DTYPES),
    "odt_f32": st.booleans(),
    "kernel": st.sampled_from(sorted(KERNELS)),
    "part": st.one_of(st.just(0), st.integers(1, 200).map(lambda k: TILE * k),
                      st.integers(1, 1 << 16)),
    "tw": st.sampled_from([0, 0, 0, 1, 2, 4, 3]),
})


def decode_plan(sh):
    Hq = sh["G"] * sh["Hkv"]
    odt = b.PA_F32 if sh["odt_f32"] else sh["dt"]
    cfg = b.PaConfig(KERNELS[sh["kernel"]], sh["part"], 0, 0, 0, sh["tw"])
    p = b.PaPlan()
    st_ = b.load().pa_decode_plan(sh["S"], Hq, sh["Hkv"], sh["D"], sh["B"], sh["NB"],
                                  sh["max_blocks"], sh["dt"], odt, ctypes.byref(cfg),
                                  ctypes.byref(p))
    return st_, p, Hq


@settings(max_examples=3000, deadline=None)
@given(shapes)
def test_decode_plan_properties(sh):
    st_, p, Hq = decode_plan(sh)
    S, Hkv, D, B, dt = sh["S"], sh["Hkv"], sh["D"], sh["B"], sh["dt"]
    max_ctx = sh["max_blocks"] * B
    req = sh["part"]
    forced = KERNELS[sh["kernel"]]
    if max_ctx > 2**31 - 1 or S > 65535 or Hq > 65535 or S * Hq > 2**31 - 1:
        assert st_ == b.PA_ERR_SHAPE
        return
    # sizes first, then types and head size, then the configuration
    if D > 512:
        assert st_ == b.PA_ERR_UNSUPPORTED
        return
    if req % TILE != 0 or sh["tw"] not in (0, 1, 2, 4):
        assert st_ == b.PA_ERR_SHAPE
        return
    if forced in (b.KERNEL_VALU, b.KERNEL_MFMA) and not supports(forced, Hq, Hkv, D, B, dt):
        assert st_ == b.PA_ERR_UNSUPPORTED
        return
    if st_ != b.PA_OK:
        # the only other refusals: a grid past the launch limits, or a forced
        # tiled kernel whose table slice cannot hold the partitions
        assert st_ in (b.PA_ERR_SHAPE, b.PA_ERR_UNSUPPORTED), st_
        return

    assert p.kernel in (b.KERNEL_GENERIC, b.KERNEL_VALU, b.KERNEL_MFMA)
    assert forced == b.KERNEL_AUTO or p.kernel == forced
    assert supports(p.kernel, Hq, Hkv, D, B, dt)
    G = Hq // Hkv
    multi_ok = (p.kernel == b.KERNEL_VALU and B % 4 == 0) or (p.kernel == b.KERNEL_MFMA and G <= 16)
    assert sh["tw"] <= 1 or multi_ok
    if sh["tw"]:
        assert p.token_waves == sh["tw"]
    else:
        assert p.token_waves in (1, 2, 4)
        if p.token_waves > 1:
            assert multi_ok and B % 4 == 0 and req == 0 and S * Hkv >= 512
            assert p.partition_tokens > 512 * p.token_waves   # at most 1024 tokens a wave
    if p.kernel == b.KERNEL_GENERIC:
        assert p.split == 0 and p.workspace_bytes == 0 and p.max_partitions == 1
        assert p.partition_tokens >= max(max_ctx, 1)
        return
    P, parts = p.partition_tokens, p.max_partitions
    assert P > 0 and P % TILE == 0
    assert parts == (ceil_div(max_ctx, P) if max_ctx > 0 else 1)
    assert 1 <= parts <= MAX_PARTS
    assert p.split == (1 if parts > 1 else 0)
    if B % 4 != 0:
        assert ceil_div(P, B) <= TABLE_LDS
    if p.kernel == b.KERNEL_MFMA:
        threads = 64 * ceil_div(G, 16) * p.token_waves
    else:
        threads = 64 * p.token_waves
    compact = S <= SCHED_MAX_SEQS and S * Hkv * parts * threads < LAUNCH_LIMIT
    rect = S * Hkv * threads < LAUNCH_LIMIT and parts <= MAX_PARTS
    assert compact or rect
    if p.split:
        assert p.workspace_bytes >= S * Hq * parts * (D + 2) * 4
    else:
        assert p.workspace_bytes == 0
    if req > 0:
        cap = TABLE_LDS * B if B % 4 != 0 else None
        single = req >= max_ctx
        too_small = req < ceil_div(max_ctx, MAX_PARTS)
        too_big = cap is not None and req > cap
        if not (single or too_small or too_big):
            assert P == req
    if forced == b.KERNEL_AUTO and req == 0 and sh["tw"] == 0 and sh["odt_f32"] is False:
        # the automatic plan is what pa_decode_workspace_bytes reports
        n = b.load().pa_decode_workspace_bytes(S, Hq, Hkv, D, B, sh["NB"], sh["max_blocks"],
                                               dt, dt)
        assert n == p.workspace_bytes


prefill_shapes = st.fixed_dictionaries({
    "S": st.one_of(st.integers(1, 64), st.integers(1, 70000), st.sampled_from(EDGE_S)),
    "T": st.one_of(st.integers(1, 4096), st.integers(1, 70000), st.sampled_from(EDGE_S)),
    "Hkv": st.sampled_from([1, 2, 4, 8, 16, 64]),
    "G": st.sampled_from([1, 2, 3, 4, 8, 16, 32, 64, 128]),
    "D": st.one_of(st.just(128), st.integers(1, 600)),
    "B": st.one_of(st.sampled_from([1, 2, 4, 8, 16, 32]), st.integers(1, 100)),
    "max_blocks": st.one_of(st.integers(0, 64), st.integers(0, 1 << 18),
                            st.sampled_from(EDGE_BLOCKS)),
    "mql": st.one_of(st.integers(1, 600), st.integers(1, 70000)),
    "dt": st.sampled_from(DTYPES),
    "kernel": st.sampled_from(["auto", "generic", "mfma"]),
    "part": st.one_of(st.just(0), st.integers(1, 200).map(lambda k: TILE * k)),
})


@settings(max_examples=3000, deadline=None)
@given(prefill_shapes)
def test_prefill_plan_properties(sh):
    S, T, Hkv, D, B, dt = sh["S"], sh["T"], sh["Hkv"], sh["D"], sh["B"], sh["dt"]
    Hq = sh["G"] * Hkv
    cfg = b.PaConfig(KERNELS[sh["kernel"]], sh["part"], 0, 0, 0)
    p = b.PaPlan()
    st_ = b.load().pa_prefill_plan(S, T, Hq, Hkv, D, B, 8, sh["max_blocks"], sh["mql"], dt, dt,
                                   ctypes.byref(cfg), ctypes.byref(p))
    max_ctx = sh["max_blocks"] * B
    # the decode validation first (sizes, then types and head size), then
    # the query rows
    if max_ctx > 2**31 - 1 or S > 65535 or Hq > 65535 or S * Hq > 2**31 - 1:
        assert st_ == b.PA_ERR_SHAPE
        return
    if D > 512:
        assert st_ == b.PA_ERR_UNSUPPORTED
        return
    if T > 65535 or T * Hq > 2**31 - 1:
        assert st_ == b.PA_ERR_SHAPE
        return
    if st_ != b.PA_OK:
        assert st_ in (b.PA_ERR_SHAPE, b.PA_ERR_UNSUPPORTED), st_
        return
    assert p.kernel in (b.KERNEL_GENERIC, b.KERNEL_MFMA)
    if p.kernel == b.KERNEL_GENERIC:
        assert p.split == 0 and p.workspace_bytes == 0
        return
    assert supports(b.KERNEL_MFMA, Hq, Hkv, D, B, dt)
    P, parts = p.partition_tokens, p.max_partitions
    assert P > 0 and P % TILE == 0
    assert parts == (ceil_div(max_ctx, P) if max_ctx > 0 else 1) and parts <= MAX_PARTS
    assert p.split == (1 if parts > 1 else 0)
    if B % 4 != 0:
        assert ceil_div(P, B) <= TABLE_LDS
    # grid x: the (sequence, kv head) pairs padded to whole XCD rounds, times
    # the query blocks of cols / G tokens, 64 threads per 32 columns; cols is
    # 64 when every sequence's rows fit them, 256 when the longest chunk
    # fills 256, else 128
    rows = sh["G"] * sh["mql"]
    cols = (PREFILL_NARROW if rows <= PREFILL_NARROW
            else PREFILL_WIDE if rows >= PREFILL_WIDE else PREFILL_COLUMNS)
    qb = ceil_div(sh["mql"], cols // sh["G"])
    assert ceil_div(S * Hkv, 8) * 8 * qb * 2 * cols < LAUNCH_LIMIT
    if p.split:
        assert p.workspace_bytes >= T * Hq * parts * (D + 2) * 4
