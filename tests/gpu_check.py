"""Shared comparison rules for the GPU parity tests.

fp32 inputs: max |gpu - oracle| <= 1e-5.
fp16 / bf16 inputs (fp32 accumulation): per element
    rel = |gpu - oracle| / max(|oracle|, 1e-2 * max_row |oracle|) <= 2e-3
for fp32 outputs (the kernel's arithmetic alone), and for outputs rounded to
the input type the final rounding is allowed on top:
    |gpu - oracle| <= 2e-3 * max(|oracle|, floor) + half an ulp of the type at oracle.
A "row" is one (sequence, head) output vector.
"""
import numpy as np
import torch

MANT_BITS = {torch.float16: 10, torch.bfloat16: 7}


def half_ulp(ref: np.ndarray, dtype) -> np.ndarray:
    mb = MANT_BITS[dtype]
    a = np.abs(ref)
    tiny = 2.0 ** (-24 if dtype == torch.float16 else -133)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    if dtype == torch.float16:
        e = np.maximum(e, -14)
    return np.maximum(2.0 ** (e - mb - 1), tiny / 2)


def check(got_t: torch.Tensor, ref: np.ndarray, in_dtype, label: str = ""):
    got = got_t.double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    if in_dtype == torch.float32:
        err = np.abs(got - ref).max(initial=0.0)
        assert err <= 1e-5, f"{label}: max abs err {err:.3e} > 1e-5"
        return {"max_abs": float(err)}
    floor = 1e-2 * np.abs(ref).max(axis=-1, keepdims=True)
    denom = np.maximum(np.abs(ref), floor)
    denom = np.where(denom > 0, denom, 1.0)
    diff = np.abs(got - ref)
    if got_t.dtype == torch.float32:
        rel = diff / denom
        worst = rel.max(initial=0.0)
        assert worst <= 2e-3, f"{label}: max rel err {worst:.3e} > 2e-3"
        return {"max_rel": float(worst)}
    bound = 2e-3 * denom + half_ulp(ref, got_t.dtype)
    ratio = (diff / bound).max(initial=0.0)
    assert ratio <= 1.0, f"{label}: error exceeds bound by {ratio:.3f}x"
    return {"bound_ratio": float(ratio)}
