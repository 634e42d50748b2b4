"""Helpers shared by the GPU tests: device upload of bf16 bit patterns and the
acceptance check against the float64 reference.

Acceptance (stated for this path): bf16 outputs within
|gpu - ref| <= 1.6e-2 + 1e-2 * |ref| elementwise, |delta LSE| <= 1e-3, an
LSE of -inf reproduced exactly together with an output of exactly +0.0 for
that (row, head), no NaN anywhere.
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import bf16_bits_to_f32

ATOL = 1.6e-2
RTOL = 1e-2
LSE_TOL = 1e-3


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_padding_exact(out_gpu: torch.Tensor, lse_gpu: torch.Tensor, what: str = "") -> None:
    """Rows with no valid key: every output bit pattern is +0.0 and every LSE is -inf."""
    assert not host_bits(out_gpu).any(), f"{what}: padding output is not exactly +0.0"
    l = lse_gpu.detach().cpu().numpy()
    assert np.isneginf(l).all(), f"{what}: padding LSE is not -inf"


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(host_bits(t)).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def check_close(out_gpu: torch.Tensor, lse_gpu: torch.Tensor, out_ref: np.ndarray,
                lse_ref: np.ndarray, what: str = "") -> dict:
    """Assert the acceptance bar; return the worst errors for reporting."""
    o = host_f64(out_gpu)
    l = host_f64(lse_gpu)
    assert o.shape == out_ref.shape and l.shape == lse_ref.shape, (o.shape, out_ref.shape)
    assert not np.isnan(o).any(), f"{what}: NaN in output"
    assert not np.isnan(l).any(), f"{what}: NaN in LSE"
    err = np.abs(o - out_ref)
    bound = ATOL + RTOL * np.abs(out_ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of tolerance, first at "
                             f"{idx.tolist()}: gpu {o[tuple(idx[0])]} ref {out_ref[tuple(idx[0])]}")
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), ninf_ref), f"{what}: -inf LSE pattern differs"
    if ninf_ref.any():
        # A (row, head) with no valid key returns exactly +0.0 (bit pattern 0), not merely
        # something inside the tolerance band.
        bits = host_bits(out_gpu) if out_gpu.dtype == torch.bfloat16 else None
        if bits is not None:
            assert not bits[ninf_ref].any(), f"{what}: a row without keys is not exactly +0.0"
        else:
            assert (o[ninf_ref] == 0).all() and not np.signbit(o[ninf_ref]).any(), \
                f"{what}: a row without keys is not exactly +0.0"
    fin = ~ninf_ref
    lerr = np.abs(l[fin] - lse_ref[fin])
    assert (lerr <= LSE_TOL).all(), f"{what}: LSE error {lerr.max()}"
    return {"max_abs_err": float(err.max(initial=0.0)),
            "max_lse_err": float(lerr.max(initial=0.0))}
