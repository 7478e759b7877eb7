"""Helpers for GPU parity tests: host arrays to device tensors and the tolerance check."""

import sys

import numpy as np
import torch

ATOL = 1e-2        # max |out - ref| over the tensor
RTOL_ROW = 2e-2    # per (node, head) row: ||out - ref|| / ||ref||
LSE_ATOL = 1e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).cuda()


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_attention(out: torch.Tensor, ref: np.ndarray, lse: torch.Tensor = None,
                    lse_ref: np.ndarray = None, label: str = ""):
    """Both bounds must hold: max-abs over the tensor and the per-row relative L2 error."""
    o = bf16_to_f64(out)
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    err = np.abs(o - ref)
    rel = np.linalg.norm(o - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    assert err.max() <= ATOL, f"{label}: max abs err {err.max():.3e}"
    assert rel.max() <= RTOL_ROW, f"{label}: max row rel err {rel.max():.3e}"
    if lse is not None:
        le = np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref)
        assert le.max() <= LSE_ATOL, f"{label}: lse err {le.max():.3e}"
    return err.max(), rel.max()
