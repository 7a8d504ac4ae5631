"""Helpers for the GPU parity tests: host<->device moves and the comparison rules."""
import sys

import numpy as np
import torch

from oracle import gemm as ogemm

DEV = "cuda"

# GEMM tolerances: the parity bar is relative L2 <= 2e-3 against the fp64 oracle;
# each element must also sit within 1e-4 of sum_k |x_k w_k| (fp32 summation of
# at most a few hundred partial sums per output is orders of magnitude tighter),
# which catches a single wrong block that an L2 norm over many rows would hide.
REL_L2 = 2e-3
ELEM = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def check_gemm(codes, scales, n, k, xbits, y_gpu, rows=None, label=""):
    """Compare GPU Y (numpy [m, n] or [m, len(rows)]) against the oracle."""
    ref = ogemm.verify_gemm(codes, scales, n, k, xbits, rows=rows)
    bound = ogemm.abs_bound(codes, scales, n, k, xbits, rows=rows)
    got = np.asarray(y_gpu, dtype=np.float64)
    assert got.shape == ref.shape, (label, got.shape, ref.shape)
    assert np.isfinite(got).all(), label
    err = got - ref
    denom = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / denom if denom > 0 else np.linalg.norm(err)
    worst = np.max(np.abs(err) - ELEM * bound)
    assert rel <= REL_L2, (label, rel)
    assert worst <= 1e-30, (label, worst, np.unravel_index(np.argmax(np.abs(err) - ELEM * bound), err.shape))
    return rel
