"""Helpers for the GPU parity tests: host arrays to device tensors, and the
attention tolerance max |gpu - ref| <= 2e-3 * (1 + |ref|), elementwise."""
import sys

import numpy as np
import torch

ATOL_REL = 2e-3


def announce(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    """numpy -> cuda tensor, bf16 bit patterns (uint16) -> torch.bfloat16."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16)
        if bf16:
            t = t.view(torch.bfloat16)
    elif a.dtype == np.uint32:
        t = t.view(torch.int32)
    return t.cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, tol: float = ATOL_REL) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = np.abs(got - ref)
    bound = tol * (1.0 + np.abs(ref))
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    ratio = float(np.max(err / bound))
    assert np.all(err <= bound), "%s: max |err| %.3g at %s (ref %.4g, got %.4g), %.2fx the bound" % (
        what, err[worst], worst, ref[worst], got[worst], ratio)
    return ratio
