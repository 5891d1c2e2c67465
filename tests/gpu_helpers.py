"""Helpers shared by the GPU parity tests: upload seeded inputs, run the library, compare."""
import sys

import numpy as np
import torch

import synth

# Parity bars. bf16 inputs with fp32 accumulation: max-abs <= 2e-2 and mean-abs <= 2e-3 on
# fp32-output runs; fp32 inputs: max-abs <= 1e-4.
BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


def note(msg: str):
    """Name the case on stdout before each GPU step, flushed, so a failing run says what ran."""
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def up(arr: np.ndarray) -> torch.Tensor:
    """Host array -> device tensor: uint16 bf16 bit patterns become bfloat16, float32 stays."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device()).view(torch.bfloat16)
    if arr.dtype == np.float32:
        return torch.from_numpy(arr).to(device())
    if arr.dtype in (np.int32, np.int64):
        return torch.from_numpy(arr.astype(np.int32)).to(device())
    raise TypeError(arr.dtype)


def down_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def rne_bits_of(t32: torch.Tensor) -> np.ndarray:
    """RNE bf16 of an fp32 device tensor, as bit patterns (computed on the host)."""
    return synth.f32_to_bf16_bits(t32.detach().cpu().numpy())


def assert_parity(got: np.ndarray, want: np.ndarray, in_dtype: str, what: str = ""):
    assert got.shape == want.shape, (got.shape, want.shape)
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    if in_dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN, "%s: max-abs %.3g mean-abs %.3g" % (what, mx, mean)
    else:
        assert mx <= F32_MAX, "%s: max-abs %.3g" % (what, mx)
    return mx, mean
