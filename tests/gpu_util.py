"""Helpers for the GPU parity tests: moving generator outputs to the device and comparing with the oracle."""
import sys

import numpy as np
import torch

import workloads as W

BF16_TOL = 2e-2     # max abs error on bf16 outputs against the fp64 oracle
FP32_TOL = 1e-4     # max abs error for the fp32 path
LSE_TOL = 1e-2      # natural-log lse of the bf16 path (fp32 arithmetic, sums of bf16-rounded probabilities)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_i32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def prefill_to_device(inp: W.PrefillInputs):
    if inp.dtype == "bf16":
        return dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    return dev_f32(inp.q), dev_f32(inp.k), dev_f32(inp.v)


def take_rows(x: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """x [B,H,N,...] on the device, rows [H,R] -> host float64 [B,H,R,...]."""
    idx = torch.from_numpy(rows).to(x.device)
    B, H = x.shape[:2]
    extra = x.shape[3:]
    g = idx.view(1, H, -1, *([1] * len(extra))).expand(B, H, idx.shape[1], *extra)
    return host64(torch.gather(x, 2, g))


def max_err(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0
