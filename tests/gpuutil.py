"""Helpers for the GPU parity tests: move seeded codes to the device, call the
library through its binding, bring results back as float64."""
from __future__ import annotations

import sys

import numpy as np
import torch

import tiled_dense_gemm_tile_amd as tg

DEV = torch.device("cuda:0")
TORCH16 = {"bf16": torch.bfloat16, "fp16": torch.float16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev16(codes: np.ndarray, in_type: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int16))
    return t.view(TORCH16[in_type]).to(DEV)


def dev8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(DEV)


def run16(in_type, A, B, C=None, out="f32", D=None):
    """A, B device tensors of TORCH16[in_type]; returns the device D."""
    fn = tg.gemm_bf16 if in_type == "bf16" else tg.gemm_fp16
    out_dtype = torch.float32 if out == "f32" else torch.bfloat16
    return fn(A, B, C, out_dtype=out_dtype, D=D)


def to_f64(D: torch.Tensor) -> np.ndarray:
    if D.dtype == torch.bfloat16:
        return D.float().cpu().numpy().astype(np.float64)
    return D.cpu().numpy().astype(np.float64)


def bf16_bits(D: torch.Tensor) -> np.ndarray:
    return D.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
