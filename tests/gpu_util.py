"""Helpers shared by the GPU tests: host <-> device conversions."""

import numpy as np
import torch

import synth


def dev_i8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a.astype(np.int8))).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a.astype(np.int32))).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a.astype(np.float32))).cuda()


def dev_bf16_bits(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint16)).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    """Round float values to bf16 (nearest even) and upload; returns (tensor, exact host values)."""
    bits = synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return dev_bf16_bits(bits), synth.bf16_bits_to_f32(bits).astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def announce(name: str):
    print(f"[gpu-case] {name}", flush=True)
