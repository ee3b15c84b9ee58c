"""Device-side generation of the seeded inputs (HIP filler in ``libsynth.so``).

Produces, directly in GPU memory, exactly the elements ``synth.values``
gives on the host.  Holds no arithmetic of the attention method.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import BF16N, BF16U4, I8U4

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_int64, ctypes.c_void_p]
        lib.synth_fill.restype = ctypes.c_int
        _lib = lib
    return _lib


def fill_(t: torch.Tensor, kind: int, seed: int, tid: int) -> torch.Tensor:
    """Fill the contiguous CUDA tensor ``t`` in place (int8 or bf16 storage)."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("fill_ needs a contiguous device tensor")
    want = torch.int8 if kind == I8U4 else torch.bfloat16
    if t.dtype != want:
        raise ValueError(f"kind {kind} fills {want}, got {t.dtype}")
    rc = _load().synth_fill(ctypes.c_void_p(t.data_ptr()), kind, seed, tid, t.numel(),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill failed with code {rc}")
    return t


def make(cfg, spec, device="cuda") -> torch.Tensor:
    """Allocate and fill one tensor of a workload on the device."""
    kind, shape, tid = spec
    dtype = torch.int8 if kind == I8U4 else torch.bfloat16
    t = torch.empty(shape, dtype=dtype, device=device)
    return fill_(t, kind, cfg.seed, tid)
