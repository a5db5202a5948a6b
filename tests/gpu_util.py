"""Device helpers for the GPU parity tests (test code only)."""
import sys

import numpy as np


def say(*a):
    """Name the case before each GPU step, flushed, so a dying run still
    leaves its last case in the log."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_device(x):
    """numpy float32 or uint16 (bf16 bit patterns) -> CUDA tensor."""
    import torch
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    elif x.dtype == np.float32:
        t = torch.from_numpy(np.ascontiguousarray(x))
    elif x.dtype == np.uint8:
        t = torch.from_numpy(np.ascontiguousarray(x))
    else:
        raise TypeError(x.dtype)
    return t.cuda()


def bf16_to_np(t):
    """CUDA bfloat16 tensor -> float64 numpy."""
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def host(t):
    return t.detach().cpu().numpy()
