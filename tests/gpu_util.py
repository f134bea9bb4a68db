"""Helpers for the GPU tests: host <-> device copies of bit patterns and the
library's entry points.  Imported only by tests marked ``gpu``."""
import os
import sys

import numpy as np
import torch

from invariant_deterministic_bi_amd import binding as B


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy bit patterns -> cuda tensor (uint16 -> bfloat16, uint8 -> uint8)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to("cuda")
    raise TypeError(a.dtype)


def host(t: torch.Tensor) -> np.ndarray:
    """cuda bfloat16 tensor -> numpy uint16 bit patterns."""
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def note(msg: str) -> None:
    """Name the case before a GPU step, so a failure can be placed."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def loaded_hip_runtimes():
    libs = set()
    with open("/proc/self/maps") as f:
        for line in f:
            p = line.split()[-1]
            if "libamdhip64" in os.path.basename(p):
                libs.add(os.path.realpath(p))
    return libs
