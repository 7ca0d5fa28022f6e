"""Helpers shared by the GPU tests (no test functions here)."""
import os

import numpy as np


class forced_env:
    """Temporarily set liblce's path-selection environment variables."""

    def __init__(self, **kv):
        self.kv = {k: str(v) for k, v in kv.items()}
        self.old = {}

    def __enter__(self):
        for k, v in self.kv.items():
            self.old[k] = os.environ.get(k)
            os.environ[k] = v

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def to_dev(arr):
    """numpy f32 -> fp32 device tensor; numpy uint16 (bf16 bits) -> bf16 device tensor."""
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()
