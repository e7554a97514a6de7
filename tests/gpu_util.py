"""Helpers for GPU tests: move seeded numpy inputs to the device and bits back."""
import numpy as np


def dev_bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bits(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().view(np.uint32)


def f32_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def say(*args):
    print("[gpu-test]", *args, flush=True)
