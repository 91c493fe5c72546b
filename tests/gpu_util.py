"""Device-tensor helpers for the GPU parity tests (torch as memory plumbing)."""
import numpy as np
import torch


def dev():
    return torch.device("cuda", 0)


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def f16_from_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(dev()).view(torch.float16)


def bf16_from_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(dev()).view(torch.bfloat16)


def bits(t):
    """uint16 bits of an fp16/bf16 device tensor as a host numpy array."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t):
    return t.detach().cpu().numpy()


def normwise(y, ref):
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-300))


def announce(msg):
    print(f"[case] {msg}", flush=True)
