"""Helpers shared by the GPU parity tests (device tensors, engines)."""
import numpy as np


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch


def dev(a, dtype=None):
    torch = require_gpu()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    require_gpu().cuda.synchronize()
    return t.detach().cpu().numpy()


def engine(cfg, weights_np, **kw):
    from diffusion_drafted_lora_amd import uno
    require_gpu()
    return uno.Engine(cfg, uno.to_device(weights_np, cfg), **kw)


def log(msg):
    print(msg, flush=True)
