"""Helpers shared by the GPU tests: move stored arrays (synth's numpy storage) to the
device and back, and the relative error measures used by the parity bars."""
import sys

import numpy as np


def torch():
    import torch as t
    return t


def to_dev(arr, dtype):
    """numpy storage array -> torch cuda tensor of the given stored dtype."""
    t = torch()
    if dtype == "bf16":
        x = t.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)).view(t.bfloat16)
    elif dtype == "f16":
        x = t.from_numpy(np.ascontiguousarray(arr, dtype=np.float16))
    elif dtype == "f32":
        x = t.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return x.to("cuda")


def to_f64(x):
    """torch tensor (any float dtype, any device) -> numpy float64."""
    return x.detach().to("cpu").to(torch().float64).numpy()


def bits(x):
    """bf16 torch tensor -> numpy uint16 bit patterns."""
    t = torch()
    return x.detach().to("cpu").contiguous().view(t.int16).numpy().view(np.uint16)


def rel_fro(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()
