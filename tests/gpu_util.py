"""Helpers shared by the GPU parity tests."""
import numpy as np
import pytest

TOL = 1e-3   # normwise bar on f32 hidden states and logits: ||gpu - oracle||_inf / ||oracle||_inf


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def np_of(t):
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32) if False else t.numpy()
    return t.numpy()


def announce(msg):
    print(f"[case] {msg}", flush=True)
