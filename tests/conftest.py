import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def read_golden(name):
    """Parse a `key = value` fixture under tests/golden (repeated keys -> list)."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out.setdefault(key, []).append(val)
    return {k: (v[0] if len(v) == 1 else v) for k, v in out.items()}


def rel_err(got, ref):
    """max |got - ref| / rms(ref) over the whole tensor (the parity metric)."""
    import numpy as np
    if hasattr(got, "detach"):
        got = got.detach().float().cpu().double().numpy()
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.abs(got - ref).max() / rms) if rms > 0 else float(np.abs(got - ref).max())


TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def gpu_device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")
