"""Helpers shared by the GPU parity tests: device transfer and comparisons."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def dev(x: np.ndarray):
    """numpy -> torch on cuda:0; uint16 arrays become bfloat16 (same bits)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(x).to("cuda")


def host(t) -> np.ndarray:
    """torch (cuda) -> numpy; bfloat16 becomes uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def zeros(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def poisoned(shape, dtype):
    """An output buffer pre-filled with an unlikely value, so unwritten
    entries show up."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if dtype in (torch.int32, torch.int64, torch.uint8, torch.int16):
        t.fill_(-7 if dtype != torch.uint8 else 77)
    else:
        t.fill_(float("nan"))
    return t


def workspace(nbytes: int):
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")


def normwise(g, o) -> float:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))


def assert_close(g, o, tol=2e-2, what=""):
    g = np.asarray(g, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = normwise(g, o)
    assert err <= tol, f"{what}: normwise error {err:.3e} > {tol}"
    return err
