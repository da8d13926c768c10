"""Helpers shared by the GPU tests (no arithmetic of the method)."""
import numpy as np
import torch

PYTEST_CONFIG = None  # set by conftest.py


def progress(msg: str) -> None:
    """A progress line of a long test, shown even when pytest captures output
    (so that a minutes-long oracle run is not silent)."""
    capman = PYTEST_CONFIG.pluginmanager.getplugin("capturemanager") if PYTEST_CONFIG else None
    if capman is None:
        print(msg, flush=True)
        return
    with capman.global_and_fixture_disabled():
        print(msg, flush=True)


def dev():
    return torch.device("cuda:0")


def bf16_dev(x: np.ndarray) -> torch.Tensor:
    """numpy fp32 -> bf16 device tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(dev())


def f32_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """The value a bf16 tensor holds, as float64."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .float().numpy().astype(np.float64)


def rel_max(a: np.ndarray, b: np.ndarray) -> float:
    """max |a - b| / max |b|."""
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-30))
