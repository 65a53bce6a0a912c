"""Helpers for the GPU tests: numpy storage arrays <-> torch device tensors,
and error summaries. Conversions move bits only."""
import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}   # max |err| gates for attention outputs


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bit patterns of a storage array (for bit-exact comparisons)."""
    a = np.ascontiguousarray(a)
    return a.view({2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def max_err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    return float(np.max(np.abs(gpu.detach().cpu().numpy().astype(np.float64) - ref)))


def say(*msg):
    print(*msg, flush=True)
