"""Helpers for the GPU parity tests: host numpy <-> device torch, comparisons."""

import numpy as np
import torch

DEV = "cuda:0"


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    t = torch.from_numpy(a).to(DEV)
    return t if dtype is None else t.to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_values(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_bytes_equal(gpu: np.ndarray, ref: np.ndarray, what: str):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    bad = gpu != ref
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first at "
                             f"{idx.tolist()}: gpu={[gpu[tuple(i)] for i in idx]} "
                             f"ref={[ref[tuple(i)] for i in idx]}")
