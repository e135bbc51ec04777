"""Helpers for GPU tests: numpy <-> torch device copies that keep bit patterns."""
import numpy as np
import torch

DEV = torch.device("cuda:0")

_VIEW = {
    np.dtype(np.uint8): (np.uint8, torch.uint8),
    np.dtype(np.int8): (np.int8, torch.int8),
    np.dtype(np.uint16): (np.int16, torch.int16),
    np.dtype(np.int16): (np.int16, torch.int16),
    np.dtype(np.uint32): (np.int32, torch.int32),
    np.dtype(np.int32): (np.int32, torch.int32),
    np.dtype(np.uint64): (np.int64, torch.int64),
    np.dtype(np.float32): (np.float32, torch.float32),
}


def to_dev(a) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    npv, _ = _VIEW[a.dtype]
    return torch.from_numpy(a.view(npv).copy()).to(DEV)


def empty(shape, np_dtype) -> torch.Tensor:
    _, tdt = _VIEW[np.dtype(np_dtype)]
    return torch.empty(shape, dtype=tdt, device=DEV)


def to_host(t: torch.Tensor, np_dtype) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np_dtype)
