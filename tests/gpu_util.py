"""Helpers shared by the GPU parity tests: host/device conversions and the
tolerance checks stated by the method's acceptance bar."""
import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev_u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).cuda()


def to_dev_u64(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint64).view(np.int64)).cuda()


def to_dev_vals(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if bf16:  # a holds bf16 bit patterns (uint16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def host_u64(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a float32 / bfloat16 tensor."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def assert_sum_close(got: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray, rel: float, what: str):
    """|got - exact| <= rel * sum|x_i| + 1e-30, element by element."""
    got = np.asarray(got, dtype=np.float64)
    bound = rel * np.asarray(abs_sum, dtype=np.float64) + 1e-30
    err = np.abs(got - exact)
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, "%s: %d elements out of tolerance, first at %d: got %r exact %r bound %r" % (
        what, bad.size, bad[0], got.flat[bad[0]], exact.flat[bad[0]], bound.flat[bad[0]])
