"""Host <-> device transfer of raw bit arrays for the GPU tests (no arithmetic)."""
import numpy as np
import pytest
import torch

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32, "int32": torch.int32}
NP_BITS = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32, "int32": np.uint32}
ESIZE = {"bf16": 2, "fp16": 2, "fp32": 4, "int32": 4}


def device():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible (these tests run on an MI355X)")
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    ib = np.int16 if bits.dtype == np.uint16 else np.int32
    return torch.from_numpy(np.ascontiguousarray(bits).view(ib)).to(device()).view(TORCH_DT[dtype])


def to_bits(t: torch.Tensor) -> np.ndarray:
    it = torch.int16 if t.element_size() == 2 else torch.int32
    a = t.detach().contiguous().view(it).cpu().numpy()
    return a.view(np.uint16 if t.element_size() == 2 else np.uint32)


def is_nan_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    b = b.astype(np.uint32)
    if dtype == "bf16":
        return (b & 0x7FFF) > 0x7F80
    if dtype == "fp16":
        return (b & 0x7FFF) > 0x7C00
    return (b & 0x7FFFFFFF) > 0x7F800000


def assert_reduce_equal(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "") -> None:
    """Bit-exact, except that NaN payloads compare by NaN-ness only."""
    assert got.shape == want.shape, (got.shape, want.shape)
    gn, wn = is_nan_bits(got, dtype), is_nan_bits(want, dtype)
    bad_nan = int((gn != wn).sum())
    diff = (got != want) & ~(gn & wn)
    nbad = int(diff.sum())
    if nbad or bad_nan:
        idx = np.flatnonzero(diff | (gn != wn))[:8]
        raise AssertionError(f"{what}: {nbad} mismatches ({bad_nan} NaN-ness); first at {idx.tolist()}: "
                             f"got {[hex(int(got[i])) for i in idx]} want {[hex(int(want[i])) for i in idx]}")
