"""Device plumbing for the GPU tests: moving seeded bf16 bit patterns to and from
HIP memory and calling the C ABI with guard bands. No arithmetic of the method."""
import numpy as np
import torch


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    """bf16/fp32 device tensor -> float64 numpy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


class Guarded:
    """A device buffer with canary bands on both sides of the region handed to a kernel."""

    PAD = 4096  # bytes on each side

    def __init__(self, nbytes: int, fill: int = 0xA5):
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * self.PAD,), fill, dtype=torch.uint8, device="cuda")
        self.fill = fill

    @property
    def ptr(self) -> int:
        return self.raw.data_ptr() + self.PAD

    def view(self, dtype, shape):
        return self.raw[self.PAD:self.PAD + self.nbytes].view(dtype).view(shape)

    def canaries_intact(self) -> bool:
        r = self.raw.cpu().numpy()
        return bool(np.all(r[:self.PAD] == self.fill) and np.all(r[self.PAD + self.nbytes:] == self.fill))
