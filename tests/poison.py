"""NaN-filled device buffers for the GPU tests.

The header promises that a decode or prefill workspace needs no
initialisation.  A split partial that a kernel forgets to write would read
back as zeros from a zero-filled workspace, and the log-sum-exp combine would
weigh those zeros away; read back from a NaN-filled one it poisons the
combined output, which the parity check then catches.  The output tensors
get the same treatment, so a row or head that no kernel writes shows up too
(the uninitialised-rescale hazard that the SharpInference PR #434 review
comment names is this class of bug).
"""
import torch

NAN = float("nan")


def nan_bytes(nbytes: int, device="cuda:0") -> torch.Tensor:
    """A 16-byte-aligned uint8 device buffer of at least nbytes, every fp32
    word of it a quiet NaN."""
    f = torch.full(((max(nbytes, 16) + 15) // 16 * 4,), NAN, dtype=torch.float32, device=device)
    return f.view(torch.uint8)


def nan_like(t: torch.Tensor) -> torch.Tensor:
    return torch.full_like(t, NAN)
