"""Host <-> device plumbing for the GPU tests (torch only moves memory)."""
import numpy as np
import torch

F32, BF16 = 0, 1
TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def to_dev(a, dtype, misalign=False):
    """Host array (float32, or uint16 bf16 patterns) -> device tensor.
    misalign=True places it one element past a 16-byte boundary."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype == BF16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    if misalign:
        buf = torch.empty(t.numel() + 8, dtype=t.dtype, device="cuda")
        v = buf[1:1 + t.numel()].view(t.shape)
        v.copy_(t.cuda())
        return v
    return t.cuda()


def from_dev(t, dtype):
    """Device tensor -> host array in the generator's storage format."""
    if dtype == BF16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def f64(t):
    """Exact float64 values of a device tensor (fp32 or bf16)."""
    return t.detach().float().cpu().numpy().astype(np.float64)
