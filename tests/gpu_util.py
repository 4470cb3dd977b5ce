"""Helpers for the GPU parity tests: device placement, canaries and the error metric."""
import numpy as np
import torch

import oracle as O
import tp_inputs as I

BF16_TOL = 1e-2   # max|err| / max|y_ref| for bf16 outputs (fp32 accumulation)
F32_TOL = 1e-5    # the fp32 path


def dev(t):
    return None if t is None else t.contiguous().cuda()


def host64(t):
    return I.as_numpy_f64(t)


def err(y_gpu, y_ref):
    return O.rel_err(host64(y_gpu), y_ref)


def canary_buffer(shape, dtype, pad=4096):
    """A device tensor of `shape` followed by `pad` NaN canaries in the same allocation."""
    n = int(np.prod(shape))
    buf = torch.full((n + pad,), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[:n].view(*shape)


def canaries_intact(buf, shape):
    n = int(np.prod(shape))
    return bool(torch.isnan(buf[n:]).all().item())


def log_case(*parts):
    """Name the case before a GPU step, flushed, so a failure can be traced to it."""
    print("CASE", *parts, flush=True)
