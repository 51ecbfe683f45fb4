"""Device storage of test operands with padded rows and offset bases."""
import numpy as np
import torch


def stored_device(values, trans, pad, offset):
    """Device storage of a logical operand: itself or its transpose, rows
    padded by `pad` floats (NaN), the whole block starting `offset` floats
    into its allocation.  Returns (keep-alive tensor, logical view, ld)."""
    S = np.ascontiguousarray(values.T) if trans else values
    rows, cols = S.shape
    ld = cols + pad
    flat = torch.full((offset + rows * ld + 4,), float("nan"), device="cuda")
    blk = flat[offset:offset + rows * ld].view(rows, ld)
    blk[:, :cols] = torch.from_numpy(S).cuda()
    view = blk[:, :cols]
    return flat, (view.t() if trans else view), ld
