"""Worker for the exhaustive fp32 -> bf16 pin: the oracle's rounding against
torch's CPU cast on one range of fp32 bit patterns (run in worker processes)."""

import numpy as np


def check_range(start: int, count: int):
    """Returns (mismatches among non-NaN inputs, first mismatching pattern or None,
    NaN inputs whose results are not NaN on either side)."""
    import torch

    from oracle import fsdp_oracle as O

    torch.set_num_threads(1)
    bits = np.arange(start, start + count, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    ours = O.bf16_round_nearest_even(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    bad = (ours != ref) & ~nan
    n_bad = int(np.count_nonzero(bad))
    first = int(bits[np.flatnonzero(bad)[0]]) if n_bad else None
    nan_bad = int(np.count_nonzero(nan & (((ours & 0x7F80) != 0x7F80) | ((ours & 0x7F) == 0)
                                          | ((ref & 0x7F80) != 0x7F80) | ((ref & 0x7F) == 0))))
    return n_bad, first, nan_bad
