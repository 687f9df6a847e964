"""The E4M3 encoding rule written as decision boundaries, for scanning every
binary32 bit pattern on the GPU with torch.

The boundaries are the midpoints between consecutive positive finite E4M3
values as the oracle decodes them; a magnitude takes the code that counts the
midpoints strictly below it, the even code at an exact midpoint, 0x7E above
the last one (saturation, infinities included); NaN gives 0x7F; the sign bit
is kept.  A CPU test checks this rule against the oracle's encoder.
"""

import numpy as np

from oracle import e4m3


def decision_midpoints():
    """Midpoints between consecutive positive finite E4M3 values (0x00 .. 0x7E)."""
    d = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    return ((d[:-1] + d[1:]) / 2.0).astype(np.float32)      # exact: <= 5 significant bits


def expected_codes_torch(torch, bits, mids):
    """Codes (int64 tensor) of int32 bit patterns `bits` under the rule above."""
    v = bits.view(torch.float32)
    a = v.abs()
    i = torch.bucketize(a, mids)
    tie = (i < mids.numel()) & (a == mids[i.clamp(max=mids.numel() - 1)])
    code = i + (tie & (i % 2 == 1)).to(i.dtype)
    code = torch.where(torch.isnan(v), torch.full_like(code, 0x7F), code)
    return code | ((bits < 0).to(code.dtype) << 7)
