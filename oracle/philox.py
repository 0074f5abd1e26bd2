"""Philox4x32-10 counter-based generator (oracle side).

Follows the published definition (Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11): a 4x32-bit counter and a 2x32-bit
key; each of the 10 rounds multiplies counter words 0 and 2 by two fixed odd
constants, mixes the high halves with the other two words and the key, and the
key advances by two Weyl constants between rounds.

The SIP sentence of the AB-Attention abstract asks for random sampling but names
no generator; Philox is the reading (a counter-based stream lets any block's
draw be computed independently, which the GPU needs). Pinned against rocRAND's
implementation in ``tests/test_oracle_philox.py``.
"""

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)
_SH32 = np.uint64(32)


def philox4x32_10(counter, key):
    """Apply Philox4x32-10.

    counter: uint32 array [..., 4]; key: uint32 array [..., 2] (broadcastable).
    Returns uint32 array [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    c0, c1, c2, c3 = (c[..., 0], c[..., 1], c[..., 2], c[..., 3])
    k0 = np.broadcast_to(k[..., 0], c0.shape).astype(np.uint32)
    k1 = np.broadcast_to(k[..., 1], c0.shape).astype(np.uint32)
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd > 0:
                k0 = k0 + _W0
                k1 = k1 + _W1
            p0 = c0.astype(np.uint64) * _M0
            p1 = c2.astype(np.uint64) * _M1
            hi0 = (p0 >> _SH32).astype(np.uint32)
            lo0 = (p0 & _MASK32).astype(np.uint32)
            hi1 = (p1 >> _SH32).astype(np.uint32)
            lo1 = (p1 & _MASK32).astype(np.uint32)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1)
