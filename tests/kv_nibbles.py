"""The device layout of a 4-bit KV block: 32 nibbles in 16 bytes, as four
little-endian dwords of 8 values each, value e (0..7) of a dword at bits
4 (e // 2) + 16 (e % 2).  The oracle keeps one nibble per array entry; these
two functions move between that form and the packed bytes the library reads
and writes (layout only: no arithmetic of the method)."""
import numpy as np

SHIFTS = np.array([4 * (e >> 1) + 16 * (e & 1) for e in range(8)], np.uint32)


def pack(nibbles):
    """uint8 nibbles [..., L] (L a multiple of 8, values 0..15) -> bytes [..., L / 2]."""
    q = np.asarray(nibbles)
    assert q.shape[-1] % 8 == 0 and q.max(initial=0) < 16
    g = q.astype(np.uint32).reshape(q.shape[:-1] + (q.shape[-1] // 8, 8))
    w = np.bitwise_or.reduce(g << SHIFTS, axis=-1).astype("<u4")
    return np.ascontiguousarray(w).view(np.uint8).reshape(q.shape[:-1] + (q.shape[-1] // 2,))


def unpack(packed):
    """bytes [..., L / 2] -> uint8 nibbles [..., L]."""
    b = np.ascontiguousarray(np.asarray(packed, np.uint8))
    assert b.shape[-1] % 4 == 0
    w = b.view("<u4").reshape(b.shape[:-1] + (b.shape[-1] // 4, 1))
    q = (w >> SHIFTS) & 0xF
    return q.astype(np.uint8).reshape(b.shape[:-1] + (b.shape[-1] * 2,))
