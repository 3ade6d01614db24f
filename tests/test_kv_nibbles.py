"""The 4-bit KV byte layout the tests hand the library (CPU only)."""
import numpy as np

import kv_nibbles


def test_layout_of_one_dword():
    # values 0..7 of one dword: 1, 2, .., 8 land at bits 0, 16, 4, 20, 8, 24, 12, 28
    q = np.arange(1, 9, dtype=np.uint8)
    b = kv_nibbles.pack(q)
    assert b.tobytes() == bytes([0x31, 0x75, 0x42, 0x86])
    assert int.from_bytes(b.tobytes(), "little") == 0x86427531


def test_roundtrip_and_order():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, (3, 5, 64)).astype(np.uint8)
    b = kv_nibbles.pack(q)
    assert b.shape == (3, 5, 32)
    assert np.array_equal(kv_nibbles.unpack(b), q)
    # a block's 32 values fill exactly its own 16 bytes
    q2 = q.copy()
    q2[1, 2, 32:] = 0
    b2 = kv_nibbles.pack(q2)
    assert np.array_equal(b2[1, 2, :16], b[1, 2, :16]) and not b2[1, 2, 16:].any()
