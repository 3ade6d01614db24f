"""Pins of the 4-bit block-32 KV cache functions of the oracle.

The pages list a 4-bit (Q4_0) KV cache type without defining it ("Lucebox
Hub", sections "Paged attention + continuous batching" and "설치·사용법");
the oracle's reading is one fp16 scale d = fp16(amax / 7) per block of 32,
codes rint(x / d) clamped to [-7, 7] and stored as nibbles q = code + 8,
value d * (q - 8).  Each pin checks a property that reading fixes, in exact
(Fraction) arithmetic where it matters; ``test_each_q4_mutant_is_caught``
plants plausible slips in a copy of the oracle's code and checks that a pin
fails for each.
"""
import inspect
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.reference as ref


def _f16(v):
    return np.asarray(v, np.float16).view(np.uint16)


def pin_zero_block(qf):
    """An all-zero block has scale 0 and nibbles 8 (value 0)."""
    x = np.zeros((2, 64))
    x[1, 32:] = np.linspace(-3, 3, 32)
    q, d = qf(x)
    return bool(np.all(q[0] == 8) and np.all(d[0] == 0) and d[1, 0] == 0 and np.all(q[1, :32] == 8))


def pin_exact_grid_round_trips(qf):
    """Blocks of k * 2^e with integers |k| <= 7 and max |k| = 7 have
    amax / 7 = 2^e, an fp16 value, so the nibbles are k + 8 and the round
    trip is exact."""
    rng = np.random.default_rng(3)
    ok = True
    for e in (-8, -3, 0, 2):
        k = rng.integers(-7, 8, (4, 64))
        k[:, 0] = 7
        k[:, 32] = -7
        x = k * 2.0 ** e
        q, d = qf(x)
        ok &= np.array_equal(q.astype(np.int64), k + 8) and np.all(oracle.f16_to_f64(d) == 2.0 ** e)
        ok &= np.array_equal(oracle.dequantize_q4_blocks(q, d), x)
    return bool(ok)


def pin_scale_is_nearest_fp16(qf):
    """d is within half an fp16 ulp of amax / 7 (exact arithmetic)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((50, 32)) * 3).astype(np.float32).astype(np.float64)
    q, d = qf(x)
    for r in range(50):
        amax = Fraction(float(np.max(np.abs(x[r]))))
        dv = Fraction(float(oracle.f16_to_f64(d[r, 0])))
        _, e = np.frexp(float(dv))
        ulp = Fraction(2) ** (int(e) - 11)
        if abs(dv - amax / 7) > ulp / 2:
            return False
    return True


def pin_codes_nearest_ties_even_clamped(qf):
    """Each code is the integer nearest x / d (exact), ties to even, clamped
    to [-7, 7]; a block with exact half-way values exercises the ties."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((40, 32)) * 2).astype(np.float32).astype(np.float64)
    x[0] = 0.0
    x[0, 0] = 7.0
    x[0, 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5, -6.5]
    q, d = qf(x)
    for r in range(40):
        dv = Fraction(float(oracle.f16_to_f64(d[r, 0])))
        for j in range(32):
            t = Fraction(float(x[r, j])) / dv
            lo = t.numerator // t.denominator
            frac = t - lo
            want = lo + 1 if (frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1)) else lo
            want = max(-7, min(7, want))
            if int(q[r, j]) - 8 != want:
                return False
    return True


def pin_clamp_at_7(qf):
    """When fp16 rounds amax / 7 down far enough that amax / d exceeds 7.5,
    the code clamps at 7: a subnormal scale of a block of tiny values."""
    a = None
    for bits in range(0x3300, 0x3900):  # bf16 2^-25 .. 2^-13
        c = float(np.array([bits << 16], np.uint32).view(np.float32)[0])
        dv = float((np.float32(c) / np.float32(7.0)).astype(np.float16))
        if dv > 0 and c / dv > 7.5:
            a = c
            break
    assert a is not None
    x = np.zeros((1, 32))
    x[0, 0] = a
    x[0, 1] = -a
    q, d = qf(x)
    return int(q[0, 0]) == 15 and int(q[0, 1]) == 1


def pin_dequant_exact_integer_dot():
    """(q - 8) times power-of-two scales give dot products exact in fp64."""
    rng = np.random.default_rng(9)
    q = rng.integers(0, 16, (3, 96)).astype(np.uint8)
    e = rng.integers(-12, -2, (3, 3))
    d = _f16(np.ldexp(1.0, e))
    w = rng.integers(-50, 50, 96)
    got = oracle.dequantize_q4_blocks(q, d) @ w
    for r in range(3):
        tot = Fraction(0)
        for b in range(3):
            s = sum((int(q[r, j]) - 8) * int(w[j]) for j in range(32 * b, 32 * b + 32))
            tot += s * Fraction(2) ** int(e[r, b])
        if got[r] != float(tot):
            return False
    return True


def pin_cache_orientation(kv_fn=None):
    """Keys are blocked along the head dim of a token, values along the tokens
    of a dim: nibbles carrying their own indices with unit scales read back as
    K[g, t, j] = nib(g, t, j) - 8 and V[g, t, j] = nib(g, j, t) - 8 (times
    the block's scale)."""
    kv_fn = kv_fn or oracle.kv_prefix_from_q4
    Hkv, cap, d, P = 2, 64, 32, 40
    kq = np.zeros((Hkv, cap, d), np.uint8)
    vq = np.zeros((Hkv, d, cap), np.uint8)
    for g in range(Hkv):
        for t in range(cap):
            for j in range(d):
                kq[g, t, j] = (g * 7 + t * 3 + j) % 16
                vq[g, j, t] = (g * 5 + t * 5 + j * 7) % 16
    ks = _f16(np.ones((Hkv, cap, 1)))
    vs = _f16(np.array([1.0, 2.0]).reshape(1, 1, 2) * np.ones((Hkv, d, 2)))
    k, v = kv_fn(kq, ks, vq, vs, P)
    if k.shape != (Hkv, P, d) or v.shape != (Hkv, P, d):
        return False
    for g in range(Hkv):
        for t in range(P):
            for j in range(d):
                if k[g, t, j] != int(kq[g, t, j]) - 8:
                    return False
                if v[g, t, j] != (int(vq[g, j, t]) - 8) * (1.0 if t < 32 else 2.0):
                    return False
    return True


QUANT_PINS = [pin_zero_block, pin_exact_grid_round_trips, pin_scale_is_nearest_fp16,
              pin_codes_nearest_ties_even_clamped, pin_clamp_at_7]


@pytest.mark.parametrize("pin", QUANT_PINS, ids=[p.__name__ for p in QUANT_PINS])
def test_quantiser_pin(pin):
    assert pin(oracle.quantize_q4_blocks)


def test_dequant_exact_integer_dot():
    assert pin_dequant_exact_integer_dot()


def test_cache_orientation():
    assert pin_cache_orientation()


def test_round_trip_error_within_half_a_step():
    # |d (q - 8) - x| <= d / 2 for every value (the clamped value is amax
    # itself, within half a step of 7 d)
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((200, 128)) * rng.uniform(0.01, 100, (200, 1))).astype(np.float32).astype(np.float64)
    q, d = oracle.quantize_q4_blocks(x)
    y = oracle.dequantize_q4_blocks(q, d)
    step = np.repeat(oracle.f16_to_f64(d), 32, axis=-1)
    assert np.all(np.abs(y - x) <= step / 2 * (1 + 1e-12) + 1e-300)


Q4_MUTANTS = [
    ("scale amax / 8", "quantize_q4_blocks", "amax / np.float32(7.0)", "amax / np.float32(8.0)"),
    ("clamp at -8", "quantize_q4_blocks", "np.clip(q, -7, 7)", "np.clip(q, -8, 7)"),
    ("truncation instead of rint", "quantize_q4_blocks",
     "np.rint(xb / np.where(dw > 0, dw, np.float32(1.0)))", "np.trunc(xb / np.where(dw > 0, dw, np.float32(1.0)))"),
    ("offset 7 instead of 8", "quantize_q4_blocks", "np.clip(q, -7, 7) + 8", "np.clip(q, -7, 7) + 7"),
    ("scale kept in fp32", "quantize_q4_blocks", ".astype(np.float32).astype(np.float16)", ".astype(np.float32)"),
    ("dequantiser offset 7", "dequantize_q4_blocks", "dtype=np.int64) - 8", "dtype=np.int64) - 7"),
    ("values blocked along the head dim", "kv_prefix_from_q4",
     "v = dequantize_q4_blocks(v_nibbles, v_scales)[:, :, :prefix_len].transpose(0, 2, 1)",
     "v = dequantize_q4_blocks(v_nibbles.transpose(0, 2, 1), v_scales.transpose(0, 2, 1))[:, :prefix_len, :]"),
]


def _mutant(fn_name, old, new):
    src = inspect.getsource(getattr(ref, fn_name))
    assert src.count(old) == 1, "mutation site not found once: %r" % old
    ns = dict(vars(ref))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[fn_name]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name,fn_name,old,new", Q4_MUTANTS, ids=[m[0] for m in Q4_MUTANTS])
def test_each_q4_mutant_is_caught(name, fn_name, old, new):
    mut = _mutant(fn_name, old, new)
    caught = []
    if fn_name == "quantize_q4_blocks":
        for p in QUANT_PINS:
            try:
                if not p(mut):
                    caught.append(p.__name__)
            except Exception:
                caught.append(p.__name__)
    elif fn_name == "dequantize_q4_blocks":
        ns = dict(vars(ref))
        ns["dequantize_q4_blocks"] = mut
        src = inspect.getsource(ref.kv_prefix_from_q4)
        exec(compile(src, "<mutant>", "exec"), ns)
        saved = oracle.dequantize_q4_blocks
        try:
            oracle.dequantize_q4_blocks = mut
            if not pin_dequant_exact_integer_dot() or not pin_cache_orientation(ns["kv_prefix_from_q4"]):
                caught.append("dequant pins")
        finally:
            oracle.dequantize_q4_blocks = saved
    else:
        try:
            if not pin_cache_orientation(mut):
                caught.append("pin_cache_orientation")
        except Exception:
            caught.append("pin_cache_orientation")
    assert caught, "no pin catches the mutant: %s" % name
