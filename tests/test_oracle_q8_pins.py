"""Pins of the int8 block-32 KV cache functions of the oracle.

The pages list an int8 (q8_0) KV cache type without defining it ("Lucebox
Hub", sections "Paged attention + continuous batching" and "설치·사용법"); the
oracle's reading is one fp16 scale d = fp16(amax / 127) per block of 32 and
codes rint(x / d) clamped to [-127, 127].  Each pin below checks a property
that reading fixes, in exact (Fraction) arithmetic where it matters, and
``test_each_q8_mutant_is_caught`` plants plausible slips in a copy of the
oracle's code and checks that a pin fails for each.
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
    """An all-zero block has scale 0 and codes 0 (no division by zero)."""
    x = np.zeros((2, 64))
    x[1, 32:] = np.linspace(-3, 3, 32)
    c, d = qf(x)
    ok = np.all(c[0] == 0) and np.all(d[0] == 0) and d[1, 0] == 0 and np.all(c[1, :32] == 0)
    return bool(ok)


def pin_exact_grid_round_trips(qf):
    """Blocks of k * 2^e with integers |k| <= 127 and max |k| = 127 have
    amax / 127 = 2^e, an fp16 value, so the codes are k and the round trip
    is exact."""
    rng = np.random.default_rng(3)
    ok = True
    for e in (-8, -3, 0, 2):
        k = rng.integers(-127, 128, (4, 64))
        k[:, 0] = 127
        k[:, 32] = -127
        x = k * 2.0 ** e
        c, d = qf(x)
        ok &= np.array_equal(c.astype(np.int64), k) and np.all(oracle.f16_to_f64(d) == 2.0 ** e)
        ok &= np.array_equal(oracle.dequantize_q8_blocks(c, d), x)
    return bool(ok)


def pin_scale_is_nearest_fp16(qf):
    """d is within half an fp16 ulp of amax / 127 (exact arithmetic)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((50, 32)) * 3).astype(np.float32).astype(np.float64)
    c, d = qf(x)
    for r in range(50):
        amax = Fraction(float(np.max(np.abs(x[r]))))
        dv = Fraction(float(oracle.f16_to_f64(d[r, 0])))
        m, e = np.frexp(float(dv))
        ulp = Fraction(2) ** (int(e) - 11)  # fp16: 11 significant bits
        if abs(dv - amax / 127) > ulp / 2:
            return False
    return True


def pin_codes_nearest_ties_even_clamped(qf):
    """Each code is the integer nearest x / d (exact), ties to even, clamped
    to [-127, 127]; blocks with an exact half-way value exercise the ties."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((40, 32)) * 2).astype(np.float32).astype(np.float64)
    # half-way values: d = 1 (amax 127), entries m + 1/2
    x[0] = 0.0
    x[0, 0] = 127.0
    x[0, 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 100.5, -126.5]
    c, d = qf(x)
    for r in range(40):
        dv = Fraction(float(oracle.f16_to_f64(d[r, 0])))
        for j in range(32):
            t = Fraction(float(x[r, j])) / dv
            lo = t.numerator // t.denominator
            frac = t - lo
            if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
                want = lo + 1
            else:
                want = lo
            want = max(-127, min(127, want))
            if int(c[r, j]) != want:
                return False
    return True


def pin_clamp_at_127(qf):
    """When fp16 rounds amax / 127 down far enough, amax / d exceeds 127.5 and
    the code is clamped: a block holding such an amax gets code 127 there.
    (Normal fp16 scales are within 2^-11 of amax / 127, so this needs a
    subnormal scale: a block of tiny values.)"""
    found = False
    for a in np.geomspace(1e-6, 1e-4, 4001):
        a = float(np.float32(a))
        dv = float(np.float16(np.float32(a) / np.float32(127.0)))
        if dv > 0 and a / dv > 127.5:
            found = True
            break
    assert found
    x = np.zeros((1, 32))
    x[0, 0] = a
    x[0, 1] = -a
    c, d = qf(x)
    return int(c[0, 0]) == 127 and int(c[0, 1]) == -127


def pin_dequant_exact_integer_dot():
    """Codes times power-of-two scales give dot products exact in fp64."""
    rng = np.random.default_rng(9)
    c = rng.integers(-127, 128, (3, 96)).astype(np.int8)
    e = rng.integers(-12, -2, (3, 3))
    d = _f16(np.ldexp(1.0, e))
    w = rng.integers(-50, 50, 96)
    got = oracle.dequantize_q8_blocks(c, d) @ w
    for r in range(3):
        tot = Fraction(0)
        for b in range(3):
            s = sum(int(c[r, j]) * int(w[j]) for j in range(32 * b, 32 * b + 32))
            tot += s * Fraction(2) ** int(e[r, b])
        if got[r] != float(tot):
            return False
    return True


def pin_cache_orientation(kv_fn=None):
    """Keys are blocked along the head dim of a token, values along the tokens
    of a dim: codes carrying their own indices with unit scales read back as
    K[g, t, j] = code(g, t, j) and V[g, t, j] = code(g, j, t)."""
    kv_fn = kv_fn or oracle.kv_prefix_from_q8
    Hkv, cap, d, P = 2, 64, 32, 40
    kc = np.zeros((Hkv, cap, d), np.int8)
    vc = np.zeros((Hkv, d, cap), np.int8)
    for g in range(Hkv):
        for t in range(cap):
            for j in range(d):
                kc[g, t, j] = (g * 37 + t * 3 + j) % 255 - 127
                vc[g, j, t] = (g * 11 + t * 5 + j * 7) % 255 - 127
    # one scale per (g, t) for K (d = 32: one block) and per (g, j, 32 tokens) for V
    ks = _f16(np.ones((Hkv, cap, 1)))
    vs = _f16(np.array([1.0, 2.0]).reshape(1, 1, 2) * np.ones((Hkv, d, 2)))
    k, v = kv_fn(kc, ks, vc, vs, P)
    if k.shape != (Hkv, P, d) or v.shape != (Hkv, P, d):
        return False
    for g in range(Hkv):
        for t in range(P):
            for j in range(d):
                if k[g, t, j] != kc[g, t, j]:
                    return False
                if v[g, t, j] != vc[g, j, t] * (1.0 if t < 32 else 2.0):
                    return False
    return True


QUANT_PINS = [pin_zero_block, pin_exact_grid_round_trips, pin_scale_is_nearest_fp16,
              pin_codes_nearest_ties_even_clamped, pin_clamp_at_127]


@pytest.mark.parametrize("pin", QUANT_PINS, ids=[p.__name__ for p in QUANT_PINS])
def test_quantiser_pin(pin):
    assert pin(oracle.quantize_q8_blocks)


def test_dequant_exact_integer_dot():
    assert pin_dequant_exact_integer_dot()


def test_cache_orientation():
    assert pin_cache_orientation()


def test_round_trip_error_within_half_a_step():
    # |d c - x| <= d / 2 for every value (clamping never adds error: the
    # clamped value is amax itself, within half a step of 127 d)
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((200, 128)) * rng.uniform(0.01, 100, (200, 1))).astype(np.float32).astype(np.float64)
    c, d = oracle.quantize_q8_blocks(x)
    y = oracle.dequantize_q8_blocks(c, d)
    step = np.repeat(oracle.f16_to_f64(d), 32, axis=-1)
    assert np.all(np.abs(y - x) <= step / 2 * (1 + 1e-12) + 1e-300)


Q8_MUTANTS = [
    ("scale amax / 128", "quantize_q8_blocks", "amax / np.float32(127.0)", "amax / np.float32(128.0)"),
    ("no clamp", "quantize_q8_blocks", "np.clip(q, -127, 127)", "np.clip(q, -128, 127)"),
    ("truncation instead of rint", "quantize_q8_blocks",
     "np.rint(xb / np.where(dw > 0, dw, np.float32(1.0)))", "np.trunc(xb / np.where(dw > 0, dw, np.float32(1.0)))"),
    ("ties away from zero", "quantize_q8_blocks",
     "np.rint(xb / np.where(dw > 0, dw, np.float32(1.0)))",
     "np.sign(xb) * np.floor(np.abs(xb / np.where(dw > 0, dw, np.float32(1.0))) + np.float32(0.5))"),
    ("scale kept in fp32", "quantize_q8_blocks", ".astype(np.float32).astype(np.float16)", ".astype(np.float32)"),
    ("values blocked along the head dim", "kv_prefix_from_q8",
     "v = dequantize_q8_blocks(v_codes, v_scales)[:, :, :prefix_len].transpose(0, 2, 1)",
     "v = dequantize_q8_blocks(v_codes.transpose(0, 2, 1), v_scales.transpose(0, 2, 1))[:, :prefix_len, :]"),
]


def _mutant(fn_name, old, new):
    src = inspect.getsource(getattr(ref, fn_name))
    assert src.count(old) == 1, "mutation site not found once: %r" % old
    ns = dict(vars(ref))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[fn_name]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name,fn_name,old,new", Q8_MUTANTS, ids=[m[0] for m in Q8_MUTANTS])
def test_each_q8_mutant_is_caught(name, fn_name, old, new):
    mut = _mutant(fn_name, old, new)
    if fn_name == "quantize_q8_blocks":
        caught = []
        for p in QUANT_PINS:
            try:
                if not p(mut):
                    caught.append(p.__name__)
            except Exception:  # a mutant that breaks the function is caught too
                caught.append(p.__name__)
    else:
        try:
            caught = [] if pin_cache_orientation(mut) else ["pin_cache_orientation"]
        except Exception:
            caught = ["pin_cache_orientation"]
    assert caught, "no pin catches the mutant: %s" % name
