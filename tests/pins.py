"""Independent checks ("pins") for the CPU oracle.

Each check takes the function under test as an argument so that the same
check can be run against the oracle (it must pass) and against deliberately
broken copies of it (it must fail): see test_oracle.py.  The expectations come
from exact rational arithmetic (fractions.Fraction), brute force over the 16
code levels, closed forms and the hand-derived fixtures in tests/golden/ --
never from the oracle itself and never from the HIP library.
"""

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32_MAX = float(np.finfo(np.float32).max)


class PinFailure(AssertionError):
    pass


def _check(cond, msg):
    if not cond:
        raise PinFailure(msg)


# ----------------------------------------------------------------------------
# exact fp32 helpers (independent of numpy's float32 division)
# ----------------------------------------------------------------------------

def f32_bits(v):
    return int(np.asarray(v, dtype=np.float32).view(np.uint32))


def bits_f32(b):
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def f32_nearest(fr):
    """fp32 value nearest to the rational `fr`, ties to even (exact search)."""
    c = np.float32(float(fr))  # within one fp32 ulp of the answer
    cands = []
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        if np.isfinite(v):
            cands.append(v)
    best = None
    for v in cands:
        dist = abs(Fraction(float(v)) - fr)
        key = (dist, f32_bits(v) & 1)  # ties: even significand first
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def nearest_level(t):
    """Brute force: the code in [-8, 7] nearest to t (a Fraction), ties away from 0."""
    best = None
    for q in range(-8, 8):
        key = (abs(t - q), -abs(q))
        if best is None or key < best[0]:
            best = (key, q)
    return best[1]


# ----------------------------------------------------------------------------
# golden fixtures
# ----------------------------------------------------------------------------

def load_groups(name):
    """Parse a tests/golden/*.txt group fixture -> list of (name, d_bits, w[128], q[128])."""
    groups = []
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "group":
                cur = {"name": tok[1], "d": None,
                       "w": np.zeros(128, dtype=np.uint32), "q": np.zeros(128, dtype=np.int64)}
            elif tok[0] == "d":
                cur["d"] = int(tok[1], 16)
            elif tok[0] == "w":
                i = int(tok[1])
                cur["w"][i] = int(tok[2], 16)
                cur["q"][i] = int(tok[3])
            elif tok[0] == "end":
                groups.append((cur["name"], cur["d"], cur["w"].view(np.float32), cur["q"]))
                cur = None
    return groups


def check_golden(quantize, fixture):
    """Each fixture group, quantized as one 1x128 row, gives exactly the listed d and codes."""
    for name, d_bits, w, q_exp in load_groups(fixture):
        q, d = quantize(w.reshape(1, 128).copy())
        _check(f32_bits(d[0, 0]) == d_bits,
               f"{fixture}:{name}: d bits {f32_bits(d[0, 0]):#010x} != {d_bits:#010x}")
        bad = np.nonzero(np.asarray(q[0], dtype=np.int64) != q_exp)[0]
        _check(bad.size == 0, f"{fixture}:{name}: codes differ at {bad[:8].tolist()}")


# ----------------------------------------------------------------------------
# exact-rational pins of the quantizer
# ----------------------------------------------------------------------------

def toy_weights(seed, N=4, K=256):
    """Small fp32 matrices with mixed magnitudes: normal, tiny, subnormal, large groups."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    G = K // 128
    for n in range(N):
        for g in range(G):
            kind = (n * G + g) % 6
            sl = slice(128 * g, 128 * g + 128)
            if kind == 1:
                W[n, sl] *= np.float32(1e-30)
            elif kind == 2:  # subnormal group
                W[n, sl] = (rng.integers(-4000, 4000, 128) * 2.0 ** -149).astype(np.float32)
            elif kind == 3:  # large group
                W[n, sl] *= np.float32(1e36)
            elif kind == 4:  # values on a coarse grid: many exact ties after division
                W[n, sl] = (rng.integers(-14, 15, 128) * 0.25).astype(np.float32)
    return W


def check_scale_exact(quantize, W):
    """d is the fp32 nearest to max|w| / 7 (exact rationals), and codes are zero when d is."""
    q, d = quantize(W)
    N, K = W.shape
    for n in range(N):
        for g in range(K // 128):
            grp = W[n, 128 * g:128 * g + 128]
            a = max(abs(Fraction(float(v))) for v in grp)
            exp = f32_nearest(a / 7)
            _check(f32_bits(d[n, g]) == f32_bits(exp),
                   f"scale ({n},{g}): got {d[n, g]!r}, nearest fp32 to a/7 is {exp!r}")


def check_codes_bruteforce(quantize, W):
    """Each code is the level in [-8, 7] nearest to fl32(w / d) (ties away from 0)."""
    q, d = quantize(W)
    N, K = W.shape
    for n in range(N):
        for k in range(K):
            dv = d[n, k // 128]
            if dv == 0:
                _check(q[n, k] == 0, f"code ({n},{k}) must be 0 when d == 0")
                continue
            t = f32_nearest(Fraction(float(W[n, k])) / Fraction(float(dv)))
            exp = nearest_level(Fraction(float(t)))
            _check(int(q[n, k]) == exp, f"code ({n},{k}): got {int(q[n, k])}, expected {exp}")


def check_round_trip(quantize, W):
    """|w - d q| <= d (1/2 + 2^-21) for every weight of a group with a normal scale."""
    q, d = quantize(W)
    N, K = W.shape
    dd = np.repeat(d.astype(np.float64), 128, axis=1)
    err = np.abs(W.astype(np.float64) - dd * q.astype(np.float64))
    normal = dd >= float(np.finfo(np.float32).tiny)
    bound = dd * (0.5 + 2.0 ** -21)
    _check(np.all(err[normal] <= bound[normal]), "round-trip bound |w - d q| <= d/2 violated")


def check_invariants(quantize, W):
    """Largest magnitude gets |q| = 7; codes in [-7, 7]; sign(q) in {sign(w), 0} (normal d)."""
    q, d = quantize(W)
    N, K = W.shape
    G = K // 128
    qg = q.reshape(N, G, 128).astype(np.int64)
    Wg = W.reshape(N, G, 128)
    normal = d >= np.finfo(np.float32).tiny
    amax = np.abs(Wg).argmax(axis=2)
    top = np.take_along_axis(qg, amax[:, :, None], axis=2)[:, :, 0]
    _check(np.all(np.abs(top[normal]) == 7), "largest weight of a group must get |q| = 7")
    _check(np.all(np.abs(qg[normal]) <= 7), "codes must lie in [-7, 7] for normal scales")
    s = np.sign(Wg).astype(np.int64)
    ok = (np.sign(qg) == s) | (qg == 0)
    _check(np.all(ok[normal]), "sign(q) must equal sign(w) or be 0")


def check_scale_equivariance(quantize, W, e):
    """quant(2^e W) = same codes and 2^e d, bit for bit (no under/overflow)."""
    q0, d0 = quantize(W)
    W1 = (W.astype(np.float64) * 2.0 ** e).astype(np.float32)
    q1, d1 = quantize(W1)
    _check(np.array_equal(q0, q1), "codes must not change under power-of-two scaling")
    _check(np.array_equal((d0.astype(np.float64) * 2.0 ** e).astype(np.float32).view(np.uint32),
                          d1.view(np.uint32)), "scales must scale exactly")


def check_group_permutation(quantize, W, seed=0):
    """Permuting weights inside a group permutes their codes and keeps the scale."""
    rng = np.random.default_rng(seed)
    q0, d0 = quantize(W)
    N, K = W.shape
    perm = np.concatenate([128 * g + rng.permutation(128) for g in range(K // 128)])
    q1, d1 = quantize(np.ascontiguousarray(W[:, perm]))
    _check(np.array_equal(q1, q0[:, perm]), "codes must follow a within-group permutation")
    _check(np.array_equal(d1.view(np.uint32), d0.view(np.uint32)), "scales must not change")


def check_group_count(quantize):
    """Group 128 along the input direction: a 9216-wide row has 72 groups (study, section 1)."""
    W = np.ones((2, 9216), dtype=np.float32)
    q, d = quantize(W)
    _check(d.shape == (2, 72), f"expected 72 groups per row, got {d.shape}")
    _check(q.shape == (2, 9216), "codes must keep the weight shape")


# ----------------------------------------------------------------------------
# 16-bit (bf16) restore scales
# ----------------------------------------------------------------------------

def bf16_nearest_bits(v32):
    """bf16 bit pattern nearest to the fp32 value v32 (exact rationals, ties to even)."""
    b = f32_bits(v32)
    base = b >> 16
    best = None
    for c in (base - 1, base, base + 1):  # same-sign neighbours around v (toward and away)
        if c < 0 or (c & 0x7F80) == 0x7F80:
            continue
        val = Fraction(float(bits_f32((c & 0xFFFF) << 16)))
        key = (abs(val - Fraction(float(v32))), c & 1)
        if best is None or key < best[0]:
            best = (key, c & 0xFFFF)
    return best[1]


def widened(quantize16):
    """A 16-bit-scale quantizer seen as one returning fp32 scales (the values the codes use)."""
    def quantize(W):
        q, d_bits = quantize16(W)
        return q, (np.asarray(d_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return quantize


def scale16_tie_weights(groups=16, seed=0):
    """Rows of one group each whose fp32 scale fl32(max|w| / 7) lies exactly halfway
    between two bf16 values (half with an even lower neighbour, half odd)."""
    rng = np.random.default_rng(seed)
    rows = []
    while len(rows) < groups:
        base = int(rng.integers(0x3800, 0x4200))
        if (base & 1) != (len(rows) & 1):
            continue
        d32 = bits_f32((base << 16) | 0x8000)
        a = np.float32(np.float64(d32) * 7.0)
        if np.float32(a / np.float32(7.0)) != d32:
            continue
        w = (rng.uniform(-1.0, 1.0, 128) * float(a)).astype(np.float32)
        w[int(rng.integers(0, 128))] = a if rng.random() < 0.5 else -a
        rows.append(w)
    return np.stack(rows)


def check_scale16_exact(quantize16, W):
    """d16 is the bf16 nearest to the fp32 scale fl32(max|w| / 7) (exact rationals)."""
    q, d_bits = quantize16(W)
    N, K = W.shape
    for n in range(N):
        for g in range(K // 128):
            grp = W[n, 128 * g:128 * g + 128]
            a = max(abs(Fraction(float(v))) for v in grp)
            exp = bf16_nearest_bits(f32_nearest(a / 7))
            _check(int(d_bits[n, g]) == exp,
                   f"16-bit scale ({n},{g}): got {int(d_bits[n, g]):#06x}, nearest bf16 is {exp:#06x}")


def check_bf16_narrowing(to_bf16, reference):
    """Narrowing fp32 -> bf16 agrees with a library's round-to-nearest-even conversion on
    random magnitudes, exact ties, the overflow threshold, subnormals and infinities."""
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-85, 85, 20000))).astype(np.float32)
    ties = ((rng.integers(0, 2 ** 31, 4000).astype(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000))
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0xFF7F8000, 0x00008000, 0x00018000, 0x80008000,
                     0x00000001, 0x7F800000, 0xFF800000, 0x00000000, 0x80000000], dtype=np.uint32)
    v = np.concatenate([v, ties.view(np.float32), edge.view(np.float32)])
    v = v[~np.isnan(v)]  # NaN payloads are not specified by round-to-nearest-even
    got = np.asarray(to_bf16(v), dtype=np.uint16)
    exp = np.asarray(reference(v), dtype=np.uint16)
    bad = np.nonzero(got != exp)[0]
    _check(bad.size == 0, f"bf16 narrowing differs at {v[bad[:4]].tolist()}")


# ----------------------------------------------------------------------------
# pins of the linear
# ----------------------------------------------------------------------------

def bf16_values(x_bits):
    return [[float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]) for b in row]
            for row in np.asarray(x_bits, dtype=np.uint16)]


def check_linear_exact(linear, x_bits, q, d):
    """fp64 y against the exact rational sum of x * d * q (4 x 128-class toys)."""
    y, absdot = linear(x_bits, q, d)
    xv = bf16_values(x_bits)
    N, K = q.shape
    for m in range(len(xv)):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                if q[n, k]:
                    acc += Fraction(xv[m][k]) * Fraction(float(d[n, k // 128])) * int(q[n, k])
            tol = 2.0 ** -50 * float(absdot[m, n]) + 1e-300
            _check(abs(Fraction(float(y[m, n])) - acc) <= Fraction(tol),
                   f"y[{m},{n}] = {y[m, n]!r} differs from exact {float(acc)!r}")


def check_linear_closed_forms(linear):
    """All-ones codes with d = 1 give row sums of x; one-hot codes pick columns of x times d."""
    rng = np.random.default_rng(7)
    K, M = 256, 3
    xf = rng.integers(-64, 64, (M, K)).astype(np.float32) * np.float32(0.125)
    x_bits = (xf.view(np.uint32) >> 16).astype(np.uint16)  # exact: few significant bits
    q = np.ones((2, K), dtype=np.int8)
    d = np.ones((2, K // 128), dtype=np.float32)
    y, _ = linear(x_bits, q, d)
    rows = xf.astype(np.float64).sum(axis=1)
    _check(np.array_equal(y[:, 0], rows) and np.array_equal(y[:, 1], rows), "row sums")
    # one-hot codes: row n has q = 1 at column pi(n) (in group pi(n)//128), scale 2^-n
    N = 5
    pi = rng.permutation(K)[:N]
    q = np.zeros((N, K), dtype=np.int8)
    d = np.zeros((N, K // 128), dtype=np.float32)
    for n in range(N):
        q[n, pi[n]] = 1 if n % 2 == 0 else -1
        d[n, pi[n] // 128] = np.float32(2.0 ** -n)
    y, _ = linear(x_bits, q, d)
    for n in range(N):
        sign = 1.0 if n % 2 == 0 else -1.0
        exp = xf[:, pi[n]].astype(np.float64) * 2.0 ** -n * sign
        _check(np.array_equal(y[:, n], exp), f"one-hot column {n}")
    # codes 7 / -8 alternating, d = 0.25, x = 1: y = 0.25 * 64 * (7 - 8) = -16 per 128 group
    q = np.tile(np.array([7, -8], dtype=np.int8), (1, 64))
    d = np.array([[0.25]], dtype=np.float32)
    one = np.full((1, 128), 0x3F80, dtype=np.uint16)
    y, absdot = linear(one, q, d)
    _check(y[0, 0] == -16.0 and absdot[0, 0] == 0.25 * 64 * 15, "alternating 7/-8 closed form")


def check_channel_scaling(quantize, linear, W, x_bits):
    """Channel scaling identity (study, section 2: W'_ij = W_ij s_j, x'_j = x_j / s_j, W'x' = Wx).

    (a) unquantized, general s: fp64 products agree to rounding;
    (b) with s a power of two constant on each 128-group, quantized codes are
        unchanged, scales scale exactly and y is bit-identical.
    """
    rng = np.random.default_rng(11)
    N, K = W.shape
    xv = np.array(bf16_values(x_bits))
    s = rng.uniform(0.25, 4.0, K)
    lhs = xv / s @ (W.astype(np.float64) * s).T
    rhs = xv @ W.astype(np.float64).T
    scale = np.abs(xv) @ np.abs(W.astype(np.float64)).T
    _check(np.all(np.abs(lhs - rhs) <= 1e-14 * scale), "W' x' must equal W x")

    e = rng.integers(-3, 4, K // 128)
    s2 = np.repeat(2.0 ** e, 128)
    q0, d0 = quantize(W)
    q1, d1 = quantize((W.astype(np.float64) * s2).astype(np.float32))
    _check(np.array_equal(q0, q1), "codes must not change under per-group power-of-two scaling")
    _check(np.array_equal((d0.astype(np.float64) * 2.0 ** e).astype(np.float32).view(np.uint32),
                          d1.view(np.uint32)), "per-group scales must scale exactly")
    xs = (xv / s2).astype(np.float32)
    xs_bits = (xs.view(np.uint32) >> 16).astype(np.uint16)
    _check(np.array_equal(((xs_bits.astype(np.uint32) << 16).view(np.float32)).astype(np.float64),
                          xv / s2), "x / s must stay exact in bf16")
    y0, _ = linear(x_bits, q0, d0)
    y1, _ = linear(xs_bits, q1, d1)
    _check(np.array_equal(y0, y1), "y must be bit-identical under paired power-of-two scaling")


# ----------------------------------------------------------------------------
# pins of the canonical packing
# ----------------------------------------------------------------------------

def check_packing(pack, unpack):
    """Byte k/2 holds code k (low nibble) and code k+1 (high nibble), offset by 8."""
    rng = np.random.default_rng(3)
    q = rng.integers(-8, 8, (3, 256)).astype(np.int8)
    b = pack(q)
    _check(b.shape == (3, 128) and b.dtype == np.uint8, "packed shape")
    for n in range(3):
        for j in range(128):
            lo, hi = int(q[n, 2 * j]) + 8, int(q[n, 2 * j + 1]) + 8
            _check(int(b[n, j]) == lo + 16 * hi, f"byte ({n},{j})")
    _check(np.array_equal(unpack(b), q), "unpack(pack(q)) == q")
    every = np.arange(256, dtype=np.uint16).astype(np.uint8).reshape(1, 256)
    _check(np.array_equal(pack(unpack(every)), every), "pack(unpack(b)) == b for all 256 bytes")


def nan_mask_equal(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b))


def is_close_f32(a, b):
    return math.isclose(float(a), float(b), rel_tol=0, abs_tol=0)


# ----------------------------------------------------------------------------
# AWQ channel scaling (study, section 2)
# ----------------------------------------------------------------------------

def awq_outlier_inputs(seed=0, N=96, K=512, T=64, share=0.01, boost=10.0):
    """Weights ~ Student-t, and calibration rows whose few 'salient' input channels are
    `boost` times larger than the rest (the situation channel scaling is for)."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_t(4, size=(N, K)) * 0.01 / np.sqrt(2)).astype(np.float32)
    S = rng.choice(K, max(1, int(round(share * K))), replace=False)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, S] *= np.float32(boost)
    return W, (x.view(np.uint32) >> 16).astype(np.uint16)


def check_awq_grid(alphas):
    """Twenty exponents k/19, k = 0..19 (study, section 2 settings table)."""
    _check(len(alphas) == 20, "the exponent grid has 20 points")
    for k, a in enumerate(alphas):
        _check(Fraction(a).limit_denominator(1000) == Fraction(k, 19), f"alpha[{k}] = {a} is not {k}/19")


def check_awq_scales(candidate_scales, m, alpha):
    """s_j proportional to m_j^alpha with geometric mean 1; inv_s the nearest fp32 to 1/s."""
    s32, inv32 = candidate_scales(m, alpha)
    ls = np.log(s32.astype(np.float64))
    _check(abs(ls.mean()) < 1e-6, "scales must have geometric mean 1")
    lm = np.log(np.maximum(np.asarray(m, dtype=np.float64), 1e-30))
    _check(np.allclose(ls - ls[0], alpha * (lm - lm[0]), atol=1e-6), "scales must follow m^alpha")
    for j in range(0, len(s32), max(1, len(s32) // 16)):
        exp = f32_nearest(1 / Fraction(float(s32[j])))
        _check(f32_bits(inv32[j]) == f32_bits(exp), f"inv_s[{j}] is not the nearest fp32 to 1/s")


def check_awq_activation_scaling(scale_activations, x_bits, inv32):
    """x' is the bf16 nearest to fl32(x * inv_s), element by element (exact rationals)."""
    xs = np.asarray(scale_activations(x_bits, inv32), dtype=np.uint16)
    T, K = x_bits.shape
    for t in range(T):
        for j in range(0, K, 7):
            xv = Fraction(float(bits_f32(int(x_bits[t, j]) << 16)))
            p = f32_nearest(xv * Fraction(float(inv32[j])))
            b = f32_bits(p) >> 16
            lo, hi = Fraction(float(bits_f32(b << 16))), Fraction(float(bits_f32((b + 1) << 16)))
            pv = Fraction(float(p))
            exp = b if (abs(pv - lo), b & 1) < (abs(hi - pv), (b + 1) & 1) else b + 1
            _check(int(xs[t, j]) == exp, f"x'[{t},{j}]: {int(xs[t, j]):#06x} != {exp:#06x}")


def check_awq_error(output_error, quantize_scaled, scale_activations, W, x_bits, s32, inv32):
    """The search objective is the mean squared *output* error of the scaled, quantized
    layer against W x, recomputed here with exact rationals."""
    got = output_error(W, x_bits, s32, inv32)
    q, d = quantize_scaled(W, s32)
    xs = np.asarray(scale_activations(x_bits, inv32), dtype=np.uint16)
    T, K = x_bits.shape
    N = W.shape[0]
    total = Fraction(0)
    for t in range(T):
        xr = [Fraction(float(bits_f32(int(x_bits[t, j]) << 16))) for j in range(K)]
        xq = [Fraction(float(bits_f32(int(xs[t, j]) << 16))) for j in range(K)]
        for n in range(N):
            yq = sum(xq[j] * Fraction(float(d[n, j // 128])) * int(q[n, j]) for j in range(K) if q[n, j])
            y = sum(xr[j] * Fraction(float(W[n, j])) for j in range(K))
            total += (yq - y) ** 2
    exp = float(total / (T * N))
    _check(abs(got - exp) <= 1e-9 * abs(exp) + 1e-300, f"output error {got!r} != exact {exp!r}")


def check_awq_identity(quantize_scaled_unused, W, x_bits, s32):
    """Channel-scaling identity W'x' = Wx (study, section 2) for the fp32-scaled weight and
    the unrounded x / s: equal to fp32 rounding of W * s."""
    Ws = (W * s32[None, :]).astype(np.float32).astype(np.float64)
    x = (np.asarray(x_bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    lhs = (x / s32.astype(np.float64)) @ Ws.T
    rhs = x @ W.astype(np.float64).T
    scale = np.abs(x) @ np.abs(W.astype(np.float64)).T
    _check(np.all(np.abs(lhs - rhs) <= 2.0 ** -22 * scale + 1e-30), "W'x' must equal Wx")


def check_awq_helps_on_salient_channels(search):
    """With a few large input channels on ordinary weights, some alpha > 0 lowers the
    output error clearly below plain RTN (alpha = 0)."""
    W, xb = awq_outlier_inputs(seed=1)
    k, s32, inv32, errors = search(W, xb)
    _check(k > 0 and errors[k] < 0.9 * errors[0], f"expected alpha > 0 to help (k={k}, {errors[k] / errors[0]:.3f})")
    _check(errors[k] == min(errors), "the chosen exponent must have the smallest error")


# ----------------------------------------------------------------------------
# GPTQ (study, section 2: the GPTQ row and settings; update rule of the
# published GPTQ algorithm).  The brute-force reference below re-solves, after
# every column, for the remaining columns that minimise the damped quadratic
# error given the columns fixed so far -- the property the Cholesky-based
# update realises -- with direct linear solves instead of the factor, and
# takes every code and scale decision in exact rationals.
# ----------------------------------------------------------------------------

def gptq_correlated_inputs(seed=0, N=3, K=256, T=64):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((K, K)) * 0.15 + np.eye(K)
    X = (rng.standard_normal((T, K)) @ A).astype(np.float32)
    xb = (X.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16 is fine for inputs
    return W, xb


def gptq_damped_hessian(x_bits, damp=0.01):
    # bf16 -> fp32 by placing the 16 bits in the top half (exact), then fp64
    X = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    H = (2.0 / X.shape[0]) * (X.T @ X)
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    return H


def gptq_bruteforce(W, x_bits, damp=0.01, scale16=False):
    H = gptq_damped_hessian(x_bits, damp)
    N, K = W.shape
    q = np.zeros((N, K), dtype=np.int8)
    d = np.zeros((N, K // 128), dtype=np.float32)
    for n in range(N):
        w0 = W[n].astype(np.float64)
        w = w0.copy()
        what = np.zeros(K)
        for j in range(K):
            if j % 128 == 0:
                a = max(abs(Fraction(float(np.float32(v)))) for v in w[j:j + 128])
                d32 = f32_nearest(a / 7)
                if scale16:  # stored as the nearest bf16, used widened
                    d32 = bits_f32(bf16_nearest_bits(d32) << 16)
                d[n, j // 128] = d32
            dv = d[n, j // 128]
            if dv == 0:
                qj = 0
            else:
                t = f32_nearest(Fraction(float(np.float32(w[j]))) / Fraction(float(dv)))
                qj = nearest_level(Fraction(float(t)))
            q[n, j] = qj
            what[j] = float(dv) * qj
            if j + 1 < K:
                F, R = slice(0, j + 1), slice(j + 1, K)
                w[R] = w0[R] - np.linalg.solve(H[R, R], H[R, F] @ (what[F] - w0[F]))
    return q, d


def check_gptq_bruteforce(gptq, scale16=False):
    """Codes and scales equal the sequential re-solve with exact-rational decisions
    (with 16-bit scales: the scales the codes use, i.e. the stored bf16 widened)."""
    W, xb = gptq_correlated_inputs(seed=3)
    q, d = gptq(W, xb)
    if scale16:
        d = (np.asarray(d, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    qb, db = gptq_bruteforce(W, xb, scale16=scale16)
    _check(np.array_equal(d.view(np.uint32), db.view(np.uint32)), "GPTQ scales differ from the brute-force re-solve")
    bad = np.argwhere(q != qb)
    _check(bad.size == 0, f"GPTQ codes differ from the brute-force re-solve at {bad[:4].tolist()}")


def check_gptq_identity_hessian_is_rtn(gptq):
    """With calibration inputs whose Hessian is a multiple of the identity nothing
    propagates, so GPTQ is RTN: the RTN pins hold for it."""
    K = 256
    xb = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0))  # X = I in bf16
    W = toy_weights(4, N=4, K=K)
    quantize = lambda Wm: gptq(Wm, xb)
    check_scale_exact(quantize, W)
    check_codes_bruteforce(quantize, W)


def check_gptq_block_width(quantize_with_block, factor, hessian):
    """The lazy block width changes only the order of the corrections: 128 and K agree."""
    W, xb = gptq_correlated_inputs(seed=5, N=4, K=512, T=96)
    U = factor(hessian(xb))
    q1, d1 = quantize_with_block(W, U, 128)
    q2, d2 = quantize_with_block(W, U, 512)
    _check(np.array_equal(q1, q2) and np.array_equal(d1, d2), "block width 128 and K must give the same codes")


def check_gptq_beats_rtn(gptq, rtn, output_error):
    """On correlated calibration inputs the column feedback lowers the output error well below RTN."""
    W, xb = gptq_correlated_inputs(seed=7, N=16, K=512, T=256)
    eg = output_error(W, *gptq(W, xb), xb)
    er = output_error(W, *rtn(W), xb)
    _check(eg < 0.6 * er, f"GPTQ error {eg:.3e} should be well below RTN {er:.3e}")


def check_gptq_dead_columns(factor, hessian):
    """A column with all-zero inputs is decoupled: its row and column of U are zero off the diagonal."""
    W, xb = gptq_correlated_inputs(seed=9, N=2, K=256, T=64)
    xb = xb.copy()
    xb[:, 17] = 0
    U = factor(hessian(xb))
    _check(np.isfinite(U).all(), "the factor must exist with a dead column")
    off = np.concatenate([U[17, :17], U[17, 18:], U[:17, 17], U[18:, 17]])
    _check(np.all(off == 0), "a dead column must not couple to the others")


def check_gptq_all_inputs_zero_is_rtn(gptq):
    """With all-zero calibration inputs every column is dead: the factor must still exist,
    nothing couples, and GPTQ is RTN."""
    K = 256
    xb = np.zeros((8, K), dtype=np.uint16)
    W = toy_weights(6, N=3, K=K)
    quantize = lambda Wm: gptq(Wm, xb)
    check_scale_exact(quantize, W)
    check_codes_bruteforce(quantize, W)


def check_gptq16_identity_hessian_is_rtn16(gptq16):
    """With 16-bit scales and an identity Hessian GPTQ is RTN with 16-bit scales: the
    16-bit-scale pins hold for it."""
    K = 256
    xb = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    W = toy_weights(5, N=4, K=K)
    quantize16 = lambda Wm: gptq16(Wm, xb)
    check_scale16_exact(quantize16, W)
    check_codes_bruteforce(widened(quantize16), W)


# ----------------------------------------------------------------------------
# when an output counts as correct (oracle/tolerance.py)
# ----------------------------------------------------------------------------

def _fmt_params(fmt):
    # (bits of significand kept, exponent-field shift into a binary32 pattern)
    return (8, 16) if fmt == "bf16" else (24, 0)


def pattern_value(bits, fmt):
    """Exact value (Fraction) of a finite bf16 / fp32 bit pattern."""
    _, shift = _fmt_params(fmt)
    v = np.array([int(bits) << shift], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(v))


def nearest_pattern(fr, fmt):
    """Bit pattern of the finite value nearest to the rational fr, ties to the even
    pattern (exact search over the patterns next to fr's truncation).  Values at or
    past halfway from the largest finite value to 2^128 give the infinity pattern."""
    _, shift = _fmt_params(fmt)
    sign = 0x8000 if fmt == "bf16" else 0x80000000
    inf = 0x7F80 if fmt == "bf16" else 0x7F800000
    mag = abs(fr)
    top = pattern_value(inf - 1, fmt)
    s = sign if fr < 0 else 0
    if mag >= (top + Fraction(2) ** 128) / 2:
        return s | inf
    t = int(np.array([abs(float(fr))], dtype=np.float32).view(np.uint32)[0]) >> shift  # near fr
    best = None
    for c in range(max(0, t - 2), min(inf - 1, t + 2) + 1):
        key = (abs(pattern_value(c, fmt) - mag), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return s | best[1]


def _ordered(bits, fmt):
    """Bit pattern -> an integer that orders patterns by value (for finite and +-inf)."""
    sign = 0x8000 if fmt == "bf16" else 0x80000000
    return -(bits & (sign - 1)) if bits & sign else bits


def check_admissible(admissible, fmt, seed=0, cases=300):
    """Brute force: the correct outputs for y_ref, tol are exactly the patterns from
    nearest(y_ref - tol) to nearest(y_ref + tol) in value order (rounding is
    monotone), computed with exact rationals; plus NaN and infinity cases."""
    rng = np.random.default_rng(seed)
    dtype = np.uint16 if fmt == "bf16" else np.uint32
    p, _ = _fmt_params(fmt)
    for _ in range(cases):
        # |y_ref| in [2^(e-1), 2^e), with e large enough that the absolute term
        # (1e-6) stays below a step of the format there
        e = int(rng.integers(-10 if fmt == "bf16" else 5, 40))
        y_ref = float(rng.choice([-1.0, 1.0]) * rng.uniform(0.5, 1.0)) * 2.0 ** e
        # tolerances from a fraction of one step of the format to a few dozen steps
        step = 2.0 ** (e - p + 1)
        absdot = abs(float(rng.uniform(0, 1))) * step * float(rng.choice([0.01, 0.3, 1.0, 8.0, 40.0])) / 2e-3
        tol = 2e-3 * absdot + 1e-6
        lo_b = nearest_pattern(Fraction(y_ref) - Fraction(tol), fmt)
        hi_b = nearest_pattern(Fraction(y_ref) + Fraction(tol), fmt)
        lo, hi = _ordered(lo_b, fmt), _ordered(hi_b, fmt)
        assert hi - lo < 4096, "test case spans too many patterns"
        cands = []
        for o in range(lo - 3, hi + 4):
            b = o if o >= 0 else (-o) | (0x8000 if fmt == "bf16" else 0x80000000)
            cands.append((b, lo <= o <= hi))
        bits = np.array([c[0] for c in cands], dtype=dtype)
        got = admissible(bits, np.full(len(cands), y_ref), np.full(len(cands), absdot), fmt)
        want = np.array([c[1] for c in cands])
        _check(np.array_equal(got, want),
               f"{fmt}: y_ref={y_ref!r} tol={tol!r}: admissible set differs at "
               f"{[hex(int(b)) for b, g, w in zip(bits, got, want) if g != w][:4]}")
    # NaN exactly where the reference is NaN; infinities only past the halfway point
    inf = 0x7F80 if fmt == "bf16" else 0x7F800000
    nan = 0x7FC0 if fmt == "bf16" else 0x7FC00000
    top = float(pattern_value(inf - 1, fmt))
    half = (top + 2.0 ** 128) / 2
    bits = np.array([nan, nan, inf, inf, inf - 1, inf | (0x8000 if fmt == "bf16" else 0x80000000)], dtype=dtype)
    y_ref = np.array([np.nan, 1.0, half * (1 + 1e-9), top, top, -half * (1 + 1e-9)])
    got = admissible(bits, y_ref, np.zeros(6), fmt)
    _check(list(got) == [True, False, True, False, True, True], f"{fmt}: special values {list(got)}")


def check_exact_rounding_is_admissible(admissible, seed=0):
    """A bf16 output that is the exactly rounded y_ref is correct even where the
    bound is tighter than half a bf16 step (|y| close to sum |w_hat x|)."""
    rng = np.random.default_rng(seed)
    y_ref = rng.uniform(0.5, 4.0, 200).astype(np.float32).astype(np.float64)
    bits = np.array([nearest_pattern(Fraction(float(v)), "bf16") for v in y_ref], dtype=np.uint16)
    got = admissible(bits, y_ref, np.abs(y_ref), "bf16")  # absdot = |y|: a same-sign row
    _check(bool(np.all(got)), "an exactly rounded bf16 output is rejected")


def check_output_error_exact(output_error, seed=0):
    """mean((x W_hat^T - x W^T)^2) against exact rationals on a toy."""
    rng = np.random.default_rng(seed)
    N, K, T = 3, 256, 2
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    q = rng.integers(-8, 8, (N, K)).astype(np.int8)
    d = (rng.uniform(0.001, 0.02, (N, K // 128))).astype(np.float32)
    xf = (rng.standard_normal((T, K))).astype(np.float32)
    x_bits = (xf.view(np.uint32) >> 16).astype(np.uint16)
    xv = bf16_values(x_bits)
    total = Fraction(0)
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(xv[t][k]) * (Fraction(float(d[n, k // 128])) * int(q[n, k]) - Fraction(float(W[n, k])))
            total += acc * acc
    exact = total / (T * N)
    got = output_error(W, q, d, x_bits)
    _check(abs(Fraction(got) - exact) <= exact * Fraction(1, 10 ** 12), f"output error {got!r} != exact {float(exact)!r}")


def check_linear_nonfinite_rows(linear, seed=0):
    """A row of x holding +inf, -inf or NaN gives NaN in every output of that row
    (even where IEEE arithmetic would give an infinity: all codes nonzero here);
    the other rows are unaffected (exact rational sums)."""
    rng = np.random.default_rng(seed)
    N, K, M = 3, 256, 4
    q = rng.integers(1, 8, (N, K)).astype(np.int8)
    d = rng.uniform(0.01, 0.1, (N, K // 128)).astype(np.float32)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[1, 5] = np.inf
    xf[2, 200] = -np.inf
    xf[3, 77] = np.nan
    x_bits = (xf.view(np.uint32) >> 16).astype(np.uint16)
    y, absdot = linear(x_bits, q, d)
    _check(bool(np.all(np.isnan(y[1:]))), "a non-finite activation must poison its whole row")
    _check(bool(np.all(np.isnan(absdot[1:]))), "absdot of a poisoned row must be NaN")
    check_linear_exact(linear, x_bits[:1], q, d)
