"""Pins of the CPU oracle (no GPU).

The oracle is checked against things other than itself: exact rationals,
brute force over the 16 code levels, closed forms, the channel-scaling
identity the study states, and hand-derived fixtures.  The second half of the
file runs the same checks against deliberately broken copies of the oracle
(one plausible mistake each) and requires every copy to be caught.
"""

import numpy as np
import pytest

import oracle
from oracle import rtn as rtn_mod
from tests import pins

Q = oracle.rtn_quantize_ref
L = oracle.w4_linear_ref


def _x_bits(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do


# ----------------------------------------------------------------------------
# the oracle passes every pin
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fixture", ["rtn_ties.txt", "rtn_special.txt"])
def test_golden_fixtures(fixture):
    pins.check_golden(Q, fixture)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_scale_exact_rational(seed):
    pins.check_scale_exact(Q, pins.toy_weights(seed))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_codes_bruteforce(seed):
    pins.check_codes_bruteforce(Q, pins.toy_weights(seed))


def test_round_trip_bound():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    pins.check_round_trip(Q, W)
    pins.check_round_trip(Q, pins.toy_weights(9, N=16, K=768))


def test_invariants():
    rng = np.random.default_rng(6)
    W = (rng.standard_t(4, size=(64, 1024)) * 0.01).astype(np.float32)
    pins.check_invariants(Q, W)


def test_scale_equivariance():
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    for e in (-10, -1, 1, 7):
        pins.check_scale_equivariance(Q, W, e)


def test_group_permutation():
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((8, 384)) * 0.02).astype(np.float32)
    pins.check_group_permutation(Q, W)


def test_group_count_matches_study():
    pins.check_group_count(Q)


def test_linear_exact_rational():
    W = pins.toy_weights(21, N=4, K=256)
    W[W == 0] = 0  # keep
    q, d = Q(W)
    pins.check_linear_exact(L, _x_bits(3, 256, 4), q, d)


def test_linear_closed_forms():
    pins.check_linear_closed_forms(L)


def test_channel_scaling_identity():
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    pins.check_channel_scaling(Q, L, W, _x_bits(2, 512, 14))


def test_packing():
    pins.check_packing(oracle.pack_canonical, oracle.unpack_canonical)


def test_nan_scale_poisons_outputs():
    W = np.zeros((2, 256), dtype=np.float32)
    W[0, 3] = np.nan
    W[1, :] = 0.01
    q, d = Q(W)
    y, _ = L(_x_bits(1, 256, 0), q, d)
    assert np.isnan(y[0, 0]) and np.isfinite(y[0, 1])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        Q(np.zeros((2, 100), dtype=np.float32))
    with pytest.raises(TypeError):
        Q(np.zeros((2, 128), dtype=np.float64))


# ----------------------------------------------------------------------------
# plausible mistakes are caught (mistakes are planted in copies of the oracle)
# ----------------------------------------------------------------------------

def _mutant_quantize(*, rounding="away", divisor=7.0, recip=False, clamp=True, poison=True,
                     zero_codes=True, abs_max=True):
    nan = rtn_mod._nan_f32()

    def quantize(W):
        N, K = W.shape
        Wg = W.reshape(N, K // 128, 128)
        finite = np.isfinite(Wg).all(axis=2)
        with np.errstate(all="ignore"):
            a = (np.abs(Wg) if abs_max else Wg).max(axis=2).astype(np.float32)
            d = (a / np.float32(divisor)).astype(np.float32)
        if poison:
            d[~finite] = nan
        usable = finite & (d != 0) if zero_codes else np.ones_like(finite)
        safe = np.where(usable, d, np.float32(1)).astype(np.float32)
        with np.errstate(all="ignore"):
            if recip:
                t = (Wg * (np.float32(1) / safe)[:, :, None]).astype(np.float32)
            else:
                t = (Wg / safe[:, :, None]).astype(np.float32)
        if rounding == "even":
            r = np.round(t.astype(np.float64))
        elif rounding == "f32floor":
            r = np.sign(t) * np.floor((np.abs(t) + np.float32(0.5)).astype(np.float32))
        elif rounding == "trunc":
            r = np.trunc(t.astype(np.float64))
        else:
            r = rtn_mod._round_half_away(t)
        if clamp:
            r = np.clip(r, -8, 7)
        r = np.nan_to_num(r, nan=0.0, posinf=127, neginf=-127)
        if zero_codes:
            r[~usable] = 0
        return r.reshape(N, K).astype(np.int8), d

    return quantize


def _all_quantizer_pins(quantize):
    pins.check_golden(quantize, "rtn_ties.txt")
    pins.check_golden(quantize, "rtn_special.txt")
    for seed in (0, 1):
        W = pins.toy_weights(seed)
        pins.check_scale_exact(quantize, W)
        pins.check_codes_bruteforce(quantize, W)
        pins.check_round_trip(quantize, W)
    rng = np.random.default_rng(6)
    pins.check_invariants(quantize, (rng.standard_t(4, size=(32, 512)) * 0.01).astype(np.float32))


@pytest.mark.parametrize("mutation", [
    dict(rounding="even"),       # numpy round: ties to even
    dict(rounding="f32floor"),   # float32 floor(|t| + 0.5)
    dict(rounding="trunc"),      # truncation instead of rounding
    dict(divisor=8.0),           # wrong range mapping
    dict(divisor=7.5),
    dict(recip=True),            # multiply by 1/d instead of dividing by d
    dict(clamp=False),           # no clip to [-8, 7]
    dict(poison=False),          # non-finite groups not flagged
    dict(zero_codes=False),      # codes of zero-scale groups not forced to 0
    dict(abs_max=False),         # max instead of max of magnitudes
])
def test_quantizer_mutants_are_caught(mutation):
    assert pins.check_golden  # the checks exist
    _all_quantizer_pins(Q)  # the oracle itself passes
    with pytest.raises(pins.PinFailure):
        _all_quantizer_pins(_mutant_quantize(**mutation))


def _mutant_linear(kind):
    def linear(x_bits, q, d):
        x = oracle.bf16_bits_to_f64(x_bits)
        N, K = q.shape
        if kind == "group_index":
            dd = d.astype(np.float64)[:, np.arange(K) % d.shape[1]]
        elif kind == "transposed_scale":
            dd = np.repeat(d.astype(np.float64), 128, axis=1)[::-1]
        else:
            dd = np.repeat(d.astype(np.float64), 128, axis=1)
        w = dd * q.astype(np.float64)
        if kind == "zero_point":
            w = dd * (q.astype(np.float64) + 8)
        if kind == "sign":
            w = -w
        if kind == "f32":
            y = (x.astype(np.float32) @ w.astype(np.float32).T).astype(np.float64)
        elif kind == "drop_last_group":
            y = x[:, :-128] @ w[:, :-128].T
        else:
            y = x @ w.T
        return y, np.abs(x) @ np.abs(w).T

    return linear


def _all_linear_pins(linear):
    W = pins.toy_weights(21, N=4, K=256)
    q, d = Q(W)
    pins.check_linear_exact(linear, _x_bits(3, 256, 4), q, d)
    pins.check_linear_closed_forms(linear)
    rng = np.random.default_rng(13)
    Wc = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    pins.check_channel_scaling(Q, linear, Wc, _x_bits(2, 512, 14))


@pytest.mark.parametrize("kind", ["group_index", "transposed_scale", "zero_point", "sign",
                                  "f32", "drop_last_group"])
def test_linear_mutants_are_caught(kind):
    _all_linear_pins(L)
    with pytest.raises(pins.PinFailure):
        _all_linear_pins(_mutant_linear(kind))


@pytest.mark.parametrize("kind", ["swap", "nooffset"])
def test_packing_mutants_are_caught(kind):
    def pack(q):
        u = (q.astype(np.int16) + (8 if kind == "swap" else 0)).astype(np.uint8) & 0x0F
        if kind == "swap":
            return (u[:, 1::2] | (u[:, 0::2] << 4)).astype(np.uint8)
        return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)

    with pytest.raises(pins.PinFailure):
        pins.check_packing(pack, oracle.unpack_canonical)


# ----------------------------------------------------------------------------
# 16-bit (bf16) restore scales
# ----------------------------------------------------------------------------

def Q16(W):
    return oracle.rtn_quantize_ref(W, "bf16")


def _torch_bf16(v):
    import torch
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_narrowing_matches_library():
    pins.check_bf16_narrowing(oracle.f32_to_bf16_bits, _torch_bf16)


def _all_scale16_pins(quantize16):
    pins.check_scale16_exact(quantize16, pins.scale16_tie_weights())
    for seed in (0, 1):
        W = pins.toy_weights(seed)
        pins.check_scale16_exact(quantize16, W)
        pins.check_codes_bruteforce(pins.widened(quantize16), W)
        pins.check_round_trip(pins.widened(quantize16), W)
    rng = np.random.default_rng(6)
    pins.check_invariants(pins.widened(quantize16), (rng.standard_t(4, size=(32, 512)) * 0.01).astype(np.float32))


def test_scale16_pins():
    _all_scale16_pins(Q16)
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    pins.check_scale_equivariance(pins.widened(Q16), W, 5)
    pins.check_group_permutation(pins.widened(Q16), W)


def test_scale16_special_groups():
    """Zero, NaN/Inf and fp32-subnormal groups under 16-bit scales."""
    W = np.zeros((4, 128), dtype=np.float32)
    W[1, 3] = np.nan
    W[2, :] = (np.arange(128) - 64).astype(np.float32) * np.float32(2.0 ** -140)
    W[3, 7] = np.inf
    q, d = Q16(W)
    assert d.dtype == np.uint16
    assert d[0, 0] == 0 and not q[0].any()
    assert d[1, 0] == 0x7FC0 and not q[1].any() and d[3, 0] == 0x7FC0 and not q[3].any()
    a = np.float32(64 * 2.0 ** -140)
    assert d[2, 0] == pins.bf16_nearest_bits(pins.f32_nearest(pins.Fraction(float(a)) / 7))


def test_scale16_linear_uses_widened_scales():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    q, d16 = Q16(W)
    x = _x_bits(2, 256, 3)
    y16, _ = L(x, q, d16)
    y32, _ = L(x, q, (d16.astype(np.uint32) << 16).view(np.float32))
    assert np.array_equal(y16, y32)


def _mutant_quantize16(kind):
    def quantize(W):
        N, K = W.shape
        Wg = W.reshape(N, K // 128, 128)
        finite = np.isfinite(Wg).all(axis=2)
        with np.errstate(all="ignore"):
            d = (np.abs(Wg).max(axis=2) / np.float32(7)).astype(np.float32)
        d[~finite] = rtn_mod._nan_f32()
        bits = d.view(np.uint32)
        if kind == "truncate":
            d16 = (bits >> 16).astype(np.uint16)
        elif kind == "ties_away":
            d16 = ((bits + np.uint32(0x8000)) >> 16).astype(np.uint16)
        else:
            d16 = oracle.f32_to_bf16_bits(d)
        dw = (d16.astype(np.uint32) << 16).view(np.float32)
        divisor = d if kind == "divide_by_f32" else dw
        usable = finite & (dw != 0)
        safe = np.where(usable, divisor, np.float32(1)).astype(np.float32)
        with np.errstate(all="ignore"):
            t = (Wg / safe[:, :, None]).astype(np.float32)
        r = np.clip(rtn_mod._round_half_away(t), -8, 7)
        r[~usable] = 0
        return r.reshape(N, K).astype(np.int8), d16
    return quantize


@pytest.mark.parametrize("kind", ["truncate", "ties_away", "divide_by_f32"])
def test_scale16_mutants_are_caught(kind):
    _all_scale16_pins(Q16)
    with pytest.raises(pins.PinFailure):
        _all_scale16_pins(_mutant_quantize16(kind))


def test_bf16_narrowing_mutant_is_caught():
    with pytest.raises(pins.PinFailure):
        pins.check_bf16_narrowing(lambda v: (np.asarray(v).view(np.uint32) >> 16).astype(np.uint16), _torch_bf16)


# ----------------------------------------------------------------------------
# AWQ channel scaling
# ----------------------------------------------------------------------------

def test_awq_grid_and_scales():
    pins.check_awq_grid(oracle.ALPHAS)
    W, xb = pins.awq_outlier_inputs(seed=2)
    m = oracle.channel_absmean_ref(xb)
    assert np.allclose(m, np.abs(pins.bf16_values(xb)).mean(axis=0), rtol=0, atol=0)
    for a in (0.0, 5 / 19, 1.0):
        pins.check_awq_scales(oracle.candidate_scales_ref, m, a)


def test_awq_alpha_zero_is_rtn():
    W, xb = pins.awq_outlier_inputs(seed=3)
    s32, inv32 = oracle.candidate_scales_ref(oracle.channel_absmean_ref(xb), 0.0)
    assert np.all(s32 == 1) and np.all(inv32 == 1)
    q1, d1 = oracle.quantize_scaled_ref(W, s32)
    q0, d0 = oracle.rtn_quantize_ref(W)
    assert np.array_equal(q1, q0) and np.array_equal(d1.view(np.uint32), d0.view(np.uint32))
    assert np.array_equal(oracle.scale_activations_ref(xb, inv32), xb)


def test_awq_activation_scaling_exact():
    W, xb = pins.awq_outlier_inputs(seed=4, T=4)
    s32, inv32 = oracle.candidate_scales_ref(oracle.channel_absmean_ref(xb), 11 / 19)
    pins.check_awq_activation_scaling(oracle.scale_activations_ref, xb, inv32)


def test_awq_error_exact_and_identity():
    W, xb = pins.awq_outlier_inputs(seed=5, N=6, K=256, T=3)
    s32, inv32 = oracle.candidate_scales_ref(oracle.channel_absmean_ref(xb), 7 / 19)
    pins.check_awq_error(oracle.awq_output_error_ref, oracle.quantize_scaled_ref, oracle.scale_activations_ref,
                         W, xb, s32, inv32)
    pins.check_awq_identity(None, W, xb, s32)


def test_awq_search_helps_on_salient_channels():
    pins.check_awq_helps_on_salient_channels(oracle.awq_search_ref)


def _awq_mutants(kind):
    """Copies of the oracle's AWQ steps with one plausible mistake each."""
    from oracle import awq as A

    def scales(m, alpha):
        a = -alpha if kind == "negative_exponent" else alpha
        p = np.power(np.maximum(np.asarray(m, dtype=np.float64), 1e-30), float(a))
        s = p if kind == "no_normalization" else p / np.exp(np.mean(np.log(p)))
        s32 = s.astype(np.float32)
        return s32, (1.0 / s32.astype(np.float64)).astype(np.float32)

    def scale_x(x_bits, inv32):
        if kind == "multiply_x":
            inv32 = (1.0 / inv32.astype(np.float64)).astype(np.float32)
        return A.scale_activations_ref(x_bits, inv32)

    def error(W, x_bits, s32, inv32):
        if kind == "weight_error":
            q, d = A.quantize_scaled_ref(W, s32)
            w_hat = np.repeat(d.astype(np.float64), 128, axis=1) * q / s32.astype(np.float64)[None, :]
            return float(np.mean((w_hat - W.astype(np.float64)) ** 2))
        q, d = A.quantize_scaled_ref(W, s32)
        y_q, _ = oracle.w4_linear_ref(scale_x(x_bits, inv32), q, d)
        y = np.asarray(pins.bf16_values(x_bits), dtype=np.float64) @ W.astype(np.float64).T
        return float(np.mean((y_q - y) ** 2))

    def search(W, x_bits):
        m = A.channel_absmean_ref(x_bits)
        grid = [k / 20 for k in range(20)] if kind == "grid_k_over_20" else A.ALPHAS
        errs = np.asarray([error(W, x_bits, *scales(m, a)) for a in grid])
        k = int(np.argmin(errs))
        return (k, *scales(m, grid[k]), errs)

    return scales, scale_x, error, search, ([k / 20 for k in range(20)] if kind == "grid_k_over_20" else A.ALPHAS)


def _all_awq_pins(scales, scale_x, error, search, grid):
    pins.check_awq_grid(grid)
    W, xb = pins.awq_outlier_inputs(seed=6, N=6, K=256, T=3)
    m = oracle.channel_absmean_ref(xb)
    pins.check_awq_scales(scales, m, 9 / 19)
    s32, inv32 = scales(m, 9 / 19)
    pins.check_awq_activation_scaling(scale_x, xb, inv32)
    pins.check_awq_error(error, oracle.quantize_scaled_ref, scale_x, W, xb, s32, inv32)
    pins.check_awq_helps_on_salient_channels(search)


@pytest.mark.parametrize("kind", ["negative_exponent", "no_normalization", "multiply_x", "weight_error",
                                  "grid_k_over_20"])
def test_awq_mutants_are_caught(kind):
    _all_awq_pins(*_awq_mutants("none"))
    with pytest.raises(pins.PinFailure):
        _all_awq_pins(*_awq_mutants(kind))


# ----------------------------------------------------------------------------
# GPTQ
# ----------------------------------------------------------------------------

def _gptq_quantize_with_block(W, U, block):
    return oracle.gptq_quantize_ref(W, U, block)


def test_gptq_bruteforce():
    pins.check_gptq_bruteforce(oracle.gptq_ref)


def test_gptq_identity_hessian_is_rtn():
    pins.check_gptq_identity_hessian_is_rtn(oracle.gptq_ref)


def test_gptq_block_width():
    pins.check_gptq_block_width(_gptq_quantize_with_block, oracle.gptq_factor_ref, oracle.gptq_hessian_ref)


def test_gptq_beats_rtn():
    pins.check_gptq_beats_rtn(oracle.gptq_ref, Q, oracle.output_error_ref)


def test_gptq_dead_columns():
    pins.check_gptq_dead_columns(oracle.gptq_factor_ref, oracle.gptq_hessian_ref)


def test_gptq_16bit_scales():
    g16 = lambda W, xb: oracle.gptq_ref(W, xb, scale_dtype="bf16")
    pins.check_gptq_bruteforce(g16, scale16=True)
    pins.check_gptq16_identity_hessian_is_rtn16(g16)


@pytest.mark.parametrize("kind", ["fp32_scale_used", "fp32_scale_stored"])
def test_gptq_16bit_scale_mutants_are_caught(kind):
    """Codes taken against the fp32 scale while the bf16 one is stored, or the fp32 scale
    stored truncated: the 16-bit pins catch both."""
    def g16(W, xb):
        U = oracle.gptq_factor_ref(oracle.gptq_hessian_ref(xb))
        q, d32 = oracle.gptq_quantize_ref(W, U)  # decisions against the fp32 scale
        if kind == "fp32_scale_used":
            return q, oracle.f32_to_bf16_bits(d32)
        return q, (d32.view(np.uint32) >> 16).astype(np.uint16)  # truncation instead of nearest
    with pytest.raises(pins.PinFailure):
        pins.check_gptq_bruteforce(g16, scale16=True)
        pins.check_gptq16_identity_hessian_is_rtn16(g16)


def test_gptq_all_inputs_zero_is_rtn():
    pins.check_gptq_all_inputs_zero_is_rtn(oracle.gptq_ref)


def test_gptq_rejects_non_finite():
    W, xb = pins.gptq_correlated_inputs()
    W = W.copy()
    W[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.gptq_ref(W, xb)


def _gptq_mutant(kind):
    """A copy of the GPTQ oracle with one plausible mistake."""
    def factor(H):
        H = np.array(H, dtype=np.float64, copy=True)
        dead = np.diag(H) == 0
        if kind != "no_dead_fix":
            H[dead, dead] = 1.0
        damp = {"damp_tenth": 0.1, "no_damping": 0.0}.get(kind, 0.01)
        H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
        if kind == "factor_of_hessian":
            return np.linalg.cholesky(H).T
        L = np.linalg.cholesky(np.linalg.inv(H))
        return L if kind == "lower_factor" else L.T

    def quantize(W, U, block=128):
        N, K = W.shape
        Wk = W.astype(np.float64)
        W0 = Wk.copy()
        q = np.zeros((N, K), dtype=np.int8)
        d = np.zeros((N, K // 128), dtype=np.float32)
        for b0 in range(0, K, block):
            b1 = min(b0 + block, K)
            E = np.zeros((N, b1 - b0))
            for j in range(b0, b1):
                if j % 128 == 0:
                    src = W0 if kind == "scale_from_original" else Wk
                    d[:, j // 128] = oracle.gptq.group_scale_ref(src[:, j:j + 128])
                dg = d[:, j // 128]
                qj = oracle.gptq.code_ref(Wk[:, j], dg)
                q[:, j] = qj.astype(np.int8)
                err = Wk[:, j] - dg.astype(np.float64) * qj
                if kind != "no_divide":
                    err = err / U[j, j]
                if kind != "no_in_block":
                    Wk[:, j + 1:b1] -= np.outer(err, U[j, j + 1:b1])
                E[:, j - b0] = err
            if kind != "no_trailing":
                Wk[:, b1:] -= E @ U[b0:b1, b1:]
        return q, d

    hessian = oracle.gptq_hessian_ref
    gptq = lambda W, xb: quantize(W, factor(hessian(xb)))
    return gptq, quantize, factor, hessian


def _all_gptq_pins(gptq, quantize, factor, hessian):
    pins.check_gptq_bruteforce(gptq)
    pins.check_gptq_identity_hessian_is_rtn(gptq)
    pins.check_gptq_block_width(quantize, factor, hessian)
    pins.check_gptq_beats_rtn(gptq, Q, oracle.output_error_ref)
    pins.check_gptq_dead_columns(factor, hessian)
    pins.check_gptq_all_inputs_zero_is_rtn(gptq)


@pytest.mark.parametrize("kind", ["no_trailing", "no_in_block", "no_divide", "scale_from_original",
                                  "factor_of_hessian", "lower_factor", "damp_tenth", "no_damping",
                                  "no_dead_fix"])
def test_gptq_mutants_are_caught(kind):
    _all_gptq_pins(*_gptq_mutant("none"))
    with pytest.raises((pins.PinFailure, np.linalg.LinAlgError)):
        _all_gptq_pins(*_gptq_mutant(kind))


# ----------------------------------------------------------------------------
# when an output counts as correct; non-finite activations; the output error
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_admissible_bruteforce(fmt):
    pins.check_admissible(oracle.admissible, fmt)


def test_exact_rounding_is_admissible():
    pins.check_exact_rounding_is_admissible(oracle.admissible)


def _admissible_mutant(kind):
    def admissible(y_bits, y_ref, absdot, fmt):
        shift = 16 if fmt == "bf16" else 0
        b = np.asarray(y_bits).astype(np.uint32) << np.uint32(shift)
        y = b.view(np.float32).astype(np.float64)
        tol = 2e-3 * np.asarray(absdot) + 1e-6
        if kind == "plain_bound":  # the bound without the output rounding
            ok = np.abs(y - y_ref) <= tol
        else:
            lo, hi = oracle.rounding_interval(np.asarray(y_bits), fmt)
            g_up, g_dn = hi - y, y - lo
            if kind == "whole_step":  # a whole step on either side instead of half
                lo, hi = y - 2 * g_dn, y + 2 * g_up
            elif kind == "symmetric_gap":  # the step above used below too (wrong at powers of two)
                lo = y - g_up
            ok = (y_ref - tol <= hi) & (y_ref + tol >= lo)
        return np.where(np.isnan(y_ref), np.isnan(y), ok)

    return admissible


@pytest.mark.parametrize("kind", ["plain_bound", "whole_step", "symmetric_gap"])
def test_admissible_mutants_are_caught(kind):
    mutant = _admissible_mutant(kind)

    def all_pins(adm):
        pins.check_admissible(adm, "bf16", cases=300)
        pins.check_exact_rounding_is_admissible(adm)
        # powers of two: the step below is half the step above
        y_ref = np.array([1.0 - 2.0 ** -10, 2.0 - 1.5 * 2.0 ** -8])
        bits = np.array([0x3F80, 0x4000], dtype=np.uint16)
        # 1 - 2^-10 rounds to 1.0; 2 - 1.5*2^-8 lies below 2.0's interval [2 - 2^-8, 2 + 2^-7]
        want = np.array([True, False])
        got = adm(bits, y_ref, np.zeros(2), "bf16")
        if not np.array_equal(got, want):
            raise pins.PinFailure(f"powers of two: {got}")

    all_pins(oracle.admissible)
    with pytest.raises(pins.PinFailure):
        all_pins(mutant)


def test_output_error_exact():
    pins.check_output_error_exact(oracle.output_error_ref)


@pytest.mark.parametrize("kind", ["f32", "mean_over_rows_only", "scale_group_index"])
def test_output_error_mutants_are_caught(kind):
    def output_error(W, q, d, x_bits):
        X = oracle.bf16_bits_to_f64(x_bits)
        G = W.shape[1] // 128
        if kind == "scale_group_index":
            What = np.asarray(d, np.float64)[:, np.arange(W.shape[1]) % G] * q
        else:
            What = (np.asarray(d, np.float64)[:, :, None] * q.reshape(q.shape[0], G, 128)).reshape(q.shape)
        if kind == "f32":
            e = (X.astype(np.float32) @ (What - W).astype(np.float32).T).astype(np.float64)
        else:
            e = X @ (What - np.asarray(W, np.float64)).T
        if kind == "mean_over_rows_only":
            return float(np.mean(np.sum(e ** 2, axis=1)))
        return float(np.mean(e ** 2))

    with pytest.raises(pins.PinFailure):
        pins.check_output_error_exact(output_error)


def test_nonfinite_activation_rows():
    pins.check_linear_nonfinite_rows(oracle.w4_linear_ref)


def test_nonfinite_activation_ieee_mutant_is_caught():
    def ieee(x_bits, q, d):  # the plain IEEE sum: +-inf where every code is nonzero
        x = oracle.bf16_bits_to_f64(x_bits)
        w = oracle.dequantize_ref(q, d)
        with np.errstate(invalid="ignore"):
            return x @ w.T, np.abs(x) @ np.abs(w).T

    with pytest.raises(pins.PinFailure):
        pins.check_linear_nonfinite_rows(ieee)
