"""Outputs where the tolerance binds, fp32 outputs, and activations at the edges
of the range -- through the C ABI on an MI355X, against the CPU oracle.

* Same-sign rows: non-negative activations against weights of one sign give
  |y| = sum_k |w_hat x|, where the bound 2e-3 * sum|w_hat x| + 1e-6 is tightest
  relative to |y|.  The fp32 outputs (the accumulated value before rounding)
  must meet the bound itself; the bf16 outputs must be the nearest-even bf16
  of such a value (oracle.admissible) and equal, bit for bit, the bf16
  rounding of the fp32 outputs.
* Non-finite activations: a NaN or infinity in row m of x makes every output
  of row m NaN, and leaves the other rows untouched (also where K is not a
  multiple of 512 and the last scale quad is padded).
* Large activations: inside the range where no fp32 intermediate overflows
  (|x| <= 2^64, |w| <= 2^38) the bound holds; past it an output may be
  non-finite where the exact value is finite, but never a wrong finite value.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_gpu_parity import CONFIGS, MFMA_ONLY, _bits, _say, check_y

pytestmark = pytest.mark.gpu


def same_sign_weight(N, K, seed, sign=1.0):
    """fp32 weights of one sign: 0.02 * (|z| + 0.25), z ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    return (sign * 0.02 * (np.abs(rng.standard_normal((N, K))) + 0.25)).astype(np.float32)


def nonneg_activations(M, K, seed, device):
    return workloads.random_activations(M, K, seed=seed, device=device).abs()


def _f32_bits(y):
    return y.cpu().numpy().view(np.uint32)


def check_rounding_of_f32(y_bf16, y_f32, what):
    """bf16 outputs are the nearest-even bf16 of the fp32 outputs, bit for bit (NaN for NaN)."""
    f = y_f32.cpu().numpy()
    want = oracle.f32_to_bf16_bits(f)
    got = _bits(y_bf16)
    nan = np.isnan(f)
    assert np.array_equal(np.isnan(oracle.bf16_bits_to_f64(got)), nan), f"{what}: NaN positions"
    assert np.array_equal(got[~nan], want[~nan]), f"{what}: bf16 outputs are not the rounding of the fp32 outputs"


def run_both(w4, x, q, d, N, path):
    yb = w4.linear(x, q, d, N, path=path)
    yf = w4.linear(x, q, d, N, path=path, out_dtype=torch.float32)
    return yb, yf


SAME_SIGN_SHAPES = [(260, 2560), (700, 1408), (37, 9216)]


@pytest.mark.parametrize("sign", [1.0, -1.0])
@pytest.mark.parametrize("path,cfg", [("gemv", None), ("gemv", "1,8"), ("gemv", "2,4"), ("mfma", None),
                                      ("mfma", "1,4"), ("mfma", "4,1"), ("mfma", "2,8s"), ("mfma", "2,4s")])
def test_same_sign_rows(w4, gpu, path, cfg, sign, monkeypatch):
    if cfg:
        monkeypatch.setenv("W4_MFMA_CFG" if path == "mfma" else "W4_GEMV_CFG", cfg)
    for i, (N, K) in enumerate(SAME_SIGN_SHAPES):
        W = same_sign_weight(N, K, seed=40 + i, sign=sign)
        q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu))
        q_ref, d_ref = oracle.rtn_quantize_ref(W)
        for M in ((1, 2, 4) if path == "gemv" else (1, 8, 16)):
            _say(f"same-sign rows sign={sign:+.0f} {N}x{K} M={M} path={path} cfg={cfg}")
            x = nonneg_activations(M, K, seed=M + 3 * i, device=gpu)
            yb, yf = run_both(w4, x, q, d, N, path)
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            assert np.allclose(np.abs(y_ref), absdot, rtol=1e-12), "the case must have |y| = sum |w_hat x|"
            check_y(yf, y_ref, absdot, f"fp32 {N}x{K} M={M}")
            check_y(yb, y_ref, absdot, f"bf16 {N}x{K} M={M}")
            check_rounding_of_f32(yb, yf, f"{N}x{K} M={M}")


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_same_sign_batched(w4, gpu, path):
    """A batch of same-sign linears with fp32 outputs and with bf16 outputs."""
    mats = []
    for i, (N, K) in enumerate(SAME_SIGN_SHAPES):
        W = same_sign_weight(N, K, seed=60 + i)
        mats.append((N, K) + w4.quantize_rtn(torch.from_numpy(W).to(gpu)) + oracle.rtn_quantize_ref(W))
    for M in ((1, 3) if path == "gemv" else (1, 8, 16)):
        _say(f"same-sign batched M={M} path={path}")
        xs = [nonneg_activations(M, K, seed=70 + M + i, device=gpu) for i, (_, K, *_) in enumerate(mats)]
        yf = w4.linear_batched([(x, q, d, N, torch.empty((M, N), dtype=torch.float32, device=gpu))
                                for x, (N, K, q, d, _, _) in zip(xs, mats)], path=path)
        yb = w4.linear_batched([(x, q, d, N, torch.empty((M, N), dtype=torch.bfloat16, device=gpu))
                                for x, (N, K, q, d, _, _) in zip(xs, mats)], path=path)
        for x, a, b, (N, K, q, d, q_ref, d_ref) in zip(xs, yf, yb, mats):
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            check_y(a, y_ref, absdot, f"batched fp32 {N}x{K} M={M}")
            check_y(b, y_ref, absdot, f"batched bf16 {N}x{K} M={M}")
            check_rounding_of_f32(b, a, f"batched {N}x{K} M={M}")


@pytest.mark.parametrize("scale_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["mfma", "gemv"])
@pytest.mark.parametrize("cfg", [c for c in CONFIGS])
def test_fp32_outputs_every_config(w4, gpu, cfg, path, scale_dtype, monkeypatch):
    """fp32 outputs of every compiled configuration meet the bound itself, and the
    bf16 outputs of the same configuration are their nearest-even rounding."""
    if cfg in MFMA_ONLY and path == "gemv":
        pytest.skip("configuration compiled for the MFMA kernel only")
    monkeypatch.setenv("W4_MFMA_CFG" if path == "mfma" else "W4_GEMV_CFG", cfg)
    sd = torch.bfloat16 if scale_dtype == "bf16" else torch.float32
    for i, (N, K) in enumerate([(700, 1408), (37, 384), (260, 2560)]):
        W = workloads.random_weight(N, K, seed=900 + i)
        q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu), scale_dtype=sd)
        q_ref, d_ref = oracle.rtn_quantize_ref(W, scale_dtype)
        for M in ((1, 3) if path == "gemv" else (1, 16, 17)):
            _say(f"fp32 outputs cfg {cfg} path={path} scales={scale_dtype} {N}x{K} M={M}")
            x = workloads.random_activations(M, K, seed=M * 13 + i, device=gpu)
            yb, yf = run_both(w4, x, q, d, N, path)
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            check_y(yf, y_ref, absdot, f"fp32 cfg {cfg} {N}x{K} M={M}")
            check_rounding_of_f32(yb, yf, f"cfg {cfg} {N}x{K} M={M}")


def _poison(x, rows):
    """Row r of x gets +inf, -inf or NaN (by r mod 3) at one position."""
    x = x.clone()
    K = x.shape[1]
    vals = (float("inf"), float("-inf"), float("nan"))
    for j, r in enumerate(rows):
        x[r, (37 * (j + 1)) % K] = vals[r % 3]
    return x


@pytest.mark.parametrize("path,cfg", [("gemv", None), ("gemv", "1,8"), ("mfma", None), ("mfma", "4,1"),
                                      ("mfma", "2,8s")])
def test_nonfinite_activations_poison_their_rows(w4, gpu, path, cfg, monkeypatch):
    if cfg:
        monkeypatch.setenv("W4_MFMA_CFG" if path == "mfma" else "W4_GEMV_CFG", cfg)
    # K = 2688: 21 groups, the last scale quad padded with three groups, whose
    # x must read as zeros (not as the start of the next row of x); a poisoned
    # value at column 37 or 74 then sits where the padding of the row before
    # would have read it
    for K in (2560, 2688):
        N = 300
        W = workloads.random_weight(N, K, seed=81)
        q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu))
        q_ref, d_ref = oracle.rtn_quantize_ref(W)
        for M, rows in ((1, [0]), (4, [1, 2]), (8, [2, 3, 7]), (16, [0, 5, 9, 10, 15])):
            if path == "gemv" and M > 4:
                continue
            _say(f"non-finite activations K={K} M={M} rows={rows} path={path} cfg={cfg}")
            x = _poison(workloads.random_activations(M, K, seed=M, device=gpu), rows)
            yb, yf = run_both(w4, x, q, d, N, path)
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            assert np.isnan(y_ref[rows]).all()
            check_y(yb, y_ref, absdot, f"bf16 K={K} M={M}")
            check_y(yf, y_ref, absdot, f"fp32 K={K} M={M}")


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_large_activations_in_range(w4, gpu, path):
    """x scaled by 2^60 (exactly, in bf16) and weights by 2^30: still within the bound."""
    N, K = 200, 4096
    W = (workloads.random_weight(N, K, seed=91) * np.float32(2.0 ** 30)).astype(np.float32)
    q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu))
    q_ref, d_ref = oracle.rtn_quantize_ref(W)
    for M in ((1, 4) if path == "gemv" else (1, 8)):
        _say(f"large activations (2^60) M={M} path={path}")
        x = workloads.random_activations(M, K, seed=M + 90, device=gpu) * (2.0 ** 60)
        yb, yf = run_both(w4, x, q, d, N, path)
        y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
        assert np.isfinite(y_ref).all()
        check_y(yf, y_ref, absdot, f"fp32 M={M}")
        check_y(yb, y_ref, absdot, f"bf16 M={M}")


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_huge_activations_never_wrong_finite(w4, gpu, path):
    """Past the range (|x| up to 3e38, so intermediate sums overflow fp32) every
    output is either correct or non-finite: never a wrong finite value."""
    N, K = 128, 1024
    W = workloads.random_weight(N, K, seed=95)
    q, d = w4.quantize_rtn(torch.from_numpy(W).to(gpu))
    q_ref, d_ref = oracle.rtn_quantize_ref(W)
    for M in ((1, 2) if path == "gemv" else (1, 8)):
        _say(f"huge activations M={M} path={path}")
        x = workloads.random_activations(M, K, seed=M + 96, device=gpu)
        x = (x / x.abs().amax(dim=1, keepdim=True).float() * 3.0e38).to(torch.bfloat16)
        assert torch.isfinite(x).all()
        yb, yf = run_both(w4, x, q, d, N, path)
        y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
        for y, bits, fmt in ((yb, _bits(yb), "bf16"), (yf, _f32_bits(yf), "f32")):
            v = (oracle.bf16_bits_to_f64(bits) if fmt == "bf16" else bits.view(np.float32).astype(np.float64))
            ok = oracle.admissible(bits, y_ref, absdot, fmt) | ~np.isfinite(v)
            assert ok.all(), f"{fmt} M={M}: {int((~ok).sum())} wrong finite outputs"
