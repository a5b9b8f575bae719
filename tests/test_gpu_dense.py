"""The dense steps of the offline quantizers on an MI355X, through the C ABI,
against the CPU oracle and fp64 NumPy on the same inputs:

* w4_gptq_hessian: H = (2/T) X^T X in fp64 -- every product of bf16 inputs is
  exact in fp64, so only the summation order differs from the oracle's;
* w4_gptq_inverse_factor: U upper triangular with (H + lambda I)^-1 = U^T U,
  against oracle.gptq_factor_ref on the same undamped H;
* w4_gptq_update: the fp32 correction of the columns after a block;
* w4_dense_linear_f32: the unquantized layer's fp32 output x W^T.

Tolerances are error bounds of the arithmetic, stated per test.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import pins
from tests.test_gpu_parity import _bits, _say

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24  # fp32 unit roundoff
U64 = 2.0 ** -53


def _x_dev(xb, gpu):
    return torch.from_numpy(xb.view(np.int16)).to(gpu).view(torch.bfloat16)


def _gamma(n, u):
    return n * u / (1 - n * u)


@pytest.mark.parametrize("T,K,kind", [(256, 1024, "correlated"), (37, 128, "correlated"), (300, 640, "recipe70b"),
                                      (1000, 2304, "recipe70b")])
def test_gptq_hessian(w4, gpu, T, K, kind):
    _say(f"gptq hessian T={T} K={K} {kind}")
    if kind == "correlated":
        _, xb = pins.gptq_correlated_inputs(seed=T + K, N=3, K=K, T=T)
    else:
        xb = _bits(workloads.activations("stack_70b", 0, "gate", T, "cpu")[:, :K].contiguous())
    H = w4.gptq_hessian(_x_dev(xb, gpu)).cpu().numpy()
    H_ref = oracle.gptq_hessian_ref(xb)
    X = np.abs(oracle.bf16_bits_to_f64(xb))
    bound = _gamma(T, U64) * (2.0 / T) * (X.T @ X) * 2  # both sums' rounding (the oracle's and the kernel's)
    assert np.array_equal(H, H.T), "H must be exactly symmetric"
    assert np.all(np.abs(H - H_ref) <= bound), f"worst {np.max(np.abs(H - H_ref) / np.maximum(bound, 1e-300)):.3f}"


@pytest.mark.parametrize("T,K,kind", [(256, 1024, "correlated"), (64, 128, "correlated"), (512, 2048, "recipe70b")])
def test_gptq_inverse_factor(w4, gpu, T, K, kind):
    """U from the library's damped Hessian against the oracle's factor of the same
    undamped Hessian (damping applied by the oracle itself).  U is fp32, so each row
    may differ by the rounding of its largest entries plus what the fp64 steps'
    different order changes; U^T U (H + lambda I) = I checks it independently."""
    _say(f"gptq inverse factor T={T} K={K} {kind}")
    if kind == "correlated":
        _, xb = pins.gptq_correlated_inputs(seed=T + K + 1, N=3, K=K, T=T)
    else:
        xb = _bits(workloads.activations("stack_70b", 1, "gate", T, "cpu")[:, :K].contiguous())
    Hg = w4.gptq_hessian(_x_dev(xb, gpu))
    H = Hg.cpu().numpy()
    w4.gptq_damp(Hg, 0.01)
    H_damped = Hg.cpu().numpy()
    U = w4.gptq_inverse_factor(Hg).cpu().numpy().astype(np.float64)
    assert np.array_equal(Hg.cpu().numpy(), H_damped), "H must not be modified"
    assert np.all(np.tril(U, -1) == 0), "U must be upper triangular"
    U_ref = oracle.gptq_factor_ref(H)
    scale = np.max(np.abs(U_ref), axis=1, keepdims=True)
    rel = np.max(np.abs(U - U_ref) / scale)
    assert rel <= 2e-5, f"U differs from the oracle's factor: {rel:.2e} of a row's largest entry"
    # U^T U is the inverse of the damped H about as well as the oracle's factor
    # rounded to fp32 is (how well depends on the conditioning of H)
    U32r = U_ref.astype(np.float32).astype(np.float64)
    resid = np.max(np.abs(U.T @ U @ H_damped - np.eye(K)))
    resid_ref = np.max(np.abs(U32r.T @ U32r @ H_damped - np.eye(K)))
    assert resid <= 4 * resid_ref + 1e-9, f"U^T U H - I: {resid:.2e} against {resid_ref:.2e} for the oracle's factor"


def test_gptq_inverse_factor_full_size(w4, gpu):
    """A 70B-class gate Hessian (K = 8192) from 256 recipe rows (outlier channels, rank
    deficient before damping): 128 diagonal blocks, the largest trailing products."""
    _say("gptq inverse factor K=8192")
    K, T = 8192, 256
    x = workloads.activations("stack_70b", 2, "gate", T, gpu)
    Hg = w4.gptq_hessian(x)
    H = Hg.cpu().numpy()
    w4.gptq_damp(Hg, 0.01)
    U = w4.gptq_inverse_factor(Hg).cpu().numpy().astype(np.float64)
    U_ref = oracle.gptq_factor_ref(H)
    scale = np.max(np.abs(U_ref), axis=1, keepdims=True)
    rel = np.max(np.abs(U - U_ref) / scale)
    assert rel <= 5e-5, f"U differs from the oracle's factor: {rel:.2e} of a row's largest entry"


@pytest.mark.parametrize("N,K,b0", [(300, 1024, 0), (300, 1024, 512), (70, 384, 128), (64, 1024, 896)])
def test_gptq_update(w4, gpu, N, K, b0):
    """W[:, b0+128:] -= err^T U[b0:b0+128, b0+128:] in fp32 against fp64: each element is
    a 128-term sum started from W, so it is within gamma_129 of the sum of magnitudes."""
    _say(f"gptq update N={N} K={K} b0={b0}")
    rng = np.random.default_rng(N + K + b0)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    U = np.triu(rng.standard_normal((K, K))).astype(np.float32)
    err = (rng.standard_normal((128, N)) * 0.01).astype(np.float32)
    Wg = torch.from_numpy(W).to(gpu)
    w4.gptq_update(Wg, torch.from_numpy(U).to(gpu), b0, torch.from_numpy(err).to(gpu))
    got = Wg.cpu().numpy().astype(np.float64)
    b1 = b0 + 128
    ref = W.astype(np.float64)
    mag = np.abs(ref).copy()
    ref[:, b1:] -= err.astype(np.float64).T @ U[b0:b1, b1:].astype(np.float64)
    mag[:, b1:] += np.abs(err.astype(np.float64)).T @ np.abs(U[b0:b1, b1:].astype(np.float64))
    assert np.array_equal(got[:, :b1], W[:, :b1].astype(np.float64)), "columns up to the block's end are untouched"
    assert np.all(np.abs(got - ref) <= _gamma(129, U32) * mag)


@pytest.mark.parametrize("T,N,K", [(37, 300, 1152), (256, 1024, 4096), (1, 70, 128)])
def test_dense_linear_f32(w4, gpu, T, N, K):
    """y = x W^T in fp32 against fp64: within gamma_K of sum |x W| (fp32 fused
    multiply-adds over k in order)."""
    _say(f"dense linear f32 T={T} N={N} K={K}")
    x = workloads.random_activations(T, K, seed=T + N, device=gpu)
    W = workloads.random_weight(N, K, seed=T + K)
    y = w4.dense_linear_f32(x, torch.from_numpy(W).to(gpu)).cpu().numpy().astype(np.float64)
    xf = oracle.bf16_bits_to_f64(_bits(x))
    ref = xf @ W.astype(np.float64).T
    mag = np.abs(xf) @ np.abs(W.astype(np.float64)).T
    assert np.all(np.abs(y - ref) <= _gamma(K, U32) * mag)
