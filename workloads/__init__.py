"""Seeded synthetic workloads: shapes, value distributions and generators.

This module is the one place both the HIP path's tests/benchmarks and the CPU
oracle draw their inputs from.  It holds none of the quantization or linear
arithmetic: it only describes matrix shapes, draws random fp32 weights and
bf16 activations, and counts the bytes a call has to move.

The pages measured whole models (Qwen3.5-4B, a 27B dense model, Llama-3.1-70B)
on public corpora; none of that is available here, so every input is synthetic
with the shapes of those models' linear layers and the value distributions
listed below.  Every draw is a pure function of (workload, layer, matrix, kind)
and the device kind it is drawn on: host draws use NumPy's PCG64, device draws
use torch's device generator.  Whichever side draws a tensor, a comparison
always hands the oracle a host copy of the very tensor the kernel consumed.
"""

from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 0
GROUP = 128


@dataclass(frozen=True)
class Matrix:
    name: str
    N: int  # outputs
    K: int  # inputs


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    matrices: tuple  # one layer's matrices, in execution order
    layers: int
    ms: tuple  # activation row counts
    weight: tuple  # weight distribution recipe
    x_channel_mult: float = 1.0  # matching-channel multiplier for x (70B recipe)
    description: str = ""
    input_groups: dict = field(default_factory=dict)  # matrix name -> shared-input tag


def _decoder_layer(hidden, ffn, q_out, kv_out):
    return (
        Matrix("q", q_out, hidden),
        Matrix("k", kv_out, hidden),
        Matrix("v", kv_out, hidden),
        Matrix("o", hidden, q_out),
        Matrix("gate", ffn, hidden),
        Matrix("up", ffn, hidden),
        Matrix("down", hidden, ffn),
    )


_DECODER_INPUTS = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
                   "gate": "mlp_in", "up": "mlp_in", "down": "down_in"}

WORKLOADS = {
    w.name: w
    for w in (
        Workload(
            "ffn_2560x9216", 1, (Matrix("ffn", 2560, 9216),), 1, (1,),
            ("normal", 0.02),
            description="single FFN matrix N=2560, K=9216, W ~ N(0, 0.02^2), "
                        "x bf16 ~ N(0,1), M=1, seed 0",
        ),
        Workload(
            "ffn_pair_outliers", 2,
            (Matrix("down", 2560, 9216), Matrix("up", 9216, 2560)), 1, (1, 8),
            ("normal_outliers", 0.02, 0.005, 0.2),
            description="2560x9216 and 9216x2560, W ~ N(0, 0.02^2) with 0.5% of "
                        "entries replaced by N(0, 0.2^2), x bf16 ~ N(0,1), M in {1, 8}",
        ),
        Workload(
            "stack_4b", 3, _decoder_layer(2560, 9216, 4096, 1024), 36, (1, 5, 7, 13),
            ("normal", 0.02),
            description="4B-class stack: hidden 2560, FFN 9216, 36 layers, "
                        "W ~ N(0, 0.02^2), M in {1, 5, 7, 13}",
            input_groups=_DECODER_INPUTS,
        ),
        Workload(
            "stack_27b", 4, _decoder_layer(5120, 17408, 6144, 1024), 64, (1, 8),
            ("normal", 0.015),
            description="27B-class stack: hidden 5120, FFN 17408, 64 layers, "
                        "W ~ N(0, 0.015^2), M in {1, 8}",
            input_groups=_DECODER_INPUTS,
        ),
        Workload(
            "stack_70b", 5, _decoder_layer(8192, 28672, 8192, 1024), 80, (1, 8, 13, 16),
            ("student_t_channels", 4.0, 0.01, 0.01, 20.0), x_channel_mult=10.0,
            description="70B-class stack: hidden 8192, FFN 28672, 80 layers, "
                        "W ~ Student-t(4) scaled to std 0.01 with 1% of input "
                        "channels x20, x bf16 ~ N(0,1) with the same channels x10, "
                        "M in {1, 8, 13, 16}",
            input_groups=_DECODER_INPUTS,
        ),
    )
}


# ----------------------------------------------------------------------------
# byte accounting (what one call must move; no arithmetic of the method)
# ----------------------------------------------------------------------------

def algorithmic_bytes(M, N, K, scale_bytes=4):
    """Bytes one linear call must move: 4-bit codes, scales (fp32, or 2 bytes for
    16-bit scales), bf16 x and y."""
    return N * K // 2 + scale_bytes * N * (K // GROUP) + 2 * M * K + 2 * M * N


def quantize_bytes(N, K, scale_bytes=4):
    """Bytes one quantize call must move: fp32 weights in, codes and scales out."""
    return 4 * N * K + N * K // 2 + scale_bytes * N * (K // GROUP)


def stack_bytes(workload, M, scale_bytes=4):
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    return w.layers * sum(algorithmic_bytes(M, m.N, m.K, scale_bytes) for m in w.matrices)


def stack_weights(workload):
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    return w.layers * sum(m.N * m.K for m in w.matrices)


# ----------------------------------------------------------------------------
# seeds
# ----------------------------------------------------------------------------

_KIND = {"weight": 1, "x": 2, "channels": 3, "test": 4}


def seed_sequence(*key):
    """np.random.SeedSequence for a tuple of small non-negative ints / strings."""
    ints = []
    for k in key:
        if isinstance(k, str):
            ints.append(int.from_bytes(k.encode()[:8].ljust(8, b"\0"), "little"))
        else:
            ints.append(int(k))
    return np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(ints))


def host_rng(*key):
    return np.random.Generator(np.random.PCG64(seed_sequence(*key)))


def torch_seed(*key):
    s = seed_sequence(*key).generate_state(2, dtype=np.uint32)
    return int(s[0]) | (int(s[1] & 0x7FFFFFFF) << 32)


# ----------------------------------------------------------------------------
# outlier channels (70B recipe): the same set for W columns and x entries
# ----------------------------------------------------------------------------

def outlier_channels(workload, layer, input_tag, K):
    """Sorted input-channel indices scaled up for one (layer, input tensor).

    1% of the K input channels, drawn without replacement; q/k/v share one set,
    gate/up share one, o and down have their own.
    """
    w = WORKLOADS[workload]
    frac = w.weight[3]
    count = int(round(frac * K))
    rng = host_rng(w.index, layer, input_tag, _KIND["channels"])
    return np.sort(rng.choice(K, size=count, replace=False)).astype(np.int64)


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------

def _recipe_host(recipe, N, K, rng, channels):
    kind = recipe[0]
    if kind == "normal":
        return rng.standard_normal((N, K), dtype=np.float32) * np.float32(recipe[1])
    if kind == "normal_outliers":
        std, frac, ostd = recipe[1:4]
        W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
        mask = rng.random((N, K), dtype=np.float32) < frac
        W[mask] = rng.standard_normal(int(mask.sum()), dtype=np.float32) * np.float32(ostd)
        return W
    if kind == "student_t_channels":
        nu, std, _, mult = recipe[1:5]
        scale = std / np.sqrt(nu / (nu - 2.0))
        W = (rng.standard_t(nu, size=(N, K)) * scale).astype(np.float32)
        if channels is not None and len(channels):
            W[:, channels] *= np.float32(mult)
        return W
    raise ValueError(kind)


def _recipe_device(recipe, N, K, gen, device, channels):
    import torch

    kind = recipe[0]
    if kind == "normal":
        return torch.randn((N, K), generator=gen, device=device, dtype=torch.float32).mul_(recipe[1])
    if kind == "normal_outliers":
        std, frac, ostd = recipe[1:4]
        W = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32).mul_(std)
        mask = torch.rand((N, K), generator=gen, device=device) < frac
        out = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32).mul_(ostd)
        return torch.where(mask, out, W)
    if kind == "student_t_channels":
        nu, std, _, mult = recipe[1:5]
        assert nu == 4.0, "device draw implements nu = 4 (chi-square with 4 dof)"
        scale = std / float(np.sqrt(nu / (nu - 2.0)))
        z = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32)
        # chi-square(4) = -2 ln(U1 U2) with U uniform on (0, 1]
        u1 = 1.0 - torch.rand((N, K), generator=gen, device=device, dtype=torch.float32)
        u2 = 1.0 - torch.rand((N, K), generator=gen, device=device, dtype=torch.float32)
        chi2 = (-2.0) * (torch.log(u1) + torch.log(u2))
        W = z.mul_(torch.rsqrt(chi2.div_(nu))).mul_(scale)
        del u1, u2, chi2
        if channels is not None and len(channels):
            idx = torch.as_tensor(channels, device=device)
            W[:, idx] *= mult
        return W
    raise ValueError(kind)


def weight(workload, layer, matrix, device="cpu"):
    """fp32 weight [N, K] of one matrix of one layer, drawn on `device`.

    device "cpu" returns a NumPy array; any other device returns a torch tensor.
    """
    w = WORKLOADS[workload]
    idx = [m.name for m in w.matrices].index(matrix)
    m = w.matrices[idx]
    channels = None
    if w.weight[0] == "student_t_channels":
        channels = outlier_channels(workload, layer, w.input_groups.get(matrix, matrix), m.K)
    key = (w.index, layer, idx, _KIND["weight"])
    if str(device) == "cpu":
        return _recipe_host(w.weight, m.N, m.K, host_rng(*key), channels)
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(*key))
    return _recipe_device(w.weight, m.N, m.K, gen, device, channels)


# ----------------------------------------------------------------------------
# activations (bf16)
# ----------------------------------------------------------------------------

def activations(workload, layer, matrix, M, device="cpu"):
    """bf16 activations [M, K] for one matrix (torch tensor on `device`).

    Drawn as fp32 N(0, 1) on the host, the recipe's outlier channels scaled
    (70B recipe), then rounded to bf16 (round to nearest even) by torch.
    """
    import torch

    w = WORKLOADS[workload]
    m = next(mm for mm in w.matrices if mm.name == matrix)
    tag = w.input_groups.get(matrix, matrix)
    rng = host_rng(w.index, layer, tag, M, _KIND["x"])
    x = rng.standard_normal((M, m.K), dtype=np.float32)
    if w.x_channel_mult != 1.0:
        ch = outlier_channels(workload, layer, tag, m.K)
        x[:, ch] *= np.float32(w.x_channel_mult)
    return torch.from_numpy(x).to(torch.bfloat16).to(device)


def random_weight(N, K, std=0.02, seed=0, device="cpu"):
    """Generic N(0, std^2) fp32 weight for tests of arbitrary shapes."""
    rng = host_rng(seed, N, K, _KIND["test"])
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    if str(device) == "cpu":
        return W
    import torch

    return torch.from_numpy(W).to(device)


def random_activations(M, K, seed=0, scale=1.0, device="cpu"):
    """Generic bf16 N(0, scale^2) activations [M, K] for tests of arbitrary shapes."""
    import torch

    rng = host_rng(seed, M, K, _KIND["test"], 1)
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(scale)
    return torch.from_numpy(x).to(torch.bfloat16).to(device)
