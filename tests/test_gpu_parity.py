"""Parity of the HIP path against the CPU oracle, on an MI355X.

Every call goes through the C ABI (via the ctypes binding).  Codes and scales
must match the oracle bit for bit (compared in canonical form after
w4_unpack).  Outputs are checked element by element with oracle.admissible:
the value the kernel accumulates must satisfy

    |v - y_ref| <= 2e-3 * sum_k |w_hat[n,k] x[m,k]| + 1e-6,

with y_ref and the sum computed in fp64 by the oracle; a bf16 output must be
the nearest-even bf16 of such a v; NaN exactly where the oracle has NaN.
Inputs come from workloads/ (seeded); the oracle always sees a host copy of
the very tensor the kernel consumed.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import pins

pytestmark = pytest.mark.gpu

def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _bits(x_bf16):
    return x_bf16.cpu().view(torch.int16).numpy().view(np.uint16)


def check_y(y_gpu, y_ref, absdot, what):
    """Outputs (bf16 or fp32 tensor) against the oracle, element by element."""
    if y_gpu.dtype == torch.float32:
        bits, fmt = y_gpu.cpu().numpy().view(np.uint32), "f32"
        y = bits.view(np.float32).astype(np.float64)
    else:
        bits, fmt = _bits(y_gpu), "bf16"
        y = oracle.bf16_bits_to_f64(bits)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y), nan_ref), f"{what}: NaN positions differ"
    ok = oracle.admissible(bits, y_ref, absdot, fmt)
    worst = oracle.worst_ratio(y, y_ref, absdot)
    assert np.all(ok), f"{what}: {int(np.sum(~ok))} {fmt} outputs out of tolerance (worst |y-y_ref|/tol {worst:.3f})"
    return worst


def _scale_bits(d_canon):
    """Canonical scales (fp32 or bf16 tensor) -> their bit patterns (uint32 / uint16)."""
    if d_canon.dtype == torch.bfloat16:
        return d_canon.cpu().view(torch.int16).numpy().view(np.uint16)
    return d_canon.cpu().numpy().view(np.uint32)


def quantize_and_compare(w4, W_dev, what, rows=None, scale_dtype=torch.float32):
    """Quantize on the GPU, unpack, compare with the oracle (all rows or a row sample)."""
    N, K = W_dev.shape
    q, d = w4.quantize_rtn(W_dev, scale_dtype=scale_dtype)
    qc, dc = w4.unpack(q, d, N, K)
    torch.cuda.synchronize()
    if rows is None:
        W_h = W_dev.cpu().numpy()
        qg, dg = qc.cpu().numpy(), _scale_bits(dc)
    else:
        idx = torch.as_tensor(rows, device=W_dev.device)
        W_h = W_dev.index_select(0, idx).cpu().numpy()
        qg, dg = qc.index_select(0, idx).cpu().numpy(), _scale_bits(dc.index_select(0, idx))
    q_ref, d_ref = oracle.rtn_quantize_ref(W_h, "bf16" if scale_dtype == torch.bfloat16 else "f32")
    d_ref_bits = d_ref if d_ref.dtype == np.uint16 else d_ref.view(np.uint32)
    assert np.array_equal(dg, d_ref_bits), f"{what}: scales differ"
    bad = np.argwhere(qg != q_ref)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:4].tolist()}"
    return q, d, q_ref, d_ref


# ----------------------------------------------------------------------------
# quantization: bit-exact codes and scales
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fixture", ["rtn_ties.txt", "rtn_special.txt"])
def test_quantize_golden(w4, gpu, fixture):
    groups = pins.load_groups(fixture)
    _say(f"quantize golden {fixture} ({len(groups)} groups)")
    W = np.stack([g[2] for g in groups]).astype(np.float32)
    W_dev = torch.from_numpy(W).to(gpu)
    q, d = w4.quantize_rtn(W_dev)
    qc, dc = w4.unpack(q, d, W.shape[0], 128)
    qc, dc = qc.cpu().numpy(), dc.cpu().numpy()
    for i, (name, d_bits, _, q_exp) in enumerate(groups):
        assert int(dc[i, 0:1].view(np.uint32)[0]) == d_bits, f"{name}: scale"
        assert np.array_equal(qc[i].astype(np.int64), q_exp), f"{name}: codes"


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_quantize_toys(w4, gpu, seed):
    _say(f"quantize toys seed={seed}")
    W = pins.toy_weights(seed, N=37, K=768)
    quantize_and_compare(w4, torch.from_numpy(W).to(gpu), f"toys{seed}")


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (37, 384), (100, 1152), (64, 9216), (257, 2560)])
def test_quantize_shapes(w4, gpu, N, K):
    _say(f"quantize N={N} K={K}")
    W = workloads.random_weight(N, K, std=0.02, seed=N + K)
    quantize_and_compare(w4, torch.from_numpy(W).to(gpu), f"{N}x{K}")


def near_tie_weights(seed, N=64, K=1024, spread_ulps=3, far=2e-5, far_share=0.125):
    """Groups whose members sit a few ulps from (k + 1/2) * d, where d is the
    group's scale as the oracle computes it: their codes depend on the last
    bit of the IEEE quotient w / d.  A share `far_share` of the members is
    instead placed about `far` (relative) from a half-integer quotient."""
    rng = np.random.default_rng(seed)
    W = np.empty((N, K), np.float32)
    for n in range(N):
        for g in range(K // 128):
            a = np.float32(rng.uniform(1e-3, 10.0))
            probe = np.zeros((1, 128), np.float32)
            probe[0, 0] = a
            d = np.float64(oracle.rtn_quantize_ref(probe)[1].reshape(-1)[0])
            k = rng.integers(-7, 7, size=127).astype(np.float64)  # quotients k + 1/2 in [-6.5, 6.5]
            shift = np.where(rng.random(127) < far_share, rng.choice([-far, far], 127), 0.0)
            vals = ((k + 0.5) * (1.0 + shift) * d).astype(np.float32)
            ulps = rng.integers(-spread_ulps, spread_ulps + 1, size=127)
            for s in range(spread_ulps):
                vals = np.where(ulps > s, np.nextafter(vals, np.float32(np.inf)), vals)
                vals = np.where(ulps < -s, np.nextafter(vals, np.float32(-np.inf)), vals)
            grp = np.concatenate([[a], vals]).astype(np.float32)
            W[n, g * 128:(g + 1) * 128] = grp[rng.permutation(128)]
    return W


@pytest.mark.parametrize("seed,far_share", [(0, 0.125), (1, 0.125), (2, 1.0)])
def test_quantize_near_ties(w4, gpu, seed, far_share):
    """Codes decided by the last bit of w / d match the oracle's IEEE quotients,
    both for quotients within a few ulps of a half-integer and (far_share = 1)
    for quotients just outside that band, everywhere in the tile."""
    _say(f"quantize near-tie weights seed={seed} far_share={far_share}")
    W = near_tie_weights(seed, far_share=far_share)
    quantize_and_compare(w4, torch.from_numpy(W).to(gpu), f"near ties {seed}/{far_share}")


@pytest.mark.parametrize("workload", ["ffn_2560x9216", "ffn_pair_outliers"])
def test_quantize_single_matrix_workloads(w4, gpu, workload):
    for m in workloads.WORKLOADS[workload].matrices:
        _say(f"quantize {workload}/{m.name} {m.N}x{m.K}")
        W = workloads.weight(workload, 0, m.name, "cpu")
        quantize_and_compare(w4, torch.from_numpy(W).to(gpu), f"{workload}/{m.name}")


@pytest.mark.parametrize("workload", ["stack_4b", "stack_27b", "stack_70b"])
def test_quantize_stack_matrices_sampled(w4, gpu, workload):
    """Full-size matrices drawn on the GPU; 96 sampled rows checked bit for bit."""
    wl = workloads.WORKLOADS[workload]
    for layer in (0, wl.layers - 1):
        for m in wl.matrices:
            _say(f"quantize {workload} layer {layer} {m.name} {m.N}x{m.K}")
            W = workloads.weight(workload, layer, m.name, gpu)
            rows = np.unique(np.concatenate([[0, m.N - 1], np.random.default_rng(layer).choice(m.N, 94)]))
            quantize_and_compare(w4, W, f"{workload}/{layer}/{m.name}", rows=rows)
            del W
            torch.cuda.empty_cache()


def test_pack_unpack_roundtrip(w4, gpu):
    _say("pack/unpack round trip N=45 K=640")
    rng = np.random.default_rng(0)
    qc = torch.from_numpy(rng.integers(-8, 8, (45, 640)).astype(np.int8)).to(gpu)
    dc = torch.from_numpy(rng.standard_normal((45, 5)).astype(np.float32)).to(gpu)
    q, d = w4.pack(qc, dc)
    qc2, dc2 = w4.unpack(q, d, 45, 640)
    assert torch.equal(qc2, qc) and torch.equal(dc2.view(torch.int32), dc.view(torch.int32))
    # padding rows (45..47) and padding groups (5..7) of the native layout hold scale 0
    dn = d.view(3, 2, 16, 4)  # [row block][scale quad][row in block][group in quad]
    assert torch.all(dn[2, :, 13:, :] == 0)
    assert torch.all(dn[:, 1, :, 1:] == 0)
    # quantize output re-packed from its canonical form is identical
    W = torch.from_numpy(workloads.random_weight(45, 640, seed=3)).to(gpu)
    q1, d1 = w4.quantize_rtn(W)
    q2, d2 = w4.pack(*w4.unpack(q1, d1, 45, 640))
    assert torch.equal(q1, q2) and torch.equal(d1.view(torch.int32), d2.view(torch.int32))


# ----------------------------------------------------------------------------
# linear: tolerance against the fp64 oracle
# ----------------------------------------------------------------------------

def linear_case(w4, gpu, M, N, K, path, seed=0, std=0.02, x_scale=1.0):
    W = torch.from_numpy(workloads.random_weight(N, K, std=std, seed=seed)).to(gpu)
    x = workloads.random_activations(M, K, seed=seed, scale=x_scale, device=gpu)
    q, d = w4.quantize_rtn(W)
    y = w4.linear(x, q, d, N, path=path)
    q_ref, d_ref = oracle.rtn_quantize_ref(W.cpu().numpy())
    y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
    return check_y(y, y_ref, absdot, f"M={M} N={N} K={K} {path}")


SHAPES = [(1, 16, 128), (1, 37, 384), (2, 50, 1152), (3, 64, 256), (4, 100, 640),
          (5, 48, 2560), (7, 33, 1024), (8, 200, 1408), (13, 17, 512), (16, 160, 896),
          (17, 40, 384), (33, 24, 256), (1, 1040, 4096)]


@pytest.mark.parametrize("path", ["mfma", "gemv", "auto"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_linear_shapes(w4, gpu, M, N, K, path):
    _say(f"linear M={M} N={N} K={K} path={path}")
    linear_case(w4, gpu, M, N, K, path, seed=M * 7 + N)


@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_linear_single_matrix_workloads(w4, gpu, path):
    for workload in ("ffn_2560x9216", "ffn_pair_outliers"):
        wl = workloads.WORKLOADS[workload]
        for m in wl.matrices:
            W = torch.from_numpy(workloads.weight(workload, 0, m.name, "cpu")).to(gpu)
            q, d = w4.quantize_rtn(W)
            q_ref, d_ref = oracle.rtn_quantize_ref(W.cpu().numpy())
            for M in wl.ms:
                _say(f"linear {workload}/{m.name} {m.N}x{m.K} M={M} path={path}")
                x = workloads.activations(workload, 0, m.name, M, gpu)
                y = w4.linear(x, q, d, m.N, path=path)
                y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
                check_y(y, y_ref, absdot, f"{workload}/{m.name} M={M}")


@pytest.mark.parametrize("workload", ["stack_4b", "stack_27b", "stack_70b"])
def test_linear_stack_matrices_sampled(w4, gpu, workload):
    """Full-size layers (first, middle, last) at every listed M; 128 sampled output rows."""
    wl = workloads.WORKLOADS[workload]
    for layer in (0, wl.layers // 2, wl.layers - 1):
        for m in wl.matrices:
            W = workloads.weight(workload, layer, m.name, gpu)
            q, d = w4.quantize_rtn(W)
            rows = np.unique(np.concatenate([[0, m.N - 1], np.random.default_rng(layer + 1).choice(m.N, 126)]))
            idx = torch.as_tensor(rows, device=gpu)
            q_ref, d_ref = oracle.rtn_quantize_ref(W.index_select(0, idx).cpu().numpy())
            del W
            for M in wl.ms:
                _say(f"linear {workload} layer {layer} {m.name} {m.N}x{m.K} M={M}")
                x = workloads.activations(workload, layer, m.name, M, gpu)
                y = w4.linear(x, q, d, m.N)
                y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
                check_y(y.index_select(1, idx), y_ref, absdot, f"{workload}/{layer}/{m.name} M={M}")
            del q, d
            torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# properties that hold at any size
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_linear_deterministic(w4, gpu, path):
    _say(f"determinism path={path}")
    W = torch.from_numpy(workloads.random_weight(2048, 4096, seed=5)).to(gpu)
    x = workloads.random_activations(8, 4096, seed=5, device=gpu)
    q, d = w4.quantize_rtn(W)
    y1 = w4.linear(x, q, d, 2048, path=path)
    y2 = w4.linear(x, q, d, 2048, path=path)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_linear_channel_scaling_bit_identical(w4, gpu, path):
    """Per-group power-of-two channel scaling (study, section 2 identity W'x' = Wx):
    codes unchanged, scales scaled exactly, outputs bit-identical."""
    _say(f"channel scaling path={path}")
    N, K, M = 96, 1024, 5
    W = workloads.random_weight(N, K, seed=17)
    x = workloads.random_activations(M, K, seed=17)
    e = np.random.default_rng(17).integers(-3, 4, K // 128)
    s = np.repeat(2.0 ** e, 128)
    W2 = (W.astype(np.float64) * s).astype(np.float32)
    x2 = (x.float().numpy().astype(np.float64) / s).astype(np.float32)
    x2 = torch.from_numpy(x2).to(torch.bfloat16)
    assert np.array_equal(x2.float().numpy().astype(np.float64), x.float().numpy() / s)
    q1, d1 = w4.quantize_rtn(torch.from_numpy(W).to(gpu))
    q2, d2 = w4.quantize_rtn(torch.from_numpy(W2).to(gpu))
    assert torch.equal(q1, q2)
    y1 = w4.linear(x.to(gpu), q1, d1, N, path=path)
    y2 = w4.linear(x2.to(gpu), q2, d2, N, path=path)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_linear_degenerate_groups(w4, gpu, path):
    """NaN scales poison exactly their rows; zero groups contribute nothing."""
    _say(f"degenerate groups path={path}")
    N, K, M = 48, 512, 3
    W = workloads.random_weight(N, K, seed=23)
    W[5, 130] = np.nan
    W[9, 0:128] = 0.0
    W[17, 300] = np.inf
    x = workloads.random_activations(M, K, seed=23)
    W_dev = torch.from_numpy(W).to(gpu)
    q, d = w4.quantize_rtn(W_dev)
    y = w4.linear(x.to(gpu), q, d, N, path=path)
    q_ref, d_ref = oracle.rtn_quantize_ref(W)
    y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
    check_y(y, y_ref, absdot, "degenerate")
    assert np.isnan(y_ref[:, 5]).all() and np.isnan(y_ref[:, 17]).all()


def test_linear_empty_is_noop(w4, gpu):
    _say("empty problems")
    q = torch.zeros(w4.packed_bytes(16, 128), dtype=torch.uint8, device=gpu)
    d = torch.zeros(w4.scale_count(16, 128), dtype=torch.float32, device=gpu)
    y = w4.linear(torch.zeros((0, 128), dtype=torch.bfloat16, device=gpu), q, d, 16)
    assert y.shape == (0, 16)
    y = w4.linear(torch.zeros((2, 128), dtype=torch.bfloat16, device=gpu), q, d, 0)
    assert y.shape == (2, 0)


# ----------------------------------------------------------------------------
# batched launches
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_linear_batched_matches_single_calls(w4, gpu, path, monkeypatch):
    """A decode layer's seven projections in one launch: bitwise equal to one call each
    (same kernel configuration), and within tolerance of the oracle."""
    monkeypatch.setenv("W4_MFMA_CFG", "1,8")
    monkeypatch.setenv("W4_GEMV_CFG", "1,8")
    shapes = [("q", 320, 512), ("k", 64, 512), ("v", 64, 512), ("o", 512, 320 + 64),
              ("gate", 700, 512), ("up", 700, 512), ("down", 512, 1408)]
    for M in (1, 3, 8):
        _say(f"batched layer M={M} path={path}")
        items, refs = [], []
        x_attn = workloads.random_activations(M, 512, seed=M, device=gpu)
        for i, (name, N, K) in enumerate(shapes):
            W = torch.from_numpy(workloads.random_weight(N, K, seed=100 + i)).to(gpu)
            q, d = w4.quantize_rtn(W)
            x = x_attn if K == 512 else workloads.random_activations(M, K, seed=M + i, device=gpu)
            items.append((x, q, d, N, torch.empty((M, N), dtype=torch.bfloat16, device=gpu)))
            refs.append(W.cpu().numpy())
        ys = w4.linear_batched(items, path=path)
        for (x, q, d, N, _), y, Wh, (name, _, _) in zip(items, ys, refs, shapes):
            y1 = w4.linear(x, q, d, N, path=path)
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"{name}: batched != single"
            q_ref, d_ref = oracle.rtn_quantize_ref(Wh)
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            check_y(y, y_ref, absdot, f"batched {name} M={M}")


# Every compiled (row blocks per wavefront, wavefronts per block) pair; the
# built-in choice picks among them by launch size, so each is checked here on
# ragged shapes: partial row panels, K not a whole number of scale quads, and
# more wavefronts per block than the matrix has quads.  "s" marks the MFMA
# kernel's shared-x form (each wavefront all of K, the x tile shared through
# LDS); it is not compiled for the dot2 kernel.
CONFIGS = ["1,4", "1,8", "2,4", "4,4", "1,2", "2,2", "4,1", "4,2", "2,8s", "2,4s"]
MFMA_ONLY = {"2,8s", "2,4s"}  # configurations compiled for the MFMA kernel only
CFG_SHAPES = [(700, 1408), (37, 384), (260, 2560)]


@pytest.mark.parametrize("scale_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["mfma", "gemv"])
@pytest.mark.parametrize("cfg", CONFIGS)
def test_linear_every_config(w4, gpu, cfg, path, scale_dtype, monkeypatch):
    monkeypatch.setenv("W4_MFMA_CFG" if path == "mfma" else "W4_GEMV_CFG", cfg)
    if cfg in MFMA_ONLY and path == "gemv":
        _say(f"config {cfg} is not compiled for the dot2 kernel")
        q = torch.zeros(w4.packed_bytes(16, 128), dtype=torch.uint8, device=gpu)
        d = torch.zeros(w4.scale_count(16, 128), dtype=torch.float32, device=gpu)
        with pytest.raises(w4.W4Error):
            w4.linear(torch.zeros((1, 128), dtype=torch.bfloat16, device=gpu), q, d, 16, path="gemv")
        return
    sd = torch.bfloat16 if scale_dtype == "bf16" else torch.float32
    mats = []
    for i, (N, K) in enumerate(CFG_SHAPES):
        W = torch.from_numpy(workloads.random_weight(N, K, seed=500 + i)).to(gpu)
        q, d = w4.quantize_rtn(W, scale_dtype=sd)
        mats.append((N, K, q, d, oracle.rtn_quantize_ref(W.cpu().numpy(), scale_dtype)))
    for M in ((1, 2, 3) if path == "gemv" else (1, 8, 16, 17)):
        _say(f"config {cfg} path={path} scales={scale_dtype} M={M}")
        xs = [workloads.random_activations(M, K, seed=M * 11 + i, device=gpu) for i, (_, K, _, _, _) in enumerate(mats)]
        items = [(x, q, d, N, torch.empty((M, N), dtype=torch.bfloat16, device=gpu))
                 for x, (N, K, q, d, _) in zip(xs, mats)]
        ys = w4.linear_batched(items, path=path)
        for x, y, (N, K, q, d, (q_ref, d_ref)) in zip(xs, ys, mats):
            y1 = w4.linear(x, q, d, N, path=path)
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            check_y(y, y_ref, absdot, f"cfg {cfg} batched {N}x{K} M={M}")
            check_y(y1, y_ref, absdot, f"cfg {cfg} single {N}x{K} M={M}")


@pytest.mark.parametrize("scale_dtype", ["f32", "bf16"])
def test_shared_x_matches_one_wavefront_panels(w4, gpu, scale_dtype, monkeypatch):
    """The shared-x MFMA form computes every output row with the same
    arithmetic in the same order as one wavefront per row panel over all of K:
    identical bits, whatever the row blocks per wavefront."""
    sd = torch.bfloat16 if scale_dtype == "bf16" else torch.float32
    shapes = [(700, 1408), (2048, 2560), (37, 384)]
    mats = []
    for i, (N, K) in enumerate(shapes):
        W = torch.from_numpy(workloads.random_weight(N, K, seed=700 + i)).to(gpu)
        mats.append((N, K) + w4.quantize_rtn(W, scale_dtype=sd))
    for M in (1, 8, 16, 23):
        _say(f"shared x vs one-wavefront panels, scales={scale_dtype} M={M}")
        xs = [workloads.random_activations(M, K, seed=M + 31 * i, device=gpu) for i, (_, K, _, _) in enumerate(mats)]
        outs = {}
        for cfg in ("4,1", "2,8s", "2,4s"):
            monkeypatch.setenv("W4_MFMA_CFG", cfg)
            items = [(x, q, d, N, torch.empty((M, N), dtype=torch.bfloat16, device=gpu))
                     for x, (N, K, q, d) in zip(xs, mats)]
            outs[cfg] = [y.view(torch.int16).clone() for y in w4.linear_batched(items, path="mfma")]
        for cfg in ("2,8s", "2,4s"):
            for a, b, (N, K, _, _) in zip(outs["4,1"], outs[cfg], mats):
                assert torch.equal(a, b), f"{cfg} differs from 4,1 on {N}x{K} M={M}"


def test_linear_unknown_config_is_an_error(w4, gpu, monkeypatch):
    q = torch.zeros(w4.packed_bytes(16, 128), dtype=torch.uint8, device=gpu)
    d = torch.zeros(w4.scale_count(16, 128), dtype=torch.float32, device=gpu)
    x = torch.zeros((1, 128), dtype=torch.bfloat16, device=gpu)
    for var, path in (("W4_MFMA_CFG", "mfma"), ("W4_GEMV_CFG", "gemv")):
        for bad in ("3,3", "2,8x", "4"):
            monkeypatch.setenv(var, bad)
            with pytest.raises(w4.W4Error):
                w4.linear(x, q, d, 16, path=path)
        monkeypatch.delenv(var)
    w4.linear(x, q, d, 16)  # and the library still works


@pytest.mark.parametrize("workload,ms", [("stack_70b", (1, 16)), ("stack_27b", (1, 2))])
def test_linear_batched_full_size_layer(w4, gpu, workload, ms):
    """One decoder layer (seven full-size matrices, short and long K mixed) in one
    launch: at M = 1 the dot2 kernel's mixed-K configurations (two row blocks per
    wavefront when the shortest K is 8192, one otherwise), then the MFMA kernel."""
    wl = workloads.WORKLOADS[workload]
    tag = workload.split("_")[1]
    mats = []
    for m in wl.matrices:
        W = workloads.weight(workload, 3, m.name, gpu)
        q, d = w4.quantize_rtn(W)
        rows = np.unique(np.concatenate([[0, m.N - 1], np.random.default_rng(7).choice(m.N, 62)]))
        idx = torch.as_tensor(rows, device=gpu)
        mats.append((m, q, d, idx, oracle.rtn_quantize_ref(W.index_select(0, idx).cpu().numpy())))
        del W
    for M in ms:
        _say(f"batched {tag} layer M={M}")
        items = []
        for (m, q, d, idx, _) in mats:
            x = workloads.activations(workload, 3, m.name, M, gpu)
            items.append((x, q, d, m.N, torch.empty((M, m.N), dtype=torch.bfloat16, device=gpu)))
        ys = w4.linear_batched(items)
        for (m, q, d, idx, (q_ref, d_ref)), (x, *_), y in zip(mats, items, ys):
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            check_y(y.index_select(1, idx), y_ref, absdot, f"{tag} batched {m.name} M={M}")


# ----------------------------------------------------------------------------
# 16-bit (bf16) scales
# ----------------------------------------------------------------------------

S16 = torch.bfloat16


@pytest.mark.parametrize("seed", [0, 1])
def test_s16_quantize_toys(w4, gpu, seed):
    _say(f"s16 quantize toys seed={seed}")
    quantize_and_compare(w4, torch.from_numpy(pins.toy_weights(seed, N=37, K=768)).to(gpu), f"s16 toys{seed}",
                         scale_dtype=S16)


def test_s16_quantize_scale_ties_and_near_ties(w4, gpu):
    _say("s16 quantize: scales halfway between bf16 values; weights near half-integer quotients")
    quantize_and_compare(w4, torch.from_numpy(pins.scale16_tie_weights(64)).to(gpu), "s16 scale ties",
                         scale_dtype=S16)
    quantize_and_compare(w4, torch.from_numpy(near_tie_weights(3)).to(gpu), "s16 near ties", scale_dtype=S16)


@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (257, 2560), (2560, 9216)])
def test_s16_quantize_shapes(w4, gpu, N, K):
    _say(f"s16 quantize N={N} K={K}")
    W = workloads.random_weight(N, K, std=0.02, seed=N + K + 1)
    quantize_and_compare(w4, torch.from_numpy(W).to(gpu), f"s16 {N}x{K}", scale_dtype=S16)


def test_s16_pack_unpack_roundtrip(w4, gpu):
    _say("s16 pack/unpack")
    N, K = 40, 640
    rng = np.random.default_rng(4)
    qc = torch.from_numpy(rng.integers(-8, 8, (N, K)).astype(np.int8)).to(gpu)
    dc = torch.from_numpy(rng.standard_normal((N, K // 128)).astype(np.float32)).to(gpu).to(torch.bfloat16)
    q, d = w4.pack(qc, dc)
    assert d.dtype == torch.bfloat16
    qc2, dc2 = w4.unpack(q, d, N, K)
    assert torch.equal(qc, qc2) and torch.equal(dc.view(torch.int16), dc2.view(torch.int16))


@pytest.mark.parametrize("path", ["mfma", "gemv", "auto"])
@pytest.mark.parametrize("M,N,K", [(1, 37, 384), (1, 1040, 4096), (4, 100, 640), (8, 200, 1408),
                                   (16, 160, 896), (33, 24, 256)])
def test_s16_linear_shapes(w4, gpu, M, N, K, path):
    _say(f"s16 linear M={M} N={N} K={K} path={path}")
    W = torch.from_numpy(workloads.random_weight(N, K, seed=M + N + K)).to(gpu)
    q, d = w4.quantize_rtn(W, scale_dtype=S16)
    x = workloads.random_activations(M, K, seed=M * 3 + N, device=gpu)
    y = w4.linear(x, q, d, N, path=path)
    q_ref, d_ref = oracle.rtn_quantize_ref(W.cpu().numpy(), "bf16")
    y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
    check_y(y, y_ref, absdot, f"s16 M={M} N={N} K={K}")


@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_s16_linear_batched_and_deterministic(w4, gpu, path):
    _say(f"s16 batched path={path}")
    shapes = [(320, 512), (64, 512), (700, 512)]
    for M in (1, 8):
        x = workloads.random_activations(M, 512, seed=M, device=gpu)
        items, refs = [], []
        for i, (N, K) in enumerate(shapes):
            W = torch.from_numpy(workloads.random_weight(N, K, seed=300 + i)).to(gpu)
            q, d = w4.quantize_rtn(W, scale_dtype=S16)
            items.append((x, q, d, N, torch.empty((M, N), dtype=torch.bfloat16, device=gpu)))
            refs.append(W.cpu().numpy())
        ys = w4.linear_batched(items, path=path)
        for (xx, q, d, N, _), y, Wh in zip(items, ys, refs):
            y1 = w4.linear(xx, q, d, N, path=path)
            y2 = w4.linear(xx, q, d, N, path=path)
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), "batched != single"
            assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"
            q_ref, d_ref = oracle.rtn_quantize_ref(Wh, "bf16")
            y_ref, absdot = oracle.w4_linear_ref(_bits(xx), q_ref, d_ref)
            check_y(y, y_ref, absdot, f"s16 batched N={N} M={M}")


def test_s16_linear_full_size_70b_layer_sampled(w4, gpu):
    """70B-class gate and down matrices at full size with 16-bit scales, M = 1 and 16; sampled rows."""
    for name in ("gate", "down"):
        m = next(mm for mm in workloads.WORKLOADS["stack_70b"].matrices if mm.name == name)
        W = workloads.weight("stack_70b", 5, name, gpu)
        q, d = w4.quantize_rtn(W, scale_dtype=S16)
        rows = np.unique(np.concatenate([[0, m.N - 1], np.random.default_rng(9).choice(m.N, 62)]))
        idx = torch.as_tensor(rows, device=gpu)
        q_ref, d_ref = oracle.rtn_quantize_ref(W.index_select(0, idx).cpu().numpy(), "bf16")
        del W
        for M in (1, 16):
            _say(f"s16 70b {name} M={M}")
            x = workloads.activations("stack_70b", 5, name, M, gpu)
            y = w4.linear(x, q, d, m.N)
            y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
            check_y(y.index_select(1, idx), y_ref, absdot, f"s16 70b {name} M={M}")
        del q, d
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# channel scaling before RTN (AWQ)
# ----------------------------------------------------------------------------

def _awq_case(gpu, seed=0, N=200, K=1024, T=64):
    W, xb = pins.awq_outlier_inputs(seed=seed, N=N, K=K, T=T)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(gpu)
    return W, xb, torch.from_numpy(W).to(gpu), x


def test_awq_steps_match_oracle(w4, gpu):
    """Channel means, candidate scales, scaled quantization (fp32 and 16-bit scales),
    scaled activations and the fused decode linear, each against the oracle."""
    _say("awq steps")
    W, xb, W_dev, x = _awq_case(gpu, seed=10)
    m = w4.channel_absmean(x)
    m_ref = oracle.channel_absmean_ref(xb)
    assert np.allclose(m.cpu().numpy(), m_ref, rtol=1e-5, atol=0), "channel means"
    for alpha in (0.0, 6 / 19, 1.0):
        s, inv = w4.awq_scales(m, alpha)
        s_h, inv_h = s.cpu().numpy(), inv.cpu().numpy()
        s_ref, _ = oracle.candidate_scales_ref(m.cpu().numpy().astype(np.float64), alpha)
        assert np.allclose(s_h, s_ref, rtol=4e-7, atol=0), f"scales alpha={alpha}"
        assert np.array_equal(inv_h, (1.0 / s_h.astype(np.float64)).astype(np.float32)), "reciprocals"
        if alpha == 0.0:
            assert np.all(s_h == 1) and np.all(inv_h == 1)
        for sd, tag in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            q, d = w4.quantize_rtn_scaled(W_dev, s, sd)
            qc, dc = w4.unpack(q, d, W.shape[0], W.shape[1])
            q_ref, d_ref = oracle.quantize_scaled_ref(W, s_h, tag)
            assert np.array_equal(qc.cpu().numpy(), q_ref), f"scaled codes alpha={alpha} {tag}"
            assert np.array_equal(_scale_bits(dc), d_ref if tag == "bf16" else d_ref.view(np.uint32)), \
                f"scaled scales alpha={alpha} {tag}"
        xs = w4.scale_activations(x, inv)
        xs_ref = oracle.scale_activations_ref(xb, inv_h)
        assert np.array_equal(_bits(xs), xs_ref), f"scaled activations alpha={alpha}"
        q, d = w4.quantize_rtn_scaled(W_dev, s)
        q_ref, d_ref = oracle.quantize_scaled_ref(W, s_h)
        for M in (1, 3, 8):
            y = w4.linear_awq(x[:M], q, d, W.shape[0], inv)
            y_sep = w4.linear(w4.scale_activations(x[:M], inv), q, d, W.shape[0], path="gemv")
            assert torch.equal(y.view(torch.int16), y_sep.view(torch.int16)), "fused scaling != separate"
            y_ref, absdot = oracle.w4_linear_ref(xs_ref[:M], q_ref, d_ref)
            check_y(y, y_ref, absdot, f"awq linear alpha={alpha} M={M}")


def test_awq_sq_error(w4, gpu):
    _say("awq squared error")
    rng = np.random.default_rng(3)
    y = torch.from_numpy(rng.standard_normal((37, 1001)).astype(np.float32)).to(gpu).to(torch.bfloat16)
    y_ref = torch.from_numpy(rng.standard_normal((37, 1001)).astype(np.float32)).to(gpu)
    got = float(w4.sq_error(y, y_ref).cpu()[0])
    exp = float(np.sum((y.float().cpu().numpy().astype(np.float64) - y_ref.cpu().numpy().astype(np.float64)) ** 2))
    assert abs(got - exp) <= 1e-12 * exp
    assert float(w4.sq_error(y[:0], y_ref[:0]).cpu()[0]) == 0.0


@pytest.mark.parametrize("seed,salient", [(1, True), (2, False)])
def test_awq_search_near_oracle_optimum(w4, gpu, seed, salient):
    """The GPU search picks an exponent whose (oracle) output error is within 2% of the
    oracle's best; with salient input channels on ordinary weights it improves on RTN."""
    from bit_group_quantized_w4_amd import awq

    _say(f"awq search seed={seed} salient={salient}")
    W, xb, W_dev, x = _awq_case(gpu, seed=seed, N=128, K=512, T=64)
    if not salient:  # outlier channels carry outlier weights too (the 70B-class recipe)
        S = np.argsort(-np.abs(pins.bf16_values(xb)).mean(axis=0))[:5]
        W[:, S] *= 20
        W_dev = torch.from_numpy(W).to(gpu)
    res = awq.search(W_dev, x)
    k_ref, _, _, err_ref = oracle.awq_search_ref(W, xb)
    m = w4.channel_absmean(x).cpu().numpy().astype(np.float64)
    s_k, inv_k = oracle.candidate_scales_ref(m, awq.ALPHAS[res["k"]])
    err_at_k = oracle.awq_output_error_ref(W, xb, s_k, inv_k)
    assert err_at_k <= 1.02 * err_ref.min(), f"k={res['k']} (oracle {k_ref}): {err_at_k} vs {err_ref.min()}"
    g = np.asarray(res["errors"])
    assert np.allclose(g, err_ref, rtol=0.05), "per-candidate errors"
    if salient:
        assert res["k"] > 0 and g[res["k"]] < 0.9 * g[0], "channel scaling should help here"


# ----------------------------------------------------------------------------
# GPTQ (the library runs it in fp32; the oracle in fp64)
# ----------------------------------------------------------------------------

def _gptq(w4, W_np, xb_np, gpu, scale_dtype=torch.float32):
    from bit_group_quantized_w4_amd import gptq
    W = torch.from_numpy(W_np).to(gpu)
    x = torch.from_numpy(xb_np.view(np.int16)).to(gpu).view(torch.bfloat16)
    q, d = gptq.quantize(W, x, scale_dtype=scale_dtype)
    qc, dc = w4.unpack(q, d, *W_np.shape)
    torch.cuda.synchronize()
    return qc.cpu().numpy(), _scale_bits(dc) if scale_dtype == torch.bfloat16 else dc.cpu().numpy()


@pytest.mark.parametrize("inputs", ["identity", "zero"])
def test_gptq_without_coupling_is_rtn(w4, gpu, inputs):
    """Calibration inputs whose Hessian couples no columns (a multiple of the identity, or all
    zero): nothing propagates, so codes and scales equal RTN's bit for bit."""
    _say(f"gptq {inputs} inputs")
    K = 256
    W = pins.toy_weights(4, N=70, K=K)  # 70 rows: a partial wavefront
    if inputs == "identity":
        xb = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    else:
        xb = np.zeros((8, K), dtype=np.uint16)
    qc, dc = _gptq(w4, W, xb, gpu)
    q_ref, d_ref = oracle.rtn_quantize_ref(W)
    assert np.array_equal(dc.view(np.uint32), d_ref.view(np.uint32)), "scales differ from RTN"
    assert np.array_equal(qc, q_ref), "codes differ from RTN"


def _gptq_compare(W, xb, qc, dc, q_ref, d_ref, what, rows=None):
    Wr = W if rows is None else W[rows]
    # The library's column loop and corrections run in fp32 (the factor in fp64), the
    # oracle's in fp64: a code decided the other way next to a tie is possible, and it
    # changes the later, error-fed weights of its row and with them that row's later
    # group maxima.  In measured runs every code was equal and scales agreed within 3e-5.
    frac = float(np.mean(qc == q_ref))
    assert frac >= 0.999, f"{what}: only {frac:.5f} of the codes equal the fp64 oracle's"
    rel = np.abs(dc.astype(np.float64) / d_ref.astype(np.float64) - 1.0)
    assert np.mean(rel <= 1e-5) >= 0.99 and rel.max() <= 0.05, f"{what}: scales drift (max {rel.max():.2e})"
    e_gpu = oracle.output_error_ref(Wr, qc, dc, xb)
    e_ref = oracle.output_error_ref(Wr, q_ref, d_ref, xb)
    q_rtn, d_rtn = oracle.rtn_quantize_ref(Wr)
    e_rtn = oracle.output_error_ref(Wr, q_rtn, d_rtn, xb)
    assert abs(e_gpu / e_ref - 1.0) <= 0.005, f"{what}: output error {e_gpu:.4e} vs oracle {e_ref:.4e}"
    assert e_gpu < 0.9 * e_rtn, f"{what}: GPTQ {e_gpu:.4e} should beat RTN {e_rtn:.4e}"
    return frac, e_gpu / e_rtn


def test_gptq_matches_oracle(w4, gpu):
    """Correlated calibration inputs, ragged rows, eight blocks: the fp32 library against the
    fp64 oracle -- codes equal but for near-tie decisions, scales equal or within rounding,
    the same output error, well below RTN's."""
    _say("gptq 300x1024, T=256, correlated inputs")
    W, xb = pins.gptq_correlated_inputs(seed=11, N=300, K=1024, T=256)
    qc, dc = _gptq(w4, W, xb, gpu)
    q_ref, d_ref = oracle.gptq_ref(W, xb)
    _gptq_compare(W, xb, qc, dc, q_ref, d_ref, "300x1024")


def test_gptq_full_size_70b_gate_sampled(w4, gpu):
    """The 70B-class gate matrix (28672 x 8192) with 256 calibration rows of the 70B recipe
    (outlier channels).  Rows are independent given the factor, so the oracle quantizes a
    sample of rows with its own fp64 factor."""
    from bit_group_quantized_w4_amd import gptq
    _say("gptq 70b gate full size")
    m = next(mm for mm in workloads.WORKLOADS["stack_70b"].matrices if mm.name == "gate")
    W = workloads.weight("stack_70b", 2, "gate", gpu)
    x = workloads.activations("stack_70b", 2, "gate", 256, gpu)
    q, d = gptq.quantize(W, x)
    qc, dc = w4.unpack(q, d, m.N, m.K)
    rows = np.unique(np.concatenate([[0, m.N - 1], np.random.default_rng(4).choice(m.N, 30)]))
    idx = torch.as_tensor(rows, device=gpu)
    qc = qc.index_select(0, idx).cpu().numpy()
    dc = dc.index_select(0, idx).cpu().numpy()
    W_rows = W.index_select(0, idx).cpu().numpy()
    xb = _bits(x)
    del q, d, W
    torch.cuda.empty_cache()
    U = oracle.gptq_factor_ref(oracle.gptq_hessian_ref(xb))
    q_ref, d_ref = oracle.gptq_quantize_ref(W_rows, U)
    _gptq_compare(W_rows, xb, qc, dc, q_ref, d_ref, "70b gate sampled")


@pytest.mark.parametrize("N,K", [(1, 128), (65, 128), (3, 384)])
def test_gptq_small_shapes(w4, gpu, N, K):
    """One row, one block (no correction product after it), a row past a full wavefront."""
    _say(f"gptq small {N}x{K}")
    W, xb = pins.gptq_correlated_inputs(seed=N + K, N=N, K=K, T=96)
    qc, dc = _gptq(w4, W, xb, gpu)
    q_ref, d_ref = oracle.gptq_ref(W, xb)
    assert np.mean(qc == q_ref) >= 0.99
    e_gpu = oracle.output_error_ref(W, qc, dc, xb)
    e_ref = oracle.output_error_ref(W, q_ref, d_ref, xb)
    assert abs(e_gpu / e_ref - 1.0) <= 0.005, f"output error {e_gpu:.4e} vs oracle {e_ref:.4e}"


def _random_cases(n_cases=36, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        N = int(rng.integers(1, 3000))
        K = 128 * int(rng.integers(1, 40))
        M = int(rng.choice([1, 1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 17, 33, 40]))
        path = ["auto", "mfma", "gemv"][i % 3]
        sd = ["f32", "bf16"][(i // 3) % 2]
        cases.append((N, K, M, path, sd))
    return cases


@pytest.mark.parametrize("N,K,M,path,scale_dtype", _random_cases())
def test_linear_random_shapes(w4, gpu, N, K, M, path, scale_dtype):
    """Seeded random shapes (ragged rows, any group count, 1-40 rows of x), every path and
    both scale formats, single and batched with a second linear of another K."""
    _say(f"random N={N} K={K} M={M} path={path} scales={scale_dtype}")
    sd = torch.bfloat16 if scale_dtype == "bf16" else torch.float32
    W = torch.from_numpy(workloads.random_weight(N, K, seed=N * 131 + K)).to(gpu)
    q, d = w4.quantize_rtn(W, scale_dtype=sd)
    x = workloads.random_activations(M, K, seed=M * 7 + K, device=gpu)
    y = w4.linear(x, q, d, N, path=path)
    q_ref, d_ref = oracle.rtn_quantize_ref(W.cpu().numpy(), scale_dtype)
    y_ref, absdot = oracle.w4_linear_ref(_bits(x), q_ref, d_ref)
    check_y(y, y_ref, absdot, f"random {N}x{K} M={M} {path} {scale_dtype}")
    # the same linear batched with another of a different K: identical bits
    K2 = 128 * (1 + (K // 128) % 7)
    W2 = torch.from_numpy(workloads.random_weight(37, K2, seed=K2)).to(gpu)
    q2, d2 = w4.quantize_rtn(W2, scale_dtype=sd)
    x2 = workloads.random_activations(M, K2, seed=M + K2, device=gpu)
    # (the batch may run another configuration than the single call, so both are held to
    # the oracle rather than to each other)
    ys = w4.linear_batched([(x, q, d, N, torch.empty((M, N), dtype=torch.bfloat16, device=gpu)),
                            (x2, q2, d2, 37, torch.empty((M, 37), dtype=torch.bfloat16, device=gpu))], path=path)
    check_y(ys[0], y_ref, absdot, "random batched")
    q2r, d2r = oracle.rtn_quantize_ref(W2.cpu().numpy(), scale_dtype)
    y2_ref, absdot2 = oracle.w4_linear_ref(_bits(x2), q2r, d2r)
    check_y(ys[1], y2_ref, absdot2, "random batched second")


def test_gptq_16bit_scales(w4, gpu):
    """16-bit scales: with an identity Hessian, RTN's 16-bit codes and scales bit for bit;
    with correlated inputs, the fp64 oracle's codes and bf16 scales."""
    _say("gptq 16-bit scales")
    K = 256
    W = pins.toy_weights(5, N=70, K=K)
    xI = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    qc, dc = _gptq(w4, W, xI, gpu, S16)
    q_ref, d_ref = oracle.rtn_quantize_ref(W, "bf16")
    assert np.array_equal(dc, d_ref) and np.array_equal(qc, q_ref), "identity Hessian must give RTN (16-bit)"
    W, xb = pins.gptq_correlated_inputs(seed=13, N=200, K=768, T=192)
    qc, dc = _gptq(w4, W, xb, gpu, S16)
    q_ref, d_ref = oracle.gptq_ref(W, xb, scale_dtype="bf16")
    assert np.mean(qc == q_ref) >= 0.999
    assert np.mean(dc == d_ref) >= 0.99
    e_gpu = oracle.output_error_ref(W, qc, dc, xb)
    e_ref = oracle.output_error_ref(W, q_ref, d_ref, xb)
    assert abs(e_gpu / e_ref - 1.0) <= 0.005, f"output error {e_gpu:.4e} vs oracle {e_ref:.4e}"
