"""Python binding of libw4.so: group-wise INT4 (RTN) quantization and the W4A16
linear layer on AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of quantization and of the linear runs
in the HIP kernels behind the C ABI declared in include/w4.h.  PyTorch provides
device memory and the current stream; nothing here computes on the CPU and
there is no fallback.  Importing this module fails loudly when libw4.so has not
been built (build it with ``python -m bit_group_quantized_w4_amd._build``).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4.so")

W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_HIP, W4_ERR_ARG, W4_ERR_SCRATCH = range(7)
PATHS = {"auto": 0, "gemv": 1, "mfma": 2}
GROUP = 128

_VP, _I64, _INT, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
MAX_BATCH = 64


class LinearDesc(ctypes.Structure):
    """ctypes mirror of w4_linear_desc."""

    _fields_ = [("x", _VP), ("M", _I64), ("K", _I64), ("q_packed", _VP), ("d_packed", _VP),
                ("N", _I64), ("y", _VP)]


class ChainLinear(ctypes.Structure):
    """ctypes mirror of w4_chain_linear."""

    _fields_ = [("x", _VP), ("M", _I64), ("K", _I64), ("q_packed", _VP), ("d_packed", _VP),
                ("N", _I64), ("y", _VP), ("stage", _I64)]


class ChainPlanC(ctypes.Structure):
    """ctypes mirror of w4_chain_plan."""

    _I32 = ctypes.c_int32
    _fields_ = [("workspace", _VP), ("linears", _I32), ("stages", _I32), ("items", _I32), ("blocks", _I32),
                ("config", _I32), ("lds_bytes", _I32), ("rows_per_item", _I32), ("waves_per_block", _I32),
                ("scale_bytes", _I32), ("rows", _I32), ("trace", _I32), ("reserved", _I32)]


# (name, restype, argtypes) of every symbol include/w4.h declares
SIGNATURES = {
    "w4_status_str": (ctypes.c_char_p, [_INT]),
    "w4_last_hip_error": (_INT, []),
    "w4_group_size": (_INT, []),
    "w4_packed_bytes": (_SZ, [_I64, _I64]),
    "w4_scale_count": (_SZ, [_I64, _I64]),
    "w4_quantize_rtn": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP]),
    "w4_linear": (_INT, [_VP, _I64, _I64, _VP, _VP, _I64, _VP, _VP]),
    "w4_linear_ex": (_INT, [_VP, _I64, _I64, _VP, _VP, _I64, _VP, _INT, _VP]),
    "w4_linear_batched": (_INT, [ctypes.POINTER(LinearDesc), _INT, _INT, _VP]),
    # fp32 outputs
    "w4_linear_f32": (_INT, [_VP, _I64, _I64, _VP, _VP, _I64, _VP, _INT, _VP]),
    "w4_linear_f32_s16": (_INT, [_VP, _I64, _I64, _VP, _VP, _I64, _VP, _INT, _VP]),
    "w4_linear_batched_f32": (_INT, [ctypes.POINTER(LinearDesc), _INT, _INT, _VP]),
    "w4_pack": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP, _VP]),
    "w4_unpack": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP, _VP]),
    # 16-bit (bf16) scales
    "w4_quantize_rtn_s16": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP]),
    "w4_linear_s16": (_INT, [_VP, _I64, _I64, _VP, _VP, _I64, _VP, _INT, _VP]),
    "w4_linear_batched_s16": (_INT, [ctypes.POINTER(LinearDesc), _INT, _INT, _VP]),
    "w4_pack_s16": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP, _VP]),
    "w4_unpack_s16": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP, _VP]),
    # channel scaling before RTN (AWQ)
    "w4_channel_absmean": (_INT, [_VP, _I64, _I64, _VP, _VP]),
    "w4_awq_scales": (_INT, [_VP, _I64, ctypes.c_double, _VP, _VP, _VP]),
    "w4_quantize_rtn_scaled": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP, _VP]),
    "w4_quantize_rtn_scaled_s16": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP, _VP]),
    "w4_scale_activations": (_INT, [_VP, _I64, _I64, _VP, _VP, _VP]),
    "w4_linear_awq": (_INT, [_VP, _I64, _I64, _VP, _VP, _I64, _VP, _VP, _VP]),
    "w4_sq_error": (_INT, [_VP, _VP, _I64, _VP, _VP]),
    # split launches (draft verification widths)
    "w4_split_workspace_bytes": (_SZ, []),
    "w4_split_workspace_init": (_INT, [_VP, _SZ, _VP]),
    "w4_split_workspace_error": (_INT, [_VP, ctypes.POINTER(ctypes.c_uint32), _VP]),
    "w4_linear_batched_split": (_INT, [ctypes.POINTER(LinearDesc), _INT, _INT, _VP, _SZ, _VP]),
    "w4_linear_batched_split_s16": (_INT, [ctypes.POINTER(LinearDesc), _INT, _INT, _VP, _SZ, _VP]),
    "w4_linear_batched_split_f32": (_INT, [ctypes.POINTER(LinearDesc), _INT, _INT, _VP, _SZ, _VP]),
    # chained decode pass
    "w4_chain_workspace_bytes": (_SZ, [_I64]),
    "w4_chain_prepare": (_INT, [ctypes.POINTER(ChainLinear), _I64, _VP, _SZ, ctypes.POINTER(ChainPlanC), _VP]),
    "w4_chain_prepare_s16": (_INT, [ctypes.POINTER(ChainLinear), _I64, _VP, _SZ, ctypes.POINTER(ChainPlanC), _VP]),
    "w4_chain_prepare_noalloc": (_INT, [ctypes.POINTER(ChainLinear), _I64, ctypes.POINTER(ChainPlanC), _VP]),
    "w4_chain_run": (_INT, [ctypes.POINTER(ChainPlanC), _VP]),
    "w4_chain_error": (_INT, [ctypes.POINTER(ChainPlanC), ctypes.POINTER(ctypes.c_uint32), _VP]),
    "w4_chain_trace": (_INT, [ctypes.POINTER(ChainPlanC), _VP, _SZ, _VP]),
    # GPTQ steps
    "w4_gptq_damp": (_INT, [_VP, _I64, ctypes.c_double, _VP]),
    "w4_gptq_hessian": (_INT, [_VP, _I64, _I64, _VP, _VP]),
    "w4_gptq_factor_workspace_bytes": (_SZ, [_I64]),
    "w4_gptq_inverse_factor": (_INT, [_VP, _I64, _VP, _SZ, _VP, _VP]),
    "w4_gptq_update": (_INT, [_VP, _I64, _I64, _I64, _VP, _VP, _VP]),
    "w4_dense_linear_f32": (_INT, [_VP, _I64, _I64, _VP, _I64, _VP, _VP]),
    "w4_gptq_block": (_INT, [_VP, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
    "w4_gptq_block_s16": (_INT, [_VP, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
}


class W4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.w4_status_str(status).decode()
        if status == W4_ERR_HIP:
            msg += f" (hipError_t {_lib.w4_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: the HIP library must be built first "
            "(python -m bit_group_quantized_w4_amd._build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library():
    """The loaded ctypes handle of libw4.so."""
    return _lib


def _check(status, where):
    if status != W4_OK:
        raise W4Error(status, where)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _one_device(tensors, what):
    """The single device of `tensors`: every buffer of one call must live on the
    GPU whose stream runs it."""
    devs = {t.device for t in tensors if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError(f"{what}: tensors on several devices ({sorted(str(d) for d in devs)})")
    return devs.pop() if devs else None


def packed_bytes(N, K):
    return int(_lib.w4_packed_bytes(N, K))


def scale_count(N, K):
    return int(_lib.w4_scale_count(N, K))


# Scale formats: fp32, or bf16 (16-bit scales; the *_s16 entry points).
SCALE_DTYPES = (torch.float32, torch.bfloat16)


def _scale_dtype(d):
    if not isinstance(d, torch.Tensor) or d.dtype not in SCALE_DTYPES:
        raise TypeError("scales must be a float32 or bfloat16 torch.Tensor")
    return d.dtype


def _empty_packed(N, K, device, scale_dtype=torch.float32):
    nb, ns = packed_bytes(N, K), scale_count(N, K)
    if nb == 0:
        _check(W4_ERR_SHAPE, "packed buffers")
    return (torch.empty(nb, dtype=torch.uint8, device=device),
            torch.empty(ns, dtype=scale_dtype, device=device))


def quantize_rtn(W, out=None, scale_dtype=torch.float32):
    """fp32 weight [N, K] on the GPU -> (codes uint8 [packed_bytes], scales [scale_count]),
    both in the library's native layout.  scale_dtype torch.bfloat16 stores 16-bit scales
    (the codes are then taken against the stored bf16 value)."""
    N, K = W.shape
    if out is not None:
        scale_dtype = _scale_dtype(out[1])
    elif scale_dtype not in SCALE_DTYPES:
        raise TypeError("scale_dtype must be torch.float32 or torch.bfloat16")
    q, d = out if out is not None else _empty_packed(N, K, W.device, scale_dtype)
    fn, name = ((_lib.w4_quantize_rtn_s16, "w4_quantize_rtn_s16") if scale_dtype == torch.bfloat16
                else (_lib.w4_quantize_rtn, "w4_quantize_rtn"))
    _check(fn(_dev(W, torch.float32, "W"), N, K, _dev(q, torch.uint8, "q"), _dev(d, scale_dtype, "d"),
              _stream(W)), name)
    return q, d


OUT_DTYPES = (torch.bfloat16, torch.float32)


class SplitWorkspace:
    """Device workspace of the split launches (w4_split_workspace_init): pass it
    as `workspace=` to linear / linear_batched.  Calls that use one workspace
    must be ordered (one stream)."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.nbytes = int(_lib.w4_split_workspace_bytes())
        self.buffer = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
        self.init()

    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def init(self):
        """(Re-)initialise on the current stream."""
        _check(_lib.w4_split_workspace_init(ctypes.c_void_p(self.buffer.data_ptr()), self.nbytes, self._stream()),
               "w4_split_workspace_init")

    def error(self):
        """The workspace's error flag (synchronises the current stream)."""
        flag = ctypes.c_uint32(0)
        _check(_lib.w4_split_workspace_error(ctypes.c_void_p(self.buffer.data_ptr()), ctypes.byref(flag),
                                             self._stream()), "w4_split_workspace_error")
        return int(flag.value)


def linear(x, q, d, N, path="auto", out=None, out_dtype=torch.bfloat16, workspace=None):
    """y [M, N] = x [M, K] bf16 times the dequantized weight (native q, d).

    y is bf16 by default; with out_dtype=torch.float32 (or an fp32 `out`) it is the
    fp32 value the kernel accumulated, before rounding (the *_f32 entry points).
    With a SplitWorkspace the MFMA kernel may split K across blocks
    (w4_linear_batched_split*)."""
    M, K = x.shape
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in OUT_DTYPES:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    if y.shape != (M, N):
        raise ValueError("out must be [M, N]")
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    if workspace is not None:
        return linear_batched([(x, q, d, N, y)], path=path, workspace=workspace)[0]
    _one_device([x, q, d, y], "linear")
    sd = _scale_dtype(d)
    if out_dtype == torch.float32:
        fn, name = ((_lib.w4_linear_f32_s16, "w4_linear_f32_s16") if sd == torch.bfloat16
                    else (_lib.w4_linear_f32, "w4_linear_f32"))
    else:
        fn, name = ((_lib.w4_linear_s16, "w4_linear_s16") if sd == torch.bfloat16
                    else (_lib.w4_linear_ex, "w4_linear"))
    _check(fn(_dev(x, torch.bfloat16, "x"), M, K, _dev(q, torch.uint8, "q"), _dev(d, sd, "d"), N,
              _dev(y, out_dtype, "y"), PATHS[path], _stream(x)), name)
    return y


def linear_batched(items, path="auto", workspace=None):
    """Several independent linears in one launch.

    items: sequence of (x [M, K] bf16, q, d, N, y [M, N]) with every y
    preallocated; at most MAX_BATCH items.  y is bf16 throughout, or fp32
    throughout (fp32 scales only: w4_linear_batched_f32).  With a
    SplitWorkspace, the split entry points.  Returns the list of y.
    """
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    items = list(items)
    descs = (LinearDesc * max(1, len(items)))()
    stream = None
    sd = _scale_dtype(items[0][2]) if items else torch.float32
    od = items[0][4].dtype if items else torch.bfloat16
    if od not in OUT_DTYPES or (od == torch.float32 and sd != torch.float32):
        raise TypeError("outputs must be bf16, or fp32 with fp32 scales")
    for i, (x, q, d, N, y) in enumerate(items):
        M, K = x.shape
        if y.shape != (M, N):
            raise ValueError(f"item {i}: y must be [M, N]")
        if _scale_dtype(d) != sd:
            raise TypeError("all items of a batch must use the same scale dtype")
        descs[i] = LinearDesc(_dev(x, torch.bfloat16, "x").value, M, K, _dev(q, torch.uint8, "q").value,
                              _dev(d, sd, "d").value, N, _dev(y, od, "y").value)
        stream = stream or _stream(x)
    dev = _one_device([t for it in items for t in (it[0], it[1], it[2], it[4])], "linear_batched")
    if workspace is not None and dev is not None and workspace.buffer.device != dev:
        raise ValueError(f"linear_batched: the workspace is on {workspace.buffer.device}, the linears on {dev}")
    # the descriptor structs of every variant have the same layout (pointers and int64s)
    if od == torch.float32:
        name = "w4_linear_batched_f32"
    else:
        name = "w4_linear_batched_s16" if sd == torch.bfloat16 else "w4_linear_batched"
    if workspace is not None:
        name = name.replace("batched", "batched_split")
        _check(getattr(_lib, name)(descs, len(items), PATHS[path], ctypes.c_void_p(workspace.buffer.data_ptr()),
                                   workspace.nbytes, stream), name)
    else:
        _check(getattr(_lib, name)(descs, len(items), PATHS[path], stream), name)
    return [it[4] for it in items]


class ChainPlan:
    """A prepared chain (w4_chain_prepare): its device workspace (None when the
    library's static scratch holds it: w4_chain_prepare_noalloc), the plan, and
    references to every tensor it names, which must stay alive while it is used."""

    def __init__(self, workspace, plan, tensors, device):
        self.workspace = workspace
        self.plan = plan
        self.device = device
        self._tensors = tensors

    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def run(self):
        """Enqueue one pass on the current stream (w4_chain_run)."""
        _check(_lib.w4_chain_run(ctypes.byref(self.plan), self._stream()), "w4_chain_run")

    def trace(self, stamps):
        """Per-item timestamps of later passes into `stamps` (int64 device tensor of
        at least 3 * items values), or None to stop (w4_chain_trace)."""
        if stamps is None:
            _check(_lib.w4_chain_trace(ctypes.byref(self.plan), None, 0, self._stream()), "w4_chain_trace")
            self._stamps = None
            return
        ptr = _dev(stamps, torch.int64, "stamps")
        if stamps.device != torch.device(self.device):
            raise ValueError(f"stamps must be on the chain's device {self.device} (got {stamps.device})")
        _check(_lib.w4_chain_trace(ctypes.byref(self.plan), ptr, stamps.numel(), self._stream()), "w4_chain_trace")
        self._stamps = stamps  # kept alive while the chain may write it

    def error(self):
        """The workspace's error flag (synchronises the current stream; w4_chain_error)."""
        flag = ctypes.c_uint32(0)
        _check(_lib.w4_chain_error(ctypes.byref(self.plan), ctypes.byref(flag), self._stream()), "w4_chain_error")
        return int(flag.value)

    @property
    def info(self):
        p = self.plan
        return {"linears": p.linears, "stages": p.stages, "items": p.items, "blocks": p.blocks,
                "rows_per_item": p.rows_per_item * 16, "waves_per_block": p.waves_per_block,
                "lds_bytes": p.lds_bytes, "scale_bytes": p.scale_bytes, "x_rows": p.rows}


def chain_prepare(stages, noalloc=False):
    """Prepare a chained pass (w4_chain_prepare): a decode step (M = 1) or a
    verification pass (M = 2..16).

    stages: sequence of stages, each a sequence of (x [M, K] bf16, q, d, N,
    y [M, N] bf16), one M throughout, with d fp32 scales throughout or bf16
    (16-bit) scales throughout.  A linear whose x lies in outputs of earlier
    stages uses no value of it before that value is written.  Returns a ChainPlan; plan.run() enqueues one
    pass.  With noalloc (fp32 scales only), the workspace is the library's
    static scratch (w4_chain_prepare_noalloc): nothing is allocated, and only
    the most recent such plan of a GPU may be run.
    """
    flat = [(s, it) for s, stage in enumerate(stages) for it in stage]
    if not flat:
        raise ValueError("a chain needs at least one linear")
    descs = (ChainLinear * len(flat))()
    tensors = []
    dev = None
    sd = _scale_dtype(flat[0][1][2])
    for i, (s, (x, q, d, N, y)) in enumerate(flat):
        M, K = x.shape
        if y.shape != (M, N):
            raise ValueError(f"linear {i}: y must be [M, N]")
        if _scale_dtype(d) != sd:
            raise TypeError("all linears of a chain must use the same scale dtype")
        # the fp32- and bf16-scale descriptor structs have the same layout
        descs[i] = ChainLinear(_dev(x, torch.bfloat16, "x").value, M, K, _dev(q, torch.uint8, "q").value,
                               _dev(d, sd, "d").value, N, _dev(y, torch.bfloat16, "y").value, s)
        tensors += [x, q, d, y]
        dev = dev or x.device
    _one_device(tensors, "chain_prepare")
    plan = ChainPlanC()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if noalloc:
        if sd != torch.float32:
            raise TypeError("w4_chain_prepare_noalloc takes fp32 scales")
        _check(_lib.w4_chain_prepare_noalloc(descs, len(flat), ctypes.byref(plan), stream), "w4_chain_prepare_noalloc")
        return ChainPlan(None, plan, tensors, dev)
    nbytes = int(_lib.w4_chain_workspace_bytes(len(flat)))
    if nbytes == 0:
        _check(W4_ERR_ARG, "w4_chain_workspace_bytes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    fn, name = ((_lib.w4_chain_prepare_s16, "w4_chain_prepare_s16") if sd == torch.bfloat16
                else (_lib.w4_chain_prepare, "w4_chain_prepare"))
    _check(fn(descs, len(flat), ctypes.c_void_p(ws.data_ptr()), nbytes, ctypes.byref(plan), stream), name)
    return ChainPlan(ws, plan, tensors, dev)


def pack(q_canon, d_canon, out=None):
    """Canonical codes int8 [N, K] and scales [N, K/128] (fp32 or bf16) -> native (q, d)."""
    N, K = q_canon.shape
    sd = _scale_dtype(d_canon)
    q, d = out if out is not None else _empty_packed(N, K, q_canon.device, sd)
    fn, name = (_lib.w4_pack_s16, "w4_pack_s16") if sd == torch.bfloat16 else (_lib.w4_pack, "w4_pack")
    _check(fn(_dev(q_canon, torch.int8, "q_canon"), _dev(d_canon, sd, "d_canon"), N, K,
              _dev(q, torch.uint8, "q"), _dev(d, sd, "d"), _stream(q_canon)), name)
    return q, d


def unpack(q, d, N, K):
    """Native (q, d) -> canonical codes int8 [N, K] and scales [N, K/128] (d's dtype)."""
    sd = _scale_dtype(d)
    qc = torch.empty((N, K), dtype=torch.int8, device=q.device)
    dc = torch.empty((N, K // GROUP), dtype=sd, device=q.device)
    fn, name = (_lib.w4_unpack_s16, "w4_unpack_s16") if sd == torch.bfloat16 else (_lib.w4_unpack, "w4_unpack")
    _check(fn(_dev(q, torch.uint8, "q"), _dev(d, sd, "d"), N, K, _dev(qc, torch.int8, "q_canon"),
              _dev(dc, sd, "d_canon"), _stream(q)), name)
    return qc, dc


# ----------------------------------------------------------------------------
# channel scaling before RTN (AWQ); the search itself is in .awq
# ----------------------------------------------------------------------------

def channel_absmean(x):
    """mean |x[:, j]| over the rows of a bf16 [T, K] tensor -> fp32 [K]."""
    T, K = x.shape
    m = torch.empty(K, dtype=torch.float32, device=x.device)
    _check(_lib.w4_channel_absmean(_dev(x, torch.bfloat16, "x"), T, K, _dev(m, torch.float32, "m"), _stream(x)),
           "w4_channel_absmean")
    return m


def awq_scales(m, alpha):
    """Candidate channel scales for one exponent: (s, inv_s), fp32 [K]."""
    K = m.shape[0]
    s = torch.empty(K, dtype=torch.float32, device=m.device)
    inv = torch.empty(K, dtype=torch.float32, device=m.device)
    _check(_lib.w4_awq_scales(_dev(m, torch.float32, "m"), K, float(alpha), _dev(s, torch.float32, "s"),
                              _dev(inv, torch.float32, "inv_s"), _stream(m)), "w4_awq_scales")
    return s, inv


def quantize_rtn_scaled(W, s, scale_dtype=torch.float32, out=None):
    """RTN of W * diag(s) (columns scaled in fp32) -> native (q, d)."""
    N, K = W.shape
    if out is not None:
        scale_dtype = _scale_dtype(out[1])
    q, d = out if out is not None else _empty_packed(N, K, W.device, scale_dtype)
    fn, name = ((_lib.w4_quantize_rtn_scaled_s16, "w4_quantize_rtn_scaled_s16") if scale_dtype == torch.bfloat16
                else (_lib.w4_quantize_rtn_scaled, "w4_quantize_rtn_scaled"))
    _check(fn(_dev(W, torch.float32, "W"), _dev(s, torch.float32, "s"), N, K, _dev(q, torch.uint8, "q"),
              _dev(d, scale_dtype, "d"), _stream(W)), name)
    return q, d


def scale_activations(x, inv_s, out=None):
    """x' = bf16(x * inv_s) column by column, bf16 [M, K]."""
    M, K = x.shape
    xo = out if out is not None else torch.empty_like(x)
    _check(_lib.w4_scale_activations(_dev(x, torch.bfloat16, "x"), M, K, _dev(inv_s, torch.float32, "inv_s"),
                                     _dev(xo, torch.bfloat16, "x_out"), _stream(x)), "w4_scale_activations")
    return xo


def linear_awq(x, q, d, N, inv_s, out=None):
    """y = W_hat' (x * inv_s): x is scaled while the dot2 kernel stages it (fp32 scales)."""
    M, K = x.shape
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(_lib.w4_linear_awq(_dev(x, torch.bfloat16, "x"), M, K, _dev(q, torch.uint8, "q"),
                              _dev(d, torch.float32, "d"), N, _dev(inv_s, torch.float32, "inv_s"),
                              _dev(y, torch.bfloat16, "y"), _stream(x)), "w4_linear_awq")
    return y


def sq_error(y, y_ref, out=None):
    """Sum of (y - y_ref)^2 in fp64 (y bf16, y_ref fp32, same shape) as a 1-element GPU tensor."""
    if y.shape != y_ref.shape:
        raise ValueError("y and y_ref must have the same shape")
    o = out if out is not None else torch.empty(1, dtype=torch.float64, device=y.device)
    _check(_lib.w4_sq_error(_dev(y, torch.bfloat16, "y"), _dev(y_ref, torch.float32, "y_ref"), y.numel(),
                            _dev(o, torch.float64, "out"), _stream(y)), "w4_sq_error")
    return o


def gptq_damp(H, damp=0.01):
    """In place on H (fp64 [K, K]): zero diagonal entries become 1, then damp * mean(diag) is added."""
    if H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise ValueError("H must be square")
    _check(_lib.w4_gptq_damp(_dev(H, torch.float64, "H"), H.shape[0], float(damp), _stream(H)), "w4_gptq_damp")
    return H


def gptq_block(W, U, b0, q_canon, d_canon, err):
    """GPTQ column loop over columns b0 .. b0+127 of W (fp32 [N, K], not modified): codes into
    q_canon (int8 [N, K]), the group scale into d_canon ([N, K/128], fp32, or bfloat16 for
    16-bit scales), the column errors into err (fp32 [128, N])."""
    N, K = W.shape
    if U.shape != (K, K) or q_canon.shape != (N, K) or d_canon.shape != (N, K // 128) or err.shape != (128, N):
        raise ValueError("shape mismatch")
    sd = _scale_dtype(d_canon)
    fn = _lib.w4_gptq_block_s16 if sd == torch.bfloat16 else _lib.w4_gptq_block
    _check(fn(_dev(W, torch.float32, "W"), N, K, int(b0), _dev(U, torch.float32, "U"),
              _dev(q_canon, torch.int8, "q_canon"), _dev(d_canon, sd, "d_canon"),
              _dev(err, torch.float32, "err"), _stream(W)), "w4_gptq_block")


def gptq_hessian(x, out=None):
    """H = (2/T) x^T x, fp64 [K, K], from bf16 calibration rows x [T, K] (w4_gptq_hessian)."""
    T, K = x.shape
    H = out if out is not None else torch.empty((K, K), dtype=torch.float64, device=x.device)
    _check(_lib.w4_gptq_hessian(_dev(x, torch.bfloat16, "x"), T, K, _dev(H, torch.float64, "H"), _stream(x)),
           "w4_gptq_hessian")
    return H


def gptq_inverse_factor(H, out=None):
    """U (fp32 [K, K], upper triangular) with H^-1 = U^T U for a damped fp64 Hessian
    (w4_gptq_inverse_factor; H is not modified)."""
    K = H.shape[0]
    if H.dim() != 2 or H.shape[1] != K:
        raise ValueError("H must be square")
    nb = int(_lib.w4_gptq_factor_workspace_bytes(K))
    if nb == 0:
        _check(W4_ERR_SHAPE, "w4_gptq_factor_workspace_bytes")
    work = torch.empty(nb, dtype=torch.uint8, device=H.device)
    U = out if out is not None else torch.empty((K, K), dtype=torch.float32, device=H.device)
    _check(_lib.w4_gptq_inverse_factor(_dev(H, torch.float64, "H"), K, ctypes.c_void_p(work.data_ptr()), nb,
                                       _dev(U, torch.float32, "U"), _stream(H)), "w4_gptq_inverse_factor")
    return U


def gptq_update(W, U, b0, err):
    """In place: W[:, b0+128:] -= err^T U[b0:b0+128, b0+128:] (w4_gptq_update); err fp32 [128, N]."""
    N, K = W.shape
    if U.shape != (K, K) or err.shape != (128, N):
        raise ValueError("shape mismatch")
    _check(_lib.w4_gptq_update(_dev(W, torch.float32, "W"), N, K, int(b0), _dev(U, torch.float32, "U"),
                               _dev(err, torch.float32, "err"), _stream(W)), "w4_gptq_update")


def dense_linear_f32(x, W, out=None):
    """y = x W^T in fp32 (x bf16 [T, K], W fp32 [N, K]; w4_dense_linear_f32)."""
    T, K = x.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K]")
    y = out if out is not None else torch.empty((T, N), dtype=torch.float32, device=x.device)
    _check(_lib.w4_dense_linear_f32(_dev(x, torch.bfloat16, "x"), T, K, _dev(W, torch.float32, "W"), N,
                                    _dev(y, torch.float32, "y"), _stream(x)), "w4_dense_linear_f32")
    return y


class W4Linear:
    """A quantized weight held in native layout, callable on bf16 activations."""

    def __init__(self, q, d, N, K):
        self.q, self.d, self.N, self.K = q, d, N, K

    @classmethod
    def from_float(cls, W, scale_dtype=torch.float32):
        q, d = quantize_rtn(W, scale_dtype=scale_dtype)
        return cls(q, d, W.shape[0], W.shape[1])

    def __call__(self, x, path="auto", out=None):
        return linear(x, self.q, self.d, self.N, path=path, out=out)


__all__ = [
    "GROUP", "LIB_PATH", "MAX_BATCH", "OUT_DTYPES", "PATHS", "SCALE_DTYPES", "SIGNATURES", "LinearDesc", "W4Error",
    "W4Linear", "SplitWorkspace",
    "awq_scales", "channel_absmean", "library", "linear", "linear_awq", "linear_batched",
    "quantize_rtn_scaled", "scale_activations", "sq_error",
    "pack", "packed_bytes", "quantize_rtn", "scale_count", "unpack",
]
