"""C-ABI contract tests that need no GPU.

They load libw4.so, check that every function include/w4.h declares is
exported, and exercise argument validation: each call here is rejected on the
host before any HIP call is made, so nothing is launched.
"""

import ctypes
import os
import re

import pytest

import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "w4.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_HIP, ERR_ARG = range(6)
FAKE = 0x10000000  # a 256-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("w4_quantize_rtn", "w4_linear", "w4_linear_ex", "w4_pack", "w4_unpack"):
        assert must in names


def test_every_declared_symbol_is_exported(w4):
    lib = ctypes.CDLL(w4.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in w4.SIGNATURES, f"binding lacks {name}"
    assert set(w4.SIGNATURES) == set(declared_functions())


def test_status_strings(w4):
    lib = w4.library()
    for s in range(7):
        assert lib.w4_status_str(s).decode().startswith("W4_")
    assert b"unknown" in lib.w4_status_str(99)
    assert lib.w4_last_hip_error() == 0


def test_size_helpers(w4):
    lib = w4.library()
    assert lib.w4_group_size() == 128
    assert lib.w4_packed_bytes(2560, 9216) == 2560 * 9216 // 2
    assert lib.w4_scale_count(2560, 9216) == 2560 * 72
    assert lib.w4_packed_bytes(37, 384) == 48 * 512 // 2  # rows padded to 16, K to 512
    assert lib.w4_scale_count(37, 384) == 48 * 4  # groups padded to whole quads of 4
    assert lib.w4_scale_count(16, 2560) == 16 * 20
    assert lib.w4_packed_bytes(0, 128) == 0
    for N, K in ((16, 100), (16, 0), (16, -128), (-1, 128)):
        assert lib.w4_packed_bytes(N, K) == 0 and lib.w4_scale_count(N, K) == 0


def _linear(lib, x=FAKE, M=1, K=128, q=FAKE + 0x100000, d=FAKE + 0x200000, N=16,
            y=FAKE + 0x300000, path=0):
    return lib.w4_linear_ex(x, M, K, q, d, N, y, path, None)


def test_linear_validation(w4):
    lib = w4.library()
    assert _linear(lib, K=100) == ERR_SHAPE
    assert _linear(lib, K=0) == ERR_SHAPE
    assert _linear(lib, M=-1) == ERR_SHAPE
    assert _linear(lib, N=-3) == ERR_SHAPE
    assert _linear(lib, M=262141) == ERR_SHAPE
    assert _linear(lib, x=None) == ERR_NULL
    assert _linear(lib, q=None) == ERR_NULL
    assert _linear(lib, d=None) == ERR_NULL
    assert _linear(lib, y=None) == ERR_NULL
    assert _linear(lib, x=FAKE + 8) == ERR_ALIGN
    assert _linear(lib, q=FAKE + 0x100004) == ERR_ALIGN
    assert _linear(lib, d=FAKE + 0x200004) == ERR_ALIGN
    assert _linear(lib, y=FAKE + 0x300001) == ERR_ALIGN
    assert _linear(lib, y=FAKE) == ERR_ARG  # output aliases x
    assert _linear(lib, y=FAKE + 0x100000 + 64) == ERR_ARG  # output inside the codes
    assert _linear(lib, path=7) == ERR_ARG
    # operands addressed with 32-bit offsets: codes below 2 GiB, x at most 1 GiB
    assert _linear(lib, N=1 << 17, K=1 << 15, x=None) == ERR_SHAPE  # codes exactly 2 GiB
    assert _linear(lib, N=(1 << 17) - 16, K=1 << 15, x=None) == ERR_NULL  # just below
    assert _linear(lib, M=(1 << 14) + 1, K=1 << 15, x=None) == ERR_SHAPE  # x above 1 GiB
    assert _linear(lib, M=1 << 14, K=1 << 15, x=None) == ERR_NULL  # x exactly 1 GiB
    # empty problems are valid no-ops that launch nothing, even with NULL buffers
    assert _linear(lib, M=0, x=None, y=None) == OK
    assert _linear(lib, N=0, q=None, d=None, y=None) == OK
    assert lib.w4_linear(None, 0, 128, None, None, 16, None, None) == OK


def test_f32_output_validation(w4):
    """fp32 outputs: 4-byte alignment, and 4 bytes per output in the overlap checks."""
    lib = w4.library()
    x, q, d, y = FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    assert lib.w4_linear_f32(x, 16, 128, q, d, 16, y + 2, 0, None) == ERR_ALIGN
    assert lib.w4_linear_f32(x, 16, 128, q, d, 16, x - 768, 0, None) == ERR_ARG  # 1 KiB from x - 768 reaches x
    assert lib.w4_linear_f32(x, 1, 100, q, d, 16, y, 0, None) == ERR_SHAPE
    assert lib.w4_linear_f32(x, 1, 128, q, d, 16, None, 0, None) == ERR_NULL
    assert lib.w4_linear_f32(x, 1, 128, q, d, 16, y, 9, None) == ERR_ARG
    assert lib.w4_linear_f32_s16(x, 1, 128, q, d + 2, 16, y, 0, None) == ERR_ALIGN
    assert lib.w4_linear_f32_s16(x, 1, 128, q, d, 16, d + 16, 0, None) == ERR_ARG  # inside the scales
    assert lib.w4_linear_f32(None, 0, 128, None, None, 16, None, 0, None) == OK
    arr = (w4.LinearDesc * 2)(w4.LinearDesc(x, 1, 128, q, d, 16, y), w4.LinearDesc(x, 1, 128, q, d, 16, y + 32))
    assert lib.w4_linear_batched_f32(arr, 2, 0, None) == ERR_ARG  # 64 fp32 bytes from y overlap y + 32


def test_batched_validation(w4):
    lib = w4.library()
    D = w4.LinearDesc
    good = dict(x=FAKE, M=1, K=128, q_packed=FAKE + 0x100000, d_packed=FAKE + 0x200000, N=16,
                y=FAKE + 0x300000)
    arr = (D * 65)(*[D(**good) for _ in range(65)])
    assert lib.w4_linear_batched(arr, 65, 0, None) == ERR_ARG  # more than W4_MAX_BATCH
    assert lib.w4_linear_batched(arr, -1, 0, None) == ERR_ARG
    assert lib.w4_linear_batched(arr, 2, 9, None) == ERR_ARG  # unknown path
    assert lib.w4_linear_batched(None, 2, 0, None) == ERR_NULL
    assert lib.w4_linear_batched(None, 0, 0, None) == OK
    # two outputs that overlap each other
    a = (D * 2)(D(**good), D(**dict(good, y=FAKE + 0x300010)))
    assert lib.w4_linear_batched(a, 2, 0, None) == ERR_ARG
    # an output that overlaps another element's input
    a = (D * 2)(D(**good), D(**dict(good, x=FAKE + 0x400000, y=FAKE)))
    assert lib.w4_linear_batched(a, 2, 0, None) == ERR_ARG
    # the first bad element's status is returned, nothing is launched
    a = (D * 2)(D(**good), D(**dict(good, K=100)))
    assert lib.w4_linear_batched(a, 2, 0, None) == ERR_SHAPE
    a = (D * 2)(D(**dict(good, M=0)), D(**dict(good, q_packed=None)))
    assert lib.w4_linear_batched(a, 2, 0, None) == ERR_NULL
    # the dot2 kernel stages x in 64 KiB of LDS: K above 32768 is refused for it
    big = (D * 1)(D(**dict(good, K=30720 + 512)))
    assert lib.w4_linear_batched(big, 1, 1, None) == ERR_SHAPE


def test_split_validation(w4):
    """The split entry points refuse a bad workspace before anything is launched."""
    lib = w4.library()
    D = w4.LinearDesc
    MiB = 1 << 20
    assert lib.w4_split_workspace_bytes() == 4 * MiB
    good = dict(x=FAKE, M=8, K=128, q_packed=FAKE + 0x100000, d_packed=FAKE + 0x200000, N=16,
                y=FAKE + 0x300000)
    a = (D * 1)(D(**good))
    ws = FAKE + 0x1000000
    for fn in (lib.w4_linear_batched_split, lib.w4_linear_batched_split_s16):
        assert fn(a, 1, 2, None, 4 * MiB, None) == ERR_NULL
        assert fn(a, 1, 2, ws + 16, 4 * MiB, None) == ERR_ALIGN
        assert fn(a, 1, 2, ws, 4 * MiB - 256, None) == ERR_ARG  # smaller than W4_SPLIT_WORKSPACE_BYTES
        assert fn(a, 1, 2, FAKE + 0x280000, 4 * MiB, None) == ERR_ARG  # covers the codes, scales and y
        assert fn(a, 1, 2, FAKE - 4 * MiB + 256, 4 * MiB, None) == ERR_ARG  # its last bytes are x
        bad = (D * 1)(D(**dict(good, K=100)))
        assert fn(bad, 1, 2, ws, 4 * MiB, None) == ERR_SHAPE
        assert fn(a, 1, 9, ws, 4 * MiB, None) == ERR_ARG  # unknown path
    f = (D * 1)(D(**dict(good, y=FAKE + 0x300002)))
    assert lib.w4_linear_batched_split_f32(f, 1, 2, ws, 4 * MiB, None) == ERR_ALIGN  # fp32 y needs 4 bytes
    assert lib.w4_split_workspace_init(None, 4 * MiB, None) == ERR_NULL
    assert lib.w4_split_workspace_init(ws + 64, 4 * MiB, None) == ERR_ALIGN
    assert lib.w4_split_workspace_init(ws, MiB, None) == ERR_ARG
    flag = ctypes.c_uint32(7)
    assert lib.w4_split_workspace_error(None, ctypes.byref(flag), None) == ERR_NULL
    assert lib.w4_split_workspace_error(ws, None, None) == ERR_NULL


def test_chain_validation(w4):
    """w4_chain_prepare refuses bad chains on the host, before any HIP call."""
    lib = w4.library()
    C = w4.ChainLinear
    plan = w4.ChainPlanC()
    # the timestamp aid checks its arguments before touching the workspace
    assert lib.w4_chain_trace(None, None, 0, None) == ERR_NULL
    assert lib.w4_chain_trace(ctypes.byref(plan), None, 0, None) == ERR_NULL  # no workspace
    plan.workspace = FAKE
    plan.items = 10
    assert lib.w4_chain_trace(ctypes.byref(plan), FAKE + 4, 30, None) == ERR_ALIGN
    assert lib.w4_chain_trace(ctypes.byref(plan), FAKE, 29, None) == ERR_ARG  # 3 values per item
    # the binding passes only a GPU int64 tensor on the chain's device (a host
    # address would become a write target of the kernel)
    import torch
    cp = w4.ChainPlan(None, plan, [], torch.device("cuda", 0))
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.trace(torch.zeros(30, dtype=torch.int64))
    with pytest.raises(TypeError, match="torch.Tensor"):
        cp.trace([0] * 30)
    # every buffer of one call on one device
    assert w4._one_device([torch.zeros(2), torch.zeros(3)], "t") == torch.device("cpu")
    with pytest.raises(ValueError, match="several devices"):
        w4._one_device([torch.zeros(2), torch.empty(2, device="meta")], "t")
    plan = w4.ChainPlanC()
    assert lib.w4_chain_workspace_bytes(0) == 0
    assert lib.w4_chain_workspace_bytes(8193) == 0
    n = lib.w4_chain_workspace_bytes(4)
    assert n > 0 and lib.w4_chain_workspace_bytes(8) > n
    ws = FAKE + 0x4000000

    def lin(i, stage, **kw):
        base = FAKE + i * 0x100000
        d = dict(x=base, M=1, K=256, q_packed=base + 0x10000, d_packed=base + 0x20000, N=32,
                 y=base + 0x30000, stage=stage)
        d.update(kw)
        return C(**d)

    def prep(items, nbytes=None, workspace=ws):
        arr = (C * max(1, len(items)))(*items)
        nb = nbytes if nbytes is not None else lib.w4_chain_workspace_bytes(max(1, len(items)))
        return lib.w4_chain_prepare(arr, len(items), workspace, nb, ctypes.byref(plan), None)

    assert prep([]) == ERR_ARG                                      # count 0
    assert lib.w4_chain_prepare(None, 1, ws, n, ctypes.byref(plan), None) == ERR_NULL
    assert prep([lin(0, 0)], workspace=None) == ERR_NULL
    assert prep([lin(0, 0)], workspace=ws + 4) == ERR_ALIGN
    assert prep([lin(0, 0, M=0)]) == ERR_SHAPE                      # M from 1 to 16
    assert prep([lin(0, 0, M=17)]) == ERR_SHAPE
    assert prep([lin(0, 0, M=2), lin(1, 1, M=1)]) == ERR_SHAPE      # one M for the whole chain
    assert prep([lin(0, 0, K=100)]) == ERR_SHAPE
    assert prep([lin(0, 0, K=30720 + 512)]) == ERR_SHAPE            # at M = 1 x must fit the LDS stage
    assert prep([lin(0, 0, N=0)]) == ERR_SHAPE
    assert prep([lin(0, 0, q_packed=None)]) == ERR_NULL
    assert prep([lin(0, 0, x=FAKE + 2)]) == ERR_ALIGN
    assert prep([lin(0, 1)]) == ERR_ARG                             # stages start at 0
    assert prep([lin(0, 0), lin(1, 2)]) == ERR_ARG                  # and step by 0 or 1
    assert prep([lin(0, 0), lin(1, 1), lin(2, 0)]) == ERR_ARG       # never go back
    # two outputs of one chain overlap
    assert prep([lin(0, 0), lin(1, 1, y=FAKE + 0x30000 + 16)]) == ERR_ARG
    # an output on weights
    assert prep([lin(0, 0), lin(1, 1, y=FAKE + 0x10000)]) == ERR_ARG
    # an output over the input of its own stage, or of an earlier one, or the
    # same 128-byte line
    assert prep([lin(0, 0, y=FAKE)]) == ERR_ARG
    assert prep([lin(0, 0), lin(1, 1, y=FAKE + 256)]) == ERR_ARG
    # x of stage 0 ends at byte 0x310 of its line; y of stage 1 starts at 0x320
    assert prep([lin(0, 0, x=FAKE + 0x210, K=128), lin(1, 1, y=FAKE + 0x320)]) == ERR_ARG
    # an input that lies partly in an earlier output and partly outside all of them
    assert prep([lin(0, 0, N=64), lin(1, 1, x=FAKE + 0x30000, K=256)]) == ERR_ARG
    # an output sharing a 128-byte line (but no byte) with weights: the codes of
    # linear 0 end at 0x12010, linear 1 writes from 0x12040
    assert prep([lin(0, 0, q_packed=FAKE + 0x10010), lin(1, 1, y=FAKE + 0x12040)]) == ERR_ARG
    # the same with scales (32 x 256 fp32: 512 bytes from 0x20010)
    assert prep([lin(0, 0, d_packed=FAKE + 0x20010), lin(1, 1, y=FAKE + 0x20220)]) == ERR_ARG
    # a later stage reading x from the line of an earlier output without reading
    # that output (stage 0 writes 64 bytes at 0x30000; stage 1 reads from 0x30040)
    assert prep([lin(0, 0), lin(1, 1, x=FAKE + 0x30040, K=128)]) == ERR_ARG
    # at M > 1 every x and y spans M rows: outputs of 2 x 32 values (128 bytes)
    # overlap where one row would not, and an input of 2 x 256 values is not
    # covered by an earlier output of 2 x 128
    assert prep([lin(0, 0, M=2), lin(1, 1, M=2, y=FAKE + 0x30040)]) == ERR_ARG
    assert prep([lin(0, 0, M=2, N=128), lin(1, 1, M=2, x=FAKE + 0x30000, K=256)]) == ERR_ARG
    # workspace too small, or overlapping a buffer of the chain
    assert prep([lin(0, 0), lin(1, 1)], nbytes=64) == ERR_ARG
    assert prep([lin(0, 0), lin(1, 1)], workspace=FAKE + 0x100000 + 0x30000 - 0x40) == ERR_ARG  # reaches y of linear 1
    # the 16-bit-scale variant checks the same (its descriptors have the same layout)
    arr = (C * 2)(lin(0, 0), lin(1, 2))
    assert lib.w4_chain_prepare_s16(arr, 2, ws, n, ctypes.byref(plan), None) == ERR_ARG
    arr = (C * 1)(lin(0, 0, M=17))
    assert lib.w4_chain_prepare_s16(arr, 1, ws, n, ctypes.byref(plan), None) == ERR_SHAPE
    # an output over 16-bit scales (32 x 256: 128 native scale slots of 2 bytes)
    arr = (C * 2)(lin(0, 0), lin(1, 1, y=FAKE + 0x20000 + 64))
    assert lib.w4_chain_prepare_s16(arr, 2, ws, n, ctypes.byref(plan), None) == ERR_ARG


def test_s16_validation(w4):
    """The 16-bit-scale entry points check their arguments like the fp32 ones."""
    lib = w4.library()
    src, q, d = FAKE, FAKE + 0x100000, FAKE + 0x200000
    assert lib.w4_quantize_rtn_s16(src, 16, 100, q, d, None) == ERR_SHAPE
    assert lib.w4_quantize_rtn_s16(None, 16, 128, q, d, None) == ERR_NULL
    assert lib.w4_quantize_rtn_s16(src, 16, 128, q, d + 8, None) == ERR_ALIGN
    assert lib.w4_quantize_rtn_s16(src, 16, 128, q, q + 512, None) == ERR_ARG  # codes/scales overlap
    assert lib.w4_quantize_rtn_s16(src, 0, 128, None, None, None) == OK
    x, y = FAKE + 0x300000, FAKE + 0x400000
    assert lib.w4_linear_s16(x, 1, 100, q, d, 16, y, 0, None) == ERR_SHAPE
    assert lib.w4_linear_s16(None, 1, 128, q, d, 16, y, 0, None) == ERR_NULL
    assert lib.w4_linear_s16(x, 1, 128, q, d + 2, 16, y, 0, None) == ERR_ALIGN
    assert lib.w4_linear_s16(x, 1, 128, q, d, 16, x, 0, None) == ERR_ARG  # output aliases x
    assert lib.w4_linear_s16(x, 1, 128, q, d, 16, d + 16, 0, None) == ERR_ARG  # output inside the scales
    assert lib.w4_linear_s16(x, 1, 128, q, d, 16, y, 7, None) == ERR_ARG
    assert lib.w4_linear_s16(None, 0, 128, None, None, 16, None, 0, None) == OK
    assert lib.w4_linear_batched_s16(None, 2, 0, None) == ERR_NULL
    assert lib.w4_linear_batched_s16(None, 0, 0, None) == OK
    assert lib.w4_pack_s16(src, d + 0x40000, 16, 256, None, d, None) == ERR_NULL
    assert lib.w4_pack_s16(src, d + 0x40000 + 1, 16, 256, q, d, None) == ERR_ALIGN  # canonical bf16: 2 bytes
    assert lib.w4_unpack_s16(q, d, -2, 256, src, src + 0x40000, None) == ERR_SHAPE


def test_quantize_pack_unpack_validation(w4):
    lib = w4.library()
    q, d, src = FAKE, FAKE + 0x100000, FAKE + 0x200000
    assert lib.w4_quantize_rtn(src, 16, 100, q, d, None) == ERR_SHAPE
    assert lib.w4_quantize_rtn(None, 16, 128, q, d, None) == ERR_NULL
    assert lib.w4_quantize_rtn(src + 4, 16, 128, q, d, None) == ERR_ALIGN
    assert lib.w4_quantize_rtn(src, 16, 128, q, q + 512, None) == ERR_ARG  # codes/scales overlap
    assert lib.w4_quantize_rtn(src, 0, 128, None, None, None) == OK
    assert lib.w4_pack(src, d + 0x40000, 16, 256, None, d, None) == ERR_NULL
    assert lib.w4_pack(src + 8, d + 0x40000, 16, 256, q, d, None) == ERR_ALIGN
    assert lib.w4_pack(src, d + 0x40000, 16, 127, q, d, None) == ERR_SHAPE
    assert lib.w4_unpack(q, d, 16, 256, None, src, None) == ERR_NULL
    assert lib.w4_unpack(q, d, 16, 256, src, src + 64, None) == ERR_ARG
    assert lib.w4_unpack(q, d, -2, 256, src, src + 0x40000, None) == ERR_SHAPE


def test_python_binding_rejects_cpu_tensors(w4):
    import torch

    with pytest.raises(ValueError):
        w4.quantize_rtn(torch.zeros(16, 128))
    with pytest.raises(ValueError):
        w4.linear(torch.zeros(1, 128, dtype=torch.bfloat16), torch.zeros(1024, dtype=torch.uint8),
                  torch.zeros(16), 16)


# ----------------------------------------------------------------------------
# byte accounting used by the roofline (hand-computed figures)
# ----------------------------------------------------------------------------

def test_algorithmic_bytes():
    # N*K/2 codes + 4*N*K/128 scales + 2*M*K x + 2*M*N y
    assert workloads.algorithmic_bytes(1, 2560, 9216) == 12_557_312
    assert workloads.algorithmic_bytes(8, 2560, 9216) == 12_722_176
    assert workloads.algorithmic_bytes(1, 9216, 2560) == 11_796_480 + 737_280 + 5_120 + 18_432
    assert round(workloads.stack_bytes("stack_4b", 1) / 1e9, 3) == 1.859
    assert round(workloads.stack_bytes("stack_27b", 1) / 1e9, 3) == 11.600
    assert round(workloads.stack_bytes("stack_70b", 1) / 1e9, 3) == 36.391
    assert workloads.stack_weights("stack_70b") == 80 * (2 * 8192 * 8192 + 2 * 1024 * 8192 + 3 * 28672 * 8192)


def test_gptq_validation(w4):
    lib = w4.library()
    W, U, qc, dc, err = FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 0x4000000

    def block(W=W, N=64, K=256, b0=0, U=U, qc=qc, dc=dc, err=err):
        return lib.w4_gptq_block(W, N, K, b0, U, qc, dc, err, None)

    assert block(N=0) == OK  # empty: nothing launched
    for bad in (dict(K=200), dict(K=0), dict(N=-1), dict(b0=64), dict(b0=256), dict(b0=-128)):
        assert block(**bad) == ERR_SHAPE, bad
    for none in ("W", "U", "qc", "dc", "err"):
        assert block(**{none: None}) == ERR_NULL, none
    assert block(W=W + 4) == ERR_ALIGN
    assert block(qc=qc + 8) == ERR_ALIGN
    assert block(U=U + 2) == ERR_ALIGN
    assert block(err=W + 64) == ERR_ARG  # output inside the weights
    assert block(dc=qc + 16) == ERR_ARG  # two outputs overlap
    assert block(qc=U + 1024) == ERR_ARG  # output inside U

    assert lib.w4_gptq_block_s16(W, 64, 256, 0, U, qc, dc + 1, err, None) == ERR_ALIGN
    assert lib.w4_gptq_block_s16(W, 64, 256, 64, U, qc, dc, err, None) == ERR_SHAPE
    assert lib.w4_gptq_block_s16(W, 64, 256, 0, U, qc, W + 2, err, None) == ERR_ARG

    assert lib.w4_gptq_damp(FAKE, 0, 0.01, None) == ERR_SHAPE
    assert lib.w4_gptq_damp(None, 16, 0.01, None) == ERR_NULL
    assert lib.w4_gptq_damp(FAKE + 4, 16, 0.01, None) == ERR_ALIGN
    for bad in (-0.5, float("nan"), float("inf")):
        assert lib.w4_gptq_damp(FAKE, 16, bad, None) == ERR_ARG, bad


def test_gptq_driver_rejects_bad_inputs(w4):
    import torch
    from bit_group_quantized_w4_amd import gptq
    W = torch.zeros((16, 256))
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        gptq.quantize(W, x)  # CPU tensors
