"""CPU checks of the C ABI boundary: the library loads, exports every function
include/*.h declares, and rejects bad arguments before touching the GPU.
No call here reaches a kernel launch."""
import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import pytest

import grouped_gemm_qgemm_amd as q
from grouped_gemm_qgemm_amd import QG, QgTensor, QgPagedKV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = []
    for h in HEADERS:
        txt = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s+\*?([A-Za-z_]\w*)\s*\(", txt, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("QG")))


@pytest.fixture(scope="module")
def lib():
    return q.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"qgemm_w4", "qgemm_w4_nk", "qgemm_w4_epilogue", "grouped_gemm", "grouped_gemm_w4", "grouped_gemm_epilogue",
            "grouped_gemm_w4_epilogue", "k_matmul_ragged_paged_scale", "kv_matmul_ragged_paged_scale",
            "qg_status_string", "qg_read_contiguous", "qg_read_strips", "qg_mfma_loop",
            "qg_empty_launch"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for s in range(9):
        assert len(q.status_string(s)) > 0
    assert q.status_string(0) == "ok"
    assert lib.qg_version() >= 100


class Buf:
    """Host memory standing in for device pointers: validation never dereferences them."""
    def __init__(self):
        self.keep = []

    def t(self, shape, dtype, misalign=False):
        n = int(np.prod(shape)) if len(shape) else 1
        arr = np.zeros(max(n, 1) * 4 + 64, np.uint8)
        self.keep.append(arr)
        base = arr.ctypes.data
        base = (base + 15) & ~15
        d = QgTensor()
        d.data = base + (2 if misalign else 0)
        d.dtype = dtype
        d.rank = len(shape)
        for i, s in enumerate(shape):
            d.shape[i] = s
        return d


def w4_call(lib, c, a, b, s, gs=128, pf=8):
    return lib.qgemm_w4(ctypes.byref(c), ctypes.byref(a), ctypes.byref(b), ctypes.byref(s), gs, pf, None)


def w4_args(bb, M=4, N=64, K=256, gs=128):
    return (bb.t((M, N), QG.F16), bb.t((M, K), QG.F16), bb.t((K // 8, N), QG.U32), bb.t((K // gs, N), QG.F16))


def test_w4_rejections(lib):
    bb = Buf()
    c, a, b, s = w4_args(bb)
    # rank-2 requirement (the page's stated error)
    assert w4_call(lib, bb.t((1, 4, 64), QG.F16), a, b, s) == QG.ERR_RANK
    assert w4_call(lib, c, a, bb.t((32 * 64,), QG.U32), s) == QG.ERR_RANK
    assert w4_call(lib, c, bb.t((4, 256), QG.BF16), b, s) == QG.ERR_DTYPE
    # bf16 activations need bf16 scales and output (one type for all three)
    cb, ab, sb = bb.t((4, 64), QG.BF16), bb.t((4, 256), QG.BF16), bb.t((2, 64), QG.BF16)
    assert w4_call(lib, cb, ab, b, s) == QG.ERR_DTYPE
    assert w4_call(lib, c, ab, b, sb) == QG.ERR_DTYPE
    assert w4_call(lib, cb, ab, b, sb, pf=4) == QG.ERR_UNSUPPORTED
    assert w4_call(lib, c, a, bb.t((32, 64), QG.I32), s) == QG.ERR_DTYPE
    assert w4_call(lib, c, a, b, s, pf=4) == QG.ERR_UNSUPPORTED
    assert w4_call(lib, c, a, b, s, gs=100) == QG.ERR_SHAPE
    assert w4_call(lib, c, a, b, bb.t((16, 64), QG.F16), gs=16) == QG.ERR_UNSUPPORTED
    assert w4_call(lib, c, a, bb.t((31, 64), QG.U32), s) == QG.ERR_SHAPE
    assert w4_call(lib, c, a, b, bb.t((3, 64), QG.F16)) == QG.ERR_SHAPE
    assert w4_call(lib, bb.t((5, 64), QG.F16), a, b, s) == QG.ERR_SHAPE
    c2, a2, b2, s2 = w4_args(bb, N=60)
    assert w4_call(lib, c2, a2, b2, s2) == QG.ERR_ALIGN
    assert w4_call(lib, bb.t((4, 64), QG.F16, misalign=True), a, b, s) == QG.ERR_ALIGN
    nul = bb.t((4, 64), QG.F16)
    nul.data = None
    assert w4_call(lib, nul, a, b, s) == QG.ERR_NULL
    assert lib.qgemm_w4(None, ctypes.byref(a), ctypes.byref(b), ctypes.byref(s), 128, 8, None) == QG.ERR_NULL


def test_w4_nk_rejections(lib):
    bb = Buf()
    M, N, K = 4, 64, 256
    c, a = bb.t((M, N), QG.F16), bb.t((M, K), QG.F16)
    b_nk, s_nk = bb.t((N, K // 8), QG.U32), bb.t((N, K // 128), QG.F16)
    call = lambda b, s, c=c: lib.qgemm_w4_nk(ctypes.byref(c), ctypes.byref(a), ctypes.byref(b), ctypes.byref(s),
                                             128, 8, None)
    assert call(bb.t((K // 8, N), QG.U32), s_nk) == QG.ERR_SHAPE     # [K/8, N] is qgemm_w4's layout
    assert call(b_nk, bb.t((K // 128, N), QG.F16)) == QG.ERR_SHAPE
    assert call(b_nk, bb.t((N, K // 128), QG.BF16)) == QG.ERR_DTYPE
    assert call(bb.t((N * K // 8,), QG.U32), s_nk) == QG.ERR_RANK
    assert call(b_nk, s_nk, c=bb.t((0, N), QG.F16)) == QG.ERR_SHAPE   # rows disagree with A
    a0 = bb.t((0, K), QG.F16)
    assert lib.qgemm_w4_nk(ctypes.byref(bb.t((0, N), QG.F16)), ctypes.byref(a0), ctypes.byref(b_nk),
                           ctypes.byref(s_nk), 128, 8, None) == QG.OK


def test_w4_empty_problem_is_a_noop(lib):
    bb = Buf()
    c, a, b, s = w4_args(bb, M=0)
    assert w4_call(lib, c, a, b, s) == QG.OK


def test_w4_zero_depth_is_rejected(lib):
    """K = 0 (a zero-depth product) is refused before anything is launched."""
    bb = Buf()
    c, a, b, s = w4_args(bb, M=4, K=0)
    assert w4_call(lib, c, a, b, s) == QG.ERR_UNSUPPORTED
    nk = lib.qgemm_w4_nk(ctypes.byref(c), ctypes.byref(a), ctypes.byref(bb.t((64, 0), QG.U32)),
                         ctypes.byref(bb.t((64, 0), QG.F16)), 128, 8, None)
    assert nk == QG.ERR_UNSUPPORTED


def epi_call(lib, c, a, b, s, flags, bias=None, res=None, gs=128):
    r = lambda t: ctypes.byref(t) if t is not None else None
    return lib.qgemm_w4_epilogue(ctypes.byref(c), ctypes.byref(a), ctypes.byref(b), ctypes.byref(s), gs, 8,
                                 flags, r(bias), r(res), None)


def test_w4_epilogue_rejections(lib):
    bb = Buf()
    M, N, K = 4, 64, 256
    c, a, b, s = w4_args(bb, M=M, N=N, K=K)
    bias, res = bb.t((N,), QG.F16), bb.t((M, N), QG.F16)
    half = bb.t((M, N // 2), QG.F16)
    # unknown flag bits
    assert epi_call(lib, c, a, b, s, 8) == QG.ERR_INVALID_ARG
    assert epi_call(lib, c, a, b, s, -1) == QG.ERR_INVALID_ARG
    # a requested operand must be given
    assert epi_call(lib, c, a, b, s, q.EPI_BIAS) == QG.ERR_NULL
    assert epi_call(lib, c, a, b, s, q.EPI_RESIDUAL, bias=bias) == QG.ERR_NULL
    # bias: rank 1, the activations' type, N entries
    assert epi_call(lib, c, a, b, s, q.EPI_BIAS, bias=bb.t((1, N), QG.F16)) == QG.ERR_RANK
    assert epi_call(lib, c, a, b, s, q.EPI_BIAS, bias=bb.t((N,), QG.BF16)) == QG.ERR_DTYPE
    assert epi_call(lib, c, a, b, s, q.EPI_BIAS, bias=bb.t((N - 8,), QG.F16)) == QG.ERR_SHAPE
    # residual: shaped like the output
    assert epi_call(lib, c, a, b, s, q.EPI_RESIDUAL, res=bb.t((M * N,), QG.F16)) == QG.ERR_RANK
    assert epi_call(lib, c, a, b, s, q.EPI_RESIDUAL, res=bb.t((M, N), QG.BF16)) == QG.ERR_DTYPE
    assert epi_call(lib, c, a, b, s, q.EPI_RESIDUAL, res=bb.t((M, N - 8), QG.F16)) == QG.ERR_SHAPE
    # SiLU gate halves N: the output (and residual) are [M, N / 2]
    assert epi_call(lib, c, a, b, s, q.EPI_SILU_GATE) == QG.ERR_SHAPE
    assert epi_call(lib, half, a, b, s, q.EPI_SILU_GATE | q.EPI_RESIDUAL, res=res) == QG.ERR_SHAPE
    c2, a2, b2, s2 = w4_args(bb, M=M, N=72, K=K)   # N % 8 == 0 but N % 16 != 0
    assert epi_call(lib, bb.t((M, 36), QG.F16), a2, b2, s2, q.EPI_SILU_GATE) == QG.ERR_ALIGN
    # empty problems with valid epilogue operands are no-ops
    c0, a0, b0, s0 = w4_args(bb, M=0, N=N, K=K)
    assert epi_call(lib, bb.t((0, N // 2), QG.F16), a0, b0, s0, 7, bias=bias,
                    res=bb.t((0, N // 2), QG.F16)) == QG.OK
    assert epi_call(lib, c0, a0, b0, s0, 0) == QG.OK


def gg_call(lib, c, a, off, b, ids, usage, tb=1, splits=None):
    u = (ctypes.c_uint32 * 2)(*usage)
    sp = (ctypes.c_int32 * 2)(*splits) if splits is not None else None
    return lib.grouped_gemm(ctypes.byref(c), ctypes.byref(a), ctypes.byref(off), ctypes.byref(b),
                            ctypes.byref(ids), u, tb, sp, None)


def test_grouped_rejections(lib):
    bb = Buf()
    T, K, N, E, G = 32, 64, 48, 4, 4
    c, a = bb.t((T, N), QG.BF16), bb.t((T, K), QG.BF16)
    off, b, ids = bb.t((G + 1,), QG.U32), bb.t((E, N, K), QG.BF16), bb.t((G,), QG.I32)
    assert gg_call(lib, c, a, off, bb.t((E * N, K), QG.BF16), ids, [8, 4]) == QG.ERR_RANK
    assert gg_call(lib, c, bb.t((T, K), QG.F16), off, b, ids, [8, 4]) == QG.ERR_DTYPE
    assert gg_call(lib, c, a, bb.t((G,), QG.U32), b, ids, [8, 4]) == QG.ERR_SHAPE
    assert gg_call(lib, c, a, off, bb.t((E, N, K + 8), QG.BF16), ids, [8, 4]) == QG.ERR_SHAPE
    assert gg_call(lib, c, a, off, b, ids, [8, 5]) == QG.ERR_INVALID_ARG
    # transpose_b == 0 takes B as [E, K, N]: the [E, N, K] buffer no longer matches K
    assert gg_call(lib, c, a, off, b, ids, [8, 4], tb=0) == QG.ERR_SHAPE
    # an expert matrix beyond 32-bit byte offsets (shape only: validation never reads the buffers)
    big = QgTensor()
    big.data, big.dtype, big.rank = b.data, QG.BF16, 3
    big.shape[0], big.shape[1], big.shape[2] = E, 65536, 32768
    big_c = QgTensor()
    big_c.data, big_c.dtype, big_c.rank = c.data, QG.BF16, 2
    big_c.shape[0], big_c.shape[1] = T, 65536
    big_a = QgTensor()
    big_a.data, big_a.dtype, big_a.rank = a.data, QG.BF16, 2
    big_a.shape[0], big_a.shape[1] = T, 32768
    assert gg_call(lib, big_c, big_a, off, big, ids, [8, 4]) == QG.ERR_UNSUPPORTED
    assert gg_call(lib, c, a, off, b, ids, [8, 0]) == QG.OK       # nothing active: no-op
    u = (ctypes.c_uint32 * 2)(8, 4)
    assert lib.grouped_gemm(ctypes.byref(c), ctypes.byref(a), ctypes.byref(off), ctypes.byref(b),
                            ctypes.byref(ids), None, 1, None, None) == QG.ERR_NULL


def test_grouped_plane_split_rejections(lib):
    """a_plane_splits (fused LoRA QKV planes of A): shape and alignment checks."""
    bb = Buf()
    T, K, N, E, G = 32, 64, 48, 4, 4
    c, a, a3 = bb.t((T, N), QG.BF16), bb.t((T, K), QG.BF16), bb.t((3 * T, K), QG.BF16)
    off, b, ids = bb.t((G + 1,), QG.U32), bb.t((E, N, K), QG.BF16), bb.t((G,), QG.I32)
    assert gg_call(lib, c, a, off, b, ids, [8, 0], splits=(8, 16)) == QG.ERR_SHAPE    # A must hold 3 planes
    assert gg_call(lib, c, a3, off, b, ids, [8, 0]) == QG.ERR_SHAPE                    # planes off: A is [T, K]
    assert gg_call(lib, c, a3, off, b, ids, [8, 0], splits=(4, 8)) == QG.ERR_ALIGN
    assert gg_call(lib, c, a3, off, b, ids, [8, 0], splits=(40, 16)) == QG.ERR_SHAPE  # past N
    assert gg_call(lib, c, a3, off, b, ids, [8, 0], splits=(-8, 16)) == QG.ERR_SHAPE
    assert gg_call(lib, c, a3, off, b, ids, [8, 0], splits=(8, 16)) == QG.OK          # nothing active: no-op
    assert gg_call(lib, c, a, off, b, ids, [8, 0], splits=(0, 0)) == QG.OK


def gw_call(lib, c, a, off, b, s, ids, usage, gs=128, pf=8):
    u = (ctypes.c_uint32 * 2)(*usage)
    return lib.grouped_gemm_w4(ctypes.byref(c), ctypes.byref(a), ctypes.byref(off), ctypes.byref(b),
                               ctypes.byref(s), ctypes.byref(ids), u, gs, pf, None)


def test_grouped_w4_rejections(lib):
    bb = Buf()
    T, K, N, E, G = 32, 256, 48, 4, 4
    c, a = bb.t((T, N), QG.F16), bb.t((T, K), QG.F16)
    off, ids = bb.t((G + 1,), QG.U32), bb.t((G,), QG.I32)
    b, s = bb.t((E, K // 8, N), QG.U32), bb.t((E, K // 128, N), QG.F16)
    assert gw_call(lib, c, a, off, bb.t((E * K // 8, N), QG.U32), s, ids, [8, 4]) == QG.ERR_RANK
    assert gw_call(lib, c, bb.t((T, K), QG.BF16), off, b, s, ids, [8, 4]) == QG.ERR_DTYPE
    cb, ab, sb = bb.t((T, N), QG.BF16), bb.t((T, K), QG.BF16), bb.t((E, K // 128, N), QG.BF16)
    assert gw_call(lib, cb, ab, off, b, s, ids, [8, 4]) == QG.ERR_DTYPE      # bf16 a and c, f16 scales
    assert gw_call(lib, cb, ab, off, b, sb, ids, [8, 0]) == QG.OK            # all bf16: accepted (no-op)
    assert gw_call(lib, c, a, off, b, bb.t((E, K // 64, N), QG.F16), ids, [8, 4]) == QG.ERR_SHAPE
    assert gw_call(lib, c, a, off, b, bb.t((E + 1, K // 128, N), QG.F16), ids, [8, 4]) == QG.ERR_SHAPE
    assert gw_call(lib, c, a, bb.t((G,), QG.U32), b, s, ids, [8, 4]) == QG.ERR_SHAPE
    assert gw_call(lib, c, a, off, b, s, ids, [8, 4], pf=4) == QG.ERR_UNSUPPORTED
    assert gw_call(lib, c, a, off, b, bb.t((E, K // 96, N), QG.F16), ids, [8, 4], gs=96) == QG.ERR_SHAPE
    assert gw_call(lib, c, a, off, b, s, ids, [8, 5]) == QG.ERR_INVALID_ARG
    assert gw_call(lib, c, a, off, b, s, ids, [8, 0]) == QG.OK       # nothing active: no-op
    assert gw_call(lib, c, a, off, b, s, ids, [8, 4], gs=0) == QG.ERR_INVALID_ARG
    u = (ctypes.c_uint32 * 2)(8, 4)
    assert lib.grouped_gemm_w4(ctypes.byref(c), ctypes.byref(a), ctypes.byref(off), ctypes.byref(b),
                               ctypes.byref(s), ctypes.byref(ids), None, 128, 8, None) == QG.ERR_NULL


def test_grouped_epilogue_rejections(lib):
    bb = Buf()
    T, K, N, E, G = 32, 64, 48, 4, 4
    a, off, ids = bb.t((T, K), QG.BF16), bb.t((G + 1,), QG.U32), bb.t((G,), QG.I32)
    b = bb.t((E, N, K), QG.BF16)
    u = (ctypes.c_uint32 * 2)(8, 4)
    r = lambda t: ctypes.byref(t) if t is not None else None

    def ge(c, flags, bias=None, res=None, bm=b):
        return lib.grouped_gemm_epilogue(ctypes.byref(c), ctypes.byref(a), ctypes.byref(off), ctypes.byref(bm),
                                         ctypes.byref(ids), u, 1, None, flags, r(bias), r(res), None)
    c, half = bb.t((T, N), QG.BF16), bb.t((T, N // 2), QG.BF16)
    assert ge(c, 8) == QG.ERR_INVALID_ARG
    assert ge(c, q.EPI_BIAS) == QG.ERR_NULL
    assert ge(c, q.EPI_BIAS, bias=bb.t((N,), QG.BF16)) == QG.ERR_RANK          # one row per expert
    assert ge(c, q.EPI_BIAS, bias=bb.t((E - 1, N), QG.BF16)) == QG.ERR_SHAPE
    assert ge(c, q.EPI_BIAS, bias=bb.t((E, N), QG.F16)) == QG.ERR_DTYPE
    assert ge(c, q.EPI_RESIDUAL, res=bb.t((T, N // 2), QG.BF16)) == QG.ERR_SHAPE
    assert ge(c, q.EPI_SILU_GATE) == QG.ERR_SHAPE                              # output is N / 2 wide
    b40 = bb.t((E, 40, K), QG.BF16)                                           # 40 % 16 != 0
    assert ge(bb.t((T, 20), QG.BF16), q.EPI_SILU_GATE, bm=b40) == QG.ERR_ALIGN
    u[1] = 0
    assert ge(half, 7, bias=bb.t((E, N), QG.BF16), res=bb.t((T, N // 2), QG.BF16)) == QG.OK   # nothing active
    # W4 experts: f16 operands
    c4, a4 = bb.t((T, 24), QG.F16), bb.t((T, 256), QG.F16)
    b4, s4 = bb.t((E, 32, N), QG.U32), bb.t((E, 2, N), QG.F16)
    u[1] = 4

    def gw(c, flags, bias=None, res=None):
        return lib.grouped_gemm_w4_epilogue(ctypes.byref(c), ctypes.byref(a4), ctypes.byref(off), ctypes.byref(b4),
                                            ctypes.byref(s4), ctypes.byref(ids), u, 128, 8, flags, r(bias), r(res),
                                            None)
    assert gw(c4, q.EPI_SILU_GATE | q.EPI_BIAS) == QG.ERR_NULL
    assert gw(c4, q.EPI_SILU_GATE | q.EPI_BIAS, bias=bb.t((E, N), QG.BF16)) == QG.ERR_DTYPE
    assert gw(bb.t((T, N), QG.F16), q.EPI_SILU_GATE) == QG.ERR_SHAPE
    assert gw(c4, -1) == QG.ERR_INVALID_ARG
    u[1] = 0
    assert gw(c4, 7, bias=bb.t((E, N), QG.F16), res=bb.t((T, 24), QG.F16)) == QG.OK


def kp_call(lib, h, offs, w, isc, wsc, blocks, layer, gran=(1, 128, 128), cl=1, pt=1, maxp=2, scales=None,
            qgran=0, fused=False):
    g = (ctypes.c_int32 * 3)(*gran)
    kv = QgPagedKV()
    kv.blocks = blocks
    kv.cache_lengths = cl
    kv.page_table = pt
    kv.max_pages_per_seq = maxp
    if scales is not None:
        kv.scales = scales
    kv.quantization_granularity = qgran
    fn = lib.kv_matmul_ragged_paged_scale if fused else lib.k_matmul_ragged_paged_scale
    return fn(ctypes.byref(h), ctypes.byref(offs), ctypes.byref(w), ctypes.byref(isc), ctypes.byref(wsc), g,
              ctypes.byref(kv), layer, None)


def test_kv_and_fp8_cache_rejections(lib):
    bb = Buf()
    T, Kh, Hkv, D, B = 10, 256, 2, 128, 2
    N = Hkv * D
    h, offs, isc = bb.t((T, Kh), QG.BF16), bb.t((B + 1,), QG.U32), bb.t((T, 2), QG.F32)
    w, wsc = bb.t((Kh, N), QG.FP8_E4M3), bb.t((2, N // 128), QG.F32)
    w2, wsc2 = bb.t((Kh, 2 * N), QG.FP8_E4M3), bb.t((2, 2 * N // 128), QG.F32)
    blocks = bb.t((2, 2, 4, 16, Hkv, D), QG.BF16)
    q8 = bb.t((2, 2, 4, 16, Hkv, D), QG.FP8_E4M3)
    sc = lambda g: bb.t((2, 2, 4, 16, Hkv, D // g), QG.F32)
    # fused keys and values: the weight has 2 * Hkv * D columns
    assert kp_call(lib, h, offs, w, isc, wsc, blocks, 0, fused=True) == QG.ERR_SHAPE
    assert kp_call(lib, h, offs, w2, isc, wsc2, blocks, 0) == QG.ERR_SHAPE
    assert kp_call(lib, h, offs, w2, isc, wsc, blocks, 0, fused=True) == QG.ERR_SHAPE   # weight_scale columns
    # per-plane width must be a multiple of 128 (three 64-wide heads: 192)
    b3 = bb.t((2, 2, 4, 16, 3, 64), QG.BF16)
    assert kp_call(lib, h, offs, bb.t((Kh, 384), QG.FP8_E4M3), isc, bb.t((2, 3), QG.F32), b3, 0,
                   fused=True) == QG.ERR_SHAPE
    # e4m3 cache: scales required, shaped [L, 2, P, S, Hkv, D / G], f32; G in {32, 64, 128} dividing D
    assert kp_call(lib, h, offs, w, isc, wsc, q8, 0, qgran=128) == QG.ERR_RANK
    assert kp_call(lib, h, offs, w, isc, wsc, q8, 0, scales=sc(64), qgran=128) == QG.ERR_SHAPE
    assert kp_call(lib, h, offs, w, isc, wsc, q8, 0, scales=bb.t((2, 2, 4, 16, Hkv, 1), QG.BF16),
                   qgran=128) == QG.ERR_DTYPE
    assert kp_call(lib, h, offs, w, isc, wsc, q8, 0, scales=sc(16), qgran=16) == QG.ERR_UNSUPPORTED
    assert kp_call(lib, h, offs, w, isc, wsc, q8, 0, scales=sc(128), qgran=0) == QG.ERR_UNSUPPORTED
    q96 = bb.t((2, 2, 4, 16, 4, 96), QG.FP8_E4M3)
    assert kp_call(lib, h, offs, bb.t((Kh, 384), QG.FP8_E4M3), isc, bb.t((2, 3), QG.F32), q96, 0,
                   scales=bb.t((2, 2, 4, 16, 4, 1), QG.F32), qgran=64) == QG.ERR_UNSUPPORTED
    # a valid e4m3-cache call with no tokens is a no-op (validation passes)
    h0, isc0 = bb.t((0, Kh), QG.BF16), bb.t((0, 2), QG.F32)
    assert kp_call(lib, h0, offs, w2, isc0, wsc2, q8, 0, scales=sc(32), qgran=32, fused=True) == QG.OK
    assert kp_call(lib, h0, offs, w, isc0, wsc, q8, 1, scales=sc(128), qgran=128) == QG.OK


def test_kproj_rejections(lib):
    bb = Buf()
    T, Kh, N, B = 10, 256, 256, 2
    h, offs = bb.t((T, Kh), QG.BF16), bb.t((B + 1,), QG.U32)
    w, isc, wsc = bb.t((Kh, N), QG.FP8_E4M3), bb.t((T, 2), QG.F32), bb.t((2, 2), QG.F32)
    blocks = bb.t((2, 2, 4, 16, 2, 128), QG.BF16)
    assert kp_call(lib, h, offs, w, isc, wsc, blocks, 2) == QG.ERR_INVALID_ARG   # layer_idx >= L
    assert kp_call(lib, h, offs, w, isc, wsc, blocks, 0, gran=(1, 64, 128)) == QG.ERR_UNSUPPORTED
    assert kp_call(lib, h, offs, w, isc, wsc, bb.t((2, 4, 16, 2, 128), QG.BF16), 0) == QG.ERR_RANK
    assert kp_call(lib, h, offs, bb.t((Kh, N), QG.BF16), isc, wsc, blocks, 0) == QG.ERR_DTYPE
    assert kp_call(lib, h, offs, w, bb.t((T, 3), QG.F32), wsc, blocks, 0) == QG.ERR_SHAPE
    assert kp_call(lib, h, offs, w, isc, wsc, bb.t((2, 2, 4, 16, 1, 128), QG.BF16), 0) == QG.ERR_SHAPE
    assert kp_call(lib, bb.t((T, 200), QG.BF16), offs, bb.t((200, N), QG.FP8_E4M3), isc, wsc, blocks, 0) == QG.ERR_SHAPE
    assert kp_call(lib, h, offs, w, isc, wsc, blocks, 0, cl=None) == QG.ERR_NULL
    h0, isc0 = bb.t((0, Kh), QG.BF16), bb.t((0, 2), QG.F32)
    assert kp_call(lib, h0, offs, w, isc0, wsc, blocks, 0) == QG.OK             # no tokens: no-op


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        q.load(str(tmp_path / "missing.so"))


def test_read_probe_rejections(lib):
    lib.qg_read_contiguous.restype = ctypes.c_int
    lib.qg_read_contiguous.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.qg_read_strips.restype = ctypes.c_int
    lib.qg_read_strips.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    buf = np.zeros(4096 + 16, np.uint8)
    base = (buf.ctypes.data + 15) & ~15
    sink = np.zeros(4, np.uint32)
    s = sink.ctypes.data
    assert lib.qg_read_contiguous(base, 4096, 4, None, None) == QG.ERR_NULL
    assert lib.qg_read_contiguous(base + 4, 4096, 4, s, None) == QG.ERR_ALIGN
    assert lib.qg_read_contiguous(base, 4008, 4, s, None) == QG.ERR_ALIGN
    assert lib.qg_read_contiguous(base, 4096, 0, s, None) == QG.ERR_INVALID_ARG
    assert lib.qg_read_contiguous(base, 0, 4, s, None) == QG.OK
    assert lib.qg_read_strips(base, 8, 512, 48, s, None) == QG.ERR_SHAPE
    assert lib.qg_read_strips(base, 8, 512, 40, s, None) == QG.ERR_ALIGN
    assert lib.qg_read_strips(base, 8, 512, 0, s, None) == QG.ERR_INVALID_ARG
    assert lib.qg_read_strips(base, 0, 512, 64, s, None) == QG.OK


def test_compute_probe_rejections(lib):
    # host checks only: every call here returns before any launch
    lib.qg_mfma_loop.restype = ctypes.c_int
    lib.qg_mfma_loop.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p]
    lib.qg_empty_launch.restype = ctypes.c_int
    lib.qg_empty_launch.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    clocks = np.zeros(8, np.uint64)
    sink = np.zeros(4, np.uint32)
    c, s = clocks.ctypes.data, sink.ctypes.data
    assert lib.qg_mfma_loop(0, 8, 4, None, s, None) == QG.ERR_NULL
    assert lib.qg_mfma_loop(0, 8, 4, c, None, None) == QG.ERR_NULL
    assert lib.qg_mfma_loop(3, 8, 4, c, s, None) == QG.ERR_INVALID_ARG
    assert lib.qg_mfma_loop(-1, 8, 4, c, s, None) == QG.ERR_INVALID_ARG
    assert lib.qg_mfma_loop(0, 0, 4, c, s, None) == QG.ERR_INVALID_ARG
    assert lib.qg_mfma_loop(1, 8, 0, c, s, None) == QG.ERR_INVALID_ARG
    assert lib.qg_empty_launch(0, 64, None) == QG.ERR_INVALID_ARG
    assert lib.qg_empty_launch(4, 0, None) == QG.ERR_INVALID_ARG
    assert lib.qg_empty_launch(4, 1025, None) == QG.ERR_INVALID_ARG


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so,
    before touching any device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout and "--gpus 1" in r.stderr
