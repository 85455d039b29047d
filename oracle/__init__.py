"""ctypes wrapper over the plain C RoLA oracle (``rola_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path (``sparse_rank_attention_amd``)
never does.  The oracle shares no code with the HIP library.

All arrays are numpy, contiguous, with the (batch, head) axes folded into one
leading ``BH`` axis: tokens ``[BH, n_pad, D]`` (bf16 as uint16 bit patterns, or
float64), pooled ``[BH, nb, D]`` float32, scores ``[BH, nb, nb]`` float32,
block map ``[BH, nb, kb]`` int32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rola_oracle.c")
_LIB = os.path.join(_HERE, "librola_oracle.so")
BLOCK = 64
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-std=c11", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sigs = {
            "ro_version": ([], ctypes.c_int),
            "ro_position": ([I64, I32, I32, P], None),
            "ro_pool": ([P, I64, I64, I64, I32, P], None),
            "ro_scores": ([P, P, I64, I32, I32, P], None),
            "ro_select": ([P, I64, I32, I32, I32, P], None),
            "ro_keep_blocks": ([ctypes.c_float, I32], ctypes.c_int),
            "ro_sparse_rows": ([P, P, P, P, I64, I64, I32, I32, D, I64, P, P], None),
            "ro_rope3d": ([P, P, P, D, I32, P], None),
            "ro_lowrank_feature": ([P, I64, P, P, D, P, I32, I32, P], None),
            "ro_lowrank_state": ([P, P, P, I64, I64, I64, I32, I32, P, P, D, P, P], None),
            "ro_lowrank_rows": ([P, P, P, P, I64, I32, I32, P, P, D, I64, P, P], None),
            "ro_e4m3_value": ([ctypes.c_uint8], D),
            "ro_e4m3_encode": ([ctypes.c_float], ctypes.c_uint8),
            "ro_quant_e4m3": ([P, I64, I64, I64, I32, P, P, P], None),
            "ro_gate": ([P, P, I32], D),
            "ro_quant_rows_e4m3": ([P, I64, I64, I64, P, P, P], None),
            "ro_gemm_w8a8": ([P, P, P, P, P, I64, I64, I64, P, P], None),
            "ro_lowrank_block_states": ([P, P, P, I64, I64, I32, I32, P, P, D, P, P], None),
            "ro_lowrank_rows_complement": ([P, P, P, P, P, I32, I64, I32, I32, P, P, D, I64, P, P], None),
            "ro_forward": ([P, P, P, P, P, P, I64, I64, I64, I32, I32, I32, P, P, D, D, I32, I32, P, P],
                           None),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_split(d_model: int):
    """Rotary dims per (t, h, w) axis: 16/24/24 at D=64, scaled in proportion otherwise."""
    dt = d_model // 4
    dh = (d_model - dt) // 2
    return (dt, dh, d_model - dt - dh)


def widen_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (np.asarray(x, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def position(n: int, grid):
    out = np.zeros(3, dtype=np.int32)
    lib().ro_position(n, grid[1], grid[2], _p(out))
    return tuple(int(v) for v in out)


def pool(x_bits: np.ndarray, n_valid: int) -> np.ndarray:
    x = _c(x_bits, np.uint16)
    bh, n_pad, d = x.shape
    out = np.zeros((bh, n_pad // BLOCK, d), dtype=np.float32)
    lib().ro_pool(_p(x), bh, n_pad, n_valid, d, _p(out))
    return out


def scores(qp: np.ndarray, kp: np.ndarray) -> np.ndarray:
    qp, kp = _c(qp, np.float32), _c(kp, np.float32)
    bh, nb, d = qp.shape
    out = np.zeros((bh, nb, nb), dtype=np.float32)
    lib().ro_scores(_p(qp), _p(kp), bh, nb, d, _p(out))
    return out


def select(s: np.ndarray, kb: int) -> np.ndarray:
    s = _c(s, np.float32)
    bh, nq, nb = s.shape
    out = np.zeros((bh, nq, kb), dtype=np.int32)
    lib().ro_select(_p(s), bh, nq, nb, kb, _p(out))
    return out


def keep_blocks(topk: float, nb: int) -> int:
    """Key blocks kept per query block for the keep ratio ``topk`` (taken as float32)."""
    return int(lib().ro_keep_blocks(float(topk), int(nb)))


def block_map(q_bits, k_bits, n_valid: int, kb: int) -> np.ndarray:
    return select(scores(pool(q_bits, n_valid), pool(k_bits, n_valid)), kb)


def sparse_rows(q, k, v, bmap, n_valid: int, rows, scale=None) -> np.ndarray:
    """Sparse branch (fp64) for flat rows bh*n_pad+n; q/k/v float64 [BH, n_pad, D]."""
    q, k, v = _c(q, np.float64), _c(k, np.float64), _c(v, np.float64)
    bmap = _c(bmap, np.int32)
    rows = _c(rows, np.int64)
    bh, n_pad, d = q.shape
    kb = bmap.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    out = np.zeros((rows.size, d), dtype=np.float64)
    lib().ro_sparse_rows(_p(q), _p(k), _p(v), _p(bmap), n_pad, n_valid, d, kb, scale, rows.size,
                         _p(rows), _p(out))
    return out


def rope3d(x, pos3, split, theta=10000.0) -> np.ndarray:
    x = _c(x, np.float64)
    y = np.zeros_like(x)
    p = _c(pos3, np.int32)
    s = _c(split, np.int32)
    lib().ro_rope3d(_p(x), _p(p), _p(s), theta, x.size, _p(y))
    return y


def lowrank_feature(x, n, grid, w, split=None, theta=10000.0) -> np.ndarray:
    x = _c(x, np.float64)
    w = _c(w, np.float32)
    d, r = w.shape
    split = default_split(d) if split is None else split
    f = np.zeros(r, dtype=np.float64)
    lib().ro_lowrank_feature(_p(x), n, _p(_c(grid, np.int32)), _p(_c(split, np.int32)), theta,
                             _p(w), d, r, _p(f))
    return f


def lowrank_state(k, v, wk, n_valid: int, grid, split=None, theta=10000.0):
    k, v, wk = _c(k, np.float64), _c(v, np.float64), _c(wk, np.float32)
    bh, n_pad, d = k.shape
    r = wk.shape[1]
    split = default_split(d) if split is None else split
    S = np.zeros((bh, r, d), dtype=np.float64)
    z = np.zeros((bh, r), dtype=np.float64)
    lib().ro_lowrank_state(_p(k), _p(v), _p(wk), bh, n_pad, n_valid, d, r,
                           _p(_c(grid, np.int32)), _p(_c(split, np.int32)), theta, _p(S), _p(z))
    return S, z


def gate(q, g) -> float:
    """Output gate sigmoid(q . w + b) of one token; ``g`` = fp32 [w_0 .. w_{D-1}, b]."""
    q, g = _c(q, np.float64), _c(g, np.float32)
    assert g.size == q.size + 1
    return lib().ro_gate(_p(q), _p(g), q.size)


def lowrank_rows(q, wq, S, z, grid, rows, split=None, theta=10000.0, gate_w=None) -> np.ndarray:
    """Low-rank output of flat rows (bh * n_pad + n); times the output gate when ``gate_w`` is set."""
    q, wq = _c(q, np.float64), _c(wq, np.float32)
    S, z = _c(S, np.float64), _c(z, np.float64)
    rows = _c(rows, np.int64)
    bh, n_pad, d = q.shape
    r = wq.shape[1]
    split = default_split(d) if split is None else split
    out = np.zeros((rows.size, d), dtype=np.float64)
    lib().ro_lowrank_rows(_p(q), _p(wq), _p(S), _p(z), n_pad, d, r, _p(_c(grid, np.int32)),
                          _p(_c(split, np.int32)), theta, rows.size, _p(rows), _p(out))
    if gate_w is not None:
        qf = q.reshape(-1, d)
        for i, row in enumerate(rows):
            out[i] *= gate(qf[row], gate_w)
    return out


def lowrank_block_states(k, v, wk, n_valid: int, grid, split=None, theta=10000.0):
    """Per-block low-rank states of one (batch, head): (Sb [nb, r, D], zb [nb, r])."""
    k, v, wk = _c(k, np.float64), _c(v, np.float64), _c(wk, np.float32)
    n_pad, d = k.shape[-2:]
    r = wk.shape[1]
    split = default_split(d) if split is None else split
    nb = n_pad // BLOCK
    Sb = np.zeros((nb, r, d), dtype=np.float64)
    zb = np.zeros((nb, r), dtype=np.float64)
    lib().ro_lowrank_block_states(_p(k), _p(v), _p(wk), n_pad, n_valid, d, r, _p(_c(grid, np.int32)),
                                  _p(_c(split, np.int32)), theta, _p(Sb), _p(zb))
    return Sb, zb


def lowrank_rows_complement(q, wq, Sb, zb, bmap, grid, rows, split=None, theta=10000.0,
                            gate_w=None) -> np.ndarray:
    """Complement-scope low-rank output of rows n of one (batch, head): the state of
    query block n // 64 covers the blocks its row of ``bmap`` [nb, kb] does not keep."""
    q, wq = _c(q, np.float64), _c(wq, np.float32)
    Sb, zb, bmap = _c(Sb, np.float64), _c(zb, np.float64), _c(bmap, np.int32)
    rows = _c(rows, np.int64)
    n_pad, d = q.shape[-2:]
    r = wq.shape[1]
    split = default_split(d) if split is None else split
    out = np.zeros((rows.size, d), dtype=np.float64)
    lib().ro_lowrank_rows_complement(_p(q), _p(wq), _p(Sb), _p(zb), _p(bmap), bmap.shape[-1], n_pad, d, r,
                                     _p(_c(grid, np.int32)), _p(_c(split, np.int32)), theta, rows.size,
                                     _p(rows), _p(out))
    if gate_w is not None:
        qf = q.reshape(-1, d)
        for i, row in enumerate(rows):
            out[i] *= gate(qf[row], gate_w)
    return out


def e4m3_value(code: int) -> float:
    return lib().ro_e4m3_value(code)


def e4m3_encode(y: float) -> int:
    return lib().ro_e4m3_encode(y)


def quant_e4m3(x_bits, n_valid: int):
    x = _c(x_bits, np.uint16)
    bh, n_pad, d = x.shape
    codes = np.zeros(x.shape, dtype=np.uint8)
    scale = np.zeros((bh, n_pad // BLOCK), dtype=np.float32)
    deq = np.zeros(x.shape, dtype=np.float64)
    lib().ro_quant_e4m3(_p(x), bh, n_pad, n_valid, d, _p(codes), _p(scale), _p(deq))
    return codes, scale, deq


def quant_rows_e4m3(x_bits):
    """Per-row e4m3 quantisation of a bf16 matrix [rows, cols] (uint16 bits).
    Returns (codes uint8 [rows, cols], scale float32 [rows], deq float64)."""
    x = _c(x_bits, np.uint16)
    rows, cols = x.shape
    codes = np.zeros(x.shape, dtype=np.uint8)
    scale = np.zeros(rows, dtype=np.float32)
    deq = np.zeros(x.shape, dtype=np.float64)
    lib().ro_quant_rows_e4m3(_p(x), rows, cols, cols, _p(codes), _p(scale), _p(deq))
    return codes, scale, deq


def gemm_w8a8(a_codes, sa, w_codes, sw, bias=None, with_abs=False):
    """y[m, n] = sa[m] sw[n] sum_k value(a[m,k]) value(w[n,k]) + bias[n], fp64.
    With ``with_abs`` also returns sa sw sum_k |products| + |bias| (error scale)."""
    a, w = _c(a_codes, np.uint8), _c(w_codes, np.uint8)
    sa, sw = _c(sa, np.float32), _c(sw, np.float32)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape[1] == K and sa.shape == (M,) and sw.shape == (N,)
    b = None if bias is None else _c(bias, np.float32)
    y = np.zeros((M, N), dtype=np.float64)
    yabs = np.zeros((M, N), dtype=np.float64) if with_abs else None
    lib().ro_gemm_w8a8(_p(a), _p(sa), _p(w), _p(sw), None if b is None else _p(b), M, N, K, _p(y),
                       None if yabs is None else _p(yabs))
    return (y, yabs) if with_abs else y


def linear_w8a8(x_bits, w_bits, bias=None, with_abs=False):
    """The whole w8a8 linear layer: x [M, K] and W [N, K] (bf16 bits) each
    quantised per row, then the scaled fp8 product plus bias."""
    ca, sa, _ = quant_rows_e4m3(x_bits)
    cw, sw, _ = quant_rows_e4m3(w_bits)
    return gemm_w8a8(ca, sa, cw, sw, bias, with_abs)


def forward(q_bits, k_bits, v_bits, wq, wk, n_valid: int, kb: int, grid, split=None,
            theta=10000.0, scale=None, fp8=False, gate_w=None, complement=False):
    """Whole RoLA forward.  Returns (block map [BH, nb, kb] int32, out [BH, n_pad, D] float64).

    ``gate_w`` (fp32 [D+1], optional): output gate on the low-rank term.
    ``complement``: low-rank state over each query block's unkept blocks only."""
    q, k, v = _c(q_bits, np.uint16), _c(k_bits, np.uint16), _c(v_bits, np.uint16)
    wq, wk = _c(wq, np.float32), _c(wk, np.float32)
    bh, n_pad, d = q.shape
    r = wq.shape[1]
    split = default_split(d) if split is None else split
    scale = d ** -0.5 if scale is None else scale
    bmap = np.zeros((bh, n_pad // BLOCK, kb), dtype=np.int32)
    out = np.zeros((bh, n_pad, d), dtype=np.float64)
    gw = None if gate_w is None else _c(gate_w, np.float32)
    assert gw is None or gw.shape == (d + 1,)
    lib().ro_forward(_p(q), _p(k), _p(v), _p(wq), _p(wk), None if gw is None else _p(gw), bh, n_pad, n_valid,
                     d, r, kb, _p(_c(grid, np.int32)), _p(_c(split, np.int32)), theta, scale, int(fp8),
                     int(bool(complement)), _p(bmap), _p(out))
    return bmap, out
