"""Python binding of librola (ctypes).  Argument marshalling only: every step of
RoLA attention runs in the HIP kernels of ``librola.so``; PyTorch provides the
device memory and the stream.  There is no CPU or PyTorch fallback: calls fail
if the library is missing or the tensors are not on a GPU.

Tensors: q, k, v (and out) are ``[B, H, n_pad, D]`` bf16 views on one device
with the last dim contiguous and identical strides; rows N..n_pad-1 of the
inputs are ignored and written as zero in the output.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from . import build as _build

ROLA_OK = 0
ROLA_PREC_BF16, ROLA_PREC_FP8 = 0, 1
ROLA_OUT_BF16, ROLA_OUT_F32 = 0, 1
ROLA_LR_GLOBAL, ROLA_LR_COMPLEMENT = 0, 1
BLOCK = 64


class RolaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class RolaConfig(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_float), ("kb_override", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("rope_split", ctypes.c_int32 * 3), ("rope_theta", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("precision", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("lowrank_scope", ctypes.c_int32)]


class RolaPlanInfo(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("nb", ctypes.c_int32), ("kb", ctypes.c_int32),
                ("n_pad", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("workspace_bytes_backward", ctypes.c_int64)]


class RolaKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


ABI_VERSION = 8  # ROLA_ABI_VERSION of include/rola.h
NOALLOC_SCRATCH_BYTES = 128 << 20  # ROLA_NOALLOC_SCRATCH_BYTES

EXPORTS = ["rola_abi_version", "rola_status_str", "rola_plan", "rola_select_blocks",
           "rola_sparse_attn", "rola_lowrank_attn", "rola_forward", "rola_backward", "rola_timing_enable",
           "rola_timing_read", "rola_mfma_probe", "rola_quant_rows", "rola_gemm_w8a8",
           "rola_forward_e4m3", "rola_forward_noalloc", "rola_forward_train", "rola_backward_saved"]

_lib = None


def library_path() -> str:
    """librola.so in the package (ROLA_LIBRARY may name another build of it)."""
    return os.environ.get("ROLA_LIBRARY") or _build.LIB


def lib():
    """Load librola.so (building it in-tree first if it is missing or stale)."""
    global _lib
    if _lib is None:
        path = library_path()
        if path == _build.LIB:
            _build.ensure_built()
        L = ctypes.CDLL(path)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        L.rola_abi_version.restype = I32
        L.rola_status_str.restype = ctypes.c_char_p
        L.rola_status_str.argtypes = [I32]
        L.rola_plan.restype = I32
        L.rola_plan.argtypes = [P, P, P]
        L.rola_select_blocks.restype = I32
        L.rola_select_blocks.argtypes = [P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.rola_sparse_attn.restype = I32
        L.rola_sparse_attn.argtypes = [P, P, P, P, P, P, P, I32, P, ctypes.c_size_t, P]
        L.rola_lowrank_attn.restype = I32
        L.rola_lowrank_attn.argtypes = [P, P, P, P, P, P, P, P, P, I32, P, ctypes.c_size_t, P]
        L.rola_forward.restype = I32
        L.rola_forward.argtypes = [P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.rola_backward.restype = I32
        L.rola_backward.argtypes = [P] * 17 + [ctypes.c_size_t, P]
        L.rola_forward_train.restype = I32
        L.rola_forward_train.argtypes = [P] * 13 + [ctypes.c_size_t, P]
        L.rola_backward_saved.restype = I32
        L.rola_backward_saved.argtypes = [P] * 19 + [ctypes.c_size_t, P]
        L.rola_timing_enable.restype = I32
        L.rola_timing_enable.argtypes = [I32]
        L.rola_timing_read.restype = I32
        L.rola_timing_read.argtypes = [P, I32]
        L.rola_mfma_probe.restype = I32
        L.rola_mfma_probe.argtypes = [I32, I32, P, P, P]
        I64 = ctypes.c_int64
        L.rola_quant_rows.restype = I32
        L.rola_quant_rows.argtypes = [P, I64, I64, I64, P, I64, P, P]
        L.rola_gemm_w8a8.restype = I32
        L.rola_gemm_w8a8.argtypes = [P, I64, P, P, I64, P, P, I64, I32, I32, P, I64, I32, P]
        L.rola_forward_noalloc.restype = I32
        L.rola_forward_noalloc.argtypes = [P] * 11
        L.rola_forward_e4m3.restype = I32
        L.rola_forward_e4m3.argtypes = [P] * 17 + [ctypes.c_size_t, P]
        if L.rola_abi_version() != ABI_VERSION:
            raise RuntimeError("%s has ABI version %d, the binding expects %d: rebuild it"
                               % (path, L.rola_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


class RolaError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status != ROLA_OK:
        raise RolaError("%s failed: %s (status %d)" % (what, lib().rola_status_str(status).decode(), status))


@dataclass
class Config:
    topk: float = 0.1
    rank: int = 32
    kb_override: int = 0
    rope_split: tuple = (0, 0, 0)
    rope_theta: float = 10000.0
    softmax_scale: float = 0.0
    precision: int = ROLA_PREC_BF16
    out_dtype: int = ROLA_OUT_BF16
    lowrank_scope: int = ROLA_LR_GLOBAL

    def c(self) -> RolaConfig:
        return RolaConfig(self.topk, self.kb_override, self.rank, (ctypes.c_int32 * 3)(*self.rope_split),
                          self.rope_theta, self.softmax_scale, self.precision, self.out_dtype,
                          self.lowrank_scope)


def problem(q: torch.Tensor, grid) -> RolaProblem:
    if q.dim() != 4:
        raise ValueError("expected [B, H, n_pad, D]")
    B, H, _, D = q.shape
    sb, sh, sn, sd = q.stride()
    if sd != 1:
        raise ValueError("head_dim must be contiguous")
    return RolaProblem(B, H, D, grid[0], grid[1], grid[2], sb, sh, sn)


def plan(prob: RolaProblem, cfg: Config) -> RolaPlanInfo:
    info = RolaPlanInfo()
    c = cfg.c()
    _check(lib().rola_plan(ctypes.byref(prob), ctypes.byref(c), ctypes.byref(info)), "rola_plan")
    return info


_ws_cache = {}


def workspace(device, nbytes: int, stream=None) -> torch.Tensor:
    """Caller-owned scratch for librola, cached per (device, stream) and grown on
    demand.  It is allocated on the stream the calls run on, so PyTorch's caching
    allocator reuses a replaced buffer only after that stream's queued kernels,
    and calls on different streams never share one."""
    dev = torch.device(device)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    key = (dev.index, s.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        _ws_cache.pop(key, None)
        with torch.cuda.stream(s):
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_tokens(q, *others):
    for t in (q,) + others:
        if t.dim() != 4:
            raise RolaError("q, k, v must be [B, H, n_pad, D] views")
        if t.dtype != torch.bfloat16:
            raise RolaError("q, k, v must be bfloat16")
        if t.shape != q.shape or t.stride() != q.stride() or t.device != q.device:
            raise RolaError("q, k, v must share shape, strides and device")


def _require_gpu(q):
    """Checked after every argument, before the workspace and the call."""
    if not q.is_cuda:
        raise RolaError("librola needs GPU tensors")


def _check_planned(q, info: RolaPlanInfo):
    """The library addresses rows 0..n_pad-1 of every token tensor."""
    if q.shape[2] != info.n_pad:
        raise RolaError("q, k, v hold %d rows; the grid needs n_pad = %d (64 * ceil(N / 64)), "
                        "rows N..n_pad-1 being padding" % (q.shape[2], info.n_pad))


def _check_out(out, q, cfg: Config):
    want = torch.float32 if cfg.out_dtype == ROLA_OUT_F32 else torch.bfloat16
    if out.dtype != want:
        raise RolaError("out must be %s for this out_dtype" % want)
    if out.shape != q.shape or out.stride() != q.stride() or out.device != q.device:
        raise RolaError("out must have the shape, strides and device of q")


def _check_proj(q, cfg: Config, *ws):
    D = q.shape[-1]
    for w in ws:
        if w.dtype != torch.float32 or tuple(w.shape) != (D, cfg.rank) or not w.is_contiguous() \
                or w.device != q.device:
            raise RolaError("wq and wk must be contiguous float32 [head_dim, rank] = [%d, %d] tensors "
                            "on the device of q" % (D, cfg.rank))


def _check_map(block_idx, q, info: RolaPlanInfo, name="block_idx"):
    B, H = q.shape[:2]
    if block_idx.dtype != torch.int32 or tuple(block_idx.shape) != (B, H, info.nb, info.kb) \
            or not block_idx.is_contiguous() or block_idx.device != q.device:
        raise RolaError("%s must be a contiguous int32 [B, H, nb, kb] = [%d, %d, %d, %d] tensor on the "
                        "device of q" % (name, B, H, info.nb, info.kb))


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _new_out(q, cfg: Config):
    dt = torch.float32 if cfg.out_dtype == ROLA_OUT_F32 else torch.bfloat16
    return torch.empty_strided(q.shape, q.stride(), dtype=dt, device=q.device)


def rola_select_blocks(q, k, grid, cfg: Config, block_idx=None, pooled_scores=None, stream=None):
    """Kept key blocks per query block: int32 [B, H, nb, kb], ascending."""
    _check_tokens(q, k)
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    B, H = q.shape[:2]
    if block_idx is None:
        block_idx = torch.empty((B, H, info.nb, info.kb), dtype=torch.int32, device=q.device)
    _check_map(block_idx, q, info)
    if pooled_scores is not None and (pooled_scores.dtype != torch.float32 or not pooled_scores.is_contiguous()
                                      or tuple(pooled_scores.shape) != (B, H, info.nb, info.nb)
                                      or pooled_scores.device != q.device):
        raise RolaError("pooled_scores must be a contiguous float32 [B, H, nb, nb] tensor on the device of q")
    _require_gpu(q)
    ws = workspace(q.device, info.workspace_bytes, stream)
    c = cfg.c()
    _check(lib().rola_select_blocks(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(block_idx),
                                    _ptr(pooled_scores), _ptr(ws), ws.numel(), _stream(stream)),
           "rola_select_blocks")
    return block_idx


def rola_sparse_attn(q, k, v, block_idx, grid, cfg: Config, out=None, accumulate=False, stream=None):
    _check_tokens(q, k, v)
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    _check_map(block_idx, q, info)
    out = _new_out(q, cfg) if out is None else out
    _check_out(out, q, cfg)
    _require_gpu(q)
    ws = workspace(q.device, info.workspace_bytes, stream)
    c = cfg.c()
    _check(lib().rola_sparse_attn(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(block_idx), _ptr(out), int(bool(accumulate)), _ptr(ws), ws.numel(),
                                  _stream(stream)), "rola_sparse_attn")
    return out


def _check_gate(gate, q):
    """The output gate is an fp32 device vector [D+1]: weights over the query, then the bias."""
    if gate is None:
        return
    if gate.dtype != torch.float32 or not gate.is_contiguous() or gate.device != q.device:
        raise RolaError("gate must be a contiguous float32 tensor on the device of q")
    if gate.numel() != q.shape[-1] + 1:
        raise RolaError("gate must hold head_dim + 1 values (weights, then bias)")


def rola_lowrank_attn(q, k, v, wq, wk, grid, cfg: Config, out=None, accumulate=False, stream=None,
                      gate=None):
    """Low-rank branch g * O_lr (g = sigmoid(q . w + b) with ``gate``, else 1)."""
    _check_tokens(q, k, v)
    _check_gate(gate, q)
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    _check_proj(q, cfg, wq, wk)
    out = _new_out(q, cfg) if out is None else out
    _check_out(out, q, cfg)
    _require_gpu(q)
    ws = workspace(q.device, info.workspace_bytes, stream)
    c = cfg.c()
    _check(lib().rola_lowrank_attn(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                   _ptr(wk), _ptr(gate), _ptr(out), int(bool(accumulate)), _ptr(ws), ws.numel(),
                                   _stream(stream)), "rola_lowrank_attn")
    return out


def rola_forward(q, k, v, wq, wk, grid, cfg: Config, out=None, block_idx_out=None, stream=None,
                 gate=None):
    """Fused RoLA forward O = O_sparse + g * O_lr (g = sigmoid(q . w + b) with ``gate``, else 1)."""
    _check_tokens(q, k, v)
    _check_gate(gate, q)
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    _check_proj(q, cfg, wq, wk)
    if block_idx_out is not None:
        _check_map(block_idx_out, q, info, "block_idx_out")
    out = _new_out(q, cfg) if out is None else out
    _check_out(out, q, cfg)
    _require_gpu(q)
    ws = workspace(q.device, info.workspace_bytes, stream)
    c = cfg.c()
    _check(lib().rola_forward(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                              _ptr(wk), _ptr(gate), _ptr(block_idx_out), _ptr(out), _ptr(ws), ws.numel(),
                              _stream(stream)), "rola_forward")
    return out


def rola_forward_train(q, k, v, wq, wk, grid, cfg: Config, out=None, block_idx_out=None, stream=None,
                       gate=None):
    """rola_forward that also keeps, for rola_backward_saved, the sparse branch's
    output O_s (fp32, the layout of q) and each row's base-2 log-sum-exp
    (fp32 [B*H, n_pad]).  Returns (out, os, lse)."""
    _check_tokens(q, k, v)
    _check_gate(gate, q)
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    _check_proj(q, cfg, wq, wk)
    if block_idx_out is not None:
        _check_map(block_idx_out, q, info, "block_idx_out")
    out = _new_out(q, cfg) if out is None else out
    _check_out(out, q, cfg)
    _require_gpu(q)
    os_ = torch.empty_strided(q.shape, q.stride(), dtype=torch.float32, device=q.device)
    lse = torch.empty((q.shape[0] * q.shape[1], info.n_pad), dtype=torch.float32, device=q.device)
    ws = workspace(q.device, info.workspace_bytes, stream)
    c = cfg.c()
    _check(lib().rola_forward_train(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                    _ptr(wk), _ptr(gate), _ptr(block_idx_out), _ptr(out), _ptr(os_), _ptr(lse),
                                    _ptr(ws), ws.numel(), _stream(stream)), "rola_forward_train")
    return out, os_, lse


def rola_forward_noalloc(q, k, v, wq, wk, grid, cfg: Config, out, block_idx_out=None, stream=None, gate=None):
    """rola_forward on the library's own per-GPU scratch (no workspace): ``out``
    is required, so the call itself allocates nothing.  Problems whose
    workspace exceeds the scratch (NOALLOC_SCRATCH_BYTES) raise RolaError."""
    _check_tokens(q, k, v)
    _check_gate(gate, q)
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    _check_proj(q, cfg, wq, wk)
    if block_idx_out is not None:
        _check_map(block_idx_out, q, info, "block_idx_out")
    _check_out(out, q, cfg)
    if info.workspace_bytes > NOALLOC_SCRATCH_BYTES:
        raise RolaError("rola_forward_noalloc: this problem needs %d workspace bytes, above the %d-byte "
                        "scratch" % (info.workspace_bytes, NOALLOC_SCRATCH_BYTES))
    _require_gpu(q)
    c = cfg.c()
    _check(lib().rola_forward_noalloc(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                      _ptr(wk), _ptr(gate), _ptr(block_idx_out), _ptr(out), _stream(stream)),
           "rola_forward_noalloc")
    return out


def rola_forward_e4m3(q, k, v, q8, k8, v8, qs, ks, vs, wq, wk, grid, cfg: Config, out=None,
                      block_idx_out=None, stream=None, gate=None):
    """rola_forward in fp8 mode with the caller's e4m3 codes (uint8, the
    shape and strides of q) and per-block scales (float32 [B, H, nb]) for the
    sparse branch; selection and the low-rank branch read the bf16 q, k, v."""
    _check_tokens(q, k, v)
    _check_gate(gate, q)
    if cfg.precision != ROLA_PREC_FP8:
        raise RolaError("rola_forward_e4m3 needs precision ROLA_PREC_FP8")
    for t in (q8, k8, v8):
        if t.dtype != torch.uint8 or t.shape != q.shape or t.stride() != q.stride() or t.device != q.device:
            raise RolaError("q8, k8, v8 must be uint8 codes with the shape and strides of q")
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    _check_proj(q, cfg, wq, wk)
    B, H = q.shape[:2]
    for t in (qs, ks, vs):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, info.nb) or not t.is_contiguous() \
                or t.device != q.device:
            raise RolaError("qs, ks, vs must be contiguous float32 [B, H, nb] on the device of q")
    if block_idx_out is not None:
        _check_map(block_idx_out, q, info, "block_idx_out")
    out = _new_out(q, cfg) if out is None else out
    _check_out(out, q, cfg)
    _require_gpu(q)
    ws = workspace(q.device, info.workspace_bytes, stream)
    c = cfg.c()
    _check(lib().rola_forward_e4m3(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(q8),
                                   _ptr(k8), _ptr(v8), _ptr(qs), _ptr(ks), _ptr(vs), _ptr(wq), _ptr(wk),
                                   _ptr(gate), _ptr(block_idx_out), _ptr(out), _ptr(ws), ws.numel(),
                                   _stream(stream)), "rola_forward_e4m3")
    return out


def rola_backward(q, k, v, wq, wk, grid, cfg: Config, block_idx, dout, gate=None, stream=None, saved=None):
    """Gradients of the forward for dL/dO = dout (the block map held constant).

    ``saved``: the (os, lse) pair of rola_forward_train on the same inputs,
    map and config (rola_backward_saved), else None (the sparse branch is
    recomputed).  Returns (dq, dk, dv, dwq, dwk, dgate): bf16 tensors like q,
    fp32 [D, rank] tensors, and the fp32 [D+1] gate gradient (None without a
    gate)."""
    _check_tokens(q, k, v)
    _check_gate(gate, q)
    want = torch.float32 if cfg.out_dtype == ROLA_OUT_F32 else torch.bfloat16
    if dout.dtype != want or dout.shape != q.shape or dout.stride() != q.stride() or dout.device != q.device:
        raise RolaError("dout must have the output dtype and the layout of q")
    prob = problem(q, grid)
    info = plan(prob, cfg)
    _check_planned(q, info)
    _check_proj(q, cfg, wq, wk)
    _check_map(block_idx, q, info)
    B, H, _, D = q.shape
    dq, dk, dv = (torch.empty_strided(q.shape, q.stride(), dtype=torch.bfloat16, device=q.device)
                  for _ in range(3))
    dwq = torch.empty((D, cfg.rank), dtype=torch.float32, device=q.device)
    dwk = torch.empty((D, cfg.rank), dtype=torch.float32, device=q.device)
    dgate = torch.empty(D + 1, dtype=torch.float32, device=q.device) if gate is not None else None
    if saved is not None:
        os_, lse = saved
        if (os_.dtype != torch.float32 or os_.shape != q.shape or os_.stride() != q.stride()
                or os_.device != q.device):
            raise RolaError("saved O_s must be fp32 with the layout of q")
        if (lse.dtype != torch.float32 or tuple(lse.shape) != (B * H, info.n_pad) or not lse.is_contiguous()
                or lse.device != q.device):
            raise RolaError("saved lse must be contiguous fp32 [B*H, n_pad]")
    _require_gpu(q)
    ws = workspace(q.device, info.workspace_bytes_backward, stream)
    c = cfg.c()
    if saved is None:
        _check(lib().rola_backward(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(wq),
                                   _ptr(wk), _ptr(gate), _ptr(block_idx), _ptr(dout), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(dwq), _ptr(dwk), _ptr(dgate), _ptr(ws), ws.numel(),
                                   _stream(stream)), "rola_backward")
    else:
        _check(lib().rola_backward_saved(ctypes.byref(prob), ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(wq), _ptr(wk), _ptr(gate), _ptr(block_idx), _ptr(dout),
                                         _ptr(os_), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwq),
                                         _ptr(dwk), _ptr(dgate), _ptr(ws), ws.numel(), _stream(stream)),
               "rola_backward_saved")
    return dq, dk, dv, dwq, dwk, dgate


def mfma_probe(precision: int, iters: int, sink, stream=None) -> float:
    """Launch the MFMA-rate probe on the stream; returns its flop count (time it with events)."""
    flop = ctypes.c_double(0.0)
    _check(lib().rola_mfma_probe(precision, iters, ctypes.byref(flop), _ptr(sink), _stream(stream)),
           "rola_mfma_probe")
    return flop.value


def timing_enable(on: bool):
    lib().rola_timing_enable(1 if on else 0)


def timing_read():
    """Per-kernel {name: (launches, total_ms)} since the last read (synchronises the events)."""
    buf = (RolaKernelTime * 32)()
    n = lib().rola_timing_read(buf, 32)
    if n < 0:
        raise RolaError("rola_timing_read failed")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n)}


# ------------------------------------------------------------ w8a8 layers
def _on_device(*ts):
    dev = ts[0].device
    for t in ts:
        if t is not None and (not t.is_cuda or t.device != dev):
            raise RolaError("librola needs all tensors on one GPU")


def _row_stride(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise RolaError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def rola_quant_rows(x, codes=None, scale=None, stream=None):
    """Per-row e4m3 quantisation of a bf16 matrix [rows, cols] (row slices of
    a wider buffer allowed).  Returns (codes uint8 [rows, cols], scale fp32 [rows])."""
    _on_device(x, codes, scale)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise RolaError("x must be a 2-D bfloat16 tensor")
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    if codes.dtype != torch.uint8 or codes.shape != (rows, cols) or scale.dtype != torch.float32 \
            or scale.numel() != rows or not scale.is_contiguous():
        raise RolaError("codes must be uint8 [rows, cols] and scale float32 [rows]")
    _check(lib().rola_quant_rows(_ptr(x), rows, cols, _row_stride(x), _ptr(codes), _row_stride(codes),
                                 _ptr(scale), _stream(stream)), "rola_quant_rows")
    return codes, scale


def rola_gemm_w8a8(x_codes, sx, w_codes, sw, bias=None, out=None, out_dtype=ROLA_OUT_BF16, stream=None):
    """out[m, n] = sx[m] sw[n] sum_k value(x[m, k]) value(w[n, k]) + bias[n].
    x_codes uint8 [M, K], w_codes uint8 [N, K]; ``out`` may be a column slice
    of a wider [M, *] buffer (unit column stride)."""
    _on_device(x_codes, sx, w_codes, sw, bias, out)
    M, K = x_codes.shape
    N = w_codes.shape[0]
    if x_codes.dtype != torch.uint8 or w_codes.dtype != torch.uint8 or w_codes.shape[1] != K:
        raise RolaError("x_codes and w_codes must be uint8 [M, K] and [N, K]")
    for t, n in ((sx, M), (sw, N)) + (((bias, N),) if bias is not None else ()):
        if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
            raise RolaError("scales and bias must be contiguous float32 vectors of the matching length")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if out_dtype == ROLA_OUT_F32 else torch.bfloat16,
                          device=x_codes.device)
    want = torch.float32 if out_dtype == ROLA_OUT_F32 else torch.bfloat16
    if out.dtype != want or tuple(out.shape) != (M, N):
        raise RolaError("out must be [M, N] of the dtype out_dtype names")
    if M == 0:
        return out
    _check(lib().rola_gemm_w8a8(_ptr(x_codes), _row_stride(x_codes), _ptr(sx), _ptr(w_codes), _row_stride(w_codes),
                                _ptr(sw), _ptr(bias), M, N, K, _ptr(out), _row_stride(out), out_dtype,
                                _stream(stream)), "rola_gemm_w8a8")
    return out


def rola_linear_w8a8(x, w_codes, sw, bias=None, out=None, out_dtype=ROLA_OUT_BF16, stream=None):
    """The whole w8a8 layer on bf16 activations: quantise x per row, then the
    scaled fp8 product (weights quantised beforehand with rola_quant_rows)."""
    xc, sx = rola_quant_rows(x, stream=stream)
    return rola_gemm_w8a8(xc, sx, w_codes, sw, bias, out, out_dtype, stream)
