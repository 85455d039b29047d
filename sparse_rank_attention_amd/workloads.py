"""Seeded synthetic inputs for RoLA attention, shared by the HIP path and the oracle.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, selection, softmax, rotary or low-rank code).

The pages measure RoLA inside Wan 2.1/2.2 video DiTs on real latents and
trained weights, none of which exist here.  The workloads below stand in for
them with the shapes of those models' self-attention (pages: "AlibabaResearch/
SparkDiffusion" README, inference section; "SparkDiffusion: 265x Faster Video
Generation ..." article, "Why Higher Resolution Benefits More").

Recipes
-------
* ``iid``   : Q, K, V ~ N(0, 1), rounded to bf16 (round-to-nearest-even).
* ``field`` : Q and K are a smooth spatio-temporal field plus noise,
  ``X[t,h,w,d] = sum_{m<8} A[m,d] sin(2 pi (ft_m t/T + fh_m h/Hg + fw_m w/W) + phi[m,d])
  + 0.5 eps`` with integer ft_m in {0,1,2}, fh_m, fw_m in {0..3},
  A ~ N(0, 1/4) (field variance ~1), phi ~ U[0, 2 pi), eps ~ N(0, 1);
  V ~ N(0, 1).  The smooth part makes pooled block energies non-uniform, as
  in real video latents, so the top-k selection has structure to find.
* Low-rank projections Wq, Wk (fp32, [D, r], shared by all heads) ~ N(0, 1/D).
* Output gate (fp32 [D+1]: weights ~ N(0, 1/D), then a bias ~ N(0, 1/4)), so
  that sigmoid(q . w + b) spreads over (0, 1) for unit-variance queries.

* w8a8 linear layers (the QKV and output projections of the same DiT blocks,
  hidden size H*D): activations x [T, H*D] ~ N(0, 1) with 1% of the input
  channels (a fixed seeded set) scaled by 8, as a stand-in for the outlier
  channels of real DiT activations; weights W [d_out, H*D] ~ N(0, 1/(H*D));
  bias ~ N(0, 0.02^2); all rounded to bf16 except the fp32 bias.  Rows of x
  draw from ``default_rng([seed, 200, row // 4096])`` in 4096-row chunks (so
  sampled rows regenerate cheaply), the outlier set from ``[seed, 201]``, W
  from ``[seed, 202]`` and the bias from ``[seed, 203]``.

Every (batch, head, tensor) draws from ``numpy.random.default_rng([seed, b, h,
tid])`` (tid 0=Q, 1=K, 2=V, 6=the output gradient of the backward tests) and the projections from ``default_rng([seed, 100+tid])``
(tid 3=Wq, 4=Wk, 5=gate), so any head can be regenerated on its own.  Tokens are in
raster (t, h, w) order; rows from N up to the padded length are zero.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple  # (T, Hg, W) latent token grid
    topk: float
    rank: int
    kind: str  # "iid" or "field"
    precision: str = "bf16"  # "bf16" or "fp8"
    seed: int = 0

    @property
    def n_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def nb(self) -> int:
        return (self.n_tokens + BLOCK - 1) // BLOCK

    @property
    def n_pad(self) -> int:
        return self.nb * BLOCK

    def dense_equiv_flop(self) -> float:
        n = self.n_tokens
        return 4.0 * n * n * self.head_dim * self.batch * self.heads

    def kept_block_flop(self, kb: int) -> float:
        """Work of the kept 64x64 block pairs when each query block keeps kb key blocks."""
        return 4.0 * self.nb * kb * BLOCK * BLOCK * self.head_dim * self.batch * self.heads


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, (4, 16, 16), 0.25, 16, "iid"),
    "wan13b_480p": Workload("wan13b_480p", 1, 12, 128, (21, 30, 52), 0.10, 32, "field"),
    "wan14b_480p": Workload("wan14b_480p", 1, 40, 128, (21, 30, 52), 0.05, 32, "field"),
    "wan14b_720p": Workload("wan14b_720p", 1, 40, 128, (21, 45, 80), 0.03, 32, "field"),
    "wan14b_720p_fp8": Workload("wan14b_720p_fp8", 1, 40, 128, (21, 45, 80), 0.03, 32,
                                "field", precision="fp8"),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _field_head(rng: np.random.Generator, grid, d: int) -> np.ndarray:
    t_n, h_n, w_n = grid
    ft = rng.integers(0, 3, size=8)
    fh = rng.integers(0, 4, size=8)
    fw = rng.integers(0, 4, size=8)
    amp = rng.normal(0.0, 0.5, size=(8, d))
    phase = rng.uniform(0.0, 2.0 * np.pi, size=(8, d))
    t = np.arange(t_n, dtype=np.float64)[:, None, None] / t_n
    h = np.arange(h_n, dtype=np.float64)[None, :, None] / h_n
    w = np.arange(w_n, dtype=np.float64)[None, None, :] / w_n
    ang = np.stack([2.0 * np.pi * (ft[m] * t + fh[m] * h + fw[m] * w) for m in range(8)], axis=-1)
    ang = ang.reshape(-1, 8)  # [N, 8], raster (t, h, w) order
    # sin(a + p) = sin(a) cos(p) + cos(a) sin(p)
    x = np.sin(ang) @ (amp * np.cos(phase)) + np.cos(ang) @ (amp * np.sin(phase))
    x += 0.5 * rng.standard_normal(size=x.shape)
    return x


def _head_tensor(w: Workload, b: int, h: int, tid: int) -> np.ndarray:
    rng = np.random.default_rng([w.seed, b, h, tid])
    n, d = w.n_tokens, w.head_dim
    if w.kind == "field" and tid in (0, 1):
        x = _field_head(rng, w.grid, d)
    else:
        x = rng.standard_normal(size=(n, d))
    out = np.zeros((w.n_pad, d), dtype=np.uint16)
    out[:n] = to_bf16_bits(x.astype(np.float32))
    return out


def make_qkv(w: Workload, heads=None, threads: int | None = None):
    """Q, K, V as bf16 bit patterns (uint16), shape [B, len(heads), N_pad, D]."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    shape = (w.batch, len(heads), w.n_pad, w.head_dim)
    outs = [np.empty(shape, dtype=np.uint16) for _ in range(3)]
    jobs = [(b, hi, h, tid) for b in range(w.batch) for hi, h in enumerate(heads) for tid in range(3)]

    def run(job):
        b, hi, h, tid = job
        outs[tid][b, hi] = _head_tensor(w, b, h, tid)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if len(jobs) > 1 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return outs[0], outs[1], outs[2]


def make_proj(w: Workload):
    """Low-rank projections Wq, Wk: float32 [D, r] ~ N(0, 1/D)."""
    out = []
    for tid in (3, 4):
        rng = np.random.default_rng([w.seed, 100 + tid])
        out.append((rng.standard_normal(size=(w.head_dim, w.rank)) / np.sqrt(w.head_dim)).astype(np.float32))
    return out[0], out[1]


def make_gate(w: Workload):
    """Output gate [w_0 .. w_{D-1}, b]: float32 [D+1], weights ~ N(0, 1/D), bias ~ N(0, 1/4)."""
    rng = np.random.default_rng([w.seed, 105])
    g = rng.standard_normal(size=w.head_dim + 1)
    g[:w.head_dim] /= np.sqrt(w.head_dim)
    g[w.head_dim] *= 0.5
    return g.astype(np.float32)


def make_dout(w: Workload, f32: bool = False):
    """Output gradient dL/dO ~ N(0, 1) of shape [B, H, N_pad, D] (rows >= N zero):
    bf16 bit patterns (uint16), or float32 values when ``f32``."""
    out = np.zeros((w.batch, w.heads, w.n_pad, w.head_dim), dtype=np.float32)
    for b in range(w.batch):
        for h in range(w.heads):
            rng = np.random.default_rng([w.seed, b, h, 6])
            out[b, h, :w.n_tokens] = rng.standard_normal((w.n_tokens, w.head_dim))
    return out if f32 else to_bf16_bits(out)


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    """A w8a8 linear layer: y [tokens, d_out] = x [tokens, d_in] W^T + bias."""
    name: str
    tokens: int
    d_in: int
    d_out: int
    seed: int = 0

    @property
    def flop(self) -> float:
        return 2.0 * self.tokens * self.d_in * self.d_out


# Wan 2.1 14B (40 heads x 128 = 5120 hidden) at 720P (21 x 45 x 80 = 75600
# latent tokens): the fused Q/K/V projection and the output projection.
LINEAR = {
    "wan14b_720p_qkv": LinearWorkload("wan14b_720p_qkv", 75600, 5120, 15360),
    "wan14b_720p_out": LinearWorkload("wan14b_720p_out", 75600, 5120, 5120),
    "wan13b_480p_qkv": LinearWorkload("wan13b_480p_qkv", 32760, 1536, 4608),
}

_LIN_CHUNK = 4096


def _outlier_channels(lw: LinearWorkload) -> np.ndarray:
    rng = np.random.default_rng([lw.seed, 201])
    return rng.choice(lw.d_in, size=max(1, lw.d_in // 100), replace=False)


def make_linear_x(lw: LinearWorkload, rows=None) -> np.ndarray:
    """Activations as bf16 bits [len(rows), d_in] (all rows when rows is None)."""
    rows = np.arange(lw.tokens) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), lw.d_in), dtype=np.uint16)
    hot = _outlier_channels(lw)
    chunks = np.unique(rows // _LIN_CHUNK)

    def run(c):
        rng = np.random.default_rng([lw.seed, 200, int(c)])
        n = min(_LIN_CHUNK, lw.tokens - c * _LIN_CHUNK)
        x = rng.standard_normal((n, lw.d_in), dtype=np.float32)
        x[:, hot] *= 8.0
        sel = np.nonzero(rows // _LIN_CHUNK == c)[0]
        out[sel] = to_bf16_bits(x[rows[sel] - c * _LIN_CHUNK])

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(run, chunks))
    return out


def make_linear_w(lw: LinearWorkload):
    """Weights as bf16 bits [d_out, d_in] and the fp32 bias [d_out]."""
    rng = np.random.default_rng([lw.seed, 202])
    w = rng.standard_normal((lw.d_out, lw.d_in), dtype=np.float32) / np.float32(np.sqrt(lw.d_in))
    bias = (np.random.default_rng([lw.seed, 203]).standard_normal(lw.d_out) * 0.02).astype(np.float32)
    return to_bf16_bits(w), bias
