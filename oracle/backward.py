"""Gradients of RoLA attention, by automatic differentiation of a plain torch fp64 forward.

TEST INFRASTRUCTURE ONLY: the tests may import this module; the product path
(``sparse_rank_attention_amd``) never does, and it shares no code with the HIP
library.

The forward is written here a second time, in torch (CPU, float64), from the
definition the C oracle follows (pages: "SparkDiffusion: 265x Faster Video
Generation on Consumer GPUs via Sparse Attention & Distillation", section
"RoLA: Preserving Global Context at Extreme Sparsity"): softmax attention
over the tokens of each query block's kept key blocks, plus the normalised
linear attention of phi(Wq^T R(q)) against phi(Wk^T R(k)) with the 3-D
rotary embedding R, optionally scaled per token by the output gate
sigmoid(q . w + b) (README "AlibabaResearch/SparkDiffusion", sparse-finetune
section, names gate_proj and gate_bias), and optionally with each query
block's low-rank sums restricted to the key blocks it does not keep.  The
training launchers on the pages need a backward kernel for this module
(README, distillation and fine-tune sections).

Its gradients are those of L = sum over valid rows of <O, dO>, taken by
torch.autograd.  The block map is a constant of the backward: the top-k
selection is piecewise constant in Q and K, so it contributes no gradient.
The dense token-level masks make this O(N^2): small sizes only.
"""
from __future__ import annotations

import numpy as np
import torch

BLOCK = 64


def _default_split(d: int):
    dt = d // 4
    dh = (d - dt) // 2
    return (dt, dh, d - dt - dh)


def _rope(x: torch.Tensor, grid, split, theta: float) -> torch.Tensor:
    """3-D rotary embedding of x [..., n, D]: axis a owns a contiguous run of
    split[a] dims; its pair p, (x[o+2p], x[o+2p+1]), turns by pos_a * theta^(-2p/split[a])."""
    n = x.shape[-2]
    idx = torch.arange(n)
    hw = grid[1] * grid[2]
    pos = (idx // hw, (idx % hw) // grid[2], idx % grid[2])
    parts, o = [], 0
    for p_axis, dax in zip(pos, split):
        pair = torch.arange(dax // 2, dtype=torch.float64)
        ang = p_axis.double()[:, None] * theta ** (-2.0 * pair / dax)[None, :]
        c, s = torch.cos(ang), torch.sin(ang)
        x0, x1 = x[..., o:o + dax:2], x[..., o + 1:o + dax:2]
        parts.append(torch.stack([x0 * c - x1 * s, x0 * s + x1 * c], dim=-1).reshape(*x.shape[:-1], dax))
        o += dax
    return torch.cat(parts, dim=-1)


def _phi(u):
    return torch.nn.functional.elu(u) + 1.0


def forward_torch(q, k, v, wq, wk, bmap, n_valid: int, grid, split=None, theta=10000.0, scale=None,
                  gate=None, complement=False):
    """O [BH, n_pad, D] from float64 tensors q, k, v [BH, n_pad, D], wq, wk [D, r],
    gate [D+1] or None, and the block map [BH, nb, kb] (numpy or tensor)."""
    bh, n_pad, d = q.shape
    split = _default_split(d) if split is None else split
    scale = d ** -0.5 if scale is None else scale
    nb = n_pad // BLOCK
    bmap = torch.as_tensor(np.asarray(bmap), dtype=torch.long)
    blk = torch.arange(n_pad) // BLOCK
    key_ok = torch.arange(n_pad) < n_valid
    outs = []
    for h in range(bh):
        kept = torch.zeros(nb, nb, dtype=torch.bool)
        kept[torch.arange(nb)[:, None], bmap[h]] = True
        tok_kept = kept[blk][:, blk] & key_ok[None, :]          # [n, m]
        logits = (q[h] @ k[h].T) * scale
        logits = logits.masked_fill(~tok_kept, float("-inf"))
        o_s = torch.softmax(logits, dim=-1) @ v[h]
        a = _phi(_rope(q[h], grid, split, theta) @ wq)           # [n, r]
        b = _phi(_rope(k[h], grid, split, theta) @ wk)
        if complement:
            lin_ok = ~kept[blk][:, blk] & key_ok[None, :]
            wts = (a @ b.T) * lin_ok
            den = wts.sum(dim=1, keepdim=True)
            o_lr = torch.where(den > 0, (wts @ v[h]) / torch.where(den > 0, den, torch.ones_like(den)),
                               torch.zeros_like(o_s))
        else:
            bv = b[:n_valid]
            o_lr = (a @ (bv.T @ v[h][:n_valid])) / (a @ bv.sum(dim=0))[:, None]
        if gate is not None:
            o_lr = o_lr * torch.sigmoid(q[h] @ gate[:d] + gate[d])[:, None]
        o = o_s + o_lr
        outs.append(torch.where((torch.arange(n_pad) < n_valid)[:, None], o, torch.zeros_like(o)))
    return torch.stack(outs)


def backward(q, k, v, wq, wk, bmap, dout, n_valid: int, grid, split=None, theta=10000.0, scale=None,
             gate=None, complement=False):
    """Gradients of sum(O * dout) over the valid rows.

    q, k, v, dout: float64 arrays [BH, n_pad, D]; wq, wk: [D, r]; gate: [D+1]
    or None.  Returns a dict of float64 arrays: dq, dk, dv [BH, n_pad, D] (zero
    on padded rows), dwq, dwk [D, r], and dgate [D+1] when a gate is given."""
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    tq, tk, tv, twq, twk = t(q), t(k), t(v), t(wq), t(wk)
    tg = t(gate) if gate is not None else None
    o = forward_torch(tq, tk, tv, twq, twk, bmap, n_valid, grid, split, theta, scale, tg, complement)
    loss = (o * torch.tensor(np.asarray(dout, dtype=np.float64))).sum()
    leaves = [tq, tk, tv, twq, twk] + ([tg] if tg is not None else [])
    grads = torch.autograd.grad(loss, leaves)
    names = ["dq", "dk", "dv", "dwq", "dwk"] + (["dgate"] if tg is not None else [])
    return {n: g.numpy() for n, g in zip(names, grads)}
