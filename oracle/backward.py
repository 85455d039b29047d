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


def _rope(x: torch.Tensor, grid, split, theta: float, inverse: bool = False) -> torch.Tensor:
    """3-D rotary embedding of x [..., n, D]: axis a owns a contiguous run of
    split[a] dims; its pair p, (x[o+2p], x[o+2p+1]), turns by pos_a * theta^(-2p/split[a])
    (by minus that angle, the transpose, when ``inverse``)."""
    n = x.shape[-2]
    idx = torch.arange(n)
    hw = grid[1] * grid[2]
    pos = (idx // hw, (idx % hw) // grid[2], idx % grid[2])
    parts, o = [], 0
    for p_axis, dax in zip(pos, split):
        pair = torch.arange(dax // 2, dtype=torch.float64)
        ang = p_axis.double()[:, None] * theta ** (-2.0 * pair / dax)[None, :]
        if inverse:
            ang = -ang
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


def backward_sampled(q_bits, k_bits, v_bits, wq, wk, bmap, dout_bits, n_valid: int, grid, q_rows, k_rows,
                     split=None, theta=10000.0, scale=None, gate=None, complement=False, heads=None):
    """The same gradients at full size, for sampled rows, from the gradient
    formulas written out (no autograd), one head at a time.

    q_bits, k_bits, v_bits, dout_bits: bf16 bit patterns [BH, n_pad, D];
    q_rows, k_rows: {head: row indices} of the dq and of the dk, dv rows wanted;
    heads: the heads to evaluate (default all; dwq, dwk and dgate then sum
    over those heads only).
    Returns ({head: dq rows}, {head: dk rows}, {head: dv rows}, dwq, dwk, dgate or None).

    With ``complement`` the low-rank sums of query block i run over the key
    blocks j it does not keep: S_i = sum_j S_j, z_i = sum_j z_j over those j
    (S_j = b_j^T v_j, z_j = sum b_j over block j's valid tokens), and L = 0 where
    that set is empty.  The per-token formulas below then use S_i, z_i, and the
    block states receive dS_j = sum of dS_i over the query blocks i that do not
    keep j (dS_i = sum over i's tokens of a dnum^T), dz_j likewise.

    Per head, with the low-rank sums over all N valid tokens:
      a = phi(R(q) Wq), b = phi(R(k) Wk), S = b^T v, z = sum b, L = a S / (a . z);
      g = sigmoid(q . w + beta) (1 without a gate); dg = dO . L; dy = dg g (1 - g);
      dnum = g dO / den, dden = -g dg / den, da = S dnum + z dden, du = da phi'(u);
      dq_lr = R^T(Wq du) + dy w, dWq = sum R(q) du^T, dS = sum a dnum^T,
      dz = sum a dden, db = dS v + dz, dv_lr = dS^T b, dw' = db phi'(.),
      dk_lr = R^T(Wk dw'), dWk = sum R(k) dw'^T;
    and for the sparse branch of each sampled query row n (its kept keys M):
      P = softmax(scale q_n . k_M), dP = dO_n . v_M, D = P . dP,
      dq_n = scale sum (P (dP - D)) k_M;
    of each sampled key m: the same rows' P and dS for every query row whose
    block kept m's block, dk_m = scale sum_n dS_nm q_n, dv_m = sum_n P_nm dO_n."""
    w16 = lambda x: torch.from_numpy((np.asarray(x, dtype=np.uint32) << 16).view(np.float32).astype(np.float64))
    bh_count, n_pad, d = q_bits.shape
    split = _default_split(d) if split is None else split
    scale = d ** -0.5 if scale is None else scale
    n = n_valid
    Wq, Wk = torch.tensor(np.asarray(wq, np.float64)), torch.tensor(np.asarray(wk, np.float64))
    G = None if gate is None else torch.tensor(np.asarray(gate, np.float64))
    dwq, dwk = torch.zeros_like(Wq), torch.zeros_like(Wk)
    dgate = torch.zeros(d + 1, dtype=torch.float64) if gate is not None else None
    dq_out, dk_out, dv_out = {}, {}, {}
    dphi = lambda u: torch.where(u > 0, torch.ones_like(u), torch.exp(u))
    for h in (range(bh_count) if heads is None else heads):
        Q, K, V, DO = w16(q_bits[h])[:n], w16(k_bits[h])[:n], w16(v_bits[h])[:n], w16(dout_bits[h])[:n]
        Rq, Rk = _rope(Q, grid, split, theta), _rope(K, grid, split, theta)
        u, wv = Rq @ Wq, Rk @ Wk
        a, b = _phi(u), _phi(wv)
        g = torch.sigmoid(Q @ G[:d] + G[d]) if G is not None else torch.ones(n, dtype=torch.float64)
        kept = np.asarray(bmap[h])
        if not complement:
            S, z = b.T @ V, b.sum(dim=0)
            den = a @ z
            L = (a @ S) / den[:, None]
            dg = (DO * L).sum(dim=1)
            dy = dg * g * (1 - g) if G is not None else torch.zeros(n, dtype=torch.float64)
            dnum = g[:, None] * DO / den[:, None]
            dden = -g * dg / den
            du = (dnum @ S.T + dden[:, None] * z[None, :]) * dphi(u)
            dS, dz = a.T @ dnum, (a * dden[:, None]).sum(dim=0)
            dw_ = (V @ dS.T + dz[None, :]) * dphi(wv)
            dv_lr = b @ dS
        else:
            nbk = (n + BLOCK - 1) // BLOCK
            blocks = [torch.arange(j * BLOCK, min(j * BLOCK + BLOCK, n)) for j in range(nbk)]
            Sj = torch.stack([b[r].T @ V[r] for r in blocks])           # [nb, r, D]
            zj = torch.stack([b[r].sum(dim=0) for r in blocks])         # [nb, r]
            off = torch.ones(nbk, nbk, dtype=torch.float64)              # off[i, j]: i does not keep j
            off[torch.arange(nbk)[:, None], torch.as_tensor(kept[:nbk], dtype=torch.long)] = 0.0
            Si = (off @ Sj.reshape(nbk, -1)).reshape(Sj.shape)
            zi = off @ zj
            dy = torch.zeros(n, dtype=torch.float64)
            du = torch.zeros_like(u)
            dSi, dzi = torch.zeros_like(Sj), torch.zeros_like(zj)
            for i, r in enumerate(blocks):
                den = a[r] @ zi[i]
                ok = den > 0                                             # empty complement: no term
                inv = torch.where(ok, 1.0 / torch.where(ok, den, torch.ones_like(den)), torch.zeros_like(den))
                L = (a[r] @ Si[i]) * inv[:, None]
                dg_i = (DO[r] * L).sum(dim=1)
                if G is not None:
                    dy[r] = dg_i * g[r] * (1 - g[r])
                dnum = g[r][:, None] * DO[r] * inv[:, None]
                dden = -g[r] * dg_i * inv
                du[r] = (dnum @ Si[i].T + dden[:, None] * zi[i][None, :]) * dphi(u[r])
                dSi[i], dzi[i] = a[r].T @ dnum, (a[r] * dden[:, None]).sum(dim=0)
            dSj = (off.T @ dSi.reshape(nbk, -1)).reshape(dSi.shape)
            dzj = off.T @ dzi
            dw_ = torch.zeros_like(wv)
            dv_lr = torch.zeros_like(V)
            for j, r in enumerate(blocks):
                dw_[r] = (V[r] @ dSj[j].T + dzj[j][None, :]) * dphi(wv[r])
                dv_lr[r] = b[r] @ dSj[j]
        dq_lr = _rope(du @ Wq.T, grid, split, theta, inverse=True) + dy[:, None] * (G[:d][None, :] if G is not None else 0)
        dwq += Rq.T @ du
        dk_lr = _rope(dw_ @ Wk.T, grid, split, theta, inverse=True)
        dwk += Rk.T @ dw_
        if G is not None:
            dgate[:d] += Q.T @ dy
            dgate[d] += dy.sum()
        keys_of = lambda i: torch.cat([torch.arange(j * BLOCK, min(j * BLOCK + BLOCK, n)) for j in sorted(kept[i])])

        def block_rows(i):  # P, dS of query block i over its kept keys
            rows = torch.arange(i * BLOCK, min(i * BLOCK + BLOCK, n))
            idx = keys_of(i)
            P = torch.softmax((Q[rows] @ K[idx].T) * scale, dim=1)
            dP = DO[rows] @ V[idx].T
            dS_ = P * (dP - (P * dP).sum(dim=1, keepdim=True))
            return rows, idx, P, dS_

        out = []
        for r in q_rows.get(h, []):
            rows, idx, P, dS_ = block_rows(r // BLOCK)
            out.append(scale * dS_[r - r // BLOCK * BLOCK] @ K[idx] + dq_lr[r])
        dq_out[h] = torch.stack(out).numpy() if out else np.zeros((0, d))
        want = list(k_rows.get(h, []))
        dk_acc = {m: torch.zeros(d, dtype=torch.float64) for m in want}
        dv_acc = {m: torch.zeros(d, dtype=torch.float64) for m in want}
        for i in range(kept.shape[0]):
            hit = [m for m in want if (m // BLOCK) in set(kept[i].tolist())]
            if not hit or i * BLOCK >= n:
                continue
            rows, idx, P, dS_ = block_rows(i)
            pos = {int(t): c for c, t in enumerate(idx)}
            for m in hit:
                cidx = pos[m]
                dk_acc[m] += scale * dS_[:, cidx] @ Q[rows]
                dv_acc[m] += P[:, cidx] @ DO[rows]
        dk_out[h] = np.stack([(dk_acc[m] + dk_lr[m]).numpy() for m in want]) if want else np.zeros((0, d))
        dv_out[h] = np.stack([(dv_acc[m] + dv_lr[m]).numpy() for m in want]) if want else np.zeros((0, d))
    return dq_out, dk_out, dv_out, dwq.numpy(), dwk.numpy(), (dgate.numpy() if dgate is not None else None)
