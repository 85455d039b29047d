"""Pins for the backward oracle (oracle/backward.py).

Its torch forward is checked against the C oracle (same outputs), and its
gradients against central finite differences of the C oracle's own fp64
branch functions: a directional derivative for Q, K, V and coordinate steps
for the fp32 projections and gate, in each scope and with and without a gate.
The written-out gradient formulas used at full size on sampled rows are
checked against the autograd gradients on every row of a small case.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as B
from sparse_rank_attention_amd.workloads import to_bf16_bits


def _case(seed, grid=(3, 7, 11), n_pad=256, d=64, r=16, bh=2, kb=2):
    rng = np.random.default_rng(seed)
    n_valid = grid[0] * grid[1] * grid[2]
    bits = lambda: to_bf16_bits(rng.standard_normal((bh, n_pad, d)).astype(np.float32))
    qb, kbits, vb = bits(), bits(), bits()
    for x in (qb, kbits, vb):
        x[:, n_valid:] = 0
    wq = (rng.standard_normal((d, r)) / np.sqrt(d)).astype(np.float32)
    wk = (rng.standard_normal((d, r)) / np.sqrt(d)).astype(np.float32)
    g = rng.standard_normal(d + 1).astype(np.float32) / 4
    bmap = oracle.block_map(qb, kbits, n_valid, kb)
    dout = rng.standard_normal((bh, n_pad, d))
    dout[:, n_valid:] = 0
    return dict(qb=qb, kb=kbits, vb=vb, q=oracle.widen_bf16(qb), k=oracle.widen_bf16(kbits), v=oracle.widen_bf16(vb),
                wq=wq, wk=wk, g=g, bmap=bmap, dout=dout, n_valid=n_valid, grid=grid, kbn=kb)


def _c_forward(c, q, k, v, wq, wk, gate, complement):
    """The C oracle's fp64 branch functions (no bf16 inputs), summed per row."""
    bh, n_pad, d = q.shape
    out = np.zeros_like(q)
    rows = np.arange(c["n_valid"])
    for h in range(bh):
        sp = oracle.sparse_rows(q[h:h + 1], k[h:h + 1], v[h:h + 1], c["bmap"][h:h + 1], c["n_valid"], rows)
        if complement:
            Sb, zb = oracle.lowrank_block_states(k[h], v[h], wk, c["n_valid"], c["grid"])
            lr = oracle.lowrank_rows_complement(q[h], wq, Sb, zb, c["bmap"][h], c["grid"], rows, gate_w=gate)
        else:
            S, z = oracle.lowrank_state(k[h:h + 1], v[h:h + 1], wk, c["n_valid"], c["grid"])
            lr = oracle.lowrank_rows(q[h:h + 1], wq, S, z, c["grid"], rows, gate_w=gate)
        out[h, :c["n_valid"]] = sp + lr
    return out


@pytest.mark.parametrize("complement", [False, True], ids=["global", "complement"])
@pytest.mark.parametrize("gated", [False, True], ids=["nogate", "gate"])
def test_torch_forward_equals_c_oracle(complement, gated):
    c = _case(61)
    g = c["g"] if gated else None
    ref = _c_forward(c, c["q"], c["k"], c["v"], c["wq"], c["wk"], g, complement)
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64))
    got = B.forward_torch(t(c["q"]), t(c["k"]), t(c["v"]), t(c["wq"]), t(c["wk"]), c["bmap"], c["n_valid"],
                          c["grid"], gate=None if g is None else t(g), complement=complement).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)
    # and the whole C forward on the bf16 inputs
    _, o = oracle.forward(c["qb"], c["kb"], c["vb"], c["wq"], c["wk"], c["n_valid"], c["kbn"], c["grid"],
                          gate_w=g, complement=complement)
    np.testing.assert_allclose(got, o, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("complement", [False, True], ids=["global", "complement"])
@pytest.mark.parametrize("gated", [False, True], ids=["nogate", "gate"])
def test_gradients_match_finite_differences(complement, gated):
    c = _case(67 + 2 * complement + gated)
    g = c["g"] if gated else None
    grads = B.backward(c["q"], c["k"], c["v"], c["wq"], c["wk"], c["bmap"], c["dout"], c["n_valid"], c["grid"],
                       gate=g, complement=complement)
    L = lambda **kw: float(np.sum(_c_forward(c, **{**dict(q=c["q"], k=c["k"], v=c["v"], wq=c["wq"], wk=c["wk"],
                                                         gate=g, complement=complement), **kw}) * c["dout"]))
    rng = np.random.default_rng(5)
    valid = (np.arange(c["q"].shape[1]) < c["n_valid"])[None, :, None]
    for name in ("q", "k", "v"):
        delta = rng.standard_normal(c[name].shape) * valid
        eps = 1e-6
        fd = (L(**{name: c[name] + eps * delta}) - L(**{name: c[name] - eps * delta})) / (2 * eps)
        an = float(np.sum(grads["d" + name] * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
        assert np.all(grads["d" + name][:, c["n_valid"]:] == 0)
    # fp32 parameters: coordinate steps of 2^-12 (exact in fp32 at these magnitudes)
    eps = 2.0 ** -12
    params = [("wq", (5, 3)), ("wq", (40, 11)), ("wk", (7, 0)), ("wk", (63, 15))]
    if gated:
        params += [("gate", (9,)), ("gate", (64,))]
    for name, idx in params:
        base = (c["g"] if name == "gate" else c[name]).copy()
        hi, lo = base.copy(), base.copy()
        hi[idx] += np.float32(eps)
        lo[idx] -= np.float32(eps)
        fd = (L(**{name: hi}) - L(**{name: lo})) / (float(hi[idx]) - float(lo[idx]))
        an = grads["dgate" if name == "gate" else "d" + name][idx]
        assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, idx, fd, an)


@pytest.mark.parametrize("complement", [False, True], ids=["global", "complement"])
@pytest.mark.parametrize("gated", [False, True], ids=["nogate", "gate"])
def test_sampled_formulas_equal_autograd(gated, complement):
    """The written-out gradient formulas (used at full size on sampled rows)
    reproduce the autograd gradients on every row of a small case, in both
    low-rank scopes."""
    c = _case(71 + gated, grid=(3, 7, 11), n_pad=256, d=64, r=16, bh=2, kb=2)
    g = c["g"] if gated else None
    dout_bits = to_bf16_bits(c["dout"].astype(np.float32))
    dout = oracle.widen_bf16(dout_bits)
    ref = B.backward(c["q"], c["k"], c["v"], c["wq"], c["wk"], c["bmap"], dout, c["n_valid"], c["grid"], gate=g,
                     complement=complement)
    rows = {h: list(range(c["n_valid"])) for h in range(2)}
    dq, dk, dv, dwq, dwk, dgate = B.backward_sampled(c["qb"], c["kb"], c["vb"], c["wq"], c["wk"], c["bmap"],
                                                     dout_bits, c["n_valid"], c["grid"], rows, rows, gate=g,
                                                     complement=complement)
    for h in range(2):
        np.testing.assert_allclose(dq[h], ref["dq"][h, :c["n_valid"]], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dk[h], ref["dk"][h, :c["n_valid"]], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dv[h], ref["dv"][h, :c["n_valid"]], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dwq, ref["dwq"], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dwk, ref["dwk"], rtol=1e-9, atol=1e-12)
    if gated:
        np.testing.assert_allclose(dgate, ref["dgate"], rtol=1e-9, atol=1e-12)


def test_sampled_formulas_empty_complement():
    """Every block kept (kb = nb): the complement is empty, the low-rank term and
    its gradients vanish, and the written-out formulas still equal autograd."""
    c = _case(75, grid=(3, 7, 11), n_pad=256, d=64, r=16, bh=2, kb=4)
    g = c["g"]
    dout_bits = to_bf16_bits(c["dout"].astype(np.float32))
    dout = oracle.widen_bf16(dout_bits)
    ref = B.backward(c["q"], c["k"], c["v"], c["wq"], c["wk"], c["bmap"], dout, c["n_valid"], c["grid"], gate=g,
                     complement=True)
    assert np.all(ref["dwq"] == 0) and np.all(ref["dwk"] == 0)
    rows = {h: list(range(c["n_valid"])) for h in range(2)}
    dq, dk, dv, dwq, dwk, dgate = B.backward_sampled(c["qb"], c["kb"], c["vb"], c["wq"], c["wk"], c["bmap"],
                                                     dout_bits, c["n_valid"], c["grid"], rows, rows, gate=g,
                                                     complement=True)
    for h in range(2):
        np.testing.assert_allclose(dq[h], ref["dq"][h, :c["n_valid"]], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dk[h], ref["dk"][h, :c["n_valid"]], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dv[h], ref["dv"][h, :c["n_valid"]], rtol=1e-9, atol=1e-12)
    assert np.all(dwq == 0) and np.all(dwk == 0) and np.all(dgate == 0)
