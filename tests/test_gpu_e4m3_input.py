"""GPU parity of rola_forward_e4m3: the fp8 forward with the caller's e4m3
codes and per-block scales for the sparse branch (selection and the low-rank
branch on the bf16 inputs, as in the library's own fp8 mode).

Bars: block maps bit-exact.  Codes made by the library's own rule (taken from
the oracle's quantiser) give exactly the output of rola_forward in fp8 mode.
Codes made by another rule (half the e4m3 range) match the oracle's sparse
branch on their dequantised values plus the bf16 low-rank branch within the
fp8 bar, 6e-2 of the output RMS.
"""
import numpy as np
import pytest

import oracle
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_fp8 import bound_ratio8, fp8_cfg
from tests.test_gpu_parity import SMALL, _full_inputs, dev, host_f64, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _torch():
    import torch
    return torch


def _flat(w, x):
    return x.reshape(w.batch * w.heads, w.n_pad, w.head_dim)


def _rule_codes(w, bits):
    """The library's own rule, from the oracle: codes [B, H, n_pad, D], scales [B, H, nb]."""
    codes, scale, _ = oracle.quant_e4m3(_flat(w, bits), w.n_tokens)
    return codes.reshape(bits.shape), scale.reshape(w.batch, w.heads, w.nb)


def _half_range_codes(w, bits):
    """Another rule: scale = absmax/224, so codes use half the e4m3 range.
    Returns codes, scales and the dequantised values value(code) * scale."""
    torch = _torch()
    x = oracle.widen_bf16(_flat(w, bits)).astype(np.float32)
    bh, n_pad, d = x.shape
    blocks = x.reshape(bh, w.nb, 64, d).copy()
    valid = (np.arange(n_pad) < w.n_tokens).reshape(w.nb, 64)
    blocks[:, ~valid] = 0.0
    amax = np.abs(blocks).max(axis=(2, 3)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(224.0) / np.where(amax > 0, amax, 1), np.float32(1)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(224.0), np.float32(1)).astype(np.float32)
    y = (blocks * inv[:, :, None, None]).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(bh, n_pad, d)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    deq = (vals.reshape(bh, w.nb, 64, d) * scale[:, :, None, None].astype(np.float64)).reshape(bh, n_pad, d)
    shape = (w.batch, w.heads, n_pad, d)
    return codes.reshape(shape), scale.reshape(w.batch, w.heads, w.nb), deq


def _call(w, q, k, v, codes, scales, cfg, bmap=None, gate=None):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    wq, wk = W.make_proj(w)
    c8 = [torch.from_numpy(np.ascontiguousarray(c)).cuda() for c in codes]
    sc = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in scales]
    return rola.rola_forward_e4m3(dev(q), dev(k), dev(v), *c8, *sc, torch.from_numpy(wq).cuda(),
                                  torch.from_numpy(wk).cuda(), w.grid, cfg, block_idx_out=bmap, gate=gate)


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
def test_library_rule_codes_reproduce_the_fp8_forward(name, w):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("e4m3 input, library rule", name)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    (cq, sq), (ck, sk), (cv, sv) = (_rule_codes(w, x) for x in (q, k, v))
    cfg = fp8_cfg(w)
    bmap = torch.empty((w.batch, w.heads, w.nb, oracle.keep_blocks(w.topk, w.nb)), dtype=torch.int32, device="cuda")
    got = _call(w, q, k, v, (cq, ck, cv), (sq, sk, sv), cfg, bmap)
    ref = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg)
    torch.cuda.synchronize()
    m_ref = oracle.block_map(_flat(w, q), _flat(w, k), w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
    np.testing.assert_array_equal(bmap.cpu().numpy().reshape(m_ref.shape), m_ref)
    assert torch.equal(got, ref)


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16out", "f32out"])
def test_other_rule_codes_match_oracle(name, w, out_f32):
    from sparse_rank_attention_amd import rola
    say("e4m3 input, half-range codes", name, "f32out" if out_f32 else "bf16out")
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    (cq, sq, dq), (ck, sk, dk), (cv, sv, dv) = (_half_range_codes(w, x) for x in (q, k, v))
    cfg = fp8_cfg(w, out_dtype=rola.ROLA_OUT_F32 if out_f32 else rola.ROLA_OUT_BF16)
    out = _call(w, q, k, v, (cq, ck, cv), (sq, sk, sv), cfg)
    got = host_f64(out).reshape(w.batch * w.heads, w.n_pad, w.head_dim)
    bmap = oracle.block_map(_flat(w, q), _flat(w, k), w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
    qf, kf, vf = (oracle.widen_bf16(_flat(w, x)) for x in (q, k, v))
    ref = np.zeros_like(got)
    for h in range(w.batch * w.heads):
        rows = np.arange(w.n_tokens)
        sp = oracle.sparse_rows(dq[h:h + 1], dk[h:h + 1], dv[h:h + 1], bmap[h:h + 1], w.n_tokens, rows)
        S, z = oracle.lowrank_state(kf[h:h + 1], vf[h:h + 1], wk, w.n_tokens, w.grid)
        lr = oracle.lowrank_rows(qf[h:h + 1], wq, S, z, w.grid, rows)
        ref[h, :w.n_tokens] = sp + lr
    assert np.all(got[:, w.n_tokens:] == 0)
    g, r = got[:, :w.n_tokens], ref[:, :w.n_tokens]
    ratio = bound_ratio8(g, r, not out_f32)
    say("e4m3 input, half-range codes", name, "err/rms", rel_err(g, r), "err/bound", ratio)
    assert ratio <= 1.0


def test_token_major_codes_and_ignored_padding():
    """Q, K, V and their codes as slices of token-major [n_pad, 3*H*D] tensors
    (stride_n = 3*H*D, stride_h = D), with NaN codes (0x7f) in the padded rows:
    the output equals the one from contiguous inputs with zero padding."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("e4m3 input, token-major")
    w = SMALL[2][1]  # ragged, D = 128, H = 2
    q, k, v = W.make_qkv(w)
    wq, wk = (torch.from_numpy(x).cuda() for x in W.make_proj(w))
    (cq, sq), (ck, sk), (cv, sv) = (_rule_codes(w, x) for x in (q, k, v))
    cfg = fp8_cfg(w, out_dtype=rola.ROLA_OUT_F32)
    H, D, n_pad = w.heads, w.head_dim, w.n_pad
    sc = [torch.from_numpy(s).cuda() for s in (sq, sk, sv)]
    plain = rola.rola_forward_e4m3(dev(q), dev(k), dev(v), *(torch.from_numpy(c).cuda() for c in (cq, ck, cv)),
                                   *sc, wq, wk, w.grid, cfg)

    def token_major(parts, dtype):
        t = torch.empty((n_pad, 3 * H * D), dtype=dtype, device="cuda")
        for i, x in enumerate(parts):
            t[:, i * H * D:(i + 1) * H * D] = x[0].permute(1, 0, 2).reshape(n_pad, H * D)
        return [t[:, i * H * D:(i + 1) * H * D].unflatten(1, (H, D)).permute(1, 0, 2).unsqueeze(0) for i in range(3)]

    bq, bk, bv = token_major([dev(x) for x in (q, k, v)], torch.bfloat16)
    codes = [torch.from_numpy(c).cuda().clone() for c in (cq, ck, cv)]
    for c in codes:
        c[:, :, w.n_tokens:] = 0x7F  # NaN codes in the padded rows
    c8q, c8k, c8v = token_major(codes, torch.uint8)
    strided = rola.rola_forward_e4m3(bq, bk, bv, c8q, c8k, c8v, *sc, wq, wk, w.grid, cfg)
    torch.cuda.synchronize()
    assert torch.equal(strided[0, :, :w.n_tokens], plain[0, :, :w.n_tokens])
    assert torch.count_nonzero(strided[0, :, w.n_tokens:]).item() == 0


def test_full_size_library_rule_reproduces_the_fp8_forward():
    """Wan 14B 720P launch (40 heads, N = 75600, 35 kept blocks): codes by the
    library's rule give exactly the fp8 forward's output."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    name = "wan14b_720p"
    say("e4m3 input, full size", name)
    w, (q, k, v), (wq, wk) = _full_inputs(name)
    cfg = fp8_cfg(w)
    codes, scales = [], []
    for x in (q, k, v):
        c, s = _rule_codes(w, x)
        codes.append(torch.from_numpy(c).cuda())
        scales.append(torch.from_numpy(s).cuda())
        del c
    qd, kd, vd = dev(q), dev(k), dev(v)
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    got = rola.rola_forward_e4m3(qd, kd, vd, *codes, *scales, wqd, wkd, w.grid, cfg)
    ref = rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("scope", ["global", "complement"])
def test_library_rule_codes_with_gate_and_scope(scope):
    """The output gate and the complement scope work unchanged on this path:
    library-rule codes give exactly rola_forward's fp8 output."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("e4m3 input, gate", scope)
    w = SMALL[2][1]
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    gate = torch.from_numpy(W.make_gate(w)).cuda()
    (cq, sq), (ck, sk), (cv, sv) = (_rule_codes(w, x) for x in (q, k, v))
    cfg = fp8_cfg(w, lowrank_scope=rola.ROLA_LR_COMPLEMENT if scope == "complement" else rola.ROLA_LR_GLOBAL)
    got = _call(w, q, k, v, (cq, ck, cv), (sq, sk, sv), cfg, gate=gate)
    ref = rola.rola_forward(dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(),
                            w.grid, cfg, gate=gate)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
