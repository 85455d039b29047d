"""GPU parity of the w8a8 linear layers (per-row e4m3 quantisation and the
scaled fp8 GEMM) against the CPU oracle.

Bars: codes and scales bit-exact.  GEMM outputs within a bound derived from
the arithmetic: the e4m3 products are exact in fp32, so the only roundings are
the fp32 accumulation over K terms, the scaling and bias, and the output
store.  The matrix core's fp32 accumulation is not assumed to round to
nearest (it measurably does not: errors grow with one sign), only to stay
within one fp32 ulp per addition, unit roundoff 2^-23; for any summation
order that gives at most K * 2^-23 of sum |products|.  With the scaling and
bias (3 * 2^-23 of the magnitude) and, for bf16 output, half a bf16 ulp:
    |got - ref| <= (K + 3) * 2^-23 * yabs + 2^-8 |ref|   (bf16 out)
where yabs = sx sw sum_k |products| + |bias| comes from the oracle.
"""
import numpy as np
import pytest

import oracle
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_parity import say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _torch():
    import torch
    return torch


def _bits_dev(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _bound_ratio(got, ref, yabs, K, bf16_out):
    bound = (K + 3) * 2.0 ** -23 * yabs + (2.0 ** -8 * np.abs(ref) if bf16_out else 2.0 ** -23 * np.abs(ref))
    bound = np.maximum(bound, 1e-30)
    return float(np.max(np.abs(got - ref) / bound))


def _mixed_rows(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-10, 8, size=(rows, 1)).astype(np.float32)
    if rows >= 3:
        x[rows // 3] = 0.0
    return W.to_bf16_bits(x)


@pytest.mark.parametrize("rows,cols,pad", [(1, 8, 0), (37, 200, 0), (300, 1536, 24), (5, 5120, 8), (3, 8200, 16)])
def test_quant_rows_bit_exact(rows, cols, pad):
    """Codes and scales equal the oracle's, also from a row slice of a wider
    buffer (pad extra columns per row)."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("quant rows", rows, cols, pad)
    rng = np.random.default_rng(rows * 7 + cols)
    xb = _mixed_rows(rng, rows, cols)
    wide = np.zeros((rows, cols + pad), dtype=np.uint16)
    wide[:, :cols] = xb
    wide[:, cols:] = W.to_bf16_bits(np.full((rows, pad), 1e4, dtype=np.float32))  # must be ignored
    xd = _bits_dev(wide)[:, :cols]
    codes, scale = rola.rola_quant_rows(xd)
    torch.cuda.synchronize()
    c_ref, s_ref, _ = oracle.quant_rows_e4m3(xb)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scale.cpu().numpy(), s_ref)


# (M, N, K): ragged token and channel tails, K of one, two, three and many stages
GEMM_CASES = [(1, 4, 64), (300, 100, 128), (257, 260, 192), (513, 512, 320), (1000, 772, 1536)]


@pytest.mark.parametrize("M,N,K", GEMM_CASES, ids=["%dx%dx%d" % c for c in GEMM_CASES])
@pytest.mark.parametrize("out_f32", [False, True], ids=["bf16out", "f32out"])
@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
def test_gemm_matches_oracle(M, N, K, out_f32, with_bias):
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("gemm", M, N, K, "f32out" if out_f32 else "bf16out", "bias" if with_bias else "nobias")
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    xb = _mixed_rows(rng, M, K)
    wb = W.to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    ca, sa, _ = oracle.quant_rows_e4m3(xb)
    cw, sw, _ = oracle.quant_rows_e4m3(wb)
    ref, yabs = oracle.gemm_w8a8(ca, sa, cw, sw, bias, with_abs=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # output written into a column slice of a wider buffer; the rest must stay untouched
    dt = torch.float32 if out_f32 else torch.bfloat16
    wide = torch.full((M, N + 16), 7.0, dtype=dt, device="cuda")
    out = wide[:, 8:8 + N]  # 16-byte aligned start, row stride N + 16
    rola.rola_gemm_w8a8(dev(ca), dev(sa), dev(cw), dev(sw), None if bias is None else dev(bias), out=out,
                        out_dtype=rola.ROLA_OUT_F32 if out_f32 else rola.ROLA_OUT_BF16)
    torch.cuda.synchronize()
    host = wide.float().cpu().numpy().astype(np.float64)
    assert np.all(host[:, :8] == 7.0) and np.all(host[:, 8 + N:] == 7.0)
    got = host[:, 8:8 + N]
    ratio = _bound_ratio(got, ref, yabs, K, not out_f32)
    rel = float(np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
    say("gemm", M, N, K, "err/bound", ratio, "rms rel", rel)
    assert ratio <= 1.0
    assert rel <= (4e-3 if not out_f32 else 1e-4)


def test_gemm_operands_from_wider_buffers():
    """x and w as column slices of wider code buffers (ld_x, ld_w > K): only
    their first K columns take part."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("gemm strided operands")
    M, N, K = 333, 196, 256
    rng = np.random.default_rng(12)
    ca, sa, _ = oracle.quant_rows_e4m3(_mixed_rows(rng, M, K))
    cw, sw, _ = oracle.quant_rows_e4m3(W.to_bf16_bits((rng.standard_normal((N, K)) / 16).astype(np.float32)))
    xw = np.full((M, K + 48), 0x7E, dtype=np.uint8)  # the extra columns hold the largest code
    ww = np.full((N, K + 32), 0x7E, dtype=np.uint8)
    xw[:, :K], ww[:, :K] = ca, cw
    xd = torch.from_numpy(xw).cuda()[:, :K]
    wd = torch.from_numpy(ww).cuda()[:, :K]
    y = rola.rola_gemm_w8a8(xd, torch.from_numpy(sa).cuda(), wd, torch.from_numpy(sw).cuda(),
                            out_dtype=rola.ROLA_OUT_F32)
    torch.cuda.synchronize()
    ref, yabs = oracle.gemm_w8a8(ca, sa, cw, sw, with_abs=True)
    assert _bound_ratio(y.cpu().numpy().astype(np.float64), ref, yabs, K, False) <= 1.0


def test_linear_layer_and_quantised_weights_on_device():
    """Weights quantised on the device, then the whole layer (activation
    quantisation + GEMM) against the oracle's linear_w8a8."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("linear layer")
    lw = W.LinearWorkload("small", 700, 640, 384, seed=3)
    xb = W.make_linear_x(lw)
    wb, bias = W.make_linear_w(lw)
    wc, sw = rola.rola_quant_rows(_bits_dev(wb))
    y = rola.rola_linear_w8a8(_bits_dev(xb), wc, sw, torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    ref, yabs = oracle.linear_w8a8(xb, wb, bias, with_abs=True)
    got = y.float().cpu().numpy().astype(np.float64)
    assert _bound_ratio(got, ref, yabs, lw.d_in, True) <= 1.0


def test_qkv_projection_feeds_attention_through_strides():
    """The fused Q/K/V projection writes a token-major [n_pad, 3*H*D] tensor;
    attention reads Q, K and V from it through strides (stride_n = 3*H*D,
    stride_h = D) and gives the same output as from contiguous copies."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("qkv -> attention strides")
    H, D, grid = 4, 64, (3, 7, 11)
    n = grid[0] * grid[1] * grid[2]
    n_pad = (n + 63) // 64 * 64
    lw = W.LinearWorkload("qkv_small", n_pad, H * D, 3 * H * D, seed=5)
    xb = W.make_linear_x(lw)
    xb[n:] = 0
    wb, bias = W.make_linear_w(lw)
    wc, sw = rola.rola_quant_rows(_bits_dev(wb))
    qkv = rola.rola_linear_w8a8(_bits_dev(xb), wc, sw, torch.from_numpy(bias).cuda())  # [n_pad, 3HD]
    view = lambda i: qkv[:, i * H * D:(i + 1) * H * D].unflatten(1, (H, D)).permute(1, 0, 2).unsqueeze(0)
    q, k, v = view(0), view(1), view(2)
    assert q.stride()[1:] == (D, 3 * H * D, 1)
    wq = torch.from_numpy((np.random.default_rng(1).standard_normal((D, 16)) / 8).astype(np.float32)).cuda()
    wk = torch.from_numpy((np.random.default_rng(2).standard_normal((D, 16)) / 8).astype(np.float32)).cuda()
    cfg = rola.Config(topk=0.3, rank=16)
    o_strided = rola.rola_forward(q, k, v, wq, wk, grid, cfg)
    o_contig = rola.rola_forward(q.contiguous(), k.contiguous(), v.contiguous(), wq, wk, grid, cfg)
    torch.cuda.synchronize()
    assert torch.equal(o_strided[0, :, :n], o_contig[0, :, :n])
    # and the projection itself, sampled, against the oracle
    rows = np.array([0, 1, 63, 64, n // 2, n - 1])
    ref, yabs = oracle.linear_w8a8(xb[rows], wb, bias, with_abs=True)
    got = qkv[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    assert _bound_ratio(got, ref, yabs, lw.d_in, True) <= 1.0


@pytest.mark.parametrize("name", ["wan14b_720p_qkv", "wan14b_720p_out", "wan13b_480p_qkv"])
def test_full_size_layer_sampled(name):
    """Wan 14B 720P projections (75600 tokens x 5120 -> 15360 or 5120) in the
    launch configuration the benchmark times, and the Wan 1.3B 480P QKV
    projection (32760 x 1536 -> 4608), checked on sampled rows: codes and
    scales bit-exact, outputs within the bound."""
    from sparse_rank_attention_amd import rola
    torch = _torch()
    say("full size", name)
    lw = W.LINEAR[name]
    xb = W.make_linear_x(lw)
    wb, bias = W.make_linear_w(lw)
    xd = _bits_dev(xb)
    del xb
    wc, sw = rola.rola_quant_rows(_bits_dev(wb))
    xc, sx = rola.rola_quant_rows(xd)
    y = rola.rola_gemm_w8a8(xc, sx, wc, sw, torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.array(sorted({0, 255, 256, lw.tokens - 1, lw.tokens - 100, *rng.integers(0, lw.tokens, 11).tolist()}))
    xs = W.make_linear_x(lw, rows)
    ca, sa, _ = oracle.quant_rows_e4m3(xs)
    cw, swr, _ = oracle.quant_rows_e4m3(wb)
    ridx = torch.from_numpy(rows).cuda()
    np.testing.assert_array_equal(xc[ridx].cpu().numpy(), ca)
    np.testing.assert_array_equal(sx[ridx].cpu().numpy(), sa)
    np.testing.assert_array_equal(wc.cpu().numpy(), cw)
    np.testing.assert_array_equal(sw.cpu().numpy(), swr)
    ref, yabs = oracle.gemm_w8a8(ca, sa, cw, swr, bias, with_abs=True)
    got = y[ridx].float().cpu().numpy().astype(np.float64)
    ratio = _bound_ratio(got, ref, yabs, lw.d_in, True)
    say("full size", name, "err/bound", ratio)
    assert ratio <= 1.0
