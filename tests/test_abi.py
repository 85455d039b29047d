"""The C ABI of librola on the host: it loads, exports every declared call, and
plans and validates without touching a device (no compute calls here)."""
import ctypes
import os
import re

import pytest

from sparse_rank_attention_amd import rola

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.byref


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "rola.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rola_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("rola_select_blocks", "rola_sparse_attn", "rola_lowrank_attn", "rola_forward", "rola_plan"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = rola.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert set(rola.EXPORTS) == set(_declared_functions())
    assert L.rola_abi_version() == rola.ABI_VERSION == 8


def _prob(B=1, H=40, D=128, grid=(21, 45, 80), sn=None):
    sn = D if sn is None else sn
    n_pad = ((grid[0] * grid[1] * grid[2] + 63) // 64) * 64
    return rola.RolaProblem(B, H, D, grid[0], grid[1], grid[2], H * n_pad * sn, n_pad * sn, sn)


def _plan(prob, cfg):
    info = rola.RolaPlanInfo()
    c = cfg.c()
    st = rola.lib().rola_plan(P(prob), P(c), P(info))
    return st, info


@pytest.mark.parametrize("grid,topk,nb,kb", [((4, 16, 16), 0.25, 16, 4), ((21, 30, 52), 0.10, 512, 51),
                                              ((21, 30, 52), 0.05, 512, 25), ((21, 45, 80), 0.03, 1182, 35),
                                              ((21, 45, 80), 0.10, 1182, 118), ((21, 45, 80), 0.05, 1182, 59),
                                              ((1, 1, 40), 0.5, 1, 1), ((21, 45, 80), 1.0, 1182, 1182)])
def test_plan_block_counts(grid, topk, nb, kb):
    st, info = _plan(_prob(grid=grid), rola.Config(topk=topk))
    assert st == 0
    assert (info.nb, info.kb) == (nb, kb)
    assert info.n_pad == 64 * nb and info.n_tokens == grid[0] * grid[1] * grid[2]
    st2, info2 = _plan(_prob(grid=grid), rola.Config(topk=topk))
    assert info2.workspace_bytes == info.workspace_bytes > 0


def test_complement_scope_plans_its_block_states():
    """The complement scope adds per-block states and per-query-block complements
    (bf16 S, fp32 z each) and the fp32 global S to the workspace."""
    prob = _prob()
    st, g = _plan(prob, rola.Config(topk=0.03))
    st2, c = _plan(prob, rola.Config(topk=0.03, lowrank_scope=rola.ROLA_LR_COMPLEMENT))
    assert st == st2 == 0 and (c.nb, c.kb) == (g.nb, g.kb)
    bh, nb, D = 40, 1182, 128
    extra = bh * nb * (D * 32 * 2 + 32 * 4) + bh * D * 32 * 4 + bh * nb * D * 32 * 2 + bh * nb * 32 * 4
    assert extra <= c.workspace_bytes - g.workspace_bytes <= extra + 4 * 256


def test_plan_rejects_bad_arguments():
    ok = rola.Config(topk=0.1)
    cases = [
        (_prob(D=96), ok, 2),                                     # head_dim unsupported
        (_prob(), rola.Config(topk=0.1, rank=8), 2),              # rank unsupported
        (_prob(), rola.Config(topk=0.0), 1),                      # topk outside (0, 1]
        (_prob(), rola.Config(topk=1.5), 1),
        (_prob(), rola.Config(topk=float("nan")), 1),
        (_prob(), rola.Config(topk=0.1, kb_override=5000), 1),    # more blocks than exist
        (_prob(), rola.Config(topk=0.1, rope_split=(32, 48, 46)), 1),  # split must sum to D
        (_prob(), rola.Config(topk=0.1, rope_split=(33, 47, 48)), 1),  # and be even
        (_prob(sn=132), ok, 3),                                   # rows not 16-byte aligned
        (_prob(sn=64), ok, 3),                                    # row shorter than D
        (_prob(grid=(1, 1, 64 * 4097)), ok, 2),                   # too many blocks
        (_prob(grid=(0, 45, 80)), ok, 1),
        (_prob(), rola.Config(topk=0.1, precision=7), 1),
        (_prob(), rola.Config(topk=0.1, out_dtype=3), 1),
        (_prob(), rola.Config(topk=0.1, lowrank_scope=2), 1),
    ]
    for prob, cfg, want in cases:
        st, _ = _plan(prob, cfg)
        assert st == want, (prob.head_dim, cfg, st)


def test_entry_points_validate_before_launch():
    """Errors are returned before any device work, so these run without a GPU."""
    L = rola.lib()
    prob, cfg = _prob(grid=(4, 16, 16), D=64, H=2), rola.Config(topk=0.25, rank=16).c()
    st, info = _plan(prob, rola.Config(topk=0.25, rank=16))
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x10008)    # not 16-byte aligned
    null = ctypes.c_void_p(0)
    big = info.workspace_bytes
    # null pointers
    assert L.rola_forward(P(prob), P(cfg), null, fake, fake, fake, fake, null, null, fake, fake, big, null) == 1
    assert L.rola_select_blocks(P(prob), P(cfg), fake, fake, null, null, fake, big, null) == 1
    # misaligned tensors
    assert L.rola_sparse_attn(P(prob), P(cfg), odd, fake, fake, fake, fake, 0, fake, big, null) == 3
    # workspace too small or missing
    assert L.rola_forward(P(prob), P(cfg), fake, fake, fake, fake, fake, null, null, fake, fake, big - 1,
                          null) == 4
    assert L.rola_lowrank_attn(P(prob), P(cfg), fake, fake, fake, fake, fake, null, fake, 0, null, big,
                               null) == 4
    # the output gate is read as 16-byte vectors
    assert L.rola_forward(P(prob), P(cfg), fake, fake, fake, fake, fake, odd, null, fake, fake, big, null) == 3
    assert L.rola_lowrank_attn(P(prob), P(cfg), fake, fake, fake, fake, fake, odd, fake, 0, fake, big,
                               null) == 3
    # bad accumulate flag
    assert L.rola_sparse_attn(P(prob), P(cfg), fake, fake, fake, fake, fake, 2, fake, big, null) == 1
    # status strings
    assert L.rola_status_str(4) == b"workspace missing or too small"


def test_backward_validates_before_launch():
    L = rola.lib()
    prob = _prob(grid=(4, 16, 16), D=64, H=2)
    cfg = rola.Config(topk=0.25, rank=16)
    st, info = _plan(prob, cfg)
    assert st == 0 and info.workspace_bytes_backward > info.workspace_bytes
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    null = ctypes.c_void_p(0)
    big = info.workspace_bytes_backward
    ok = [fake] * 5 + [null] + [fake] * 7 + [null]  # q, k, v, wq, wk; gate; block_idx .. dwk; dgate

    def call(c, args, ws_bytes=big):
        return L.rola_backward(P(prob), P(c.c()), *args, fake, ws_bytes, null)

    args = list(ok)
    args[0] = null
    assert call(cfg, args) == 1                               # q missing
    args = list(ok)
    args[5] = fake
    assert call(cfg, args) == 1                               # gate without dgate
    args = list(ok)
    args[7] = odd
    assert call(cfg, args) == 3                               # dout misaligned
    assert call(cfg, ok, big - 1) == 4                        # workspace too small
    assert call(rola.Config(topk=0.25, rank=16, precision=rola.ROLA_PREC_FP8), ok) == 2
    # the complement scope plans per-block states and per-block gradient sums
    # on top, and checks for them before launching
    comp = rola.Config(topk=0.25, rank=16, lowrank_scope=rola.ROLA_LR_COMPLEMENT)
    st, cinfo = _plan(prob, comp)
    assert st == 0 and cinfo.workspace_bytes_backward > big
    assert call(comp, ok, cinfo.workspace_bytes_backward - 1) == 4


def test_training_pair_validates_before_launch():
    """rola_forward_train needs both saved outputs and bf16 precision; rola_backward_saved
    needs both saved inputs (aligned) and otherwise checks as rola_backward does."""
    L = rola.lib()
    prob = _prob(grid=(4, 16, 16), D=64, H=2)
    cfg = rola.Config(topk=0.25, rank=16)
    fp8 = rola.Config(topk=0.25, rank=16, precision=rola.ROLA_PREC_FP8)
    st, info = _plan(prob, cfg)
    assert st == 0
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    odd4 = ctypes.c_void_p(0x10002)
    null = ctypes.c_void_p(0)
    # forward_train: q, k, v, wq, wk, gate, block_idx_out, out, os, lse
    fwd = [fake] * 5 + [null, null, fake, fake, fake]

    def ftrain(c, args, ws_bytes=info.workspace_bytes):
        return L.rola_forward_train(P(prob), P(c.c()), *args, fake, ws_bytes, null)

    for i in (8, 9):
        args = list(fwd)
        args[i] = null
        assert ftrain(cfg, args) == 1                          # os or lse missing
    args = list(fwd)
    args[8] = odd
    assert ftrain(cfg, args) == 3                              # os misaligned
    args = list(fwd)
    args[9] = odd4
    assert ftrain(cfg, args) == 3                              # lse misaligned
    assert ftrain(cfg, fwd, info.workspace_bytes - 1) == 4     # workspace too small
    assert ftrain(fp8, fwd) == 2                               # fp8: no training pair
    # backward_saved: q, k, v, wq, wk, gate, block_idx, dout, os, lse, dq, dk, dv, dwq, dwk, dgate
    bwd = [fake] * 5 + [null] + [fake] * 9 + [null]

    def bsaved(c, args, ws_bytes=info.workspace_bytes_backward):
        return L.rola_backward_saved(P(prob), P(c.c()), *args, fake, ws_bytes, null)

    for i in (8, 9):
        args = list(bwd)
        args[i] = null
        assert bsaved(cfg, args) == 1                          # os or lse missing
    args = list(bwd)
    args[8] = odd
    assert bsaved(cfg, args) == 3                              # os misaligned
    args = list(bwd)
    args[0] = null
    assert bsaved(cfg, args) == 1                              # q missing
    assert bsaved(cfg, bwd, info.workspace_bytes_backward - 1) == 4
    assert bsaved(fp8, bwd) == 2


def test_mfma_probe_validates_before_launch():
    L = rola.lib()
    flop = ctypes.c_double(-1.0)
    fake = ctypes.c_void_p(0x10000)
    assert L.rola_mfma_probe(rola.ROLA_PREC_BF16, 0, P(flop), fake, None) == 1
    assert L.rola_mfma_probe(7, 100, P(flop), fake, None) == 1
    assert L.rola_mfma_probe(rola.ROLA_PREC_FP8, 100, None, fake, None) == 1
    assert L.rola_mfma_probe(rola.ROLA_PREC_FP8, 100, P(flop), None, None) == 1
    assert flop.value == -1.0


def test_timing_read_without_launches_is_empty():
    assert rola.lib().rola_timing_read(None, 4) == -1
    assert rola.timing_read() == {}


def test_plan_fp8_adds_code_images_to_workspace():
    """fp8 mode keeps one 64*D-byte e4m3 K tile image and 64 rows of V codes as fp16 values
    (128*D bytes) per (batch, head, block), plus three scales (compared at fp32 output, where
    the bf16 path keeps no fp16 copy of V)."""
    prob = _prob(grid=(21, 45, 80))
    f32 = dict(topk=0.03, out_dtype=rola.ROLA_OUT_F32)
    st, b = _plan(prob, rola.Config(**f32))
    st8, f = _plan(prob, rola.Config(precision=rola.ROLA_PREC_FP8, **f32))
    assert st == st8 == 0
    bh_nb = prob.batch * prob.heads * f.nb
    assert f.workspace_bytes - b.workspace_bytes >= bh_nb * (192 * prob.head_dim + 16)
    assert f.workspace_bytes - b.workspace_bytes <= bh_nb * (192 * prob.head_dim + 16) + 5 * 256


def test_plan_bf16_output_adds_fp16_copy_of_v():
    """bf16 output with bf16 operands keeps an fp16 copy of V ([B*H][nb*64][D]) and two range
    flags per (batch*head, pass-1 chunk); fp32 output does not, and fp8 mode keeps its fp16 V
    codes at either output type."""
    prob = _prob(grid=(21, 45, 80))
    st, a = _plan(prob, rola.Config(topk=0.03))
    st32, b = _plan(prob, rola.Config(topk=0.03, out_dtype=rola.ROLA_OUT_F32))
    st8a, c = _plan(prob, rola.Config(topk=0.03, precision=rola.ROLA_PREC_FP8))
    st8b, d = _plan(prob, rola.Config(topk=0.03, precision=rola.ROLA_PREC_FP8, out_dtype=rola.ROLA_OUT_F32))
    assert st == st32 == st8a == st8b == 0
    bh = prob.batch * prob.heads
    copy = bh * a.nb * 64 * prob.head_dim * 2
    # flags: two per pass-1 chunk (at most two per block), 4 bytes each; two 256-byte alignments
    assert copy < a.workspace_bytes - b.workspace_bytes <= copy + bh * a.nb * 8 + 2 * 256
    assert c.workspace_bytes == d.workspace_bytes


def test_plan_rejects_token_stride_beyond_32bit_tile_offsets():
    st, _ = _plan(_prob(sn=(1 << 24) + 8), rola.Config(topk=0.1))
    assert st == 2
    st, _ = _plan(_prob(sn=1 << 24), rola.Config(topk=0.1))
    assert st == 0


def test_w8a8_entries_validate_before_launch():
    """The row quantisation and the fp8 GEMM reject bad shapes, strides and
    alignment before any device work."""
    L = rola.lib()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    odd4 = ctypes.c_void_p(0x10002)
    null = ctypes.c_void_p(0)
    q = L.rola_quant_rows
    assert q(null, 10, 64, 64, fake, 64, fake, null) == 1
    assert q(fake, 10, 60, 64, fake, 64, fake, null) == 1        # cols not a multiple of 8
    assert q(fake, 10, 64, 32, fake, 64, fake, null) == 1        # ld_x < cols
    assert q(fake, 10, 64, 64, fake, 60, fake, null) == 1        # ld_codes not a multiple of 8
    assert q(odd, 10, 64, 64, fake, 64, fake, null) == 3
    assert q(fake, 10, 64, 64, fake, 64, odd4, null) == 3       # scale not 4-byte aligned
    assert q(fake, 0, 64, 64, fake, 64, fake, null) == 0         # no rows: nothing to do
    g = L.rola_gemm_w8a8
    ok = dict(x=fake, ldx=128, sx=fake, w=fake, ldw=128, sw=fake, bias=null, M=100, N=64, K=128, out=fake,
              ldo=64, dt=0)

    def call(**kw):
        a = {**ok, **kw}
        return g(a["x"], a["ldx"], a["sx"], a["w"], a["ldw"], a["sw"], a["bias"], a["M"], a["N"], a["K"],
                 a["out"], a["ldo"], a["dt"], null)
    assert call(x=null) == 1 and call(sw=null) == 1 and call(out=null) == 1
    assert call(K=96) == 1 and call(K=0) == 1                    # K a positive multiple of 64
    assert call(N=66) == 1 and call(M=-1) == 1
    assert call(M=0) == 0                                        # no tokens: nothing to do
    assert call(ldx=64) == 1 and call(ldw=136) == 1 and call(ldo=60) == 1 and call(ldo=66) == 1
    assert call(ldx=1 << 24) == 1
    assert call(dt=2) == 1
    assert call(x=odd) == 3 and call(out=odd) == 3 and call(sw=odd) == 3 and call(bias=odd) == 3
    assert call(sx=odd4) == 3


def test_forward_e4m3_validates_before_launch():
    L = rola.lib()
    prob = _prob(grid=(4, 16, 16), D=64, H=2)
    fp8 = rola.Config(topk=0.25, rank=16, precision=rola.ROLA_PREC_FP8)
    st, info = _plan(prob, fp8)
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    odd4 = ctypes.c_void_p(0x10002)
    null = ctypes.c_void_p(0)
    big = info.workspace_bytes

    def call(cfg, **kw):
        a = dict(q=fake, k=fake, v=fake, q8=fake, k8=fake, v8=fake, qs=fake, ks=fake, vs=fake, wq=fake, wk=fake,
                 gate=null, map=null, out=fake)
        a.update(kw)
        return L.rola_forward_e4m3(P(prob), P(cfg.c()), a["q"], a["k"], a["v"], a["q8"], a["k8"], a["v8"],
                                   a["qs"], a["ks"], a["vs"], a["wq"], a["wk"], a["gate"], a["map"], a["out"],
                                   fake, kw.get("ws", big), null)
    assert call(rola.Config(topk=0.25, rank=16)) == 1          # bf16 precision
    assert call(fp8, k8=null) == 1 and call(fp8, vs=null) == 1
    assert call(fp8, q8=odd) == 3 and call(fp8, qs=odd4) == 3
    assert call(fp8, ws=big - 1) == 4
