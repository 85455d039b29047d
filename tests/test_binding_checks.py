"""The Python binding checks every argument against the plan before anything
reaches the library's compute calls: wrong row counts, output dtype, shape or
strides, projection shapes and block-map shapes raise RolaError.  Runs on the
host: well-formed CPU tensors get as far as the GPU check and stop there."""
import pytest
import torch

from sparse_rank_attention_amd import rola

GRID = (2, 5, 9)            # N = 90 tokens -> nb = 2, n_pad = 128
B, H, D, NPAD, NB = 1, 2, 64, 128, 2


def _qkv(rows=NPAD, dtype=torch.bfloat16):
    return [torch.zeros((B, H, rows, D), dtype=dtype) for _ in range(3)]


def _cfg(**kw):
    return rola.Config(topk=0.5, rank=16, **kw)


def _proj(shape=(D, 16)):
    return torch.zeros(shape, dtype=torch.float32), torch.zeros(shape, dtype=torch.float32)


def test_well_formed_host_tensors_reach_the_gpu_check():
    q, k, v = _qkv()
    wq, wk = _proj()
    with pytest.raises(rola.RolaError, match="GPU"):
        rola.rola_forward(q, k, v, wq, wk, GRID, _cfg())
    with pytest.raises(rola.RolaError, match="GPU"):
        rola.rola_select_blocks(q, k, GRID, _cfg())


def test_unpadded_rows_are_rejected():
    q, k, v = _qkv(rows=90)  # N rows, not n_pad
    wq, wk = _proj()
    with pytest.raises(rola.RolaError, match="n_pad = 128"):
        rola.rola_forward(q, k, v, wq, wk, GRID, _cfg())
    with pytest.raises(rola.RolaError, match="n_pad"):
        rola.rola_lowrank_attn(q, k, v, wq, wk, GRID, _cfg())


@pytest.mark.parametrize("bad", ["dtype", "shape", "strides"])
def test_output_must_match_the_config_and_layout(bad):
    q, k, v = _qkv()
    wq, wk = _proj()
    out = torch.zeros_like(q)
    cfg = _cfg()
    if bad == "dtype":
        cfg = _cfg(out_dtype=rola.ROLA_OUT_F32)  # bf16 out with an fp32 out_dtype
    elif bad == "shape":
        out = torch.zeros((B, H, NPAD, D + 8), dtype=torch.bfloat16)[..., :D + 8]
    else:
        out = torch.zeros((B, NPAD, H, D), dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(rola.RolaError, match="out must"):
        rola.rola_forward(q, k, v, wq, wk, GRID, cfg, out=out)


@pytest.mark.parametrize("shape,dtype", [((D, 32), torch.float32), ((D, 16), torch.float64), ((16, D), torch.float32)])
def test_projections_must_be_fp32_head_dim_by_rank(shape, dtype):
    q, k, v = _qkv()
    wq = torch.zeros(shape, dtype=dtype)
    wk = torch.zeros((D, 16), dtype=torch.float32)
    with pytest.raises(rola.RolaError, match="wq and wk"):
        rola.rola_forward(q, k, v, wq, wk, GRID, _cfg())
    with pytest.raises(rola.RolaError, match="wq and wk"):
        rola.rola_lowrank_attn(q, k, v, wk, wq, GRID, _cfg())


def test_block_maps_must_match_the_plan():
    q, k, v = _qkv()
    wq, wk = _proj()
    kb = 1  # floor(0.5 * 2)
    for bad in (torch.zeros((B, H, NB, kb + 1), dtype=torch.int32),
                torch.zeros((B, H, NB, kb), dtype=torch.int64),
                torch.zeros((B, H, NB, 2 * kb), dtype=torch.int32)[..., ::2]):
        with pytest.raises(rola.RolaError, match="block_idx"):
            rola.rola_sparse_attn(q, k, v, bad, GRID, _cfg())
        with pytest.raises(rola.RolaError, match="block_idx_out"):
            rola.rola_forward(q, k, v, wq, wk, GRID, _cfg(), block_idx_out=bad)
        with pytest.raises(rola.RolaError, match="block_idx"):
            rola.rola_select_blocks(q, k, GRID, _cfg(), block_idx=bad)


def test_token_tensors_must_agree():
    q, k, v = _qkv()
    wq, wk = _proj()
    with pytest.raises(rola.RolaError, match="bfloat16"):
        rola.rola_forward(q.float(), k, v, wq, wk, GRID, _cfg())
    with pytest.raises(rola.RolaError, match="share shape"):
        rola.rola_forward(q, k[:, :1], v, wq, wk, GRID, _cfg())


def test_training_pair_arguments():
    """rola_forward_train checks as rola_forward does; the saved pair handed to
    rola_backward must be fp32 O_s with the layout of q and contiguous fp32
    [B*H, n_pad] log-sum-exps."""
    q, k, v = _qkv()
    wq, wk = _proj()
    with pytest.raises(rola.RolaError, match="GPU"):
        rola.rola_forward_train(q, k, v, wq, wk, GRID, _cfg())
    with pytest.raises(rola.RolaError, match="n_pad"):
        rola.rola_forward_train(*_qkv(rows=90), wq, wk, GRID, _cfg())
    bmap = torch.zeros((B, H, NB, 1), dtype=torch.int32)
    dout = torch.zeros_like(q)
    good_os = torch.zeros((B, H, NPAD, D), dtype=torch.float32)
    good_lse = torch.zeros((B * H, NPAD), dtype=torch.float32)
    with pytest.raises(rola.RolaError, match="GPU"):
        rola.rola_backward(q, k, v, wq, wk, GRID, _cfg(), bmap, dout, saved=(good_os, good_lse))
    for os_, lse, msg in ((good_os.to(torch.bfloat16), good_lse, "O_s"),
                          (good_os[:, :, :90], good_lse, "O_s"),
                          (good_os, good_lse[:, :90], "lse"),
                          (good_os, good_lse.t().contiguous().t(), "lse"),
                          (good_os, good_lse.to(torch.float64), "lse")):
        with pytest.raises(rola.RolaError, match=msg):
            rola.rola_backward(q, k, v, wq, wk, GRID, _cfg(), bmap, dout, saved=(os_, lse))
