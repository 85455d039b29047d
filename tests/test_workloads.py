"""The seeded input generators: shapes, padding, determinism and per-head independence."""
import numpy as np

from sparse_rank_attention_amd import workloads as W


def test_shapes_padding_and_determinism():
    w = W.WORKLOADS["tiny"]
    q, k, v = W.make_qkv(w)
    assert q.shape == (1, 2, 1024, 64) and q.dtype == np.uint16
    q2, _, _ = W.make_qkv(w)
    np.testing.assert_array_equal(q, q2)
    wq, wk = W.make_proj(w)
    assert wq.shape == (64, 16) and wq.dtype == np.float32
    assert not np.array_equal(wq, wk)


def test_field_heads_regenerate_alone_and_pad_with_zero():
    w = W.Workload("t", 1, 3, 64, (3, 5, 7), 0.25, 16, "field")
    assert w.n_tokens == 105 and w.n_pad == 128 and w.nb == 2
    q, k, v = W.make_qkv(w)
    q1, k1, v1 = W.make_qkv(w, heads=[1])
    np.testing.assert_array_equal(q[:, 1:2], q1)
    np.testing.assert_array_equal(v[:, 1:2], v1)
    assert np.all(q[:, :, 105:] == 0) and np.all(v[:, :, 105:] == 0)
    qf = W.bf16_bits_to_f32(q[0, :, :105])
    assert 0.5 < qf.std() < 2.0


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], dtype=np.float32)
    b = W.bf16_bits_to_f32(W.to_bf16_bits(x))
    np.testing.assert_array_equal(b, np.array([1.0, 1.0 + 2.0 ** -6, 1.0], dtype=np.float32))


def test_linear_inputs_regenerate_by_rows():
    """Sampled rows of the w8a8 activations equal the same rows of the whole
    matrix (chunked seeding), and the weights are reproducible."""
    lw = W.LinearWorkload("t", 9000, 64, 32, seed=4)
    full = W.make_linear_x(lw)
    rows = np.array([0, 1, 4095, 4096, 8191, 8999])
    np.testing.assert_array_equal(W.make_linear_x(lw, rows), full[rows])
    w1, b1 = W.make_linear_w(lw)
    w2, b2 = W.make_linear_w(lw)
    np.testing.assert_array_equal(w1, w2)
    np.testing.assert_array_equal(b1, b2)
    # the outlier channels carry about 8x the scale of the others
    x = W.bf16_bits_to_f32(full)
    hot = W._outlier_channels(lw)
    cold = np.setdiff1d(np.arange(lw.d_in), hot)
    ratio = x[:, hot].std() / x[:, cold].std()
    assert 7.0 < ratio < 9.0
