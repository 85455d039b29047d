"""Block selection on rows with ties, bit-exact against the oracle.

The selection kernel narrows each row to the keys at or above the kb-th
largest of its 64 lane maxima when kb <= 64 and at most 128 keys reach that
bound, and searches the whole row otherwise.  These cases drive both paths
with ties at the threshold: every pooled score of a row equal (nb = 100: the
narrowed path; nb = 150: more than 128 candidates, the whole-row path), and
inputs with few distinct values (partial ties), at kb below and above 64.
Ties must go to the lowest key-block indices, as the oracle takes them."""
import numpy as np
import pytest

import oracle
from sparse_rank_attention_amd import workloads as W
from tests.conftest import gpu_available
from tests.test_gpu_parity import dev, say

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _bits(x):
    """float32 values exactly representable in bf16 -> bf16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xffff) == 0)
    return (u >> 16).astype(np.uint16)


def _case(kind, nb, topk, seed):
    w = W.Workload("ties", 1, 2, 64, (1, 1, nb * 64 - 17), topk, 16, "iid", seed=seed)
    rng = np.random.default_rng(seed)
    shape = (1, w.heads, w.n_pad, w.head_dim)
    if kind == "equal_scores":   # every key row the same: all scores of a query row tie
        q = rng.integers(-4, 5, size=shape).astype(np.float32) * 0.25
        k = np.broadcast_to(rng.integers(-4, 5, size=(1, w.heads, 1, w.head_dim)).astype(np.float32) * 0.25,
                            shape).copy()
    else:                        # few distinct values: partial ties
        q = rng.integers(-1, 2, size=shape).astype(np.float32)
        k = rng.integers(-1, 2, size=shape).astype(np.float32)
    q[:, :, w.n_tokens:] = 0.0
    k[:, :, w.n_tokens:] = 0.0
    return w, _bits(q), _bits(k)


CASES = [("equal_scores", 100, 0.25), ("equal_scores", 150, 0.25), ("equal_scores", 150, 0.6),
         ("few_values", 100, 0.3), ("few_values", 150, 0.2), ("few_values", 150, 0.5)]


@pytest.mark.parametrize("kind,nb,topk", CASES, ids=["%s-nb%d-top%g" % c for c in CASES])
def test_select_blocks_with_ties(kind, nb, topk):
    from sparse_rank_attention_amd import rola
    w, q, k = _case(kind, nb, topk, seed=nb)
    say("ties", kind, "nb", w.nb, "kb", oracle.keep_blocks(w.topk, w.nb))
    bmap = rola.rola_select_blocks(dev(q), dev(k), w.grid, rola.Config(topk=w.topk, rank=w.rank))
    qp = oracle.pool(q.reshape(-1, w.n_pad, w.head_dim), w.n_tokens)
    kp = oracle.pool(k.reshape(-1, w.n_pad, w.head_dim), w.n_tokens)
    m_ref = oracle.select(oracle.scores(qp, kp), oracle.keep_blocks(w.topk, w.nb))
    np.testing.assert_array_equal(bmap.cpu().numpy().reshape(m_ref.shape), m_ref)
