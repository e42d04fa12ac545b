"""Pins of the oracle's logits: the full-vocabulary LM head against an
explicit dot product per (position, id), whatever the row-chunk size, and
the gathered legal logits against the full logits restricted to each
position's legal set (VFlash paper §2.5: the constraints act on logits that
are already computed, so restricting them is the whole effect)."""
import math

import numpy as np
import pytest

from block_draft_decoding_amd import synth
from oracle import fpd_oracle as O


def _model(V, H=48, dtype="f32"):
    s = synth.DrafterShape(hidden=H, n_q=2, n_kv=1, head_dim=16, n_layers=1, inter=64, vocab=V, n_fused=1,
                           dtype=dtype, weight_std=0.3)
    return O.Model(s, synth.make_weights(s, 17))


def _dot_logits(h, W):
    """z[b, p, v] = sum_k h[b, p, k] W[v, k], each sum exactly rounded (fsum)."""
    B, P, H = h.shape
    z = np.empty((B, P, W.shape[0]))
    for b in range(B):
        for p in range(P):
            for v in range(W.shape[0]):
                z[b, p, v] = math.fsum(float(x) * float(y) for x, y in zip(h[b, p], W[v]))
    return z


@pytest.mark.parametrize("chunk", [1, 7, 64, 100, 299, 300, 301, 8192])
def test_full_logits_is_the_dot_product_for_every_chunk_size(chunk):
    # V = 300 is not a multiple of most chunk sizes: the last chunk is ragged
    m = _model(300)
    rng = np.random.default_rng(3)
    h = rng.standard_normal((2, 3, 48))
    want = _dot_logits(h, m.w.w_lm.astype(np.float64))
    got = O.full_logits(m, h, chunk_rows=chunk)
    assert got.shape == (2, 3, 300)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_full_logits_of_bf16_weights_use_the_stored_values():
    # bf16 workloads hold bf16 values; the logits are their exact products
    m = _model(130, dtype="bf16")
    w = m.w.w_lm.astype(np.float64)
    assert np.array_equal(w, O.bf16_round(w))
    h = O.bf16_round(np.random.default_rng(4).standard_normal((1, 2, 48)))
    np.testing.assert_allclose(O.full_logits(m, h, chunk_rows=64), _dot_logits(h, w), rtol=1e-12, atol=1e-12)


def test_full_logits_one_hot_hidden_reads_a_column():
    # h = e_k gives z[v] = W[v, k] exactly
    m = _model(77)
    h = np.zeros((1, 1, 48))
    h[0, 0, 5] = 1.0
    assert np.array_equal(O.full_logits(m, h, chunk_rows=10)[0, 0], m.w.w_lm[:, 5].astype(np.float64))


def _layout():
    # sets of 1, 3 and 6 ids given out of order (stored ascending), one free
    # position, one position per set more than once
    schema = dict(kind="custom", block_len=7, sets=[[9], [40, 2, 17], [5, 1, 33, 8, 29, 13]],
                  pos_set=[-2, 1, 0, 2, -1, 1, 2], pairs=[], fields=[], off_id=-1, fill_id=-1, digit0_id=-1,
                  coord_base=0, coord_count=0)
    return O.build_layout(schema, 50)


def test_gathered_logits_are_the_restriction_of_the_full_logits():
    lay = _layout()
    rng = np.random.default_rng(5)
    z = rng.standard_normal((2, lay.L - 1, 50))
    got = O.gathered_logits(z, lay)
    assert got.shape == (2, 6, 50)           # a free position makes the row as wide as the vocabulary
    legal = {1: [2, 17, 40], 2: [9], 3: [1, 5, 8, 13, 29, 33], 4: list(range(50)), 5: [2, 17, 40],
             6: [1, 5, 8, 13, 29, 33]}
    for b in range(2):
        for p, ids in legal.items():
            row = got[b, p - 1]
            for i, v in enumerate(ids):
                assert row[i] == z[b, p - 1, v]
            assert np.all(np.isneginf(row[len(ids):]))


def test_gathered_logits_width_without_free_positions():
    schema = dict(kind="custom", block_len=4, sets=[[3, 1], [7, 6, 5, 4]], pos_set=[-2, 0, 1, 0], pairs=[],
                  fields=[], off_id=-1, fill_id=-1, digit0_id=-1, coord_base=0, coord_count=0)
    lay = O.build_layout(schema, 10)
    z = np.arange(30, dtype=np.float64).reshape(1, 3, 10)
    got = O.gathered_logits(z, lay)
    want = np.array([[[1, 3, -np.inf, -np.inf], [14, 15, 16, 17], [21, 23, -np.inf, -np.inf]]])
    assert np.array_equal(got, want)


def test_masked_argmax_equals_argmax_of_the_gathered_row():
    # the decision on the gathered row (first maximum, ascending ids) is the
    # masked argmax over the full logits
    lay = _layout()
    rng = np.random.default_rng(6)
    z = rng.integers(-3, 3, size=(4, lay.L - 1, 50)).astype(np.float64)     # ties
    toks = O.masked_argmax(z, lay)
    g = O.gathered_logits(z, lay)
    for b in range(4):
        for p in range(1, lay.L):
            assert toks[b, p - 1] == lay.legal(p)[int(np.argmax(g[b, p - 1]))]
