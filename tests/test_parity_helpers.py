"""CPU checks of the GPU tests' comparison helpers: the oracle decision
computed from gathered legal logits (compact vocabulary) equals the oracle's
own decision on full logits, and the decision margins agree between the
two logit layouts."""
import numpy as np
import pytest

from oracle import fpd_oracle as O
from tests.gpu_cases import (legal_logits, legal_rms, logit_scale, rel_close, rel_close_logits, tokens_from_legal,
                             top2_gap)


def _layout(kind, V=4099, **over):
    cb = V - 1020
    schema = dict(kind=kind, start_id=V - 4, mask_id=V - 1, delim_id=cb + 1001, off_id=-1, plus_id=cb + 1003,
                  minus_id=cb + 1004, digit0_id=cb + 1005, fill_id=cb + 1015, coord_base=cb, coord_count=1001)
    schema.update(over)
    return O.build_layout(schema, V)


@pytest.mark.parametrize("kind,over", [("traj2d3d", dict(n_points=9, off_id=4099 - 1020 + 1002)),
                                       ("points3d_text", dict(n_points=3)), ("traj2d", dict(n_points=5)),
                                       ("boxes2d", dict(n_points=4))])
def test_compact_decision_equals_full_decision(kind, over):
    lay = _layout(kind, **over)
    rng = np.random.default_rng(1)
    H, V = 32, 4099
    w = rng.standard_normal((V, H)) * 0.2
    if lay.off_id >= 0:
        w[lay.off_id] *= 6.0          # OFF wins some pairs
    h = rng.standard_normal((3, lay.L - 1, H))
    z = h @ w.T
    # dense ties in a few rows exercise the lowest-id rule
    z[0, :4] = np.round(z[0, :4])
    zg = legal_logits(h, w, lay)
    zg[0, :4] = O.gathered_logits(z, lay)[0, :4]
    np.testing.assert_allclose(zg, O.gathered_logits(z, lay), rtol=1e-12, atol=1e-12)
    assert np.array_equal(tokens_from_legal(zg, lay), O.constrained_tokens(z, lay))
    np.testing.assert_allclose(top2_gap(zg, lay, gathered=True), top2_gap(z, lay), rtol=0, atol=1e-12)
    np.testing.assert_allclose(legal_rms(zg, lay, gathered=True), legal_rms(z, lay), rtol=1e-12)
    if lay.off_id >= 0:
        assert (O.constrained_tokens(z, lay) == lay.off_id).any()


def test_logit_scale_is_the_rms_of_a_logit():
    # for hidden rows in random directions, h . w_t has rms ||h|| ||w_t|| / sqrt(H)
    schema = dict(kind="custom", block_len=4, sets=[list(range(100))], pos_set=[-2, 0, 0, 0], pairs=[], fields=[],
                  off_id=-1, fill_id=-1, digit0_id=-1, coord_base=0, coord_count=0)
    lay = O.build_layout(schema, 100)
    rng = np.random.default_rng(2)
    w = rng.standard_normal((100, 64)).astype(np.float32) * rng.uniform(0.01, 0.3, size=(100, 1)).astype(np.float32)
    h = rng.standard_normal((4000, 3, 64))
    s = logit_scale(h, w, lay)
    z = h @ w.astype(np.float64).T
    ratio = np.sqrt(np.mean(z * z, axis=(0, 1))) / np.sqrt(np.mean(s * s, axis=(0, 1)))
    np.testing.assert_allclose(ratio, 1.0, rtol=0.05)


def test_rel_close_rules():
    want = np.array([[1.0, -2.0, 0.5], [3.0, -np.inf, -np.inf]])
    rel_close(want * (1 + 1e-3), want, "bf16", "scaled")
    with pytest.raises(AssertionError):
        rel_close(want * 1.05, want, "bf16", "too far")
    # a single entry far off its value but within 2e-2 of the row scale passes
    # only when the row scale is given
    w1 = np.array([[1e-3]])
    with pytest.raises(AssertionError):
        rel_close(w1 + 1e-3, w1, "bf16", "singleton")
    rel_close(w1 + 1e-3, w1, "bf16", "singleton", scale=np.array([[1.0]]))
    with pytest.raises(AssertionError):        # -inf padding must match
        rel_close(np.array([[1.0, 0.0]]), np.array([[1.0, -np.inf]]), "bf16", "pattern")


def test_small_sets_are_compared_per_id_across_positions():
    # 6 positions: three use a 1-id set, three a 20-id set
    schema = dict(kind="custom", block_len=7, sets=[[5], list(range(20, 40))], pos_set=[-2, 0, 1, 0, 1, 0, 1],
                  pairs=[], fields=[], off_id=-1, fill_id=-1, digit0_id=-1, coord_base=0, coord_count=0)
    lay = O.build_layout(schema, 50)
    rng = np.random.default_rng(3)
    z = rng.standard_normal((2, 6, 50))
    want = O.gathered_logits(z, lay)
    got = want.copy()
    # a delimiter logit 5% off: within 2e-2 of its column (3 values of scale ~1)?  no:
    # 0.05 / sqrt(3) is above 2e-2 when the column's norm is small, so scale it
    got[0, 0, 0] += 0.01
    rel_close_logits(got, want, lay, "bf16", "delim")
    got[0, 0, 0] += 0.2
    with pytest.raises(AssertionError):
        rel_close_logits(got, want, lay, "bf16", "delim far")
