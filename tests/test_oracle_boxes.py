"""Pins of the oracle's box partial acceptance (VFlash paper §2.5: for boxes
the drafts before the first uncertain coordinate are kept; reading R25 in the
oracle's header) and of the box layout.  Worked examples by hand, special
cases that reduce to the schema validator, monotonicity in the threshold, and
a brute force over every certain/uncertain pattern of a one-box block."""
import itertools

import numpy as np
import pytest

from oracle import fpd_oracle as O

V = 4099
CB = V - 1020
IDS = dict(start_id=V - 4, mask_id=V - 1, delim_id=CB + 1001, off_id=-1, plus_id=CB + 1003,
           minus_id=CB + 1004, digit0_id=CB + 1005, fill_id=CB + 1015, coord_base=CB, coord_count=1001)
DELIM = IDS["delim_id"]


def box_layout(n):
    return O.build_layout(dict(kind="boxes2d", n_points=n, **IDS), V)


def valid_boxes(n, rng, B=1):
    t = np.empty((B, 5 * n), np.int32)
    for b in range(B):
        for i in range(n):
            t[b, 5 * i:5 * i + 4] = CB + rng.integers(0, 1001, 4)
            t[b, 5 * i + 4] = DELIM
    return t


def test_box_layout_roles():
    lay = box_layout(3)
    assert lay.L == 16
    roles = [lay.is_coord(p) for p in range(1, lay.L)]
    assert roles == [True, True, True, True, False] * 3
    assert [len(lay.legal(p)) for p in range(1, 6)] == [1001, 1001, 1001, 1001, 1]
    assert lay.legal(5).tolist() == [DELIM]


def test_coordinate_positions_of_other_layouts():
    t3 = O.build_layout(dict(kind="traj2d3d", n_points=2, **{**IDS, "off_id": CB + 1002}), V)
    assert [t3.is_coord(p) for p in range(1, t3.L)] == [True] * 5 + [False] + [True] * 5 + [False]
    pts = O.build_layout(dict(kind="points3d_text", n_points=1, **IDS), V)
    assert not any(pts.is_coord(p) for p in range(1, pts.L))
    txt = O.build_layout(dict(kind="text", block_len=5, **IDS), V)
    assert not any(txt.is_coord(p) for p in range(1, txt.L))
    # a custom set mixing coordinates with another id is not a coordinate position
    cus = O.build_layout(dict(kind="custom", block_len=4, sets=[[CB, CB + 1], [CB, 7], [CB + 5]],
                              pos_set=[-2, 0, 1, 2], pairs=[], fields=[], **{**IDS, "fill_id": -1}), V)
    assert [cus.is_coord(p) for p in range(1, 4)] == [True, False, True]


def test_worked_examples():
    lay = box_layout(2)
    tok = np.array([[CB + 10, CB + 20, CB + 300, CB + 400, DELIM, CB + 1, CB + 2, CB + 3, CB + 4, DELIM]], np.int32)
    conf = np.array([[0.9, 0.9, 0.2, 0.9, 0.0, 0.9, 0.9, 0.9, 0.9, 0.0]], np.float32)
    k, fi, fu = O.accept_boxes(tok, conf, 0.5, lay)
    assert (k[0], fi[0], fu[0]) == (2, -1, 2)          # x2 of the first box is uncertain: keep x1, y1
    # delimiter confidences are never read
    k, fi, fu = O.accept_boxes(tok, np.where(conf == 0.0, np.nan, 0.9).astype(np.float32), 0.5, lay)
    assert (k[0], fi[0], fu[0]) == (10, -1, -1)
    # a confidence equal to the threshold is certain; NaN is not
    c = np.full((1, 10), 0.5, np.float32)
    assert O.accept_boxes(tok, c, 0.5, lay)[0][0] == 10
    c[0, 6] = np.nan
    assert O.accept_boxes(tok, c, 0.5, lay)[0][0] == 6
    # a schema failure before the first uncertain coordinate decides k
    bad = tok.copy()
    bad[0, 4] = CB + 7                                  # coordinate where the delimiter belongs
    c[0, 6] = 0.1
    k, fi, fu = O.accept_boxes(bad, c, 0.5, lay)
    assert (k[0], fi[0], fu[0]) == (4, 4, 6)
    # ... and an uncertain coordinate before a later schema failure
    bad = tok.copy()
    bad[0, 9] = CB
    k, fi, fu = O.accept_boxes(bad, c, 0.5, lay)
    assert (k[0], fi[0], fu[0]) == (6, 9, 6)


def test_all_certain_reduces_to_the_validator():
    rng = np.random.default_rng(5)
    lay = box_layout(6)
    tok = valid_boxes(6, rng, B=40)
    rows = rng.choice(40, 20, replace=False)
    tok[rows, rng.integers(0, 30, 20)] = rng.integers(0, V, 20)       # plant schema errors
    for conf in (np.full(tok.shape, np.inf, np.float32), rng.uniform(0.5, 1.0, tok.shape).astype(np.float32)):
        k, fi, fu = O.accept_boxes(tok, conf, 0.5, lay)
        kv, fv = O.validate_primitive(tok, lay)
        assert np.array_equal(fi, fv) and (fu == -1).all()
        assert np.array_equal(k, np.where(fv >= 0, fv, tok.shape[1]))


def test_all_uncertain_keeps_nothing():
    rng = np.random.default_rng(6)
    lay = box_layout(4)
    tok = valid_boxes(4, rng, B=8)
    for conf in (np.full(tok.shape, np.nan, np.float32), np.zeros(tok.shape, np.float32)):
        k, fi, fu = O.accept_boxes(tok, conf, 0.25, lay)
        assert (k == 0).all() and (fu == 0).all() and (fi == -1).all()


def test_monotone_in_the_threshold():
    rng = np.random.default_rng(7)
    lay = box_layout(8)
    tok = valid_boxes(8, rng, B=30)
    conf = rng.uniform(0, 1, tok.shape).astype(np.float32)
    prev = None
    for tau in np.linspace(0, 1, 21):
        k = O.accept_boxes(tok, conf, tau, lay)[0]
        if prev is not None:
            assert (k <= prev).all()
        prev = k
    assert (prev <= 40).all()


def test_brute_force_one_box():
    """Every certain/uncertain pattern over the 4 coordinates of one valid box
    and every delimiter slot content: k is the length of the longest prefix
    whose coordinates are all certain and whose tokens are all legal."""
    lay = box_layout(1)
    base = np.array([CB + 1, CB + 2, CB + 3, CB + 4, DELIM], np.int32)
    for pattern in itertools.product([0, 1], repeat=4):
        for last in (DELIM, CB + 9):
            tok = base.copy()
            tok[4] = last
            conf = np.array(list(pattern) + [0], np.float32)
            k, fi, fu = O.accept_boxes(tok[None], conf[None], 1.0, lay)
            good = 0
            while good < 5:
                legal = tok[good] in lay.legal(good + 1)
                certain = good == 4 or pattern[good] == 1
                if not (legal and certain):
                    break
                good += 1
            assert k[0] == good, (pattern, last, k[0], good)


@pytest.mark.parametrize("n", [1, 2, 64])
def test_block_length_counts_one_anchor_and_five_per_box(n):
    assert box_layout(n).L == 1 + 5 * n
