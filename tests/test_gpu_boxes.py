"""GPU parity of box partial acceptance (VFlash paper §2.5: for boxes the
drafts before the first uncertain coordinate are kept) and of box blocks
end to end: the drafted box tokens within the bf16 bar, then k, the first
schema failure and the first uncertain coordinate bit-exact against the
oracle on the same tokens and confidences.  Confidences stand in for the
external spatial-confidence model: seeded uniform values, with NaN, values
equal to the threshold and planted schema errors mixed in."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_draft_decoding_amd import synth
from oracle import fpd_oracle as O
from tests.gpu_cases import GpuCase, oracle_result, progress, small_ids, workload_inputs
from tests.test_gpu_parity import SMALL, compare_all, run_both, small_workload

pytestmark = pytest.mark.gpu


def _accept(fpd, lay_d, toks, conf, tau):
    B = toks.shape[0]
    k = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    fi = torch.full_like(k, -7)
    fu = torch.full_like(k, -7)
    fpd.fpd_accept_boxes(lay_d, torch.from_numpy(np.ascontiguousarray(toks)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(conf)).cuda(), tau, k, fi, fu)
    torch.cuda.synchronize()
    return k.cpu().numpy(), fi.cpu().numpy(), fu.cpu().numpy()


def _check(fpd, lay_d, lay, toks, conf, tau, what):
    got = _accept(fpd, lay_d, toks, conf, tau)
    want = O.accept_boxes(toks, conf, tau, lay)
    for name, g, w in zip(("k", "first_invalid", "first_uncertain"), got, want):
        bad = np.nonzero(g != w)[0]
        assert bad.size == 0, (what, name, bad[:5], g[bad[:5]], w[bad[:5]])
    return want


def _mixed_conf(B, P, seed, tau):
    conf = synth.make_box_conf(B, P, seed)
    rng = np.random.default_rng(seed)
    n = B * P // 50
    conf.reshape(-1)[rng.integers(0, B * P, n)] = np.float32(tau)      # exactly the threshold: certain
    conf.reshape(-1)[rng.integers(0, B * P, max(1, n // 20))] = np.nan
    return conf


def _legal_tokens(lay, B, rng, n_bad):
    toks = np.empty((B, lay.L - 1), np.int32)
    for p in range(1, lay.L):
        ids = lay.legal(p)
        toks[:, p - 1] = ids[rng.integers(0, len(ids), size=B)]
    rows = rng.choice(B, n_bad, replace=False)
    toks[rows, rng.integers(0, lay.L - 1, n_bad)] = rng.integers(-2, lay.vocab + 2, n_bad)
    return toks


def test_small_box_block_end_to_end():
    wl = small_workload("boxes2d", 3, 77, seed=70, n_points=9)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", "small boxes", inp.weights.w_lm)
    lay = res["layout"]
    toks = g.toks.cpu().numpy()
    P = lay.L - 1
    for tau in (0.0, 0.02, 0.3):
        _check(g.fpd, g.lay, lay, toks, _mixed_conf(wl.batch, P, 71, tau), tau, f"small tau={tau}")
    # all certain: the validator's decision
    k, fi, fu = _accept(g.fpd, g.lay, toks, np.ones((wl.batch, P), np.float32), 0.5)
    kv, fv = g.validate()
    assert np.array_equal(fi, fv.cpu().numpy()) and (fu == -1).all()
    assert np.array_equal(k, np.where(fi >= 0, fi, P))


@pytest.mark.parametrize("kind,over", [
    ("boxes2d", dict(n_points=150)),                       # L = 751: positions past one pass of the workgroup
    ("traj2d3d", dict(n_points=40, off_id=4099 - 1020 + 1002)),
    ("traj2d", dict(n_points=3)),
])
def test_accept_many_rows_bit_exact(kind, over):
    from block_draft_decoding_amd import fpd
    shape = replace(SMALL, n_layers=1)
    schema = dict(kind=kind, **small_ids(shape.vocab))
    schema.update(over)
    w = fpd.weights_to_device(synth.make_weights(shape, seed=13), torch.bfloat16)
    d = fpd.fpd_drafter_create(fpd.make_config(shape), w)
    lay_d = fpd.fpd_layout_create(d, schema)
    lay = O.build_layout(schema, shape.vocab)
    rng = np.random.default_rng(72)
    B = 384
    toks = _legal_tokens(lay, B, rng, B // 3)
    progress(f"[boxes] {kind} L={lay.L} B={B}")
    for tau in (0.001, 0.01, 0.5, -np.inf, np.inf):
        conf = _mixed_conf(B, lay.L - 1, 73, tau)
        want = _check(fpd, lay_d, lay, toks, conf, tau, f"{kind} tau={tau}")
        if tau == 0.001:
            k = want[0]
            assert len(np.unique(k)) > 8          # many distinct kept lengths
            assert 0 < (k == lay.L - 1).sum() or kind == "boxes2d"


def test_custom_layout_reads_only_coordinate_positions():
    """A custom set that mixes coordinates with another id is not a
    coordinate position: its confidence is never read."""
    from block_draft_decoding_amd import fpd
    shape = replace(SMALL, n_layers=1)
    ids = small_ids(shape.vocab)
    cb = ids["coord_base"]
    schema = dict(kind="custom", block_len=6, sets=[[cb, cb + 1, cb + 2], [cb, 7], [cb + 5]],
                  pos_set=[-2, 0, 1, 2, -1, 0], pairs=[], fields=[], **{**ids, "fill_id": -1})
    w = fpd.weights_to_device(synth.make_weights(shape, seed=14), torch.bfloat16)
    d = fpd.fpd_drafter_create(fpd.make_config(shape), w)
    lay_d = fpd.fpd_layout_create(d, schema)
    lay = O.build_layout(schema, shape.vocab)
    toks = np.array([[cb + 1, 7, cb + 5, 100, cb + 2]] * 4, np.int32)
    conf = np.array([[0.9, 0.0, 0.9, 0.0, 0.9],       # uncertain values only at non-coordinate slots
                     [0.9, 0.9, 0.0, 0.9, 0.9],
                     [np.nan, 0.9, 0.9, 0.9, 0.9],
                     [0.9, 0.9, 0.9, 0.9, 0.1]], np.float32)
    k, fi, fu = _check(fpd, lay_d, lay, toks, conf, 0.5, "custom")
    assert k.tolist() == [5, 2, 0, 4]


def test_full_size_box_list():
    """64 boxes (L = 321) from the 4B-class drafter over a 2048-position
    context: the block within the bf16 bar, then acceptance bit-exact."""
    name = "boxes64"
    wl, inp = workload_inputs(name)
    g = GpuCase(wl, inp)
    g.fuse()
    g.draft()
    lg = g.argmax(logits=True)
    torch.cuda.synchronize()
    progress(f"[gpu] {name} done")
    res = oracle_result(name)
    compare_all(wl, g, lg, res, "bf16", f"full {name}", inp.weights.w_lm)
    lay = res["layout"]
    toks = g.toks.cpu().numpy()
    conf = synth.make_box_conf(wl.batch, lay.L - 1, 4000 + wl.seed_index)
    for tau in (0.0, 0.004, 0.05):
        k, fi, fu = _check(g.fpd, g.lay, lay, toks, conf, tau, f"full tau={tau}")
        progress(f"[boxes64] tau={tau}: k={k.tolist()} first_uncertain={fu.tolist()}")
