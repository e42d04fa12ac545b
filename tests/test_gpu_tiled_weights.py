"""GPU parity of the K-tile-contiguous weight copies (fpd_drafter_prepare):
a prepared drafter reads its projections from the copies, which changes
only the addresses the GEMMs load from, so its outputs must equal those of
the same drafter unprepared bit for bit, and the oracle within the bf16
bar.  The cases cover every GEMM plan the drafter takes: few rows (split K
over 32-row tiles), up to 64 rows, a last 128-row tile that carries
leftover rows, partly filled tiles, 128x128 tiles of 8 waves for a few
hundred rows, a ragged last column tile (an MLP width that is not a multiple
of the tile) and a context long enough for the large-tile fusion path."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_draft_decoding_amd import synth
from tests.gpu_cases import GpuCase, progress
from tests.test_gpu_parity import SMALL, compare_all, run_both, small_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,L,C,inter", [
    (1, 16, 64, 1408),     # 16 rows: split-K 32-row tiles
    (2, 25, 77, 1472),     # 50 rows; ragged MLP columns
    (1, 129, 200, 1408),   # 129 rows: the 128x256 tile split along K, a one-row last tile; context 200 rows
    (2, 100, 600, 1472),   # 200 rows (partly filled last tile); context 1200 rows
    (2, 150, 64, 1408),    # 300 rows: 128x128 8-wave tiles, K split (gate/up via the split-K sum)
])
def test_tiled_copies_match_row_major_bitwise(B, L, C, inter):
    shape = replace(SMALL, inter=inter)
    wl = small_workload("text", B, C, seed=90 + L, shape=shape, block_len=L)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", f"tiled weights B={B} L={L} C={C} I={inter}", inp.weights.w_lm)
    row = GpuCase(wl, inp, prepare=False)
    row.fuse()
    row.draft()
    lg_row = row.argmax(logits=True)
    torch.cuda.synchronize()
    progress(f"[tiled-vs-row-major B={B} L={L} C={C}] comparing")
    assert torch.equal(g.hidden, row.hidden)
    assert torch.equal(lg, lg_row) and torch.equal(g.toks, row.toks)
    if C > 0:  # the C written positions (the capacity is padded to a multiple of 8)
        for x, y in zip(g.ctx_np(), row.ctx_np()):
            assert np.array_equal(x, y)


def test_prepare_is_idempotent_and_f32_is_a_no_op():
    from block_draft_decoding_amd import fpd
    wl = small_workload("text", 1, 64, seed=95, block_len=80)
    inp = synth.make_inputs(wl)
    g = GpuCase(wl, inp)
    fpd.fpd_drafter_prepare(g.d)  # second call: no new copy, same results
    g.fuse()
    g.draft()
    h1 = g.hidden.clone()
    g.draft()
    torch.cuda.synchronize()
    assert torch.equal(h1, g.hidden)
    shape32 = replace(synth.DRAFTER_TINY, n_layers=1)
    w32 = fpd.weights_to_device(synth.make_weights(shape32, seed=3), torch.float32)
    d32 = fpd.fpd_drafter_create(fpd.make_config(shape32), w32)
    fpd.fpd_drafter_prepare(d32)
    d32.close()
