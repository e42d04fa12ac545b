"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact for token ids, masks and accepted lengths.
Floating point: every hidden row, context row and position's legal logits
within 2e-2 (bf16) / 1e-4 (fp32) relative per vector, with an elementwise
guard; the LM head, masked argmax and pairing on the GPU's own hidden states
must give the oracle's ids wherever the top-2 legal gap exceeds 1e-2; end to
end (through five bf16 layers) ids must agree wherever the gap exceeds 5e-2
of the position's legal-logit rms, and closer disagreements are counted.
tests/gpu_cases.py states the rules and their derivation."""
import itertools
import time
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_draft_decoding_amd import synth
from oracle import fpd_oracle as O
from tests.gpu_cases import (GpuCase, check_head_stage, check_tokens_e2e, legal_logits, logit_scale,
                             oracle_result, progress, rel_close, rel_close_logits, small_ids, to_np,
                             tokens_from_legal, workload_inputs)

pytestmark = pytest.mark.gpu

SMALL = synth.DrafterShape(hidden=512, n_q=8, n_kv=2, head_dim=128, n_layers=2, inter=1408, vocab=4099,
                           n_fused=3, dtype="bf16", weight_std=0.02)


def small_workload(kind, B, C, seed, shape=SMALL, shared_ctx=False, **schema_over):
    ids = small_ids(shape.vocab)
    schema = dict(kind=kind, **ids)
    schema.update(schema_over)
    return synth.Workload(f"small-{kind}", shape, batch=B, ctx=C, schema=schema, seed_index=seed,
                          off_row_std=0.06 if schema.get("off_id", -1) >= 0 else None, shared_ctx=shared_ctx)


def run_both(wl, n_layers=None, logits=True):
    """GPU run and oracle run of one workload: (inputs, GpuCase, logits, oracle result)."""
    inp = synth.make_inputs(wl)
    g = GpuCase(wl, inp, n_layers=n_layers)
    g.fuse()
    g.draft()
    lg = g.argmax(logits=logits)
    torch.cuda.synchronize()
    shape = wl.shape if n_layers is None else replace(wl.shape, n_layers=n_layers)
    w = inp.weights if n_layers is None else replace(inp.weights, layers=inp.weights.layers[:n_layers])
    res = O.run_block(O.Model(shape, w), inp.feats, inp.tokens, wl.schema, want_logits=True,
                      shared_ctx=wl.shared_ctx)
    return inp, g, lg, res


def compare_all(wl, g, lg, res, dtype, name="", w_lm=None):
    """Every parity rule on one run: context K/V, hidden states, legal
    logits and tokens end to end, then the head stage on the GPU's own
    hidden states (w_lm given), and legality of every id."""
    stats = {}
    if wl.ctx > 0:
        ck, cv = g.ctx_np()
        stats["ctx_k"] = rel_close(ck, res["ctx_k"], dtype, "ctx_k")
        stats["ctx_v"] = rel_close(cv, res["ctx_v"], dtype, "ctx_v")
    stats["hidden"] = rel_close(to_np(g.hidden), res["hidden"], dtype, "hidden")
    lay = res["layout"]
    if lg is not None:
        sc = logit_scale(res["hidden"], w_lm, lay) if w_lm is not None else None
        stats["logits"] = rel_close_logits(to_np(lg), O.gathered_logits(res["logits"], lay), lay, dtype, "logits",
                                           scale=sc)
    got = g.toks.cpu().numpy()
    stats["tokens"] = check_tokens_e2e(got, res["tokens"], res["logits"], lay, dtype, "tokens")
    if w_lm is not None:
        herr, hcnt = check_head_stage(g, lg, lay, w_lm, dtype, name)
        if herr is not None:
            stats["head logits"] = herr
        stats["head tokens"] = hcnt
    for b in range(got.shape[0]):
        for p in range(1, lay.L):
            assert got[b, p - 1] in lay.legal(p)
    progress(f"[parity {name}] " + ", ".join(
        f"{k}: row {v[0]:.2e} elem {v[1]:.2e}" for k, v in stats.items() if "tokens" not in k) +
        f"; tokens agree/differ(gap>1e-2)/differ(gap<=1e-2) end to end {stats['tokens']}" +
        (f", head stage {stats['head tokens']}" if "head tokens" in stats else ""))
    return stats


# The constrained LM head takes 32-column chunks for all but the text cases;
# their work items split K four ways (traj2d: 33 items; traj2d3d, B = 2: 97
# and B = 4: 161 items); the full-size 2D+3D block (322 items) splits two
# ways.  test_head_without_k_groups covers a hidden size whose K tiles
# cannot be split.
@pytest.mark.parametrize("kind,B,C,over", [
    ("text", 2, 300, dict(block_len=37)),
    ("traj2d3d", 2, 300, dict(n_points=7, off_id=4099 - 1020 + 1002)),
    ("traj2d3d", 4, 64, dict(n_points=7, off_id=4099 - 1020 + 1002)),
    ("points3d_text", 3, 77, dict(n_points=2)),
    ("traj2d", 1, 0, dict(n_points=1)),
    ("text", 1, 64, dict(block_len=2)),
])
def test_small_bf16_end_to_end(kind, B, C, over):
    wl = small_workload(kind, B, C, seed=40 + B, **over)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", f"small {kind} B={B} C={C}", inp.weights.w_lm)
    lay = res["layout"]
    if kind != "text":
        k, f = g.validate(torch.from_numpy(res["tokens"]).cuda())
        ko, fo = O.validate_primitive(res["tokens"], lay)
        assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(f.cpu().numpy(), fo)
    if kind == "traj2d3d":
        n_off = int((res["tokens"] == lay.off_id).sum())
        progress(f"[pairs] off-frame tokens {n_off} of {res['tokens'].size}")


# Context fusion over B x C = 4,096 rows takes 32 row tiles of 128 (split K
# two ways), so the GEMM launch walks its tiles in groups of four row tiles
# across the column tiles; 2,100 rows end in a partly filled 17th row tile,
# which keeps the row-tiles-first order with that tile last.  ctx_k / ctx_v
# are compared row by row.
@pytest.mark.parametrize("B,C", [(2, 2048), (1, 2100)])
def test_grouped_tile_order_context_fusion(B, C):
    wl = small_workload("traj2d3d", B, C, seed=47 + B, n_points=7, off_id=4099 - 1020 + 1002)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", f"grouped tile order B={B} C={C}", inp.weights.w_lm)


# 4L packed rows per KV head (n_q = 8, n_kv = 2): L = 65 and 72 end in a
# tail tile of 4 and 32 rows, which runs in its own two-split workgroups
# while the full tile takes 3 (C = 300) or 7 (C = 1000) key splits; L = 73
# leaves 36 rows, more than one wave holds, and keeps the plain plan.  The
# shared case has three blocks read one context through the tail workgroups.
@pytest.mark.parametrize("B,C,L,shared", [(2, 300, 65, False), (1, 1000, 72, False), (2, 300, 73, False),
                                          (3, 300, 65, True)])
def test_tail_query_tile(B, C, L, shared):
    wl = small_workload("text", B, C, seed=80 + L, block_len=L, shared_ctx=shared)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", f"tail tile B={B} C={C} L={L} shared={shared}", inp.weights.w_lm)


def test_head_without_k_groups():
    """Hidden 320 = 5 K tiles: the narrow-chunk LM head cannot split K into
    wave groups and runs one wave per item."""
    shape = replace(SMALL, hidden=320)
    wl = small_workload("traj2d3d", 2, 64, seed=74, shape=shape, n_points=7, off_id=4099 - 1020 + 1002)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", "hidden 320", inp.weights.w_lm)


def test_more_than_eight_split_partials():
    """A narrow drafter with a wide MLP (hidden 512, MLP 4096): at 16 block
    rows the down projection splits K 32 ways (one pass of workgroups over
    the CUs), so its split-K sums take the four-group residual + RMSNorm
    kernel."""
    shape = replace(SMALL, inter=4096)
    wl = small_workload("text", 1, 64, seed=73, shape=shape, block_len=16)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", "16-way split-K sums", inp.weights.w_lm)


def test_folded_rows_fill_both_halves_of_the_extra_slab():
    """A wide MLP (I = 9,728: 76 paired column tiles) over 396 block rows =
    3 x 128 + 12: the gate/up projection carries the 12 leftover rows in its
    last row tile.  The 16-row slab of extra rows is filled by two different
    loading waves, 8 rows each, so 12 rows use both halves with the second
    one partly clamped (1 and 16 leftover rows are the 385-row and the
    16 x 25-row full-size blocks)."""
    shape = replace(SMALL, inter=9728)
    wl = small_workload("text", 1, 64, seed=91, shape=shape, block_len=396)
    inp, g, lg, res = run_both(wl)
    compare_all(wl, g, lg, res, "bf16", "12 folded rows", inp.weights.w_lm)


@pytest.mark.parametrize("n_layers", [1, 2, 3])
def test_per_layer_hidden_parity(n_layers):
    shape = replace(SMALL, n_layers=3)
    wl = small_workload("text", 1, 200, seed=50, shape=shape, block_len=21)
    inp, g, lg, res = run_both(wl, n_layers=n_layers, logits=False)
    r = rel_close(to_np(g.hidden), res["hidden"], "bf16", f"hidden after {n_layers} layers")
    progress(f"[layers {n_layers}] hidden row {r[0]:.2e} elem {r[1]:.2e}")


def test_tiny_fp32_workload():
    wl, inp = workload_inputs("tiny")
    g = GpuCase(wl, inp)
    g.fuse()
    g.draft()
    lg = g.argmax(logits=True)
    torch.cuda.synchronize()
    res = O.run_block(O.Model(wl.shape, inp.weights), inp.feats, inp.tokens, wl.schema, want_logits=True)
    compare_all(wl, g, lg, res, "f32", "tiny fp32", inp.weights.w_lm)
    k, f = g.validate()
    ko, fo = O.validate_primitive(g.toks.cpu().numpy(), res["layout"])
    assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(f.cpu().numpy(), fo)
    # text verification with every planted prefix length 0..15
    draft = np.repeat(res["tokens"], 16, axis=0)
    tgt = synth.plant_targets(draft, np.arange(16), wl.shape.vocab, 3001)
    kk = torch.empty(16, dtype=torch.int32, device="cuda")
    nx = torch.empty_like(kk)
    g.fpd.fpd_verify_prefix(torch.from_numpy(draft).cuda(), torch.from_numpy(tgt).cuda(), kk, nx)
    ko, no = O.verify_prefix(draft, tgt)
    assert np.array_equal(kk.cpu().numpy(), np.arange(16)) and np.array_equal(kk.cpu().numpy(), ko)
    assert np.array_equal(nx.cpu().numpy(), no)


def test_rope_shift_invariance_on_gpu():
    wl, inp = workload_inputs("tiny")
    g = GpuCase(wl, inp)
    g.fuse(pos0=0)
    g.draft()
    a = to_np(g.hidden)
    g.fuse(pos0=1000)
    g.draft(block_pos=wl.ctx + 1000)
    b = to_np(g.hidden)
    # fp32 angles at positions ~1000 carry ~1e-4 relative rounding, so the
    # invariance holds to that level rather than to the 1e-4 parity bound
    rows = np.linalg.norm(b - a, axis=-1) / np.linalg.norm(a, axis=-1)
    assert rows.max() < 1e-3, rows.max()


def test_zero_lm_head_ties_pick_lowest_ids():
    wl = small_workload("traj2d3d", 2, 50, seed=61, n_points=3, off_id=4099 - 1020 + 1002)
    inp = synth.make_inputs(wl)
    inp.weights.w_lm[...] = 0.0
    g = GpuCase(wl, inp)
    g.fuse()
    g.draft()
    g.argmax()
    torch.cuda.synchronize()
    lay = O.build_layout(wl.schema, wl.shape.vocab)
    want = np.array([[lay.legal(p)[0] for p in range(1, lay.L)]] * 2, np.int32)
    assert np.array_equal(g.toks.cpu().numpy(), want)


def test_validator_planted_errors_bit_exact():
    wl = small_workload("points3d_text", 1, 16, seed=62, n_points=6)
    inp = synth.make_inputs(wl)
    g = GpuCase(wl, inp)
    lay = O.build_layout(wl.schema, wl.shape.vocab)
    sch = wl.schema
    rng = np.random.default_rng(9)
    B = 512
    toks = np.empty((B, lay.L - 1), np.int32)
    for p in range(1, lay.L):
        ids = lay.legal(p)
        toks[:, p - 1] = ids[rng.integers(0, len(ids), size=B)]
    for (p0, w) in lay.fields:      # well-formed fields: FILL^j DIGIT^(w-j)
        j = rng.integers(0, w, size=B)
        for i in range(w):
            dig = sch["digit0_id"] + rng.integers(0, 10, size=B)
            toks[:, p0 - 1 + i] = np.where(i < j, sch["fill_id"], dig)
    # plant errors in half the rows: fill after a digit, foreign ids, out-of-vocabulary ids
    for b in range(0, B, 2):
        for _ in range(rng.integers(1, 3)):
            toks[b, rng.integers(0, lay.L - 1)] = rng.choice([sch["fill_id"], 5, -3, 10 ** 6])
    k, f = g.validate(torch.from_numpy(toks).cuda())
    ko, fo = O.validate_primitive(toks, lay)
    assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(f.cpu().numpy(), fo)
    assert B // 2 <= int((ko > 0).sum()) < B


def test_verify_brute_force_v3_l5():
    from block_draft_decoding_amd import fpd
    V, L = 3, 5
    drafts = np.array(list(itertools.product(range(V), repeat=L - 1)), np.int32)
    targets = np.array(list(itertools.product(range(V), repeat=L)), np.int32)
    D = np.ascontiguousarray(np.repeat(drafts, len(targets), axis=0))
    T = np.ascontiguousarray(np.tile(targets, (len(drafts), 1)))
    k = torch.empty(D.shape[0], dtype=torch.int32, device="cuda")
    nx = torch.empty_like(k)
    fpd.fpd_verify_prefix(torch.from_numpy(D).cuda(), torch.from_numpy(T).cuda(), k, nx)
    ko, no = O.verify_prefix(D, T)
    assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(nx.cpu().numpy(), no)


def test_layout_masks_on_device_match_oracle():
    wl, inp = workload_inputs("tiny")
    g = GpuCase(wl, inp)
    from block_draft_decoding_amd import fpd
    for name in ("text", "traj2d", "traj2d3d", "points3d"):
        w = synth.WORKLOADS[name]
        small = replace(w, shape=replace(SMALL, vocab=151_936), schema=w.schema)
        # masks only depend on the schema and the vocabulary
        m = fpd.fpd_schema_expand(small.schema, 151_936)
        lay = O.build_layout(small.schema, 151_936)
        offs, ids = lay.csr()
        assert np.array_equal(m["pos_set"], lay.pos_set) and np.array_equal(m["set_ids"], ids)
    m = fpd.fpd_layout_masks(g.lay)
    lay = O.build_layout(wl.schema, wl.shape.vocab)
    assert np.array_equal(m["pos_set"], lay.pos_set)
    assert np.array_equal(m["set_offsets"], lay.csr()[0]) and np.array_equal(m["set_ids"], lay.csr()[1])


def test_determinism_bitwise():
    wl = small_workload("traj2d3d", 1, 300, seed=63, n_points=5, off_id=4099 - 1020 + 1002)
    inp = synth.make_inputs(wl)
    g = GpuCase(wl, inp)
    outs = []
    for _ in range(2):
        g.fuse()
        g.draft()
        lg = g.argmax(logits=True)
        torch.cuda.synchronize()
        outs.append((g.hidden.clone(), g.toks.clone(), lg.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2], outs[1][2])


# ---- full-size workloads ------------------------------------------------------------

@pytest.mark.parametrize("name", ["text", "traj2d", "traj2d3d", "flashdrive8", "flashdrive16",
                                  "traj2d_shared16"])
def test_full_size_workload(name):
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
    if wl.schema["kind"] == "text":
        n = lay.L                  # every accepted length 0 .. L-1
        draft = np.repeat(res["tokens"], n, axis=0)
        tgt = synth.plant_targets(draft, np.arange(n), wl.shape.vocab, 3000 + wl.seed_index)
        kk = torch.empty(n, dtype=torch.int32, device="cuda")
        nx = torch.empty_like(kk)
        g.fpd.fpd_verify_prefix(torch.from_numpy(draft).cuda(), torch.from_numpy(tgt).cuda(), kk, nx)
        assert np.array_equal(kk.cpu().numpy(), np.arange(n))
        assert np.array_equal(nx.cpu().numpy(), tgt[np.arange(n), np.arange(n)])
    else:
        k, f = g.validate()
        ko, fo = O.validate_primitive(g.toks.cpu().numpy(), lay)
        assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(f.cpu().numpy(), fo)
        if name == "traj2d3d":
            # the pairing rule fires: some pairs go off-frame, and some need the
            # joint decision (exactly one of the pair prefers OFF on its own)
            t = g.toks.cpu().numpy()
            n_off = int((t == lay.off_id).sum())
            joint = 0
            for (pu, pv) in lay.pairs:
                own = [lay.legal(p)[int(np.argmax(res["logits"][0, p - 1, lay.legal(p)]))] == lay.off_id
                       for p in (pu, pv)]
                joint += own[0] != own[1]
            progress(f"[pairs] off-frame tokens {n_off} of {t.size}; pairs decided jointly {joint}")
            assert n_off >= 2 and joint >= 1


def test_full_size_two_trajectory_blocks():
    """Two 8-waypoint blocks in one call (M = 50 rows, each with its own
    context): the 64-row GEMM tiles with their split-K sums at the drafter's
    real widths."""
    wl = synth.scaled_workload("traj2d", batch=2)
    inp = synth.make_inputs(wl)
    g = GpuCase(wl, inp)
    g.fuse()
    g.draft()
    lg = g.argmax(logits=True)
    torch.cuda.synchronize()
    progress("[gpu] traj2d x2 done")
    res = O.run_block(O.Model(wl.shape, inp.weights), inp.feats, inp.tokens, wl.schema, want_logits=True)
    compare_all(wl, g, lg, res, "bf16", "full traj2d x2", inp.weights.w_lm)
    k, f = g.validate()
    ko, fo = O.validate_primitive(g.toks.cpu().numpy(), res["layout"])
    assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(f.cpu().numpy(), fo)


def test_full_size_points3d_requests_against_the_oracle():
    """B = 8 independent requests, L = 2433, C = 4096 (M = 19,464 projection
    rows: 128x256 tiles whose last row tile carries the 8 rows past 152 x 128,
    for the QKV, O, gate/up and down projections).  The oracle runs requests 0
    and 7 on their own (request 7 holds the carried rows): their context K/V,
    hidden states, legal logits, tokens and acceptance are compared in full.
    The LM head, argmax and validator are compared on all eight requests from
    the GPU's own hidden states."""
    wl, inp = workload_inputs("points3d")
    g = GpuCase(wl, inp)
    g.fuse()
    g.draft()
    lg = g.argmax(logits=True)
    torch.cuda.synchronize()
    progress("[gpu] points3d done")
    lay = O.build_layout(wl.schema, wl.shape.vocab)
    m = O.Model(wl.shape, inp.weights)
    w_lm = inp.weights.w_lm
    # every request: head stage on the GPU's hidden states, legality, validator
    herr, hcnt = check_head_stage(g, lg, lay, w_lm, "bf16", "points3d")
    toks = g.toks.cpu().numpy()
    for p in range(1, lay.L):
        assert np.isin(toks[:, p - 1], lay.legal(p)).all()
    k, f = g.validate()
    ko, fo = O.validate_primitive(toks, lay)
    assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(f.cpu().numpy(), fo)
    progress(f"[points3d head stage] logits row {herr[0]:.2e} elem {herr[1]:.2e}; tokens {hcnt}")
    ck_all, cv_all = g.ctx_np()
    hid_all = to_np(g.hidden)
    lg_all = to_np(lg)
    for b in (0, 7):
        t = time.time()
        ck, cv = O.fuse_context_kv(m, inp.feats[b:b + 1])
        hid = O.draft_block(m, inp.tokens[b:b + 1], ck, cv)
        zg = legal_logits(hid, w_lm, lay)
        otoks = tokens_from_legal(zg, lay)
        progress(f"[oracle] points3d request {b} in {time.time() - t:.1f}s")
        e_k = rel_close(ck_all[:, b:b + 1], ck, "bf16", f"request {b} ctx_k")
        e_v = rel_close(cv_all[:, b:b + 1], cv, "bf16", f"request {b} ctx_v")
        e_h = rel_close(hid_all[b:b + 1], hid, "bf16", f"request {b} hidden")
        e_z = rel_close_logits(lg_all[b:b + 1], zg, lay, "bf16", f"request {b} logits",
                               scale=logit_scale(hid, w_lm, lay))
        cnt = check_tokens_e2e(toks[b:b + 1], otoks, zg, lay, "bf16", f"request {b} tokens", gathered=True)
        kb, fb = O.validate_primitive(otoks, lay)
        if cnt[1] + cnt[2] == 0:   # identical tokens: identical acceptance
            assert int(ko[b]) == int(kb[0]) and int(fo[b]) == int(fb[0])
        progress(f"[parity points3d request {b}] ctx_k {e_k[0]:.2e}/{e_k[1]:.2e} ctx_v {e_v[0]:.2e}/{e_v[1]:.2e} "
                 f"hidden {e_h[0]:.2e}/{e_h[1]:.2e} logits {e_z[0]:.2e}/{e_z[1]:.2e} (row/elem); "
                 f"tokens agree/differ(gap>1e-2)/differ(gap<=1e-2) {cnt}; first_invalid gpu {int(fo[b])} "
                 f"oracle {int(fb[0])}")


def test_padding_memory_never_reaches_outputs():
    """Context capacity past the valid keys and every workspace byte hold NaN
    before the calls.  Padding keys are masked out of the scores and their
    value columns are zeroed before the P V product, and every workspace
    buffer is written before it is read, so the outputs still match the
    oracle."""
    from block_draft_decoding_amd import fpd
    wl = small_workload("traj2d3d", 2, 300, seed=64, n_points=7, off_id=4099 - 1020 + 1002)
    inp = synth.make_inputs(wl)
    g = GpuCase(wl, inp)
    cap = 456                      # 156 keys of NaN capacity past C = 300 (not a tile multiple)
    g.cap = cap
    g.ws = fpd.alloc_workspace(g.d, g.B, cap, g.L)
    g.ctx_k, g.ctx_v = fpd.alloc_context(g.d, g.B, cap)
    g.ctx_k.fill_(float("nan"))
    g.ctx_v.fill_(float("nan"))
    g.ws.fill_(255)                # all-ones bytes: NaN in every float and bf16 view
    g.fuse()
    g.draft()
    lg = g.argmax(logits=True)
    torch.cuda.synchronize()
    assert torch.isfinite(g.hidden.float()).all()
    res = O.run_block(O.Model(wl.shape, inp.weights), inp.feats, inp.tokens, wl.schema, want_logits=True)
    compare_all(wl, g, lg, res, "bf16", "NaN padding", inp.weights.w_lm)


def test_validator_large_sets_from_global_memory():
    """Legal-id sets too large to stage in LDS are searched in global memory;
    results must stay bit-exact with the oracle."""
    from block_draft_decoding_amd import fpd
    V = 70_000
    shape = replace(SMALL, vocab=V, n_layers=1)
    rng = np.random.default_rng(11)
    sets = [sorted(rng.choice(V - 8, 20_000, replace=False).tolist()) for _ in range(3)]
    L = 41
    pos_set = [-2] + [int(rng.integers(-1, 3)) for _ in range(L - 1)]
    schema = dict(kind="custom", block_len=L, sets=sets, pos_set=pos_set, pairs=[], fields=[], off_id=-1,
                  fill_id=-1, digit0_id=-1, coord_base=0, coord_count=0, start_id=V - 4, mask_id=V - 1,
                  delim_id=-1, plus_id=-1, minus_id=-1)
    w = fpd.weights_to_device(synth.make_weights(shape, seed=12), torch.bfloat16)
    d = fpd.fpd_drafter_create(fpd.make_config(shape), w)
    lay_d = fpd.fpd_layout_create(d, schema)
    lay = O.build_layout(schema, V)
    B = 256
    toks = np.empty((B, L - 1), np.int32)
    for p in range(1, L):
        ids = lay.legal(p)
        toks[:, p - 1] = ids[rng.integers(0, len(ids), size=B)]
    for b in range(0, B, 2):       # foreign and out-of-vocabulary ids in half the rows
        toks[b, rng.integers(0, L - 1)] = rng.choice([V - 5, -1, V + 3, int(rng.integers(0, V))])
    k = torch.empty(B, dtype=torch.int32, device="cuda")
    f = torch.empty_like(k)
    fpd.fpd_validate_primitive(lay_d, torch.from_numpy(toks).cuda(), k, f)
    ko, fo = O.validate_primitive(toks, lay)
    assert np.array_equal(k.cpu().numpy(), ko) and np.array_equal(f.cpu().numpy(), fo)
    assert 0 < int((ko == 0).sum()) < B


def test_append_context_in_pieces_matches_one_fusion():
    """Incremental context: the context appended in three pieces at their
    own positions (the decode loop after each committed block) gives the
    oracle's caches of one fusion of the whole context, and the same block
    output; keys before each piece are untouched by it."""
    from block_draft_decoding_amd import fpd
    wl = small_workload("traj2d3d", 2, 40, seed=66, n_points=3, off_id=4099 - 1020 + 1002)
    inp = synth.make_inputs(wl)
    g = GpuCase(wl, inp)
    cap = 48
    g.cap = cap
    g.ws = fpd.alloc_workspace(g.d, g.B, cap, g.L)
    g.ctx_k, g.ctx_v = fpd.alloc_context(g.d, g.B, cap)
    for a, b in ((0, 7), (7, 16), (16, 40)):
        before_k = g.ctx_k[:, :, :, :a].clone()
        fpd.fpd_append_context_kv(g.d, g.feats[:, :, a:b].contiguous(), g.ctx_k, g.ctx_v, g.ws, pos0=a)
        torch.cuda.synchronize()
        assert torch.equal(g.ctx_k[:, :, :, :a], before_k)
    g.draft()
    lg = g.argmax(logits=True)
    torch.cuda.synchronize()
    res = O.run_block(O.Model(wl.shape, inp.weights), inp.feats, inp.tokens, wl.schema, want_logits=True)
    compare_all(wl, g, lg, res, "bf16", "appended context", inp.weights.w_lm)


def test_blocks_share_one_context():
    """Several primitives against one observation: three blocks with their
    own anchors attend to one shared context (no copy per block)."""
    wl = small_workload("traj2d3d", 3, 77, seed=67, shared_ctx=True, n_points=5, off_id=4099 - 1020 + 1002)
    inp, g, lg, res = run_both(wl)
    assert g.ctx_k.shape[1] == 1
    compare_all(wl, g, lg, res, "bf16", "shared context", inp.weights.w_lm)
    toks = res["tokens"]
    assert not np.array_equal(toks[0], toks[1])   # distinct anchors give distinct blocks
