"""The drafted-block step (fpd_draft_block + fpd_constrained_argmax +
fpd_validate_primitive) captured into a HIP graph and replayed: the library
only enqueues kernels on the caller's stream, so a captured step must
reproduce the eager step bit for bit.  Each replay follows eager work on
other inputs that overwrites every output buffer, and the host synchronises
between them; every replay is checked."""
import pytest
import torch

from block_draft_decoding_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["traj2d", "traj2d3d"])
def test_graph_replays_match_eager(name):
    from block_draft_decoding_amd import fpd
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    s = wl.shape
    w = fpd.weights_to_device(inp.weights, torch.bfloat16)
    d = fpd.fpd_drafter_create(fpd.make_config(s), w)
    fpd.fpd_drafter_prepare(d)
    lay = fpd.fpd_layout_create(d, wl.schema)
    B, C, L = wl.batch, wl.ctx, lay.L
    cap = (C + 7) // 8 * 8
    ws = fpd.alloc_workspace(d, B, cap, L)
    ck, cv = fpd.alloc_context(d, B, cap)
    stream = torch.cuda.Stream()
    tokens = torch.from_numpy(inp.tokens).cuda()
    other = tokens.clone()
    other[:, 0] = (other[:, 0] + 1) % s.vocab   # another anchor: different outputs
    hidden = torch.empty(B, L - 1, s.hidden, dtype=torch.bfloat16, device="cuda")
    toks = torch.empty(B, L - 1, dtype=torch.int32, device="cuda")
    k = torch.empty(B, dtype=torch.int32, device="cuda")
    f = torch.empty(B, dtype=torch.int32, device="cuda")

    def step(tok):
        fpd.fpd_draft_block(d, tok, ck, cv, C, hidden, ws, stream=stream)
        fpd.fpd_constrained_argmax(d, lay, hidden, toks, ws, stream=stream)
        fpd.fpd_validate_primitive(lay, toks, k, f, stream=stream)

    with torch.cuda.stream(stream):
        fpd.fpd_fuse_context_kv(d, fpd.to_device(inp.feats, torch.bfloat16), ck, cv, ws, stream=stream)
        step(tokens)
    stream.synchronize()
    ref = [x.clone() for x in (hidden, toks, k, f)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(tokens)
    stream.synchronize()

    for rep in range(3):
        with torch.cuda.stream(stream):
            step(other)
        stream.synchronize()
        assert not torch.equal(hidden, ref[0]), "the eager step on other inputs must overwrite the outputs"
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        for got, want, what in zip((hidden, toks, k, f), ref, ("hidden", "tokens", "k", "first_invalid")):
            assert torch.equal(got, want), f"replay {rep}: {what} differs from the eager step"
