#!/usr/bin/env python3
"""Throughput of the block-drafter hot path on one MI355X.

A step is one drafted block: fpd_draft_block (embedding, 5 non-causal
GQA + SwiGLU layers, final norm) + fpd_constrained_argmax (legal-row LM
head, masked argmax, off-frame pairing) + acceptance (schema validator;
prefix verification for text blocks; for box lists the validator plus the
first uncertain coordinate of a per-position confidence vector that stands
in for the external spatial-confidence model), with the fused context K/V resident
in HBM.  Context fusion (fpd_fuse_context_kv) runs once per context and is
timed and reported separately.  The default workload is the 64-waypoint
2D+3D trajectory primitive (L = 385, context 4,096, bf16, batch 1).

With --graph the step is also captured into a HIP graph (the library only
enqueues kernels on the caller's stream, so its launches capture as they
are), its outputs are checked bitwise against an eager step, and the
timed steps replay it; the eager time per step is reported beside it.
Replay measured about 1% slower than eager launches at L = 385 and 25, so
eager launches are the default.

Prints one JSON line.  The dominant kernel's roofline uses HIP events
recorded by the library around its launches (same stream) over a second
pass of the timed steps; the CPU baseline is the float64 oracle on the
host's cores over a bounded sample of the same workload.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
BOX_TAU = 0.004             # confidence threshold of the box workloads' acceptance


TRIMMED = ("gemm_o", "gemm_gate_up", "gemm_down")


def launch_rows(tag, s, B, L, layer):
    """Rows one layer's launch of a kernel tag works on.  With one request the
    last layer's O projection and MLP run on the L-1 rows whose hidden states
    feed the LM head (the anchor row's output is never read)."""
    if B == 1 and layer == s.n_layers - 1 and tag in TRIMMED:
        return L - 1
    return B * L


def kernel_work(tag, s, B, L, C, lay_info, M=None):
    """Algorithmic (flops, bytes) of one launch of a kernel tag on M rows
    (default: the per-launch average over the block's layers): what the
    method must compute and move (weights once, activations in and out),
    without padding or re-reads."""
    H, nq, nkv, d, I = s.hidden, s.n_q, s.n_kv, s.head_dim, s.inter
    if M is None:
        M = sum(launch_rows(tag, s, B, L, i) for i in range(s.n_layers)) / s.n_layers
    e = 2  # bf16
    nqkv = (nq + 2 * nkv) * d
    if tag == "gemm_qkv":
        return 2.0 * M * H * nqkv, e * (nqkv * H + M * H + M * nqkv)
    if tag == "gemm_o":
        return 2.0 * M * nq * d * H, e * (H * nq * d + M * nq * d) + 8.0 * M * H
    if tag == "gemm_gate_up":
        return 2.0 * M * H * 2 * I, e * (2 * I * H + M * H + M * I)
    if tag == "gemm_down":
        return 2.0 * M * I * H, e * (H * I + M * I) + 8.0 * M * H
    if tag == "attention":
        T = C + L
        return 4.0 * B * nq * L * T * d, e * (2 * B * nkv * T * d + 2 * B * nq * L * d)
    if tag == "lm_head":
        rows_cols, n_ids = lay_info
        return 2.0 * B * rows_cols * H, e * (n_ids * H + B * (L - 1) * H)
    return None


def block_work(s, B, L, C, lay_info):
    """Algorithmic (flops, bytes) of one drafted block: every layer's four
    projections and attention over the rows launch_rows gives, plus the
    constrained LM head; bytes are the weights read once, the context K/V and the legal
    LM-head rows (activations are small next to them)."""
    flops = 0.0
    for tag in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention"):
        for i in range(s.n_layers):
            flops += kernel_work(tag, s, B, L, C, lay_info, M=launch_rows(tag, s, B, L, i))[0]
    flops += kernel_work("lm_head", s, B, L, C, lay_info)[0]
    H, d, I = s.hidden, s.head_dim, s.inter
    nqkv = (s.n_q + 2 * s.n_kv) * d
    weights = s.n_layers * (nqkv * H + H * s.n_q * d + 2 * I * H + H * I) * 2
    ctx_kv = s.n_layers * 2 * B * s.n_kv * C * d * 2
    lm_rows = lay_info[1] * H * 2
    return flops, weights + ctx_kv + lm_rows


def host_description():
    """CPU model and the BLAS numpy uses, for the CPU baseline."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')} ({b.get('openblas configuration', '').strip()})"
    except Exception:
        pass
    return model, blas


def cpu_baseline(wl, inp, budget_s):
    """The oracle's warm block (layers, full-vocabulary logits, masked argmax,
    pairing, acceptance) on the host cores; context fusion done beforehand."""
    import numpy as np
    from block_draft_decoding_amd import synth
    from oracle import fpd_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    m = O.Model(wl.shape, inp.weights)
    t = time.time()
    ck, cv = O.fuse_context_kv(m, inp.feats)
    fuse_s = time.time() - t
    lay = O.build_layout(wl.schema, wl.shape.vocab)
    times = []
    t_all = time.time()
    while len(times) < 3 and (not times or time.time() - t_all + times[-1] < budget_s):
        t = time.time()
        hid = (O.draft_blocks_shared if wl.shared_ctx else O.draft_block)(m, inp.tokens, ck, cv)
        z = O.full_logits(m, hid)
        toks = O.constrained_tokens(z, lay)
        if wl.schema["kind"] == "text":
            O.verify_prefix(toks, np.zeros((toks.shape[0], toks.shape[1] + 1), np.int32))
        elif wl.schema["kind"] == "boxes2d":
            O.accept_boxes(toks, synth.make_box_conf(wl.batch, lay.L - 1, 4000 + wl.seed_index), BOX_TAU, lay)
        else:
            O.validate_primitive(toks, lay)
        times.append(time.time() - t)
    blk = statistics.median(times)
    tokens = wl.batch * (lay.L - 1)
    model, blas = host_description()
    return {"value": tokens / blk, "unit": "drafted tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{len(times)} warm block(s) of the same workload (batch {wl.batch}, L={lay.L}, "
                      f"C={wl.ctx}), median {blk:.2f} s per block; context fusion {fuse_s:.2f} s not counted"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="traj2d3d")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time replays of the step captured into a HIP graph")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work (bounded sample)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 256 MiB device buffer 5 times (reference for the FETCH_SIZE / WRITE_SIZE "
                         "counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from block_draft_decoding_amd import fpd, profiling, synth

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return

    wl = synth.WORKLOADS[args.workload]
    s = wl.shape
    t0 = time.time()
    inp = synth.make_inputs(wl)
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    w = fpd.weights_to_device(inp.weights, dt)
    d = fpd.fpd_drafter_create(fpd.make_config(s), w)
    fpd.fpd_drafter_prepare(d)
    lay = fpd.fpd_layout_create(d, wl.schema)
    L, B, C = lay.L, wl.batch, wl.ctx
    cap = (C + 7) // 8 * 8
    ws = fpd.alloc_workspace(d, B, cap, L)
    shared = wl.shared_ctx          # several blocks against one observation
    ck, cv = fpd.alloc_context(d, 1 if shared else B, cap)
    draft = fpd.fpd_draft_blocks_shared_ctx if shared else fpd.fpd_draft_block
    feats = fpd.to_device(inp.feats, dt)
    tokens = torch.from_numpy(inp.tokens).cuda()
    hidden = torch.empty(B, L - 1, s.hidden, dtype=dt, device="cuda")
    toks = torch.empty(B, L - 1, dtype=torch.int32, device="cuda")
    k_out = torch.empty(B, dtype=torch.int32, device="cuda")
    aux = torch.empty(B, dtype=torch.int32, device="cuda")
    text = wl.schema["kind"] == "text"
    boxes = wl.schema["kind"] == "boxes2d"
    if boxes:
        conf = torch.from_numpy(synth.make_box_conf(B, L - 1, 4000 + wl.seed_index)).cuda()
        unc = torch.empty(B, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    setup_s = time.time() - t0

    with torch.cuda.stream(stream):
        fpd.fpd_fuse_context_kv(d, feats, ck, cv, ws, stream=stream)
        draft(d, tokens, ck, cv, C, hidden, ws, stream=stream)
        fpd.fpd_constrained_argmax(d, lay, hidden, toks, ws, stream=stream)
    stream.synchronize()
    target = None
    if text:
        target = torch.from_numpy(synth.plant_targets(toks.cpu().numpy(), 7, s.vocab, 3000 + wl.seed_index)).cuda()

    def step():
        draft(d, tokens, ck, cv, C, hidden, ws, stream=stream)
        fpd.fpd_constrained_argmax(d, lay, hidden, toks, ws, stream=stream)
        if text:
            fpd.fpd_verify_prefix(toks, target, k_out, aux, stream=stream)
        elif boxes:
            fpd.fpd_accept_boxes(lay, toks, conf, BOX_TAU, k_out, aux, unc, stream=stream)
        else:
            fpd.fpd_validate_primitive(lay, toks, k_out, aux, stream=stream)

    def timed(run_step):
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                run_step()
            stream.synchronize()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            ev[0].record(stream)
            for i in range(args.steps):
                run_step()
                ev[i + 1].record(stream)
            stream.synchronize()
            torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)], ev[0].elapsed_time(ev[-1]) / args.steps

    per_eager, eager_ms = timed(step)
    launch = "eager"
    per, ms = per_eager, eager_ms
    if args.graph:
        ref = [x.clone() for x in (hidden, toks, k_out, aux)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for x in (hidden, toks, k_out, aux):
            x.zero_()
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        for a, b in zip((hidden, toks, k_out, aux), ref):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay differs from the eager step")
        per, ms = timed(graph.replay)
        launch = "hip_graph"
    drafted = B * (L - 1)

    # context fusion, once per context (reported, not in the step)
    with torch.cuda.stream(stream):
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        f0.record(stream)
        for _ in range(reps):
            fpd.fpd_fuse_context_kv(d, feats, ck, cv, ws, stream=stream)
        f1.record(stream)
        stream.synchronize()
    fuse_ms = f0.elapsed_time(f1) / reps

    # incremental context: the last 8 positions re-appended at their offset,
    # as a decode loop does after each committed block
    n_app = min(8, C)
    feats_tail = feats[:, :, C - n_app:].contiguous()
    with torch.cuda.stream(stream):
        fpd.fpd_append_context_kv(d, feats_tail, ck, cv, ws, pos0=C - n_app, stream=stream)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(reps):
            fpd.fpd_append_context_kv(d, feats_tail, ck, cv, ws, pos0=C - n_app, stream=stream)
        a1.record(stream)
        stream.synchronize()
    append_ms = a0.elapsed_time(a1) / reps

    # coordinate codec on the drafted block: tokens -> bin values, as a caller
    # reads the trajectory out of each block
    vals = torch.empty(toks.numel(), dtype=torch.float64, device="cuda")
    cb = wl.schema.get("coord_base", 0)
    with torch.cuda.stream(stream):
        fpd.fpd_tokens_to_coords(toks, vals, cb, stream=stream)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(reps):
            fpd.fpd_tokens_to_coords(toks, vals, cb, stream=stream)
        c1.record(stream)
        stream.synchronize()
    decode_ms = c0.elapsed_time(c1) / reps

    # per-kernel durations: library-recorded HIP events over a second pass of the steps
    nprof = min(args.steps, 20)
    with torch.cuda.stream(stream):
        fpd.fpd_profile_enable(True)
        for _ in range(nprof):
            step()
        stream.synchronize()
        recs = fpd.fpd_profile_records()
        fpd.fpd_profile_enable(False)
    kern = {}
    for tag, kms in recs:
        c = kern.setdefault(tag, [0, 0.0])
        c[0] += 1
        c[1] += kms
    dom = max(kern, key=lambda t: kern[t][1])
    m = fpd.fpd_layout_masks(lay)
    rows_cols = 0
    for p in range(1, L):
        sidx = m["pos_set"][p]
        rows_cols += s.vocab if sidx < 0 else int(m["set_offsets"][sidx + 1] - m["set_offsets"][sidx])
    n_ids = int(m["set_ids"].size) + (s.vocab if (m["pos_set"][1:] == -1).any() else 0)
    work = kernel_work(dom, s, B, L, C, (rows_cols, n_ids))
    avg_ms = kern[dom][1] / kern[dom][0]
    roof = None
    if work:
        flops, nbytes = work
        if flops / nbytes >= RIDGE:
            ach = flops / (avg_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
        else:
            ach = nbytes / (avg_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
        roof["traffic"] = profiling.read_traffic(dom, args.workload)
        roof.update({"kernel": dom, "avg_launch_ms": round(avg_ms, 4), "launches_per_step": kern[dom][0] // nprof,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes})
    kernels = {t: {"launches_per_step": round(c[0] / nprof, 2), "ms_per_step": round(c[1] / nprof, 4)}
               for t, c in sorted(kern.items(), key=lambda kv: -kv[1][1])}
    # the whole block against the chip: algorithmic work / measured step time
    bflops, bbytes = block_work(s, B, L, C, (rows_cols, n_ids))
    t_s = ms * 1e-3
    block_roof = {"bound": "mfma" if bflops / bbytes >= RIDGE else "hbm",
                  "algorithmic_flops": bflops, "algorithmic_bytes": bbytes,
                  "achieved_tflops": round(bflops / t_s / 1e12, 2),
                  "mfma_frac": round(bflops / t_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "achieved_gbs": round(bbytes / t_s / 1e9, 1),
                  "hbm_frac": round(bbytes / t_s / 1e9 / PEAK_HBM_GBS, 4),
                  "roofline_ms": round(max(bflops / (PEAK_BF16_TFLOPS * 1e12), bbytes / (PEAK_HBM_GBS * 1e9)) * 1e3, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, args.cpu_budget)

    per_sorted = sorted(per)
    out = {
        "metric": "drafted block tokens/sec, L=385 ctx=4096 bf16 batch 1; % HBM/MFMA roofline"
        if args.workload == "traj2d3d" else f"drafted block tokens/sec ({args.workload})",
        "value": round(drafted / (ms * 1e-3), 1),
        "unit": "drafted tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.notes}", "block_len": L, "ctx": C, "batch": B,
                   "drafted_tokens_per_step": drafted},
        "latency_ms": {"p50": round(per_sorted[len(per) // 2], 4), "p90": round(per_sorted[int(len(per) * 0.9)], 4)},
        "fuse_context_ms": round(fuse_ms, 4),
        f"append_context_{n_app}_ms": round(append_ms, 4),
        "decode_coords_ms": round(decode_ms, 4),
        "launch": launch,
        "eager_ms_per_step": round(eager_ms, 4),
        "cold_ms_per_step": round(fuse_ms + ms, 4),
        "accepted_k": k_out[:8].tolist(),
        "roofline": roof,
        "block_roofline": block_roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
