"""Writes tests/golden/noise_floor_<workload>.json: how far a second faithful
implementation of the bf16 drafter is from the float64 oracle.

The second implementation keeps every bf16 storage point of the oracle
(fused context rows, context K/V, normed GEMM inputs, Q/K/V after RoPE,
attention output, SwiGLU product, final hidden state) and differs only in
accumulating its matrix products in float32 instead of float64; attention
probabilities are not rounded.  Its distance from the oracle is the floor
that any float32-accumulating implementation of the same arithmetic sits
at: each storage rounding turns a tiny pre-rounding difference into
whole-ulp flips of some elements, and after a layer or two the two runs sit
about one bf16 ulp apart.  Uses only the oracle and the seeded inputs.

    python tests/golden/noise_floor.py traj2d3d
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from block_draft_decoding_amd import synth  # noqa: E402
from oracle import fpd_oracle as O  # noqa: E402


def f32_products(m: O.Model):
    """The float32-accumulating composition over the oracle's model m."""
    S = lambda x: O._store(x, m.dtype)
    W32 = [{k: np.asarray(v, np.float32) for k, v in lw.items()} for lw in m.w.layers]
    fc32 = np.asarray(m.w.w_fc, np.float32)
    emb = m.w.embed
    nq, nkv, d, H, I = m.nq, m.nkv, m.d, m.H, m.I

    def mm(a, b32):
        return (np.asarray(a, np.float32) @ b32).astype(np.float64)

    def fuse(feats):
        f = np.asarray(feats, np.float64)
        B, nt, C, _ = f.shape
        X = np.concatenate([f[:, t] for t in range(nt)], axis=-1)
        Zn = S(O.rmsnorm(mm(X, fc32.T), m.w.g_fc, m.eps))
        pos = np.arange(C)
        ks, vs = [], []
        for lw in W32:
            k = mm(Zn, lw["w_qkv"][nq * d:(nq + nkv) * d].T).reshape(B, C, nkv, d)
            v = mm(Zn, lw["w_qkv"][(nq + nkv) * d:].T).reshape(B, C, nkv, d)
            ks.append(S(m._rope(k, pos)))
            vs.append(S(v))
        return np.stack(ks), np.stack(vs)

    def attention(q, k, v):
        T = q.shape[0]
        out = np.empty((T, nq, d))
        for i in range(nq):
            j = (i * nkv) // nq
            s = mm(q[:, i], np.asarray(k[:, j].T, np.float32)) / np.sqrt(d)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[:, i] = mm(p, np.asarray(v[:, j], np.float32)) / p.sum(axis=1, keepdims=True)
        return out

    def draft(tokens, ck, cv):
        B, L = tokens.shape
        C = ck.shape[2]
        pos = C + np.arange(L)
        out = np.empty((B, L - 1, H))
        for b in range(B):
            h = np.asarray(emb[tokens[b]], np.float64)
            for li, lw in enumerate(W32):
                g = m.layer(li)
                a = S(O.rmsnorm(h, g["g_attn"], m.eps))
                qkv = mm(a, lw["w_qkv"].T)
                q = S(m._rope(qkv[:, :nq * d].reshape(L, nq, d), pos))
                kb = S(m._rope(qkv[:, nq * d:(nq + nkv) * d].reshape(L, nkv, d), pos))
                vb = S(qkv[:, (nq + nkv) * d:].reshape(L, nkv, d))
                o = S(attention(q, np.concatenate([ck[li, b], kb]), np.concatenate([cv[li, b], vb]))
                      .reshape(L, nq * d))
                h = h + mm(o, lw["w_o"].T)
                mmx = S(O.rmsnorm(h, g["g_mlp"], m.eps))
                gu = mm(mmx, lw["w_gu"].T)
                h = h + mm(S(O.silu(gu[:, :I]) * gu[:, I:]), lw["w_d"].T)
            out[b] = S(O.rmsnorm(h[1:], m.w.g_final, m.eps))
        return out

    return fuse, draft


def elem_stats(got, want, scale=None, tol=2e-2):
    """Elementwise |g - o| / max(|o|, s), s = each entry's natural scale, or
    the tensor's rms where none is given."""
    fin = np.isfinite(want)
    g, w = got[fin], want[fin]
    floor = scale[fin] if scale is not None else float(np.sqrt(np.mean(w * w)))
    e = np.abs(g - w) / np.maximum(np.abs(w), floor)
    return {"elem_max": float(e.max()), "elem_p99_9": float(np.percentile(e, 99.9)),
            f"n_elem_over_{tol:g}": int((e > tol).sum()), "n_elem": int(e.size)}


def logit_entry_scale(hid, w_lm, lay):
    """||h_p|| ||w_t|| / sqrt(H) for every gathered legal logit (0 in the padding)."""
    B, P, H = hid.shape
    width = max(len(lay.legal(p)) for p in range(1, lay.L))
    out = np.zeros((B, P, width))
    hn = np.linalg.norm(hid, axis=-1)
    for p in range(1, lay.L):
        ids = lay.legal(p)
        wn = np.linalg.norm(np.asarray(w_lm[ids], np.float64), axis=1) / np.sqrt(H)
        out[:, p - 1, :len(ids)] = hn[:, p - 1, None] * wn[None, :]
    return out


def logit_rows(got, want, scale, lay, min_ids=16):
    """Largest ||g - o|| / max(||o||, ||s||) over positions with min_ids legal ids or more."""
    worst = 0.0
    for p in range(1, lay.L):
        n = len(lay.legal(p))
        if n < min_ids:
            continue
        d = np.linalg.norm(got[:, p - 1, :n] - want[:, p - 1, :n], axis=-1)
        den = np.maximum(np.linalg.norm(want[:, p - 1, :n], axis=-1), np.linalg.norm(scale[:, p - 1, :n], axis=-1))
        worst = max(worst, float((d / den).max()))
    return worst


def main(name: str) -> None:
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    m = O.Model(wl.shape, inp.weights)
    lay = O.build_layout(wl.schema, wl.shape.vocab)
    t = time.time()
    ck, cv = O.fuse_context_kv(m, inp.feats)
    hid = O.draft_block(m, inp.tokens, ck, cv)
    z = O.full_logits(m, hid)
    toks = O.constrained_tokens(z, lay)
    t_ref = time.time() - t
    fuse, draft = f32_products(m)
    t = time.time()
    ck2, cv2 = fuse(inp.feats)
    hid2 = draft(inp.tokens, ck2, cv2)
    z2 = O.full_logits(m, hid2)
    toks2 = O.constrained_tokens(z2, lay)
    t_f32 = time.time() - t
    zg, zg2 = O.gathered_logits(z, lay), O.gathered_logits(z2, lay)
    sc = logit_entry_scale(hid, inp.weights.w_lm, lay)
    rows = np.linalg.norm(hid2 - hid, axis=-1) / np.linalg.norm(hid, axis=-1)
    diff = toks2 != toks
    gaps = []
    for b, p0 in zip(*np.nonzero(diff)):
        ids = lay.legal(int(p0) + 1)
        v = np.sort(z[b, p0, ids])
        gaps.append(float(v[-1] - v[-2]))
    out = {
        "workload": name,
        "what": "float64 oracle vs the same arithmetic with float32 accumulation (same bf16 storage points); "
                "row_max: largest relative L2 error of a hidden row or of a position's legal logits (sets of 16 "
                "ids or more); elem: |g - o| / max(|o|, s) with s the tensor rms (context, hidden) or each "
                "logit's natural scale ||h_p|| ||w_t|| / sqrt(H)",
        "command": f"python tests/golden/noise_floor.py {name}",
        "ctx_k": elem_stats(ck2, ck), "ctx_v": elem_stats(cv2, cv),
        "hidden": dict(row_max=float(rows.max()), **elem_stats(hid2, hid)),
        "logits": dict(row_max=logit_rows(zg2, zg, sc, lay), **elem_stats(zg2, zg, sc)),
        "tokens": {"positions": int(toks.size), "differ": int(diff.sum()), "top2_gaps_at_differences": gaps},
        "seconds": {"oracle": round(t_ref, 1), "float32_accumulation": round(t_f32, 1)},
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"noise_floor_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "traj2d3d")
