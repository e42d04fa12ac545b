"""CPU oracle for the Flash Primitive Decoding block-drafter path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this file: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library and does not
import the package that holds it.

It is a plain, slow, float64 NumPy transcription of what the pages say the
drafter computes:

* VFlash paper (Chinese translation), §2.1 "Preliminaries": features of
  selected target layers are fused and injected as key/value into every
  drafter layer; given the block's first (observed) token, one
  bidirectional forward predicts all masked positions of the block;
  greedy verification accepts drafts up to the first disagreement with the
  target.
* VFlash paper, §2.2 "Flash Primitive Decoding": a schema fixes the block
  length (one observed start token and L-1 masked tokens) and every
  position is predicted conditionally independently in one pass.
* VFlash paper, §2.3 "Token representation": 1,001 coordinate tokens;
  fixed-width numeric fields of one sign and five digits whose unused high
  digits hold a fill token.
* VFlash paper, §2.5 "Inference": per-position legal vocabularies, a
  cross-position rule that pairs off-frame image coordinates, both applied
  to logits that are already computed; acceptance by a schema validator.
* VFlash blog summary, "Method": text blocks of 16 positions (anchor and 15
  proposals) keep the longest matching prefix plus the target's next token.
* FlashDrive, §3.2 "Decode: Speculative Reasoning": fused target hidden
  states form the draft layers' KV cache.

Where the pages are silent the readings below are taken (each also listed
in the repository's design notes):
  R1  fusion = concatenate the n_t target layers along features, one
      bias-free linear map W_fc, then RMSNorm (gain g_fc);
  R2  each drafter layer projects the fused features with its own K/V rows
      of W_qkv; context keys get RoPE at positions ctx_pos0..ctx_pos0+C-1;
  R3  pre-norm RMSNorm, y = x / sqrt(mean(x^2) + eps) * g; no biases;
  R4  rotate-half RoPE on (i, i + d/2), inv_freq_i = theta^(-2i/d); block
      positions follow the context: block_pos..block_pos+L-1;
  R6  positions 1..L-1 each predict their own token; position 0 none;
  R8  no attention mask; query head i reads KV head floor(i*n_kv/n_q);
      scale 1/sqrt(d);
  R9  masked argmax: lowest id among the maxima; NaN counts as the maximum;
  R10 image-coordinate pairs (u, v): the legal set of each is the
      coordinate ids plus OFF; the pair is decided by a joint argmax over
      (OFF, OFF) and all on-frame (a, b); a tie between the branches goes
      to on-frame, ties inside a branch to the lowest ids;
  R11 trajectory acceptance is all or nothing: k = (L-1) * a(y);
  R12 a numeric field's five digit positions read FILL^j DIGIT^(5-j),
      0 <= j <= 4;
  R13 text acceptance: k = longest prefix with t_i = g_{i-1}; next = g_k;
  R15 bf16 workloads store weights/features in bf16 and round to bf16 at
      exactly these points: the normed GEMM inputs (fused context, attention
      and MLP inputs, final hidden), Q/K/V after RoPE, context K/V, the
      attention output and the SwiGLU product.  Everything else is carried
      at full precision (float64 here).  f32 workloads round nowhere.
  R22 incremental context: features of newly committed target positions
      pos0.. are fused exactly as the first context (R1, R2) and their K/V
      written at cache rows pos0.. (cache row = target position);
  R23 several primitives from one observation: blocks of one length, each
      with its own anchor, attend to one shared context and to their own
      block only (no attention between blocks);
  R24 coordinate codec: bin = clamp(round-half-even((x - lo) * s), 0, 1000)
      with s = 1000 / (hi - lo) (2D: lo 0, hi 1000, s = 1; 3D: the
      predefined range, a parameter since its values are not printed); a bin
      decodes to lo + bin * (hi - lo) / 1000; fields hold |n| <= 99,999;
  R25 box acceptance: a box is [x1, y1, x2, y2, DELIM]; an external
      confidence per drafted position is given, and a coordinate position
      (legal set inside the coordinate ids, OFF allowed) is uncertain when
      its confidence is not >= tau (NaN is uncertain); the drafts kept are
      those before the first uncertain coordinate and before the first
      schema failure, k = min(first_uncertain, first_invalid), L-1 if none.

Functions whose result has no independent pin say so in their docstring.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# numeric helpers
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value of each float64 entry (ties to even), as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2^-126 the spacing is fixed at 2^-133."""
    x = np.asarray(x, F64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Apply the storage rounding of the workload's dtype (R15)."""
    return bf16_round(x) if dtype == "bf16" else np.asarray(x, F64)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """R3: x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, F64)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """R4: rotate-half rotary embedding over the last axis (head dim d).

    x: [..., T, heads, d]; positions: [T].  Entry i is paired with i + d/2
    and turned by the angle position * theta^(-2i/d)."""
    x = np.asarray(x, F64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-np.arange(half, dtype=F64) * 2.0 / d)
    ang = np.asarray(positions, F64)[:, None] * inv_freq[None, :]       # [T, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def _f64(a) -> np.ndarray:
    return np.asarray(a, F64)


# ---------------------------------------------------------------------------
# model description
# ---------------------------------------------------------------------------

class Model:
    """Weights and shape, as float64 arrays.  ``weights`` is any object with
    the attributes w_fc, g_fc, embed, w_lm, g_final, layers (list of dicts
    with g_attn, w_qkv, w_o, g_mlp, w_gu, w_d); ``shape`` any object with
    hidden, n_q, n_kv, head_dim, n_layers, inter, vocab, n_fused, dtype,
    rope_theta, use_rope, rms_eps."""

    def __init__(self, shape, weights):
        self.s = shape
        self.w = weights
        self.H = shape.hidden
        self.nq, self.nkv, self.d = shape.n_q, shape.n_kv, shape.head_dim
        self.I = shape.inter
        self.V = shape.vocab
        self.dtype = shape.dtype
        self.eps = float(shape.rms_eps)
        self.theta = float(shape.rope_theta)
        self.use_rope = bool(shape.use_rope)
        self._layers = None

    def layer(self, i: int) -> Dict[str, np.ndarray]:
        if self._layers is None:
            self._layers = [{k: _f64(v) for k, v in lw.items()} for lw in self.w.layers]
        return self._layers[i]

    @property
    def n_layers(self) -> int:
        return len(self.w.layers)

    def _rope(self, x, positions):
        return rope(x, positions, self.theta) if self.use_rope else np.asarray(x, F64)


# ---------------------------------------------------------------------------
# step 1: context fusion (VFlash paper §2.1; FlashDrive §3.2) -- R1, R2, R3
# ---------------------------------------------------------------------------

def fuse_context_kv(m: Model, feats: np.ndarray, ctx_pos0: int = 0):
    """Fused target features -> per-layer context K/V.

    feats: [B, n_t, C, H].  Returns (ctx_k, ctx_v), each
    [n_layers, B, C, n_kv, d]; keys already rotated (R2)."""
    feats = _f64(feats)
    B, nt, C, H = feats.shape
    X = np.concatenate([feats[:, t] for t in range(nt)], axis=-1)        # [B, C, nt*H]
    Z = X @ _f64(m.w.w_fc).T                                             # [B, C, H]
    Zn = _store(rmsnorm(Z, m.w.g_fc, m.eps), m.dtype)
    pos = ctx_pos0 + np.arange(C)
    nq, nkv, d = m.nq, m.nkv, m.d
    ks, vs = [], []
    for li in range(m.n_layers):
        w = m.layer(li)["w_qkv"]
        wk = w[nq * d:(nq + nkv) * d]
        wv = w[(nq + nkv) * d:(nq + 2 * nkv) * d]
        k = (Zn @ wk.T).reshape(B, C, nkv, d)
        v = (Zn @ wv.T).reshape(B, C, nkv, d)
        ks.append(_store(m._rope(k, pos), m.dtype))
        vs.append(_store(v, m.dtype))
    return np.stack(ks), np.stack(vs)


def append_context_kv(m: Model, ctx_k: np.ndarray, ctx_v: np.ndarray, feats: np.ndarray, pos0: int):
    """Incremental context: after a block is accepted the target's forward
    pass updates its cache and the context features (VFlash paper §2.5), and
    the drafter is conditioned on the newest target positions (FlashDrive
    §3.2, Fig. 4: the hidden states of the last eight target tokens).  feats [B, n_t, C_new, H] are the
    fused-layer features of target positions pos0 .. pos0 + C_new - 1; their
    K/V (keys rotated at those positions) replace rows pos0 .. of the given
    caches [n_layers, B, C, n_kv, d], which grow if needed (R22).  Rows
    before pos0 are returned unchanged."""
    nk, nv = fuse_context_kv(m, feats, ctx_pos0=pos0)
    Cn = nk.shape[2]
    N, B, C0 = ctx_k.shape[0], ctx_k.shape[1], ctx_k.shape[2]
    C = max(C0, pos0 + Cn)
    out_k = np.zeros((N, B, C) + ctx_k.shape[3:], np.float64)
    out_v = np.zeros((N, B, C) + ctx_v.shape[3:], np.float64)
    out_k[:, :, :C0] = ctx_k
    out_v[:, :, :C0] = ctx_v
    out_k[:, :, pos0:pos0 + Cn] = nk
    out_v[:, :, pos0:pos0 + Cn] = nv
    return out_k, out_v


# ---------------------------------------------------------------------------
# step 2-4: the drafter forward over one block (VFlash paper §2.1, §2.2)
# ---------------------------------------------------------------------------

def attention(m: Model, q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """R8: non-causal GQA attention.  q [T, n_q, d]; k, v [S, n_kv, d].
    Two-pass softmax.  Returns [T, n_q, d]."""
    T = q.shape[0]
    out = np.empty((T, m.nq, m.d), F64)
    scale = 1.0 / np.sqrt(m.d)
    for i in range(m.nq):
        j = (i * m.nkv) // m.nq
        s = (q[:, i, :] @ k[:, j, :].T) * scale                          # [T, S]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, i, :] = p @ v[:, j, :]
    return out


def draft_block(m: Model, tokens: np.ndarray, ctx_k: np.ndarray, ctx_v: np.ndarray,
                block_pos: Optional[int] = None, return_residuals: bool = False):
    """Drafter forward over a block (R3-R8, R15).

    tokens: [B, L] (anchor, then masked positions); ctx_k/ctx_v:
    [n_layers, B, C, n_kv, d].  block_pos defaults to C (the block follows
    its context).  Returns the final hidden states h_f [B, L-1, H] of
    positions 1..L-1 (R6), and optionally the residual stream after each
    layer ([n_layers, B, L, H])."""
    tokens = np.asarray(tokens)
    B, L = tokens.shape
    C = ctx_k.shape[2]
    if block_pos is None:
        block_pos = C
    pos = block_pos + np.arange(L)
    nq, nkv, d, H = m.nq, m.nkv, m.d, m.H
    out = np.empty((B, L - 1, H), F64)
    resid = []
    for b in range(B):
        h = _f64(m.w.embed[tokens[b]])                                   # [L, H]
        rb = []
        for li in range(m.n_layers):
            w = m.layer(li)
            a = _store(rmsnorm(h, w["g_attn"], m.eps), m.dtype)
            qkv = a @ w["w_qkv"].T
            q = qkv[:, :nq * d].reshape(L, nq, d)
            kb = qkv[:, nq * d:(nq + nkv) * d].reshape(L, nkv, d)
            vb = qkv[:, (nq + nkv) * d:].reshape(L, nkv, d)
            q = _store(m._rope(q, pos), m.dtype)
            kb = _store(m._rope(kb, pos), m.dtype)
            vb = _store(vb, m.dtype)
            kk = np.concatenate([_f64(ctx_k[li, b]), kb], axis=0)
            vv = np.concatenate([_f64(ctx_v[li, b]), vb], axis=0)
            o = _store(attention(m, q, kk, vv).reshape(L, nq * d), m.dtype)
            h = h + o @ w["w_o"].T
            mm = _store(rmsnorm(h, w["g_mlp"], m.eps), m.dtype)
            gu = mm @ w["w_gu"].T
            u = _store(silu(gu[:, :m.I]) * gu[:, m.I:], m.dtype)
            h = h + u @ w["w_d"].T
            rb.append(h.copy())
        out[b] = _store(rmsnorm(h[1:], m.w.g_final, m.eps), m.dtype)
        resid.append(np.stack(rb))
    if return_residuals:
        return out, np.stack(resid, axis=1)
    return out


def draft_blocks_shared(m: Model, tokens: np.ndarray, ctx_k: np.ndarray, ctx_v: np.ndarray,
                        block_pos: Optional[int] = None) -> np.ndarray:
    """Several blocks against one shared observation (VFlash paper,
    conclusion / future work: complementary primitives from one
    observation): every block of tokens [B, L] attends to the single
    context ctx_k / ctx_v [n_layers, 1, C, n_kv, d] (R23).  Returns [B, L-1, H]."""
    B = np.asarray(tokens).shape[0]
    bk = np.broadcast_to(ctx_k, ctx_k.shape[:1] + (B,) + ctx_k.shape[2:])
    bv = np.broadcast_to(ctx_v, ctx_v.shape[:1] + (B,) + ctx_v.shape[2:])
    return draft_block(m, tokens, bk, bv, block_pos=block_pos)


def full_logits(m: Model, hidden: np.ndarray, chunk_rows: int = 8192) -> np.ndarray:
    """Full-vocabulary logits z = h_f W_lm^T, [B, L-1, V].  The vocabulary is
    converted to float64 in row chunks only to bound memory."""
    hidden = _f64(hidden)
    B, P, H = hidden.shape
    z = np.empty((B, P, m.V), F64)
    flat = hidden.reshape(B * P, H)
    for lo in range(0, m.V, chunk_rows):
        wl = _f64(m.w.w_lm[lo:lo + chunk_rows])
        z[:, :, lo:lo + chunk_rows] = (flat @ wl.T).reshape(B, P, -1)
    return z


# ---------------------------------------------------------------------------
# layouts (VFlash paper §2.2, §2.3 and the blog's "Method")
# ---------------------------------------------------------------------------

class Layout:
    """Per-position roles of a block.

    pos_set[p] for block position p in 0..L-1: -2 anchor, -1 free (whole
    vocabulary), s >= 0 index of a legal set.  sets: list of ascending id
    arrays.  pairs: (p_u, p_v) block positions of paired image
    coordinates.  fields: (p_first_digit, 5) for each numeric field.
    Sets are numbered in order of first appearance along the block."""

    def __init__(self, L, pos_set, sets, pairs, fields, off_id, fill_id, digit_ids, vocab, coord_range=(0, 0)):
        self.L = L
        self.coord_range = (int(coord_range[0]), int(coord_range[1]))   # (first coordinate id, count)
        self.pos_set = np.asarray(pos_set, np.int32)
        self.sets = [np.asarray(s, np.int64) for s in sets]
        self.pairs = [tuple(p) for p in pairs]
        self.fields = [tuple(f) for f in fields]
        self.off_id = off_id
        self.fill_id = fill_id
        self.digit_ids = set(int(x) for x in digit_ids)
        self.vocab = vocab

    def legal(self, p: int) -> np.ndarray:
        s = int(self.pos_set[p])
        if s == -1:
            return np.arange(self.vocab, dtype=np.int64)
        if s < 0:
            raise ValueError("position 0 is the anchor and has no legal set")
        return self.sets[s]

    def is_coord(self, p: int) -> bool:
        """Position p holds a coordinate: its legal set is non-empty, every id
        in it is a coordinate id or OFF, and at least one is a coordinate id
        (R25)."""
        s = int(self.pos_set[p])
        if s < 0:
            return False
        lo, n = self.coord_range
        ids = self.sets[s]
        coord = (ids >= lo) & (ids < lo + n)
        return bool(coord.any()) and bool(np.all(coord | (ids == self.off_id)))

    def csr(self):
        offs = np.zeros(len(self.sets) + 1, np.int32)
        for i, s in enumerate(self.sets):
            offs[i + 1] = offs[i] + len(s)
        ids = np.concatenate(self.sets).astype(np.int32) if self.sets else np.zeros(0, np.int32)
        return offs, ids


def build_layout(schema: Dict, vocab: int) -> Layout:
    """Schema -> layout.  Per-point position orders (the pages' Table 1
    body is not available, so these are readings):
      traj2d        [x, y, DELIM] per waypoint;
      traj2d3d      [u, v, X, Y, Z, DELIM] per waypoint, (u, v) paired when
                    an OFF id is declared, u and v then also allow OFF;
      boxes2d       [x1, y1, x2, y2, DELIM] per box (R25);
      points3d_text ([SIGN, D, D, D, D, D] x 3 axes, DELIM) per point;
      text          every position free;
      custom        explicit sets and per-position indices."""
    kind = schema["kind"]
    roles: List[Tuple] = []            # one entry per block position 1..L-1
    pairs, fields = [], []
    coords = tuple(range(schema["coord_base"], schema["coord_base"] + schema["coord_count"]))
    digits = tuple(schema["digit0_id"] + i for i in range(10)) if schema.get("digit0_id", -1) >= 0 else ()
    off = schema.get("off_id", -1)
    if kind == "text":
        L = int(schema["block_len"])
        roles = [None] * (L - 1)
    elif kind == "traj2d":
        for _ in range(schema["n_points"]):
            roles += [coords, coords, (schema["delim_id"],)]
    elif kind == "traj2d3d":
        img = tuple(sorted(coords + (off,))) if off >= 0 else coords
        for _ in range(schema["n_points"]):
            p = 1 + len(roles)
            if off >= 0:
                pairs.append((p, p + 1))
            roles += [img, img, coords, coords, coords, (schema["delim_id"],)]
    elif kind == "boxes2d":
        for _ in range(schema["n_points"]):
            roles += [coords] * 4 + [(schema["delim_id"],)]
    elif kind == "points3d_text":
        sign = tuple(sorted((schema["plus_id"], schema["minus_id"])))
        dig = tuple(sorted(digits + (schema["fill_id"],)))
        for _ in range(schema["n_points"]):
            for _axis in range(3):
                p = 1 + len(roles)
                fields.append((p + 1, 5))
                roles += [sign] + [dig] * 5
            roles.append((schema["delim_id"],))
    elif kind == "custom":
        L = int(schema["block_len"])
        given = [tuple(sorted(set(int(i) for i in s))) for s in schema["sets"]]
        ps = list(schema["pos_set"])
        if len(ps) != L or ps[0] != -2:
            raise ValueError("custom pos_set must have L entries and start with -2")
        lay = Layout(L, ps, given, schema.get("pairs", []), schema.get("fields", []), off,
                     schema.get("fill_id", -1), digits, vocab,
                     coord_range=(schema.get("coord_base", 0), schema.get("coord_count", 0)))
        return lay
    else:
        raise ValueError(f"unknown schema kind {kind!r}")
    L = 1 + len(roles)
    sets: List[Tuple] = []
    index: Dict[Tuple, int] = {}
    pos_set = [-2]
    for r in roles:
        if r is None:
            pos_set.append(-1)
            continue
        if r not in index:
            index[r] = len(sets)
            sets.append(r)
        pos_set.append(index[r])
    return Layout(L, pos_set, sets, pairs, fields, off, schema.get("fill_id", -1), digits, vocab,
                  coord_range=(schema["coord_base"], schema["coord_count"]))


# ---------------------------------------------------------------------------
# step 5: constrained decoding (VFlash paper §2.5) -- R9, R10
# ---------------------------------------------------------------------------

def masked_argmax(z: np.ndarray, lay: Layout) -> np.ndarray:
    """t_p = lowest id attaining the maximum of z_p over S_p (R9).
    z: full logits [B, L-1, V] of positions 1..L-1.  Returns int32 [B, L-1]."""
    B, P, V = z.shape
    out = np.empty((B, P), np.int32)
    for p in range(1, lay.L):
        ids = lay.legal(p)
        out[:, p - 1] = ids[np.argmax(z[:, p - 1, ids], axis=1)]
    return out


def pair_off_frame(z: np.ndarray, tokens: np.ndarray, lay: Layout) -> np.ndarray:
    """R10: joint decision of each (u, v) pair over {(OFF, OFF)} and all
    on-frame combinations, written out over the whole product set.
    Returns a copy of tokens with every pair replaced by its joint choice."""
    out = np.array(tokens, np.int32, copy=True)
    if not lay.pairs:
        return out
    off = lay.off_id
    for (pu, pv) in lay.pairs:
        A = lay.legal(pu)
        A = A[A != off]
        Bs = lay.legal(pv)
        Bs = Bs[Bs != off]
        for b in range(z.shape[0]):
            zu, zv = z[b, pu - 1], z[b, pv - 1]
            joint = zu[A][:, None] + zv[Bs][None, :]
            flat = int(np.argmax(joint))                     # first maximum: lowest a, then b
            ia, ib = divmod(flat, len(Bs))
            s_on = joint[ia, ib]
            s_off = zu[off] + zv[off]
            if s_off > s_on:
                out[b, pu - 1], out[b, pv - 1] = off, off
            else:
                out[b, pu - 1], out[b, pv - 1] = A[ia], Bs[ib]
    return out


def constrained_tokens(z: np.ndarray, lay: Layout) -> np.ndarray:
    """Masked argmax followed by the pairing rule."""
    return pair_off_frame(z, masked_argmax(z, lay), lay)


def gathered_logits(z: np.ndarray, lay: Layout) -> np.ndarray:
    """Logits restricted to each position's legal set, ascending id order,
    padded with -inf to the widest set (the whole vocabulary if any position
    is free).  [B, L-1, W]."""
    B, P, V = z.shape
    widths = [len(lay.legal(p)) for p in range(1, lay.L)]
    W = max(widths) if widths else 0
    out = np.full((B, P, W), -np.inf, F64)
    for p in range(1, lay.L):
        ids = lay.legal(p)
        out[:, p - 1, :len(ids)] = z[:, p - 1, ids]
    return out


# ---------------------------------------------------------------------------
# step 6: acceptance (VFlash paper §2.1, §2.5; VFlash blog "Method") -- R11-R13
# ---------------------------------------------------------------------------

def _field_first_bad(toks, fill_id, digit_ids) -> int:
    """Index of the first entry of a 5-digit field that breaks
    FILL^j DIGIT^(5-j) with j <= 4, or -1 (R12)."""
    in_digits = False
    n = len(toks)
    for i, t in enumerate(toks):
        t = int(t)
        if t in digit_ids:
            in_digits = True
            continue
        if t == fill_id and not in_digits and i < n - 1:
            continue
        return i
    return -1


def validate_primitive(tokens: np.ndarray, lay: Layout):
    """Schema validator a(y) (R11, R12).  tokens: [B, L-1] for positions
    1..L-1.  Returns (k [B], first_invalid [B]) where first_invalid is the
    smallest failing index into the drafted tokens (-1 if valid) and
    k = (L-1) if valid else 0."""
    tokens = np.asarray(tokens)
    B, P = tokens.shape
    k = np.zeros(B, np.int32)
    first = np.full(B, -1, np.int32)
    for b in range(B):
        bad = []
        for p in range(1, lay.L):
            t = int(tokens[b, p - 1])
            s = int(lay.pos_set[p])
            ok = (0 <= t < lay.vocab) if s == -1 else bool(np.any(lay.sets[s] == t))
            if not ok:
                bad.append(p - 1)
        for (pu, pv) in lay.pairs:
            iu = tokens[b, pu - 1] == lay.off_id
            iv = tokens[b, pv - 1] == lay.off_id
            if iu != iv:
                bad.append(pu - 1)
        for (p0, w) in lay.fields:
            i = _field_first_bad(tokens[b, p0 - 1:p0 - 1 + w], lay.fill_id, lay.digit_ids)
            if i >= 0:
                bad.append(p0 - 1 + i)
        if bad:
            first[b] = min(bad)
        else:
            k[b] = P
    return k, first


def accept_boxes(tokens: np.ndarray, conf: np.ndarray, tau: float, lay: Layout):
    """Box partial acceptance (VFlash paper §2.5: for boxes, the positions
    before the first uncertain coordinate are kept; R25).  tokens, conf:
    [B, L-1] (conf float32, one value per drafted position; only coordinate
    positions are read).  Returns (k [B], first_invalid [B], first_uncertain
    [B]); the last two are -1 when there is none."""
    tokens = np.asarray(tokens)
    conf = np.asarray(conf, np.float32)
    B, P = tokens.shape
    _, first_invalid = validate_primitive(tokens, lay)
    tau32 = np.float32(tau)
    k = np.full(B, P, np.int32)
    first_unc = np.full(B, -1, np.int32)
    coord_pos = [p for p in range(1, lay.L) if lay.is_coord(p)]
    for b in range(B):
        for p in coord_pos:
            if not conf[b, p - 1] >= tau32:          # NaN is uncertain
                first_unc[b] = p - 1
                break
        stops = [i for i in (first_invalid[b], first_unc[b]) if i >= 0]
        if stops:
            k[b] = min(stops)
    return k, first_invalid, first_unc


def verify_prefix(draft: np.ndarray, target: np.ndarray):
    """Greedy longest-prefix verification (R13).  draft: [B, L-1] holding
    t_1..t_{L-1}; target: [B, L] holding g_0..g_{L-1}, g_j the target's
    greedy token after the anchor and t_1..t_j.  Returns (k [B], next [B]):
    k = number of leading drafts equal to the target's tokens, next = g_k."""
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, P = draft.shape
    k = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        i = 0
        while i < P and draft[b, i] == target[b, i]:
            i += 1
        k[b] = i
        nxt[b] = target[b, i]
    return k, nxt


# ---------------------------------------------------------------------------
# whole block
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# coordinate codec (VFlash paper §2.3; §3.1 "Base VLM") -- R24, R12
# ---------------------------------------------------------------------------

N_COORD = 1001   # coordinate tokens per axis


def coords_to_tokens(values, coord_base: int, lo: float = 0.0, hi: float = 1000.0) -> np.ndarray:
    """Coordinate value -> one of the 1,001 coordinate tokens (R24).  2D
    image coordinates are already normalised to 0..1000 (lo 0, hi 1000); 3D
    coordinates are quantised uniformly over the predefined range [lo, hi].
    bin = clamp(round_half_even((x - lo) * s), 0, 1000) with the scale
    s = 1000 / (hi - lo) (exactly 1 for the 2D range); a NaN value gives -1."""
    x = np.asarray(values, F64)
    scale = F64(N_COORD - 1) / (F64(hi) - F64(lo))
    t = (x - F64(lo)) * scale
    b = np.clip(np.rint(t), 0, N_COORD - 1)
    out = np.where(np.isnan(x), -1, coord_base + np.nan_to_num(b)).astype(np.int32)
    return out


def tokens_to_coords(tokens, coord_base: int, lo: float = 0.0, hi: float = 1000.0) -> np.ndarray:
    """Coordinate token -> the value of its bin, lo + i * w with the bin
    width w = (hi - lo) / 1000, for i = token - coord_base in 0..1000; NaN
    for any other token (R24)."""
    t = np.asarray(tokens, np.int64)
    i = t - coord_base
    ok = (i >= 0) & (i < N_COORD)
    width = (F64(hi) - F64(lo)) / F64(N_COORD - 1)
    v = F64(lo) + i.astype(F64) * width
    return np.where(ok, v, np.nan)


def ints_to_fields(values, plus_id: int, minus_id: int, digit0_id: int, fill_id: int) -> np.ndarray:
    """Integer -> a fixed-width field of a sign and five digit positions
    [n, 6] (VFlash paper §2.3): sign PLUS for n >= 0 else MINUS; |n| written
    with five digits whose leading zeros become FILL, except the last digit
    (R12: FILL^j DIGIT^(5-j), j <= 4).  A value with |n| > 99,999 does not
    fit and gives six -1 tokens."""
    v = np.asarray(values, np.int64)
    out = np.empty(v.shape + (6,), np.int32)
    out[..., 0] = np.where(v < 0, minus_id, plus_id)
    a = np.abs(v)
    for j in range(5):                       # most significant digit first
        d = (a // 10 ** (4 - j)) % 10
        lead = a < 10 ** (4 - j)             # nothing but zeros so far
        out[..., 1 + j] = np.where(lead & (j < 4), fill_id, digit0_id + d)
    out[np.abs(v) > 99_999] = -1
    return out


def fields_to_ints(fields, plus_id: int, minus_id: int, digit0_id: int, fill_id: int):
    """Inverse of ints_to_fields on [n, 6] tokens.  Returns (values [n],
    valid [n]): a field is valid when its sign is PLUS or MINUS and its digits
    read FILL^j DIGIT^(5-j) with j <= 4 (R12); invalid fields give 0."""
    f = np.asarray(fields, np.int64).reshape(-1, 6)
    n = f.shape[0]
    vals = np.zeros(n, np.int32)
    valid = np.zeros(n, np.int32)
    digits = set(range(digit0_id, digit0_id + 10))
    for r in range(n):
        sgn = f[r, 0]
        if sgn not in (plus_id, minus_id) or _field_first_bad(f[r, 1:], fill_id, digits) >= 0:
            continue
        a = 0
        for t in f[r, 1:]:
            a = a * 10 + (int(t) - digit0_id if int(t) in digits else 0)
        vals[r] = -a if sgn == minus_id else a
        valid[r] = 1
    return vals, valid


def run_block(m: Model, feats, tokens, schema: Dict, targets=None, ctx_pos0: int = 0,
              block_pos: Optional[int] = None, want_logits: bool = False, shared_ctx: bool = False):
    """Fuse, draft, decode under the layout, then accept.  Returns a dict
    with ctx_k, ctx_v, hidden, tokens, (logits), k_prim/first_invalid for
    primitive layouts and k_text/next when target tokens are given.
    shared_ctx: feats hold one context that every block attends to (R23)."""
    lay = build_layout(schema, m.V)
    ck, cv = fuse_context_kv(m, feats, ctx_pos0)
    C = ck.shape[2]
    bp = (C + ctx_pos0) if block_pos is None else block_pos
    if shared_ctx:
        hidden = draft_blocks_shared(m, tokens, ck, cv, block_pos=bp)
    else:
        hidden = draft_block(m, tokens, ck, cv, block_pos=bp)
    z = full_logits(m, hidden)
    toks = constrained_tokens(z, lay)
    res = dict(ctx_k=ck, ctx_v=cv, hidden=hidden, tokens=toks, layout=lay)
    if want_logits:
        res["logits"] = z
    if targets is not None:
        res["k_text"], res["next"] = verify_prefix(toks, targets)
    if schema["kind"] != "text":
        res["k_prim"], res["first_invalid"] = validate_primitive(toks, lay)
    return res
