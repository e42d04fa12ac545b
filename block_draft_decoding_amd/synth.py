"""Seeded synthetic inputs for the block-drafter path.

This module only *draws* inputs: weights, target features, block tokens,
schemas and planted target tokens.  It holds none of the drafter's
arithmetic, so the HIP path (through the Python binding) and the CPU
oracle can both be fed from it without sharing any of the computation.

Shapes follow the workloads the pages describe:
  * the tiny fp32 drafter (hidden 256, 2 layers, 16-token block);
  * sub-task text blocks of 16 positions (one anchor and 15 proposals) in
    the verified speculative mode (VFlash, "Method"; VFlash paper §2.5);
  * an 8-waypoint 2D trajectory (NAVSIM-shaped, VFlash paper §2.3);
  * a 64-waypoint 2D+3D trajectory (Alpamayo-shaped, VFlash "Method");
  * a dense 3D point-motion block written as fixed-width sign + 5 digit
    fields (VFlash paper §2.3, §3.1).
The datasets those pages evaluate on, and every trained checkpoint, are not
available; only their shapes are reproduced, with N(0, sigma) weights and
N(0, 1) target features.

Determinism: every tensor has its own ``numpy.random.SeedSequence`` keyed
by (seed, tensor index) and is filled in fixed chunks of ``_CHUNK``
elements, each from its own spawned child stream.  The values therefore do
not depend on the number of threads used to draw them.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

_CHUNK = 1 << 22

# Token ids of the bf16 workloads.  The pages print no ids; these are the
# fixed choices made for the synthetic vocabulary of 151,936 entries:
# 1,001 coordinate tokens (value v <-> id COORD_BASE + v, v in [0, 1000]),
# then the structural tokens.
COORD_BASE = 150_000
COORD_COUNT = 1001
DELIM_ID = 151_001
OFF_ID = 151_002
PLUS_ID = 151_003
MINUS_ID = 151_004
DIGIT0_ID = 151_005          # digits 0..9 are 151_005 .. 151_014
FILL_ID = 151_015            # fill for unused high digits of a numeric field
START_ID = 151_016           # typed primitive start token (block anchor)
MASK_ID = 151_935            # input token of every masked block position

# The tiny fp32 drafter: vocabulary 2,048 with coordinate ids 1000..2000.
TINY_COORD_BASE = 1000
TINY_MASK_ID = 2047


@dataclass(frozen=True)
class DrafterShape:
    """Shape of the drafter (the model), independent of any block."""
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    n_layers: int
    inter: int
    vocab: int
    n_fused: int                 # number of target layers fused into the context
    dtype: str                   # "bf16" or "f32"
    rope_theta: float = 1.0e6
    use_rope: int = 1
    rms_eps: float = 1.0e-6
    weight_std: float = 0.02


@dataclass
class Workload:
    name: str
    shape: DrafterShape
    batch: int
    ctx: int
    schema: Dict
    seed_index: int
    # std of the LM head's OFF row when it is drawn apart from the other rows.  The
    # masked positions' final hidden states are strongly aligned (one MASK input
    # token at every position), so OFF's logit moves together across positions;
    # at 0.3 (15x the other rows) OFF wins 7 of the 64 image-coordinate pairs of
    # the 64-waypoint block and 4 pairs need the joint decision.
    off_row_std: Optional[float] = None
    k_star: Optional[List[int]] = None    # planted accepted lengths for text verification
    notes: str = ""
    shared_ctx: bool = False              # all blocks share one context (features of batch 1)

    @property
    def block_len(self) -> int:
        return schema_block_len(self.schema)


def schema_block_len(schema: Dict) -> int:
    """Block length implied by a schema's kind and point count (counting rule
    only: one anchor plus the positions of the declared layout)."""
    kind = schema["kind"]
    if kind in ("text", "custom"):
        return int(schema["block_len"])
    per_point = {"traj2d": 3, "traj2d3d": 6, "points3d_text": 19, "boxes2d": 5}[kind]
    return 1 + per_point * int(schema["n_points"])


def _bf16_ids(**over) -> Dict:
    d = dict(start_id=START_ID, mask_id=MASK_ID, delim_id=DELIM_ID, off_id=-1,
             plus_id=PLUS_ID, minus_id=MINUS_ID, digit0_id=DIGIT0_ID, fill_id=FILL_ID,
             coord_base=COORD_BASE, coord_count=COORD_COUNT)
    d.update(over)
    return d


DRAFTER_4B = DrafterShape(hidden=2560, n_q=32, n_kv=8, head_dim=128, n_layers=5,
                          inter=9728, vocab=151_936, n_fused=5, dtype="bf16")
# FlashDrive's drafter: two layers, conditioned on the last 8 target tokens;
# its widths are not printed, so the same 2560-wide layers are used.
DRAFTER_2L = DrafterShape(hidden=2560, n_q=32, n_kv=8, head_dim=128, n_layers=2,
                          inter=9728, vocab=151_936, n_fused=5, dtype="bf16")
DRAFTER_TINY = DrafterShape(hidden=256, n_q=4, n_kv=2, head_dim=64, n_layers=2,
                            inter=704, vocab=2048, n_fused=2, dtype="f32")


def _tiny_schema() -> Dict:
    # 16 positions: anchor, then odd positions restricted to the coordinate
    # ids 1000..2000, even positions free.
    L = 16
    coord = list(range(TINY_COORD_BASE, TINY_COORD_BASE + 1001))
    pos_set = [-2] + [0 if p % 2 == 1 else -1 for p in range(1, L)]
    return dict(kind="custom", block_len=L, sets=[coord], pos_set=pos_set, pairs=[], fields=[],
                start_id=-1, mask_id=TINY_MASK_ID, delim_id=-1, off_id=-1, plus_id=-1,
                minus_id=-1, digit0_id=-1, fill_id=-1, coord_base=TINY_COORD_BASE,
                coord_count=1001)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", DRAFTER_TINY, batch=1, ctx=64, schema=_tiny_schema(), seed_index=1,
                     k_star=list(range(16)),
                     notes="fp32 tiny drafter, context 64 from 2 fused layers, L=16"),
    "text": Workload("text", DRAFTER_4B, batch=1, ctx=2048,
                     schema=dict(kind="text", block_len=16, **_bf16_ids()), seed_index=2,
                     k_star=list(range(16)),
                     notes="sub-task text block, L=16 (anchor + 15 proposals), full vocabulary"),
    "traj2d": Workload("traj2d", DRAFTER_4B, batch=1, ctx=2048,
                       schema=dict(kind="traj2d", n_points=8, **_bf16_ids()), seed_index=3,
                       notes="NAVSIM-shaped 2D trajectory, 8 waypoints x (x, y, delim), L=25"),
    "traj2d3d": Workload("traj2d3d", DRAFTER_4B, batch=1, ctx=4096,
                         schema=dict(kind="traj2d3d", n_points=64, **_bf16_ids(off_id=OFF_ID)),
                         seed_index=4, off_row_std=0.3,
                         notes="Alpamayo-shaped 2D+3D trajectory, 64 waypoints x "
                               "(u, v, X, Y, Z, delim), L=385, paired off-frame rule"),
    "flashdrive8": Workload("flashdrive8", DRAFTER_2L, batch=1, ctx=8,
                            schema=dict(kind="text", block_len=8, **_bf16_ids()), seed_index=6,
                            k_star=list(range(8)),
                            notes="FlashDrive-shaped reasoning block: 2 layers, context = last 8 target "
                                  "tokens, L=8, full vocabulary, prefix verification"),
    "flashdrive16": Workload("flashdrive16", DRAFTER_2L, batch=1, ctx=8,
                             schema=dict(kind="text", block_len=16, **_bf16_ids()), seed_index=7,
                             k_star=list(range(16)),
                             notes="FlashDrive-shaped reasoning block: 2 layers, context = last 8 target "
                                   "tokens, L=16, full vocabulary, prefix verification"),
    "traj2d_shared16": Workload("traj2d_shared16", DRAFTER_4B, batch=16, ctx=2048,
                                schema=dict(kind="traj2d", n_points=8, **_bf16_ids()), seed_index=8,
                                shared_ctx=True,
                                notes="16 NAVSIM-shaped 2D-trajectory blocks (L=25) against one shared "
                                      "context of 2048 positions: M = 400 projection rows"),
    "boxes64": Workload("boxes64", DRAFTER_4B, batch=1, ctx=2048,
                        schema=dict(kind="boxes2d", n_points=64, **_bf16_ids()), seed_index=9,
                        notes="Dense200-shaped box list, 64 boxes x (x1, y1, x2, y2, delim), L=321; "
                              "partial acceptance against an external per-coordinate confidence"),
    "points3d": Workload("points3d", DRAFTER_4B, batch=8, ctx=4096,
                         schema=dict(kind="points3d_text", n_points=128, **_bf16_ids()),
                         seed_index=5,
                         notes="dense 3D point motion, 128 points x 3 axes x (sign + 5 digits) "
                               "+ delim, L=2433, 8 independent requests"),
}


# --------------------------------------------------------------------------
# drawing helpers
# --------------------------------------------------------------------------

def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed: int, key: int, shape, std: float) -> np.ndarray:
    """float32 N(0, std^2) draws, deterministic in (seed, key)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, np.float32)
    nchunks = max(1, math.ceil(n / _CHUNK))
    children = np.random.SeedSequence(entropy=seed, spawn_key=(key,)).spawn(nchunks)

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        np.random.Generator(np.random.PCG64(children[i])).standard_normal(
            dtype=np.float32, out=out[lo:hi])

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    if std != 1.0:
        np.multiply(out, np.float32(std), out=out)
    return out.reshape(shape)


def round_to_bf16_inplace(x: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bfloat16 values (ties to even),
    in place, keeping float32 storage.  Input preparation only: bf16
    workloads are drawn in float32 and stored in bfloat16."""
    assert x.dtype == np.float32 and x.flags.c_contiguous
    u = x.reshape(-1).view(np.uint32)
    step = 1 << 22
    for lo in range(0, u.size, step):
        seg = u[lo:lo + step]
        bias = ((seg >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        seg += bias
        seg &= np.uint32(0xFFFF0000)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of a float32 array whose values are bf16-exact."""
    return (x.reshape(-1).view(np.uint32) >> np.uint32(16)).astype(np.uint16).reshape(x.shape)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        round_to_bf16_inplace(x)
    return x


@dataclass
class Weights:
    """Drafter weights in torch ``Linear`` layout ([out, in]), float32 storage
    holding exactly the values of the stored dtype."""
    w_fc: np.ndarray              # [H, n_t*H]
    g_fc: np.ndarray              # [H]
    embed: np.ndarray             # [V, H]
    w_lm: np.ndarray              # [V, H]
    g_final: np.ndarray           # [H]
    layers: List[Dict[str, np.ndarray]] = field(default_factory=list)
    # per layer: g_attn [H], w_qkv [(n_q+2 n_kv) d, H], w_o [H, n_q d],
    #            g_mlp [H], w_gu [2 I, H] (gate rows, then up rows), w_d [H, I]


def make_weights(shape: DrafterShape, seed: int, off_row: Optional[int] = None,
                 off_row_std: Optional[float] = None, zero: tuple = ()) -> Weights:
    """Draw all drafter weights.  Norm gains are 1.  ``zero`` names weight
    kinds (e.g. ("w_o", "w_d")) to set to zero, for closed-form checks."""
    H, V, d = shape.hidden, shape.vocab, shape.head_dim
    std = shape.weight_std
    qkv = (shape.n_q + 2 * shape.n_kv) * d
    key = iter(range(10_000))

    def w(name, shp, s=std):
        a = _normal(seed, next(key), shp, s)
        if name in zero:
            a[...] = 0
        return _store(a, shape.dtype)

    def ones(n):
        return np.ones(n, np.float32)

    w_fc = w("w_fc", (H, shape.n_fused * H))
    embed = w("embed", (V, H))
    w_lm = w("w_lm", (V, H))
    if off_row is not None and off_row_std is not None:
        w_lm[off_row] = _store(_normal(seed, 9_999, (H,), off_row_std), shape.dtype)
    layers = []
    for _ in range(shape.n_layers):
        layers.append(dict(
            g_attn=ones(H),
            w_qkv=w("w_qkv", (qkv, H)),
            w_o=w("w_o", (H, shape.n_q * d)),
            g_mlp=ones(H),
            w_gu=w("w_gu", (2 * shape.inter, H)),
            w_d=w("w_d", (H, shape.inter)),
        ))
    return Weights(w_fc=w_fc, g_fc=ones(H), embed=embed, w_lm=w_lm, g_final=ones(H),
                   layers=layers)


def make_features(shape: DrafterShape, batch: int, ctx: int, seed: int) -> np.ndarray:
    """Frozen target-layer features [B, n_t, C, H], N(0, 1)."""
    f = _normal(seed, 0, (batch, shape.n_fused, ctx, shape.hidden), 1.0)
    return _store(f, shape.dtype)


def make_block_tokens(shape: DrafterShape, schema: Dict, batch: int, seed: int,
                      distinct_anchors: bool = False) -> np.ndarray:
    """Block input tokens [B, L]: anchor then MASK at every other position.
    Primitive blocks start with the typed start token; text blocks (and the
    tiny drafter) start with a drawn anchor.  distinct_anchors: blocks after
    the first draw their anchor (several primitives from one observation
    differ by their start token)."""
    L = schema_block_len(schema)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(1,))))
    tok = np.full((batch, L), schema["mask_id"], np.int32)
    if schema["kind"] == "text":
        tok[:, 0] = rng.integers(0, shape.vocab - 1, size=batch)
    elif schema["kind"] == "custom":
        tok[:, 0] = rng.integers(0, 1000, size=batch)
    else:
        tok[:, 0] = schema["start_id"]
    if distinct_anchors and batch > 1:
        tok[1:, 0] = rng.integers(0, shape.vocab - 1, size=batch - 1)
    return tok


def plant_targets(draft: np.ndarray, k_star, vocab: int, seed: int) -> np.ndarray:
    """Target tokens g_0..g_{L-1} [B, L] built around given draft tokens
    t_1..t_{L-1} [B, L-1] so that exactly the first k* drafts agree:
    g_{i-1} = t_i for i <= k*, g_{k*} differs from t_{k*+1}, the rest are
    uniform.  Stands in for the target model's greedy tokens."""
    draft = np.asarray(draft, np.int32)
    B, Lm1 = draft.shape
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(2,))))
    ks = np.broadcast_to(np.asarray(k_star, np.int64), (B,))
    tgt = rng.integers(0, vocab, size=(B, Lm1 + 1)).astype(np.int32)
    for b in range(B):
        k = int(ks[b])
        assert 0 <= k <= Lm1
        tgt[b, :k] = draft[b, :k]
        if k < Lm1:
            r = int(rng.integers(0, vocab - 1))
            tgt[b, k] = (int(draft[b, k]) + 1 + r) % vocab
    return tgt


def make_box_conf(batch: int, n_drafted: int, seed: int) -> np.ndarray:
    """Stand-in for the external spatial-confidence model's output: one
    float32 per drafted position [B, L-1], uniform on [0, 1)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(3,))))
    return rng.random((batch, n_drafted), dtype=np.float32)


@dataclass
class Inputs:
    workload: Workload
    weights: Weights
    feats: np.ndarray
    tokens: np.ndarray


def make_inputs(wl: Workload, weights: Optional[Weights] = None, zero: tuple = ()) -> Inputs:
    k = wl.seed_index
    if weights is None:
        off_row = wl.schema.get("off_id", -1)
        weights = make_weights(wl.shape, 1000 + k,
                               off_row=off_row if (off_row is not None and off_row >= 0) else None,
                               off_row_std=wl.off_row_std, zero=zero)
    feats = make_features(wl.shape, 1 if wl.shared_ctx else wl.batch, wl.ctx, 2000 + k)
    tokens = make_block_tokens(wl.shape, wl.schema, wl.batch, 3000 + k, distinct_anchors=wl.shared_ctx)
    return Inputs(wl, weights, feats, tokens)


def scaled_workload(name: str, **over) -> Workload:
    """A copy of a named workload with some drafter-shape or block fields
    replaced (used for small parity cases that keep the structure)."""
    wl = WORKLOADS[name]
    shape_over = {k: v for k, v in over.items() if k in DrafterShape.__dataclass_fields__}
    wl_over = {k: v for k, v in over.items() if k not in shape_over}
    return replace(wl, shape=replace(wl.shape, **shape_over), **wl_over)
