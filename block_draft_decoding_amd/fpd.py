"""Python binding of libfpd (ctypes).  Argument marshalling only: every step
of the block-drafter path runs in the library's gfx950 kernels; PyTorch
provides device memory and streams.

The functions carry the C ABI's names (include/fpd.h).  Shapes are read from
the tensors passed in; tensors must be contiguous and on the GPU.  A missing
or unloadable library raises ``ImportError`` at import time -- there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfpd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libfpd.so not found at {LIB_PATH}: build it with "
                      "`python block_draft_decoding_amd/csrc/build.py` (or __graft_entry__.build())")
try:
    _lib = ctypes.CDLL(LIB_PATH)
except OSError as e:  # pragma: no cover
    raise ImportError(f"cannot load {LIB_PATH}: {e}") from e

# ---- constants (mirror include/fpd.h) ---------------------------------------
FPD_OK, FPD_E_ARG, FPD_E_SHAPE, FPD_E_DTYPE, FPD_E_SCHEMA, FPD_E_WORKSPACE, FPD_E_UNSUPPORTED, FPD_E_HIP = range(8)
FPD_DTYPE_F32, FPD_DTYPE_BF16 = 0, 1
SCHEMA_KINDS = {"text": 0, "traj2d": 1, "traj2d3d": 2, "points3d_text": 3, "custom": 4, "boxes2d": 5}

i32 = ctypes.c_int32
vp = ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)


class fpd_config(ctypes.Structure):
    _fields_ = [("hidden", i32), ("n_q", i32), ("n_kv", i32), ("head_dim", i32), ("n_layers", i32),
                ("inter", i32), ("vocab", i32), ("n_fused", i32), ("dtype", i32), ("use_rope", i32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class fpd_layer_weights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("g_attn", "w_qkv", "w_o", "g_mlp", "w_gu", "w_d")]


class fpd_weights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("w_fc", "g_fc", "embed", "w_lm", "g_final")] + \
               [("layers", ctypes.POINTER(fpd_layer_weights))]


class fpd_schema(ctypes.Structure):
    _fields_ = [("kind", i32), ("n_points", i32), ("block_len", i32),
                ("start_id", i32), ("mask_id", i32), ("delim_id", i32), ("off_id", i32),
                ("plus_id", i32), ("minus_id", i32), ("digit0_id", i32), ("fill_id", i32),
                ("coord_base", i32), ("coord_count", i32),
                ("n_sets", i32), ("set_offsets", P_i32), ("set_ids", P_i32), ("pos_set", P_i32),
                ("n_pairs", i32), ("pairs", P_i32), ("n_fields", i32), ("fields", P_i32)]


class fpd_layout_sizes(ctypes.Structure):
    _fields_ = [("L", i32), ("n_sets", i32), ("n_set_ids", i32), ("n_pairs", i32), ("n_fields", i32),
                ("width", i32)]


def _proto(name, args):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = i32
    return f


_lib.fpd_status_string.argtypes = [i32]
_lib.fpd_status_string.restype = ctypes.c_char_p
_lib.fpd_last_error.argtypes = []
_lib.fpd_last_error.restype = ctypes.c_char_p
_create = _proto("fpd_drafter_create", [ctypes.POINTER(fpd_config), ctypes.POINTER(fpd_weights), ctypes.POINTER(vp)])
_destroy = _proto("fpd_drafter_destroy", [vp])
_prepare = _proto("fpd_drafter_prepare", [vp, vp])
_expand = _proto("fpd_schema_expand", [ctypes.POINTER(fpd_schema), i32, ctypes.POINTER(fpd_layout_sizes),
                                       P_i32, P_i32, P_i32, P_i32, P_i32])
_lay_create = _proto("fpd_layout_create", [vp, ctypes.POINTER(fpd_schema), ctypes.POINTER(vp), P_i32])
_lay_destroy = _proto("fpd_layout_destroy", [vp])
_lay_masks = _proto("fpd_layout_masks", [vp, ctypes.POINTER(fpd_layout_sizes), P_i32, P_i32, P_i32, P_i32, P_i32])
_ws_size = _proto("fpd_workspace_size", [vp, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)])
_fuse = _proto("fpd_fuse_context_kv", [vp, vp, i32, i32, i32, vp, vp, i32, vp, ctypes.c_size_t, vp])
_append = _proto("fpd_append_context_kv", [vp, vp, i32, i32, i32, vp, vp, i32, vp, ctypes.c_size_t, vp])
_draft = _proto("fpd_draft_block", [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, ctypes.c_size_t, vp])
_draft_noalloc = _proto("fpd_draft_block_noalloc", [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp])
_draft_shared = _proto("fpd_draft_blocks_shared_ctx", [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, ctypes.c_size_t, vp])
_argmax = _proto("fpd_constrained_argmax", [vp, vp, vp, i32, vp, vp, vp, ctypes.c_size_t, vp])
_validate = _proto("fpd_validate_primitive", [vp, vp, i32, vp, vp, vp])
_verify = _proto("fpd_verify_prefix", [vp, vp, i32, i32, vp, vp, vp])
f64 = ctypes.c_double
_boxes = _proto("fpd_accept_boxes", [vp, vp, vp, ctypes.c_float, i32, vp, vp, vp, vp])
_c2t = _proto("fpd_coords_to_tokens", [vp, i32, f64, f64, i32, vp, vp])
_t2c = _proto("fpd_tokens_to_coords", [vp, i32, f64, f64, i32, vp, vp])
_i2f = _proto("fpd_ints_to_fields", [vp, i32, i32, i32, i32, i32, vp, vp])
_f2i = _proto("fpd_fields_to_ints", [vp, i32, i32, i32, i32, i32, vp, vp, vp])


class FpdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.fpd_last_error().decode(errors="replace")
        super().__init__(f"{where}: {fpd_status_string(status)} ({status}): {msg}")


def fpd_status_string(status: int) -> str:
    return _lib.fpd_status_string(status).decode()


def fpd_last_error() -> str:
    return _lib.fpd_last_error().decode(errors="replace")


def _check(st: int, where: str) -> None:
    if st != FPD_OK:
        raise FpdError(st, where)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


TORCH_DT = {FPD_DTYPE_F32: torch.float32, FPD_DTYPE_BF16: torch.bfloat16}


# ---- handles -----------------------------------------------------------------

class Drafter:
    """Owns an fpd_drafter handle and keeps the borrowed weight tensors alive."""

    def __init__(self, cfg: fpd_config, weights: Dict, keep):
        self.cfg = cfg
        self._keep = keep
        self._layers = (fpd_layer_weights * cfg.n_layers)()
        for i, lw in enumerate(weights["layers"]):
            for k in ("g_attn", "w_qkv", "w_o", "g_mlp", "w_gu", "w_d"):
                setattr(self._layers[i], k, _ptr(lw[k], k, TORCH_DT[cfg.dtype]))
        w = fpd_weights()
        for k in ("w_fc", "g_fc", "embed", "w_lm", "g_final"):
            setattr(w, k, _ptr(weights[k], k, TORCH_DT[cfg.dtype]))
        w.layers = self._layers
        h = vp()
        _check(_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)), "fpd_drafter_create")
        self.handle = h

    @property
    def dtype(self) -> torch.dtype:
        return TORCH_DT[self.cfg.dtype]

    @property
    def value_dtype(self) -> torch.dtype:
        """dtype of the context values ctx_v: float16 for bf16 drafters."""
        return torch.float16 if self.dtype == torch.bfloat16 else self.dtype

    def close(self) -> None:
        if getattr(self, "handle", None):
            _destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


class Layout:
    def __init__(self, handle, L: int, drafter: Drafter):
        self.handle = handle
        self.L = L
        self.drafter = drafter

    def close(self) -> None:
        if getattr(self, "handle", None):
            _lay_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


def make_config(shape) -> fpd_config:
    """fpd_config from any object with the drafter-shape attributes."""
    return fpd_config(shape.hidden, shape.n_q, shape.n_kv, shape.head_dim, shape.n_layers, shape.inter,
                      shape.vocab, shape.n_fused, FPD_DTYPE_BF16 if shape.dtype == "bf16" else FPD_DTYPE_F32,
                      int(shape.use_rope), float(shape.rope_theta), float(shape.rms_eps))


def fpd_drafter_create(cfg: fpd_config, weights: Dict) -> Drafter:
    """weights: dict of device tensors w_fc, g_fc, embed, w_lm, g_final and
    layers (list of dicts g_attn, w_qkv, w_o, g_mlp, w_gu, w_d)."""
    return Drafter(cfg, weights, weights)


def fpd_drafter_destroy(d: Drafter) -> None:
    d.close()


def fpd_drafter_prepare(d: Drafter, stream=None) -> None:
    """Register-tile copies of the bf16 projections (no-op for f32)."""
    _check(_prepare(d.handle, _stream(stream)), "fpd_drafter_prepare")


def _schema_struct(schema: Dict):
    s = fpd_schema()
    s.kind = SCHEMA_KINDS[schema["kind"]]
    s.n_points = int(schema.get("n_points", 0))
    s.block_len = int(schema.get("block_len", 0))
    for k in ("start_id", "mask_id", "delim_id", "off_id", "plus_id", "minus_id", "digit0_id", "fill_id",
              "coord_base", "coord_count"):
        setattr(s, k, int(schema.get(k, -1)))
    keep = []

    def arr(a):
        x = np.ascontiguousarray(np.asarray(a, np.int32).reshape(-1))
        keep.append(x)
        return x.ctypes.data_as(P_i32)

    if schema["kind"] == "custom":
        sets = schema.get("sets", [])
        offs = np.zeros(len(sets) + 1, np.int32)
        for i, st in enumerate(sets):
            offs[i + 1] = offs[i] + len(st)
        s.n_sets = len(sets)
        s.set_offsets = arr(offs)
        s.set_ids = arr(np.concatenate([np.asarray(x, np.int32) for x in sets]) if sets else np.zeros(1, np.int32))
        s.pos_set = arr(schema["pos_set"])
        pairs = np.asarray(schema.get("pairs", []), np.int32).reshape(-1)
        fields = np.asarray(schema.get("fields", []), np.int32).reshape(-1)
        s.n_pairs = pairs.size // 2
        s.pairs = arr(pairs if pairs.size else np.zeros(1, np.int32))
        s.n_fields = fields.size // 2
        s.fields = arr(fields if fields.size else np.zeros(1, np.int32))
    return s, keep


def _tables(fn, first_arg, sizes: fpd_layout_sizes) -> Dict[str, np.ndarray]:
    out = dict(pos_set=np.zeros(sizes.L, np.int32), set_offsets=np.zeros(sizes.n_sets + 1, np.int32),
               set_ids=np.zeros(max(1, sizes.n_set_ids), np.int32), pairs=np.zeros(max(1, 2 * sizes.n_pairs), np.int32),
               fields=np.zeros(max(1, 2 * sizes.n_fields), np.int32))
    p = lambda a: a.ctypes.data_as(P_i32)
    st = fn(*first_arg, ctypes.byref(sizes), p(out["pos_set"]), p(out["set_offsets"]), p(out["set_ids"]),
            p(out["pairs"]), p(out["fields"]))
    _check(st, fn.__name__)
    out["set_ids"] = out["set_ids"][:sizes.n_set_ids]
    out["pairs"] = out["pairs"][:2 * sizes.n_pairs].reshape(-1, 2)
    out["fields"] = out["fields"][:2 * sizes.n_fields].reshape(-1, 2)
    out["L"] = sizes.L
    out["width"] = sizes.width
    return out


def fpd_schema_expand(schema: Dict, vocab: int) -> Dict[str, np.ndarray]:
    """Host-only schema expansion (no GPU)."""
    s, keep = _schema_struct(schema)
    sizes = fpd_layout_sizes()
    _check(_expand(ctypes.byref(s), vocab, ctypes.byref(sizes), None, None, None, None, None), "fpd_schema_expand")
    return _tables(_expand, (ctypes.byref(s), vocab), sizes)


def fpd_layout_create(d: Drafter, schema: Dict) -> Layout:
    s, keep = _schema_struct(schema)
    h = vp()
    L = i32()
    _check(_lay_create(d.handle, ctypes.byref(s), ctypes.byref(h), ctypes.byref(L)), "fpd_layout_create")
    return Layout(h, L.value, d)


def fpd_layout_destroy(lay: Layout) -> None:
    lay.close()


def fpd_layout_masks(lay: Layout) -> Dict[str, np.ndarray]:
    sizes = fpd_layout_sizes()
    _check(_lay_masks(lay.handle, ctypes.byref(sizes), None, None, None, None, None), "fpd_layout_masks")
    return _tables(_lay_masks, (lay.handle,), sizes)


def fpd_workspace_size(d: Drafter, B: int, C: int, L: int) -> int:
    n = ctypes.c_size_t()
    _check(_ws_size(d.handle, B, C, L, ctypes.byref(n)), "fpd_workspace_size")
    return n.value


def alloc_workspace(d: Drafter, B: int, C: int, L: int, device=None) -> torch.Tensor:
    return torch.empty(max(1, fpd_workspace_size(d, B, C, L)), dtype=torch.uint8, device=device or "cuda")


def alloc_context(d: Drafter, B: int, cap: int, device=None):
    """ctx_k [n_layers, B, n_kv, cap, d] (drafter dtype) and ctx_v
    [n_layers, B, n_kv, d, cap] (float16 for bf16 drafters: the bf16-rounded
    values held exactly; float32 for f32 drafters)."""
    c = d.cfg
    dev = device or "cuda"
    vdt = d.value_dtype
    return (torch.empty(c.n_layers, B, c.n_kv, cap, c.head_dim, dtype=d.dtype, device=dev),
            torch.empty(c.n_layers, B, c.n_kv, c.head_dim, cap, dtype=vdt, device=dev))


# ---- hot path ------------------------------------------------------------------

def fpd_fuse_context_kv(d: Drafter, feats: torch.Tensor, ctx_k: torch.Tensor, ctx_v: torch.Tensor,
                        ws: torch.Tensor, pos0: int = 0, stream=None) -> None:
    B, nt, C, H = feats.shape
    cap = ctx_k.shape[3]
    _check(_fuse(d.handle, _ptr(feats, "feats", d.dtype), B, C, pos0, _ptr(ctx_k, "ctx_k", d.dtype),
                 _ptr(ctx_v, "ctx_v", d.value_dtype), cap, _ptr(ws, "ws"), ws.numel(), _stream(stream)),
           "fpd_fuse_context_kv")


def fpd_append_context_kv(d: Drafter, feats: torch.Tensor, ctx_k: torch.Tensor, ctx_v: torch.Tensor,
                          ws: torch.Tensor, pos0: int, stream=None) -> None:
    """feats [B, n_fused, C_new, H]: features of target positions pos0.. ."""
    B, nt, C_new, H = feats.shape
    cap = ctx_k.shape[3]
    _check(_append(d.handle, _ptr(feats, "feats", d.dtype), B, C_new, pos0, _ptr(ctx_k, "ctx_k", d.dtype),
                   _ptr(ctx_v, "ctx_v", d.value_dtype), cap, _ptr(ws, "ws"), ws.numel(), _stream(stream)),
           "fpd_append_context_kv")


def fpd_draft_block(d: Drafter, tokens: torch.Tensor, ctx_k: Optional[torch.Tensor],
                    ctx_v: Optional[torch.Tensor], C: int, hidden_out: torch.Tensor, ws: torch.Tensor,
                    block_pos: Optional[int] = None, stream=None) -> None:
    B, L = tokens.shape
    cap = ctx_k.shape[3] if ctx_k is not None else 0
    _check(_draft(d.handle, _ptr(tokens, "tokens", torch.int32), B, L, _ptr(ctx_k, "ctx_k", d.dtype),
                  _ptr(ctx_v, "ctx_v", d.value_dtype), C, cap, C if block_pos is None else block_pos,
                  _ptr(hidden_out, "hidden_out", d.dtype), _ptr(ws, "ws"), ws.numel(), _stream(stream)),
           "fpd_draft_block")



def fpd_draft_block_noalloc(d: Drafter, tokens: torch.Tensor, ctx_k: Optional[torch.Tensor],
                            ctx_v: Optional[torch.Tensor], C: int, hidden_out: torch.Tensor,
                            block_pos: Optional[int] = None, stream=None) -> None:
    """fpd_draft_block on the library's static scratch (no workspace)."""
    B, L = tokens.shape
    cap = ctx_k.shape[3] if ctx_k is not None else 0
    _check(_draft_noalloc(d.handle, _ptr(tokens, "tokens", torch.int32), B, L, _ptr(ctx_k, "ctx_k", d.dtype),
                          _ptr(ctx_v, "ctx_v", d.value_dtype), C, cap, C if block_pos is None else block_pos,
                          _ptr(hidden_out, "hidden_out", d.dtype), _stream(stream)),
           "fpd_draft_block_noalloc")


def fpd_draft_blocks_shared_ctx(d: Drafter, tokens: torch.Tensor, ctx_k: torch.Tensor, ctx_v: torch.Tensor,
                                C: int, hidden_out: torch.Tensor, ws: torch.Tensor,
                                block_pos: Optional[int] = None, stream=None) -> None:
    """tokens [B, L]; ctx_k / ctx_v hold one context (their batch axis is 1)."""
    B, L = tokens.shape
    cap = ctx_k.shape[3]
    _check(_draft_shared(d.handle, _ptr(tokens, "tokens", torch.int32), B, L, _ptr(ctx_k, "ctx_k", d.dtype),
                         _ptr(ctx_v, "ctx_v", d.value_dtype), C, cap, C if block_pos is None else block_pos,
                         _ptr(hidden_out, "hidden_out", d.dtype), _ptr(ws, "ws"), ws.numel(), _stream(stream)),
           "fpd_draft_blocks_shared_ctx")

def fpd_constrained_argmax(d: Drafter, lay: Layout, hidden: torch.Tensor, tokens_out: torch.Tensor,
                           ws: torch.Tensor, logits_out: Optional[torch.Tensor] = None, stream=None) -> None:
    B = hidden.shape[0]
    _check(_argmax(d.handle, lay.handle, _ptr(hidden, "hidden", d.dtype), B,
                   _ptr(tokens_out, "tokens_out", torch.int32), _ptr(logits_out, "logits_out", torch.float32),
                   _ptr(ws, "ws"), ws.numel(), _stream(stream)), "fpd_constrained_argmax")


def fpd_validate_primitive(lay: Layout, tokens: torch.Tensor, k_out: torch.Tensor, first_invalid_out: torch.Tensor,
                           stream=None) -> None:
    B = tokens.shape[0]
    _check(_validate(lay.handle, _ptr(tokens, "tokens", torch.int32), B, _ptr(k_out, "k_out", torch.int32),
                     _ptr(first_invalid_out, "first_invalid_out", torch.int32), _stream(stream)),
           "fpd_validate_primitive")


def fpd_accept_boxes(lay: Layout, tokens: torch.Tensor, conf: torch.Tensor, tau: float, k_out: torch.Tensor,
                     first_invalid_out: torch.Tensor, first_uncertain_out: torch.Tensor, stream=None) -> None:
    B = tokens.shape[0]
    if conf.shape != tokens.shape:
        raise ValueError(f"conf must have the shape of tokens {tuple(tokens.shape)}, got {tuple(conf.shape)}")
    _check(_boxes(lay.handle, _ptr(tokens, "tokens", torch.int32), _ptr(conf, "conf", torch.float32), tau, B,
                  _ptr(k_out, "k_out", torch.int32), _ptr(first_invalid_out, "first_invalid_out", torch.int32),
                  _ptr(first_uncertain_out, "first_uncertain_out", torch.int32), _stream(stream)),
           "fpd_accept_boxes")


def fpd_verify_prefix(draft: torch.Tensor, target: torch.Tensor, k_out: torch.Tensor, next_out: torch.Tensor,
                      stream=None) -> None:
    B, L = target.shape
    _check(_verify(_ptr(draft, "draft", torch.int32), _ptr(target, "target", torch.int32), B, L,
                   _ptr(k_out, "k_out", torch.int32), _ptr(next_out, "next_out", torch.int32), _stream(stream)),
           "fpd_verify_prefix")


# ---- coordinate codec ---------------------------------------------------------------

def fpd_coords_to_tokens(values: torch.Tensor, tokens_out: torch.Tensor, coord_base: int, lo: float = 0.0,
                         hi: float = 1000.0, stream=None) -> None:
    n = values.numel()
    _check(_c2t(_ptr(values, "values", torch.float32), n, lo, hi, coord_base,
                _ptr(tokens_out, "tokens_out", torch.int32), _stream(stream)), "fpd_coords_to_tokens")


def fpd_tokens_to_coords(tokens: torch.Tensor, values_out: torch.Tensor, coord_base: int, lo: float = 0.0,
                         hi: float = 1000.0, stream=None) -> None:
    n = tokens.numel()
    _check(_t2c(_ptr(tokens, "tokens", torch.int32), n, lo, hi, coord_base,
                _ptr(values_out, "values_out", torch.float64), _stream(stream)), "fpd_tokens_to_coords")


def fpd_ints_to_fields(values: torch.Tensor, fields_out: torch.Tensor, plus_id: int, minus_id: int,
                       digit0_id: int, fill_id: int, stream=None) -> None:
    n = values.numel()
    _check(_i2f(_ptr(values, "values", torch.int32), n, plus_id, minus_id, digit0_id, fill_id,
                _ptr(fields_out, "fields_out", torch.int32), _stream(stream)), "fpd_ints_to_fields")


def fpd_fields_to_ints(fields: torch.Tensor, values_out: torch.Tensor, valid_out: torch.Tensor, plus_id: int,
                       minus_id: int, digit0_id: int, fill_id: int, stream=None) -> None:
    n = fields.numel() // 6
    _check(_f2i(_ptr(fields, "fields", torch.int32), n, plus_id, minus_id, digit0_id, fill_id,
                _ptr(values_out, "values_out", torch.int32), _ptr(valid_out, "valid_out", torch.int32),
                _stream(stream)), "fpd_fields_to_ints")


# ---- device upload of host arrays -------------------------------------------------

def to_device(x: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """Upload a float32 host array holding values exact in `dtype`."""
    if dtype == torch.bfloat16:
        bits = (np.ascontiguousarray(x, np.float32).reshape(-1).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16).reshape(x.shape)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device).to(dtype)


def weights_to_device(w, dtype: torch.dtype, device="cuda") -> Dict:
    """Device copies of a weight container with attributes w_fc, g_fc, embed,
    w_lm, g_final, layers."""
    up = lambda a: to_device(a, dtype, device)
    return dict(w_fc=up(w.w_fc), g_fc=up(w.g_fc), embed=up(w.embed), w_lm=up(w.w_lm), g_final=up(w.g_final),
                layers=[{k: up(v) for k, v in lw.items()} for lw in w.layers])


# ---- per-launch timing (diagnostics) ------------------------------------------------
_prof_enable = _proto("fpd_profile_enable", [i32])
_prof_count = _proto("fpd_profile_count", [P_i32])
_prof_read = _proto("fpd_profile_read", [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)])


def fpd_profile_enable(on: bool) -> None:
    _check(_prof_enable(1 if on else 0), "fpd_profile_enable")


def fpd_profile_records():
    """[(tag, ms)] of the recorded launches; call after synchronising."""
    n = i32()
    _check(_prof_count(ctypes.byref(n)), "fpd_profile_count")
    out = []
    for i in range(n.value):
        tag = ctypes.c_char_p()
        ms = ctypes.c_float()
        _check(_prof_read(i, ctypes.byref(tag), ctypes.byref(ms)), "fpd_profile_read")
        out.append((tag.value.decode(), ms.value))
    return out
