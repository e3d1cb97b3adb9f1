"""Thin Python binding of libivc.so (include/ivc.h), argument marshalling only.

Every function here has the name of the C entry point it calls and takes the
same arguments; torch tensors are passed as their device pointers and
``stream`` defaults to torch's current stream.  All computation happens in
the HIP kernels behind the C ABI: if the library is missing, importing this
module's functions raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

# IVC_LIBRARY may name another build of the same library (the host-sanitized
# debug build the CPU tests load); the default is the in-tree libivc.so
LIB_PATH = os.environ.get("IVC_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libivc.so")

IVC_OK = 0
IVC_F32, IVC_BF16 = 0, 1
IVC_POOL_KV, IVC_POOL_FOLDED = 0, 1
SHUFFLE64_ORDERS = ("direct", "twice_r2")  # ivc_shuffle64_order values 0, 1
IVC_DEV_OK = 0
IVC_DEV_ERR_IMG_COUNT = 1
IVC_DEV_ERR_VALID_TOKENS = 2
IVC_DEV_ERR_TILE_COUNT = 4
IVC_DEV_ERR_SEQ_LAYOUT = 8
MAX_POOL_LAYERS = 8
GATE_BLOCKS = 4


class IvcError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class ivc_config(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("vit_width", c_int32), ("grid", c_int32), ("has_cls", c_int32),
        ("llm_width", c_int32), ("mlp1_hidden", c_int32), ("flash", c_int32),
        ("mlp2_hidden", c_int32), ("pool_layers", c_int32), ("pool_heads", c_int32),
        ("gate_hidden", c_int32), ("gate_expansion", c_int32), ("pool_mode", c_int32),
        ("ps_version", c_int32), ("shuffle64_order", c_int32), ("ln_fold", c_int32),
        ("rel_quantile", c_double), ("abs_threshold", c_double),
        ("ln_eps", c_float),
    ]


_VP8 = c_void_p * MAX_POOL_LAYERS
_VP4 = c_void_p * GATE_BLOCKS


class ivc_weights(ctypes.Structure):
    _fields_ = [
        ("mlp1_ln_w", c_void_p), ("mlp1_ln_b", c_void_p), ("mlp1_w1", c_void_p),
        ("mlp1_b1", c_void_p), ("mlp1_w2", c_void_p), ("mlp1_b2", c_void_p),
        ("mlp2_ln_w", c_void_p), ("mlp2_ln_b", c_void_p), ("mlp2_w1", c_void_p),
        ("mlp2_b1", c_void_p), ("mlp2_w2", c_void_p), ("mlp2_b2", c_void_p),
        ("mlp2_w3", c_void_p), ("mlp2_b3", c_void_p),
        ("pool_query", c_void_p),
        ("pool_wq", _VP8), ("pool_bq", _VP8), ("pool_wk", _VP8), ("pool_bk", _VP8),
        ("pool_wv", _VP8), ("pool_bv", _VP8), ("pool_wo", _VP8), ("pool_bo", _VP8),
        ("gate_w1", _VP4), ("gate_b1", _VP4), ("gate_w2", _VP4), ("gate_b2", _VP4),
        ("gate_ln_w", _VP4), ("gate_ln_b", _VP4),
        ("gate_cls_w", c_void_p), ("gate_cls_b", c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libivc.so (built in-tree by vlm_visual_token_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m vlm_visual_token_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    sig = {
        "ivc_connector_create": (c_int32, [POINTER(ivc_config), POINTER(ivc_weights), P, POINTER(P)]),
        "ivc_connector_destroy": (None, [P]),
        "ivc_connector_workspace_bytes": (c_size_t, [P, c_int32, c_int64]),
        "ivc_connector_run": (c_int32, [P, P, c_int32, P, P, P, c_size_t, P]),
        "ivc_connector_run_routed": (c_int32, [P, P, c_int32, P, P, P, P, c_size_t, P]),
        "ivc_connector_route": (c_int32, [P, P, P, c_int32, P, P, P, P, P, P, c_size_t, P]),
        "ivc_connector_forward": (c_int32, [P, P, P, c_int32, P, P, P, P, P, P, P, P, c_size_t, P]),
        "ivc_connector_compact": (c_int32, [P, P, P, c_int64, c_int32, P, P, P, c_int32, P, P, P,
                                            P, P, P, P, c_size_t, P]),
        "ivc_connector_forward_compact": (c_int32, [P, P, P, c_int32, P, P, P, P, P, P, P, P, P,
                                                    c_int64, c_int32, P, P, P, P, P, P, c_size_t,
                                                    P]),
        "ivc_connector_forward_compact_workspace_bytes": (c_size_t, [P, c_int32, c_int64]),
        "ivc_connector_compact_noalloc": (c_int32, [P, P, P, c_int64, c_int32, P, P, P, c_int32, P,
                                                    P, P, P, P, P, P]),
        "ivc_connector_compact_batch": (c_int32, [P, P, P, c_int32, P, c_int64, c_int32, P, P, P,
                                                  P, c_int32, P, P, P, P, P, P, P, c_size_t, P]),
        "ivc_connector_compact_batch_workspace_bytes": (c_size_t, [P, c_int32, c_int64, c_int32]),
        "ivc_route_decide": (c_int32, [P, c_int32, c_double, c_double, P, P, P]),
        "ivc_tile_offsets": (c_int32, [P, c_int32, P, P, P]),
        "ivc_pixel_shuffle": (c_int32, [c_int32, P, c_int32, c_int32, c_int32, c_int32, c_int32,
                                        c_int32, c_int32, P, P]),
        "ivc_profile_enable": (None, [c_int32]),
        "ivc_profile_reset": (None, []),
        "ivc_profile_read": (c_int32, [POINTER(c_char_p), POINTER(c_double), POINTER(c_int64), c_int32]),
        "ivc_status_string": (c_char_p, [c_int32]),
        "ivc_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> list[str]:
    return [
        "ivc_connector_create", "ivc_connector_destroy", "ivc_connector_workspace_bytes",
        "ivc_connector_run", "ivc_connector_run_routed", "ivc_connector_route", "ivc_connector_forward",
        "ivc_connector_compact", "ivc_connector_compact_noalloc",
        "ivc_connector_forward_compact", "ivc_connector_forward_compact_workspace_bytes",
        "ivc_connector_compact_batch", "ivc_connector_compact_batch_workspace_bytes", "ivc_route_decide",
        "ivc_tile_offsets",
        "ivc_pixel_shuffle", "ivc_profile_enable", "ivc_profile_reset", "ivc_profile_read",
        "ivc_status_string", "ivc_last_error",
    ]


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"expected a tensor, int or None, got {type(x)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(st: int, where: str):
    if st != IVC_OK:
        lib = load()
        raise IvcError(st, where, lib.ivc_last_error().decode())


# ---------------------------------------------------------------------------
# config and weight tables
# ---------------------------------------------------------------------------
def make_config(cfg: dict) -> ivc_config:
    """ivc_config from a workload dict (keys as in the synthetic workloads)."""
    c = ivc_config()
    c.dtype = IVC_BF16 if cfg["dtype"] == "bf16" else IVC_F32
    c.vit_width = cfg["C"]
    c.grid = cfg["P"]
    c.has_cls = cfg["has_cls"]
    c.llm_width = cfg["D"]
    c.mlp1_hidden = cfg["mlp1_hidden"]
    c.flash = cfg["flash"]
    c.mlp2_hidden = cfg["mlp2_hidden"]
    c.pool_layers = cfg["pool_layers"]
    c.pool_heads = cfg["pool_heads"]
    c.gate_hidden = cfg["gate_hidden"]
    c.gate_expansion = cfg["gate_expansion"]
    c.pool_mode = cfg.get("pool_mode", IVC_POOL_KV)
    c.ps_version = cfg.get("ps_version", 2)
    c.shuffle64_order = SHUFFLE64_ORDERS.index(cfg.get("shuffle64_order", "direct"))
    c.ln_fold = int(cfg.get("ln_fold", 0))
    c.rel_quantile = cfg["rel_quantile"]
    c.abs_threshold = cfg["abs_threshold"]
    c.ln_eps = cfg["ln_eps"]
    return c


def make_weights(cfg: dict, w: dict) -> ivc_weights:
    """ivc_weights from named device tensors ("mlp1.ln.w", "pool.0.q.w", ...)."""
    t = ivc_weights()
    p = lambda k: _ptr(w[k])  # noqa: E731
    t.mlp1_ln_w, t.mlp1_ln_b = p("mlp1.ln.w"), p("mlp1.ln.b")
    t.mlp1_w1, t.mlp1_b1 = p("mlp1.l1.w"), p("mlp1.l1.b")
    t.mlp1_w2, t.mlp1_b2 = p("mlp1.l2.w"), p("mlp1.l2.b")
    if cfg["flash"]:
        t.mlp2_ln_w, t.mlp2_ln_b = p("mlp2.ln.w"), p("mlp2.ln.b")
        t.mlp2_w1, t.mlp2_b1 = p("mlp2.l1.w"), p("mlp2.l1.b")
        t.mlp2_w2, t.mlp2_b2 = p("mlp2.l2.w"), p("mlp2.l2.b")
        t.mlp2_w3, t.mlp2_b3 = p("mlp2.l3.w"), p("mlp2.l3.b")
        t.pool_query = p("pool.query")
        for l in range(cfg["pool_layers"]):
            t.pool_wq[l], t.pool_bq[l] = p(f"pool.{l}.q.w"), p(f"pool.{l}.q.b")
            t.pool_wk[l], t.pool_bk[l] = p(f"pool.{l}.k.w"), p(f"pool.{l}.k.b")
            t.pool_wv[l], t.pool_bv[l] = p(f"pool.{l}.v.w"), p(f"pool.{l}.v.b")
            t.pool_wo[l], t.pool_bo[l] = p(f"pool.{l}.o.w"), p(f"pool.{l}.o.b")
        for b in range(GATE_BLOCKS):
            t.gate_w1[b], t.gate_b1[b] = p(f"gate.{b}.l1.w"), p(f"gate.{b}.l1.b")
            t.gate_w2[b], t.gate_b2[b] = p(f"gate.{b}.l2.w"), p(f"gate.{b}.l2.b")
            t.gate_ln_w[b], t.gate_ln_b[b] = p(f"gate.{b}.ln.w"), p(f"gate.{b}.ln.b")
        t.gate_cls_w, t.gate_cls_b = p("gate.cls.w"), p("gate.cls.b")
    return t


# ---------------------------------------------------------------------------
# entry points (same names and argument order as include/ivc.h)
# ---------------------------------------------------------------------------
def ivc_connector_create(cfg: ivc_config, weights: ivc_weights, stream=None) -> int:
    lib = load()
    h = c_void_p()
    _check(lib.ivc_connector_create(ctypes.byref(cfg), ctypes.byref(weights), _stream(stream),
                                    ctypes.byref(h)), "ivc_connector_create")
    return h.value


def ivc_connector_destroy(h: int) -> None:
    load().ivc_connector_destroy(h)


def ivc_connector_workspace_bytes(h: int, max_tiles: int, max_seq_len: int) -> int:
    return int(load().ivc_connector_workspace_bytes(h, max_tiles, max_seq_len))


def ivc_connector_run(h, vit, T, out256, out64, ws, ws_bytes, stream=None) -> None:
    _check(load().ivc_connector_run(h, _ptr(vit), T, _ptr(out256), _ptr(out64), _ptr(ws),
                                    ws_bytes, _stream(stream)), "ivc_connector_run")


def ivc_connector_run_routed(h, vit, T, use64, out256, out64, ws, ws_bytes, stream=None) -> None:
    _check(load().ivc_connector_run_routed(h, _ptr(vit), T, _ptr(use64), _ptr(out256), _ptr(out64),
                                           _ptr(ws), ws_bytes, _stream(stream)),
           "ivc_connector_run_routed")


def ivc_connector_route(h, vit, valid_tokens, T, gate, threshold, use64, pooled, dev_status, ws,
                        ws_bytes, stream=None) -> None:
    _check(load().ivc_connector_route(h, _ptr(vit), _ptr(valid_tokens), T, _ptr(gate),
                                      _ptr(threshold), _ptr(use64), _ptr(pooled),
                                      _ptr(dev_status), _ptr(ws), ws_bytes, _stream(stream)),
           "ivc_connector_route")


def ivc_connector_forward(h, vit, valid_tokens, T, gate, threshold, use64, pooled, dev_status,
                          out256, out64, ws, ws_bytes, stream=None) -> None:
    _check(load().ivc_connector_forward(h, _ptr(vit), _ptr(valid_tokens), T, _ptr(gate),
                                        _ptr(threshold), _ptr(use64), _ptr(pooled),
                                        _ptr(dev_status), _ptr(out256), _ptr(out64), _ptr(ws),
                                        ws_bytes, _stream(stream)), "ivc_connector_forward")


def ivc_connector_compact(h, ids, embeds, L, img_context_id, use64, out256, out64, T, out_ids,
                          out_pos, keep_map, out_embeds, out_len, dev_status, ws, ws_bytes,
                          stream=None) -> None:
    _check(load().ivc_connector_compact(h, _ptr(ids), _ptr(embeds), L, img_context_id,
                                        _ptr(use64), _ptr(out256), _ptr(out64), T, _ptr(out_ids),
                                        _ptr(out_pos), _ptr(keep_map), _ptr(out_embeds),
                                        _ptr(out_len), _ptr(dev_status), _ptr(ws), ws_bytes,
                                        _stream(stream)), "ivc_connector_compact")


def ivc_connector_forward_compact_workspace_bytes(h, max_tiles, max_seq_len) -> int:
    return int(load().ivc_connector_forward_compact_workspace_bytes(h, max_tiles, max_seq_len))


def ivc_connector_forward_compact(h, vit, valid_tokens, T, gate, threshold, use64, pooled,
                                  dev_status, out256, out64, ids, embeds, L, img_context_id,
                                  out_ids, out_pos, keep_map, out_embeds, out_len, ws, ws_bytes,
                                  stream=None) -> None:
    _check(load().ivc_connector_forward_compact(
        h, _ptr(vit), _ptr(valid_tokens), T, _ptr(gate), _ptr(threshold), _ptr(use64),
        _ptr(pooled), _ptr(dev_status), _ptr(out256), _ptr(out64), _ptr(ids), _ptr(embeds), L,
        img_context_id, _ptr(out_ids), _ptr(out_pos), _ptr(keep_map), _ptr(out_embeds),
        _ptr(out_len), _ptr(ws), ws_bytes, _stream(stream)), "ivc_connector_forward_compact")


def ivc_connector_compact_noalloc(h, ids, embeds, L, img_context_id, use64, out256, out64, T,
                                  out_ids, out_pos, keep_map, out_embeds, out_len, dev_status,
                                  stream=None) -> None:
    _check(load().ivc_connector_compact_noalloc(h, _ptr(ids), _ptr(embeds), L, img_context_id,
                                                _ptr(use64), _ptr(out256), _ptr(out64), T,
                                                _ptr(out_ids), _ptr(out_pos), _ptr(keep_map),
                                                _ptr(out_embeds), _ptr(out_len), _ptr(dev_status),
                                                _stream(stream)), "ivc_connector_compact_noalloc")


def ivc_connector_compact_batch(h, ids, cu_seqlens, B, embeds, L, img_context_id, tile_offsets,
                                use64, out256, out64, T, out_ids, out_pos, keep_map, out_embeds,
                                out_cu_seqlens, dev_status, ws, ws_bytes, stream=None) -> None:
    _check(load().ivc_connector_compact_batch(
        h, _ptr(ids), _ptr(cu_seqlens), B, _ptr(embeds), L, img_context_id, _ptr(tile_offsets),
        _ptr(use64), _ptr(out256), _ptr(out64), T, _ptr(out_ids), _ptr(out_pos), _ptr(keep_map),
        _ptr(out_embeds), _ptr(out_cu_seqlens), _ptr(dev_status), _ptr(ws), ws_bytes,
        _stream(stream)), "ivc_connector_compact_batch")


def ivc_connector_compact_batch_workspace_bytes(h, max_tiles: int, max_total_len: int,
                                                max_seqs: int) -> int:
    return load().ivc_connector_compact_batch_workspace_bytes(h, max_tiles, max_total_len,
                                                              max_seqs)


def ivc_route_decide(gate, T, rel_quantile, abs_threshold, threshold, use64, stream=None) -> None:
    _check(load().ivc_route_decide(_ptr(gate), T, rel_quantile, abs_threshold, _ptr(threshold),
                                   _ptr(use64), _stream(stream)), "ivc_route_decide")


def ivc_tile_offsets(tiles_per_image, B, offsets, dev_status, stream=None) -> None:
    _check(load().ivc_tile_offsets(_ptr(tiles_per_image), B, _ptr(offsets), _ptr(dev_status),
                                   _stream(stream)), "ivc_tile_offsets")


def ivc_pixel_shuffle(dtype, vit, T, P, C, has_cls, r, out, stream=None, ps_version=2,
                      shuffle64_order=0) -> None:
    _check(load().ivc_pixel_shuffle(dtype, _ptr(vit), T, P, C, has_cls, r, ps_version,
                                    shuffle64_order, _ptr(out),
                                    _stream(stream)), "ivc_pixel_shuffle")


def ivc_profile_enable(on) -> None:
    """False/0: off; True/1: per-kernel events, projector chains on one stream;
    2: per-kernel events, chains on their two streams."""
    load().ivc_profile_enable(int(on))


def ivc_profile_reset() -> None:
    load().ivc_profile_reset()


def ivc_profile_read(cap: int = 64) -> dict:
    """{kernel name: (total ms, launches)} of the kernels timed since the last reset."""
    lib = load()
    names = (c_char_p * cap)()
    ms = (c_double * cap)()
    n = (c_int64 * cap)()
    k = lib.ivc_profile_read(names, ms, n, cap)
    return {names[i].decode(): (ms[i], int(n[i])) for i in range(min(k, cap))}


def ivc_status_string(s: int) -> str:
    return load().ivc_status_string(s).decode()


def ivc_last_error() -> str:
    return load().ivc_last_error().decode()
