"""Convenience wrapper over the C ABI: owns a handle and a workspace, and
allocates output tensors with torch (device memory only; every step of the
computation runs in the library's kernels)."""
from __future__ import annotations

import torch

from . import ivc

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


class Connector:
    def __init__(self, cfg: dict, weights: dict, max_tiles: int, max_seq_len: int = 0,
                 device: str = "cuda", stream=None):
        self.cfg = cfg
        self.device = torch.device(device)
        self.dtype = _TORCH_DT[cfg["dtype"]]
        self._weights = weights  # keep the source tensors alive until create() has copied them
        self.c_cfg = ivc.make_config(cfg)
        self.c_w = ivc.make_weights(cfg, weights)
        self.h = ivc.ivc_connector_create(self.c_cfg, self.c_w, stream)
        self._weights = None
        self.ws_bytes = ivc.ivc_connector_workspace_bytes(self.h, max_tiles, max_seq_len)
        if cfg.get("flash") and max_seq_len > 0:  # room for forward_compact too
            self.ws_bytes = max(self.ws_bytes, ivc.ivc_connector_forward_compact_workspace_bytes(
                self.h, max_tiles, max_seq_len))
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.S = (cfg["P"] // 2) ** 2
        self.S64 = (cfg["P"] // 4) ** 2

    def close(self):
        if self.h:
            ivc.ivc_connector_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, vit: torch.Tensor, out256=None, out64=None, stream=None):
        T = vit.shape[0]
        D = self.cfg["D"]
        if out256 is None:
            out256 = torch.empty((T, self.S, D), dtype=self.dtype, device=self.device)
        if self.cfg["flash"] and out64 is None:
            out64 = torch.empty((T, self.S64, D), dtype=self.dtype, device=self.device)
        ivc.ivc_connector_run(self.h, vit, T, out256, out64, self.ws, self.ws_bytes, stream)
        return out256, out64

    def run_routed(self, vit: torch.Tensor, use64: torch.Tensor, out256=None, out64=None,
                   stream=None):
        T = vit.shape[0]
        D = self.cfg["D"]
        if out256 is None:
            out256 = torch.empty((T, self.S, D), dtype=self.dtype, device=self.device)
        if out64 is None:
            out64 = torch.empty((T, self.S64, D), dtype=self.dtype, device=self.device)
        ivc.ivc_connector_run_routed(self.h, vit, T, use64, out256, out64, self.ws, self.ws_bytes,
                                     stream)
        return out256, out64

    def route(self, vit: torch.Tensor, valid=None, with_pooled=True, stream=None, out=None):
        T = vit.shape[0]
        if out is None:
            out = dict(
                gate=torch.empty((T, 2), dtype=torch.float32, device=self.device),
                thr=torch.empty(1, dtype=torch.float64, device=self.device),
                use64=torch.empty(T, dtype=torch.uint8, device=self.device),
                pooled=(torch.empty((T, self.cfg["C"]), dtype=torch.float32, device=self.device)
                        if with_pooled else None),
                status=torch.zeros(1, dtype=torch.int32, device=self.device),
            )
        ivc.ivc_connector_route(self.h, vit, valid, T, out["gate"], out["thr"], out["use64"],
                                out["pooled"], out["status"], self.ws, self.ws_bytes, stream)
        return out

    def forward(self, vit: torch.Tensor, valid=None, with_pooled=True, stream=None, out=None):
        """route + route-first run in one call (ivc_connector_forward)."""
        T = vit.shape[0]
        D = self.cfg["D"]
        if out is None:
            out = dict(
                gate=torch.empty((T, 2), dtype=torch.float32, device=self.device),
                thr=torch.empty(1, dtype=torch.float64, device=self.device),
                use64=torch.empty(T, dtype=torch.uint8, device=self.device),
                pooled=(torch.empty((T, self.cfg["C"]), dtype=torch.float32, device=self.device)
                        if with_pooled else None),
                status=torch.zeros(1, dtype=torch.int32, device=self.device),
                out256=torch.empty((T, self.S, D), dtype=self.dtype, device=self.device),
                out64=torch.empty((T, self.S64, D), dtype=self.dtype, device=self.device),
            )
        ivc.ivc_connector_forward(self.h, vit, valid, T, out["gate"], out["thr"], out["use64"],
                                  out["pooled"], out["status"], out["out256"], out["out64"],
                                  self.ws, self.ws_bytes, stream)
        return out

    def forward_compact(self, vit: torch.Tensor, ids, embeds, img_context_id: int, valid=None,
                        with_pooled=True, stream=None, out=None):
        """forward + compact of its outputs in one call (ivc_connector_forward_compact):
        the forward's outputs and the compaction's (ids, pos, keep_map, embeds, len)."""
        T = vit.shape[0]
        L = ids.shape[0]
        D = self.cfg["D"]
        if out is None:
            out = dict(
                gate=torch.empty((T, 2), dtype=torch.float32, device=self.device),
                thr=torch.empty(1, dtype=torch.float64, device=self.device),
                use64=torch.empty(T, dtype=torch.uint8, device=self.device),
                pooled=(torch.empty((T, self.cfg["C"]), dtype=torch.float32, device=self.device)
                        if with_pooled else None),
                status=torch.zeros(1, dtype=torch.int32, device=self.device),
                out256=torch.empty((T, self.S, D), dtype=self.dtype, device=self.device),
                out64=torch.empty((T, self.S64, D), dtype=self.dtype, device=self.device),
                ids=torch.empty(L, dtype=torch.int32, device=self.device),
                pos=torch.empty(L, dtype=torch.int32, device=self.device),
                keep_map=torch.empty(L, dtype=torch.int32, device=self.device),
                embeds=torch.empty((L, D), dtype=self.dtype, device=self.device),
                len=torch.zeros(1, dtype=torch.int64, device=self.device),
            )
        ivc.ivc_connector_forward_compact(
            self.h, vit, valid, T, out["gate"], out["thr"], out["use64"], out["pooled"],
            out["status"], out["out256"], out["out64"], ids, embeds, L, img_context_id,
            out["ids"], out["pos"], out["keep_map"], out["embeds"], out["len"], self.ws,
            self.ws_bytes, stream)
        return out

    def compact(self, ids, embeds, use64, out256, out64, img_context_id: int, stream=None,
                out=None):
        L = ids.shape[0]
        T = use64.shape[0]
        if out is None:
            out = dict(
                ids=torch.empty(L, dtype=torch.int32, device=self.device),
                pos=torch.empty(L, dtype=torch.int32, device=self.device),
                keep_map=torch.empty(L, dtype=torch.int32, device=self.device),
                embeds=torch.empty((L, self.cfg["D"]), dtype=self.dtype, device=self.device),
                len=torch.zeros(1, dtype=torch.int64, device=self.device),
                status=torch.zeros(1, dtype=torch.int32, device=self.device),
            )
        ivc.ivc_connector_compact(self.h, ids, embeds, L, img_context_id, use64, out256, out64, T,
                                  out["ids"], out["pos"], out["keep_map"], out["embeds"],
                                  out["len"], out["status"], self.ws, self.ws_bytes, stream)
        return out

    def compact_batch(self, ids, cu_seqlens, embeds, tile_offsets, use64, out256, out64,
                      img_context_id: int, stream=None, out=None, ws=None):
        """Variable-length batch compaction (ivc_connector_compact_batch).
        ``ws`` defaults to a workspace sized for this call."""
        L = ids.shape[0]
        B = cu_seqlens.shape[0] - 1
        T = use64.shape[0]
        if out is None:
            out = dict(
                ids=torch.empty(L, dtype=torch.int32, device=self.device),
                pos=torch.empty(L, dtype=torch.int32, device=self.device),
                keep_map=torch.empty(L, dtype=torch.int32, device=self.device),
                embeds=torch.empty((L, self.cfg["D"]), dtype=self.dtype, device=self.device),
                cu=torch.zeros(B + 1, dtype=torch.int32, device=self.device),
                status=torch.zeros(1, dtype=torch.int32, device=self.device),
            )
        if ws is None:
            n = ivc.ivc_connector_compact_batch_workspace_bytes(self.h, T, L, B)
            ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        ivc.ivc_connector_compact_batch(self.h, ids, cu_seqlens, B, embeds, L, img_context_id,
                                        tile_offsets, use64, out256, out64, T, out["ids"],
                                        out["pos"], out["keep_map"], out["embeds"], out["cu"],
                                        out["status"], ws, ws.numel(), stream)
        return out
