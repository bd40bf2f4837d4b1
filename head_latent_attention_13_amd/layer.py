"""Device buffers of one MLA layer, driven through the C ABI.

``MLALayer`` owns the absorbed weights and the workspace (torch tensors on
the GPU) and forwards each step to the library; it does no arithmetic.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _lib as L


class MLALayer:
    def __init__(self, dims: L.mla_dims, raw: Dict[str, torch.Tensor], max_batch: int, max_nq: int = 1,
                 device: str = "cuda", stream=None):
        self.dims = dims
        self.device = device
        _, _, total = L.mla_absorbed_layout(dims)
        self.absorbed = torch.empty(total, dtype=torch.uint8, device=device)
        L.mla_absorb_weights(dims, raw, self.absorbed, stream)
        self.ws_bytes = L.mla_workspace_size(dims, max_batch, max_nq)
        # zero once: the first 256 bytes hold the sticky device error word
        self.workspace = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)

    @property
    def act_dtype(self):
        return torch.bfloat16 if self.dims.dtype == L.MLA_BF16 else torch.float32

    def append(self, x: torch.Tensor, pos: torch.Tensor, batch: int, n_q: int, cache: L.Cache, stream=None):
        L.mla_compress_append(self.dims, self.absorbed, x, pos, batch, n_q, cache, self.workspace, stream)

    def store_rows(self, rows, pos, batch, n_q, cache: L.Cache, stream=None):
        L.mla_cache_store_rows(self.dims, rows, pos, batch, n_q, cache, self.workspace, stream)

    def q_proj(self, x, kv_len, batch, n_q, q, stream=None):
        L.mla_q_proj(self.dims, self.absorbed, x, kv_len, batch, n_q, q, self.workspace, stream)

    def attention(self, q, kv_len, batch, n_q, cache: L.Cache, o_lat, lse: Optional[torch.Tensor] = None,
                  stream=None):
        L.mla_attention(self.dims, q, kv_len, batch, n_q, cache, o_lat, lse, self.workspace, stream)

    def decode(self, x, kv_len, batch, n_q, cache: L.Cache, o_lat, lse: Optional[torch.Tensor] = None,
               stream=None):
        L.mla_decode(self.dims, self.absorbed, x, kv_len, batch, n_q, cache, o_lat, lse, self.workspace, stream)

    def out_proj(self, o_lat, n_tok, y, stream=None):
        L.mla_out_proj(self.dims, self.absorbed, o_lat, n_tok, y, self.workspace, stream)

    def prefill_expanded(self, x, kv_len, batch, n_q, cache: L.Cache, y, lse: Optional[torch.Tensor] = None,
                         stream=None):
        """Expanded-form chunked prefill (factored weights, contiguous cache);
        its workspace, sized for (batch, n_q, cache.s_max), is kept until a
        larger one is needed."""
        need = L.mla_prefill_workspace_size(self.dims, batch, n_q, cache.s_max)
        if getattr(self, "pf_workspace", None) is None or self.pf_workspace.numel() < need:
            self.pf_workspace = torch.zeros(need, dtype=torch.uint8, device=self.device)
        L.mla_prefill_expanded(self.dims, self.absorbed, x, kv_len, batch, n_q, cache, y, lse, self.pf_workspace,
                               stream)

    def prefill_error(self, stream=None) -> int:
        ws = getattr(self, "pf_workspace", None)
        return 0 if ws is None else L.mla_read_device_error(ws, stream)

    def device_error(self, stream=None) -> int:
        return L.mla_read_device_error(self.workspace, stream)
