"""Device-side setup shared by the GPU tests, smoke() and bench.py: allocate a workload's
tensors in HBM (through torch), build the RoPE table, size the workspace, and call the
C ABI. Marshalling only; all arithmetic of the path runs in liblla.so.
"""

from __future__ import annotations

import torch

from . import lla
from .inputs import Workload, decode_inputs, teacher_inputs


def dims_for(w: Workload, n_max: int | None = None, batch: int | None = None) -> lla.lla_dims:
    return lla.make_dims(w.T, w.D, w.H, w.d, w.r_k, w.r_v, batch or w.batch, n_max or w.n,
                         lla.LLA_PER_HEAD if w.variant == "per_head" else lla.LLA_2D,
                         lla.LLA_F32 if w.dtype == "f32" else lla.LLA_BF16, w.rope_base, w.scale)


class DeviceLatentStore:
    """A latent cache plus decode-side codec for one workload, resident on ``device``."""

    def __init__(self, w: Workload, seed: int, device="cuda", n_alloc: int | None = None,
                 tensors: dict | None = None, with_q: bool = True):
        self.w = w
        self.device = torch.device(device)
        self.n_max = n_alloc or w.n
        t = tensors if tensors is not None else decode_inputs(w, seed, device, self.n_max, with_q)
        self.t = {k: v.to(self.device).contiguous() for k, v in t.items()}
        self.dims = dims_for(w, self.n_max)
        tb = lla.lla_rope_table_bytes(self.dims)
        self.rope = torch.empty(tb, dtype=torch.uint8, device=self.device)
        lla.lla_rope_table_build(self.dims, self.rope)
        self.codec = lla.make_codec(self.t.get("w_down_k_t"), self.t["mu_k"], self.t["w_up_k"],
                                    self.t.get("w_down_v_t"), self.t["mu_v"], self.t["w_up_v"],
                                    self.rope)
        self.cache = lla.make_cache(self.t["c_k"], self.t["c_v"])
        self._ws = None

    def workspace(self, n_ctx: int, loop_count: int, opts=None) -> torch.Tensor:
        nb = lla.lla_decode_workspace_bytes(self.dims, n_ctx, loop_count, opts)
        if self._ws is None or self._ws.numel() < nb:
            self._ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def decode(self, layer: int, loop_begin: int, loop_count: int, q: torch.Tensor | None = None,
               n_ctx: int | None = None, ctx_lens: torch.Tensor | None = None, opts=None,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        w = self.w
        n_ctx = w.n if n_ctx is None else n_ctx
        if q is None:
            # stored per (layer, loop) as [B][H][d]; the call wants [B][H][L][d]
            if loop_count == 1:
                q = self.t["q"][layer, loop_begin]
            else:
                q = self.t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).contiguous()
        if out is None:
            out = torch.empty(w.batch, w.H, loop_count, w.d, dtype=torch.float32, device=self.device)
        ws = self.workspace(n_ctx, loop_count, opts)
        lla.lla_decode_attn(self.dims, self.codec, self.cache, layer, n_ctx, ctx_lens, q,
                            loop_begin, loop_count, out, ws, ws.numel(), opts, stream)
        return out

    def absorbed_workspace(self, n_ctx: int, loop_count: int, opts=None) -> torch.Tensor:
        nb = lla.lla_decode_absorbed_workspace_bytes(self.dims, self.w.d_rope, n_ctx, loop_count, opts)
        if self._ws is None or self._ws.numel() < nb:
            self._ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def decode_absorbed(self, layer: int, loop_begin: int, loop_count: int,
                        q: torch.Tensor | None = None, n_ctx: int | None = None,
                        ctx_lens: torch.Tensor | None = None, opts=None,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Decoupled-RoPE absorbed decode over this store's latents and rotary keys."""
        w = self.w
        n_ctx = w.n if n_ctx is None else n_ctx
        if q is None:
            if loop_count == 1:
                q = self.t["q"][layer, loop_begin]
            else:
                q = self.t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).contiguous()
        if out is None:
            out = torch.empty(w.batch, w.H, loop_count, w.d, dtype=torch.float32, device=self.device)
        ws = self.absorbed_workspace(n_ctx, loop_count, opts)
        lla.lla_decode_attn_absorbed(self.dims, self.codec, self.cache, self.t["k_rope"], w.d_rope,
                                     layer, n_ctx, ctx_lens, q, loop_begin, loop_count, out, ws,
                                     ws.numel(), opts, stream)
        return out

    def paginate(self, seed: int, spare_pages: int = 0, shuffle: bool = True):
        """Move this store's dense latent cache into a page pool: logical page p of
        sequence b goes to a random physical page (in order with shuffle=False) (spare pages are filled with NaN, so a
        read of a page the table does not name shows). Sets self.pages / self.block_table
        and replaces c_k, c_v by the pools [D][num_pages][Hc][16][r] (and k_rope, when the
        store has rotary keys, by [D][num_pages][H][16][d_rope]); the dense tensors stay in
        self.dense."""
        w = self.w
        npg = (self.n_max + 15) // 16
        num_pages = w.batch * npg + spare_pages
        g = torch.Generator(device="cpu").manual_seed(seed)
        perm = (torch.randperm(num_pages, generator=g) if shuffle
                else torch.arange(num_pages))[:w.batch * npg]
        table = perm.reshape(w.batch, npg).to(torch.int32)
        keys = [k for k in ("c_k", "c_v", "k_rope") if k in self.t]
        self.dense = {k: self.t[k] for k in keys}
        for key in keys:
            x = self.t[key]  # [D][B][heads][n][r]
            nh, r = x.shape[2], x.shape[-1]
            pad = npg * 16 - x.shape[3]
            if pad:
                x = torch.cat([x, torch.zeros(*x.shape[:3], pad, r, dtype=x.dtype, device=x.device)], 3)
            pool = torch.full((w.D, num_pages, nh, 16, r), float("nan"), dtype=x.dtype,
                              device=self.device)
            pages = x.reshape(w.D, w.batch, nh, npg, 16, r).permute(0, 1, 3, 2, 4, 5)
            pool[:, perm.to(self.device)] = pages.reshape(w.D, w.batch * npg, nh, 16, r)
            self.t[key] = pool
        self.block_table = table.to(self.device)
        self.pages = lla.make_pages(self.block_table, npg, num_pages)
        self.cache = lla.make_cache(self.t["c_k"], self.t["c_v"])
        return table

    def decode_paged(self, layer: int, loop_begin: int, loop_count: int, q=None, n_ctx=None,
                     ctx_lens=None, opts=None, out=None, stream=None) -> torch.Tensor:
        w = self.w
        n_ctx = w.n if n_ctx is None else n_ctx
        if q is None:
            if loop_count == 1:
                q = self.t["q"][layer, loop_begin]
            else:
                q = self.t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).contiguous()
        if out is None:
            out = torch.empty(w.batch, w.H, loop_count, w.d, dtype=torch.float32, device=self.device)
        nb = lla.lla_decode_paged_workspace_bytes(self.dims, n_ctx, loop_count, opts)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        lla.lla_decode_attn_paged(self.dims, self.codec, self.cache, self.pages, layer, n_ctx,
                                  ctx_lens, q, loop_begin, loop_count, out, ws, ws.numel(), opts,
                                  stream)
        return out

    def decode_absorbed_paged(self, layer: int, loop_begin: int, loop_count: int, q=None,
                              n_ctx=None, ctx_lens=None, opts=None, out=None,
                              stream=None) -> torch.Tensor:
        """Decoupled-RoPE absorbed decode over the paged cache (after paginate)."""
        w = self.w
        n_ctx = w.n if n_ctx is None else n_ctx
        if q is None:
            if loop_count == 1:
                q = self.t["q"][layer, loop_begin]
            else:
                q = self.t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).contiguous()
        if out is None:
            out = torch.empty(w.batch, w.H, loop_count, w.d, dtype=torch.float32, device=self.device)
        nb = lla.lla_decode_absorbed_paged_workspace_bytes(self.dims, w.d_rope, n_ctx, loop_count, opts)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        lla.lla_decode_attn_absorbed_paged(self.dims, self.codec, self.cache, self.pages,
                                           self.t["k_rope"], w.d_rope, layer, n_ctx, ctx_lens, q,
                                           loop_begin, loop_count, out, ws, ws.numel(), opts, stream)
        return out

    def reconstruct(self, layer: int, loop_begin: int, loop_count: int, pos_start: int = 0,
                    n_tok: int | None = None, k_out: torch.Tensor | None = None,
                    v_out: torch.Tensor | None = None, keys: bool = True, values: bool = True,
                    stream=None):
        """Rebuilt K/V of a slot range, [loop_count][B][H][n_max][d] in the cache dtype."""
        w = self.w
        n_tok = self.n_max - pos_start if n_tok is None else n_tok
        shape = (loop_count, w.batch, w.H, self.n_max, w.d)
        if keys and k_out is None:
            k_out = torch.zeros(shape, dtype=w.torch_dtype, device=self.device)
        if values and v_out is None:
            v_out = torch.zeros(shape, dtype=w.torch_dtype, device=self.device)
        lla.lla_reconstruct(self.dims, self.codec, self.cache, layer, loop_begin, loop_count,
                            pos_start, n_tok, k_out if keys else None, v_out if values else None,
                            stream)
        return k_out, v_out

    def encode(self, layer: int, x_k: torch.Tensor, x_v: torch.Tensor, pos_start: int,
               n_new: int, stream=None) -> None:
        lla.lla_encode(self.dims, self.codec, self.cache, layer, x_k, x_v, pos_start, n_new, stream)


class DeviceTeacherCache:
    """An uncompressed per-loop key/value cache for one workload, resident on ``device``."""

    def __init__(self, w: Workload, seed: int, device="cuda", n_alloc: int | None = None,
                 tensors: dict | None = None, with_q: bool = True):
        self.w = w
        self.device = torch.device(device)
        self.n_max = n_alloc or w.n
        t = tensors if tensors is not None else teacher_inputs(w, seed, device, self.n_max, with_q)
        self.t = {k: v.to(self.device).contiguous() for k, v in t.items()}
        self.dims = dims_for(w, self.n_max)
        self._ws = None

    def workspace(self, n_ctx: int, loop_count: int, opts=None) -> torch.Tensor:
        nb = lla.lla_decode_teacher_workspace_bytes(self.dims, n_ctx, loop_count, opts)
        if self._ws is None or self._ws.numel() < nb:
            self._ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def decode(self, layer: int, loop_begin: int, loop_count: int, q: torch.Tensor | None = None,
               n_ctx: int | None = None, ctx_lens: torch.Tensor | None = None, opts=None,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        w = self.w
        n_ctx = w.n if n_ctx is None else n_ctx
        if q is None:
            if loop_count == 1:
                q = self.t["q"][layer, loop_begin]
            else:
                q = self.t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).contiguous()
        if out is None:
            out = torch.empty(w.batch, w.H, loop_count, w.d, dtype=torch.float32, device=self.device)
        ws = self.workspace(n_ctx, loop_count, opts)
        lla.lla_decode_attn_teacher(self.dims, self.t["k_cache"], self.t["v_cache"], layer, n_ctx,
                                    ctx_lens, q, loop_begin, loop_count, out, ws, ws.numel(), opts,
                                    stream)
        return out
