"""Thin ctypes binding of ``liblla.so`` (the C ABI in include/lla.h).

Argument marshalling only: every step of the decode and encode path runs in the
library's gfx950 kernels. Functions carry the C names; device buffers may be passed as
torch tensors (their ``data_ptr()`` is used) or as integer addresses. ``stream=None``
uses torch's current HIP stream. A non-OK status raises :class:`LLAError`.

The library is loaded on first use; if it has not been built (``python -m
latent_decode_attention_lla_amd.build``) the call fails loudly. There is no fallback.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# LLA_LIBRARY names another build of the same library (the host-ASan build of build.py)
LIB_PATH = os.environ.get("LLA_LIBRARY") or os.path.join(HERE, "liblla.so")

LLA_OK = 0
LLA_ERR_INVALID_ARG = -1
LLA_ERR_UNSUPPORTED = -2
LLA_ERR_WORKSPACE = -3
LLA_ERR_HIP = -4

LLA_F32 = 0
LLA_BF16 = 1
LLA_PER_HEAD = 0
LLA_2D = 1
LLA_PATH_AUTO = 0
LLA_PATH_RECONSTRUCT = 1
LLA_PATH_ROTARY_FOLD = 2

EXPORTED = (
    "lla_status_string", "lla_compression_ratio", "lla_cache_bytes_per_token",
    "lla_rope_table_bytes", "lla_rope_table_build", "lla_encode",
    "lla_decode_workspace_bytes", "lla_decode_attn", "lla_decode_num_splits",
    "lla_decode_absorbed_workspace_bytes", "lla_decode_attn_absorbed",
    "lla_decode_absorbed_supported", "lla_decode_absorbed_paged_workspace_bytes",
    "lla_decode_attn_absorbed_paged",
    "lla_decode_teacher_workspace_bytes", "lla_decode_attn_teacher", "lla_decode_teacher_supported",
    "lla_decode_teacher_num_splits", "lla_decode_paged_num_splits", "lla_reconstruct",
    "lla_encode_paged", "lla_decode_paged_workspace_bytes", "lla_decode_attn_paged",
    "lla_decode_attn_noalloc", "lla_stream_ceiling", "lla_encode_fused_acc_bytes",
    "lla_encode_fused",
)

# bytes of the fixed split-partial array lla_decode_attn_noalloc uses (include/lla.h)
LLA_NOALLOC_SCRATCH_BYTES = 8 << 20


class LLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({lla_status_string(status)})")


class lla_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("r_k", ctypes.c_int32), ("r_v", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("scale", ctypes.c_float)]


class lla_codec(ctypes.Structure):
    _fields_ = [("w_down_k_t", ctypes.c_void_p), ("mu_k", ctypes.c_void_p),
                ("w_up_k", ctypes.c_void_p), ("w_down_v_t", ctypes.c_void_p),
                ("mu_v", ctypes.c_void_p), ("w_up_v", ctypes.c_void_p),
                ("rope_table", ctypes.c_void_p)]


class lla_cache(ctypes.Structure):
    _fields_ = [("c_k", ctypes.c_void_p), ("c_v", ctypes.c_void_p)]


class lla_proj(ctypes.Structure):
    _fields_ = [("w_k", ctypes.c_void_p), ("w_v", ctypes.c_void_p), ("d_model", ctypes.c_int32)]


class lla_pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class lla_decode_opts(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("path", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load liblla.so (once). Raises if it is missing: the HIP path is the only path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"LLA HIP library not built: {LIB_PATH} is missing "
                           "(run python -m latent_decode_attention_lla_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.lla_status_string.argtypes = [i32]
    lib.lla_status_string.restype = ctypes.c_char_p
    lib.lla_compression_ratio.argtypes = [P(lla_dims)]
    lib.lla_compression_ratio.restype = ctypes.c_double
    lib.lla_cache_bytes_per_token.argtypes = [P(lla_dims)]
    lib.lla_cache_bytes_per_token.restype = ctypes.c_double
    lib.lla_rope_table_bytes.argtypes = [P(lla_dims)]
    lib.lla_rope_table_bytes.restype = sz
    lib.lla_rope_table_build.argtypes = [P(lla_dims), vp, vp]
    lib.lla_rope_table_build.restype = i32
    lib.lla_encode.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache), i32, vp, vp, i32, i32, vp]
    lib.lla_encode.restype = i32
    lib.lla_encode_fused_acc_bytes.argtypes = [P(lla_dims), i32]
    lib.lla_encode_fused_acc_bytes.restype = sz
    lib.lla_encode_fused.argtypes = [P(lla_dims), P(lla_codec), P(lla_proj), P(lla_cache), i32, i32,
                                     vp, i32, i32, vp, sz, vp]
    lib.lla_encode_fused.restype = i32
    lib.lla_decode_workspace_bytes.argtypes = [P(lla_dims), i32, i32, P(lla_decode_opts)]
    lib.lla_decode_workspace_bytes.restype = sz
    lib.lla_decode_num_splits.argtypes = [P(lla_dims), i32, i32, P(lla_decode_opts)]
    lib.lla_decode_num_splits.restype = i32
    lib.lla_decode_attn.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache), i32, i32, vp, vp,
                                    i32, i32, vp, vp, sz, P(lla_decode_opts), vp]
    lib.lla_decode_attn_noalloc.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache), i32, i32, vp,
                                            vp, i32, i32, vp, P(lla_decode_opts), vp]
    lib.lla_decode_attn_noalloc.restype = i32
    lib.lla_stream_ceiling.argtypes = [i32, vp, vp, sz, i32, vp]
    lib.lla_stream_ceiling.restype = i32
    lib.lla_decode_attn.restype = i32
    lib.lla_decode_absorbed_workspace_bytes.argtypes = [P(lla_dims), i32, i32, i32,
                                                        P(lla_decode_opts)]
    lib.lla_decode_absorbed_workspace_bytes.restype = sz
    lib.lla_decode_attn_absorbed.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache), vp, i32,
                                             i32, i32, vp, vp, i32, i32, vp, vp, sz,
                                             P(lla_decode_opts), vp]
    lib.lla_decode_attn_absorbed.restype = i32
    lib.lla_decode_absorbed_supported.argtypes = [P(lla_dims), i32]
    lib.lla_decode_absorbed_supported.restype = i32
    lib.lla_decode_absorbed_paged_workspace_bytes.argtypes = [P(lla_dims), i32, i32, i32,
                                                              P(lla_decode_opts)]
    lib.lla_decode_absorbed_paged_workspace_bytes.restype = sz
    lib.lla_decode_attn_absorbed_paged.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache),
                                                   P(lla_pages), vp, i32, i32, i32, vp, vp, i32,
                                                   i32, vp, vp, sz, P(lla_decode_opts), vp]
    lib.lla_decode_attn_absorbed_paged.restype = i32
    lib.lla_decode_teacher_workspace_bytes.argtypes = [P(lla_dims), i32, i32, P(lla_decode_opts)]
    lib.lla_decode_teacher_workspace_bytes.restype = sz
    lib.lla_decode_attn_teacher.argtypes = [P(lla_dims), vp, vp, i32, i32, vp, vp, i32, i32, vp,
                                            vp, sz, P(lla_decode_opts), vp]
    lib.lla_decode_attn_teacher.restype = i32
    lib.lla_decode_teacher_supported.argtypes = [P(lla_dims)]
    lib.lla_decode_teacher_supported.restype = i32
    lib.lla_decode_teacher_num_splits.argtypes = [P(lla_dims), i32, i32, P(lla_decode_opts)]
    lib.lla_decode_teacher_num_splits.restype = i32
    lib.lla_decode_paged_num_splits.argtypes = [P(lla_dims), i32, i32, P(lla_decode_opts)]
    lib.lla_decode_paged_num_splits.restype = i32
    lib.lla_reconstruct.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache), i32, i32, i32, i32,
                                    i32, vp, vp, vp]
    lib.lla_reconstruct.restype = i32
    lib.lla_encode_paged.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache), P(lla_pages), i32, vp,
                                     vp, i32, i32, vp]
    lib.lla_encode_paged.restype = i32
    lib.lla_decode_paged_workspace_bytes.argtypes = [P(lla_dims), i32, i32, P(lla_decode_opts)]
    lib.lla_decode_paged_workspace_bytes.restype = sz
    lib.lla_decode_attn_paged.argtypes = [P(lla_dims), P(lla_codec), P(lla_cache), P(lla_pages), i32,
                                          i32, vp, vp, i32, i32, vp, vp, sz, P(lla_decode_opts), vp]
    lib.lla_decode_attn_paged.restype = i32
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != LLA_OK:
        raise LLAError(fn, status)


def make_dims(T, D, H, d_head, r_k, r_v, batch, n_max, variant=LLA_PER_HEAD, dtype=LLA_BF16,
              rope_base=10000.0, scale=0.0) -> lla_dims:
    return lla_dims(T, D, H, d_head, r_k, r_v, batch, n_max, variant, dtype, rope_base, scale)


def make_codec(w_down_k_t=None, mu_k=None, w_up_k=None, w_down_v_t=None, mu_v=None, w_up_v=None,
               rope_table=None) -> lla_codec:
    return lla_codec(_ptr(w_down_k_t), _ptr(mu_k), _ptr(w_up_k), _ptr(w_down_v_t), _ptr(mu_v),
                     _ptr(w_up_v), _ptr(rope_table))


def make_cache(c_k, c_v) -> lla_cache:
    return lla_cache(_ptr(c_k), _ptr(c_v))


def make_opts(num_splits=0, path=LLA_PATH_AUTO) -> lla_decode_opts:
    return lla_decode_opts(num_splits, path)


def lla_status_string(status: int) -> str:
    return load().lla_status_string(status).decode()


def lla_compression_ratio(dims: lla_dims) -> float:
    return load().lla_compression_ratio(ctypes.byref(dims))


def lla_cache_bytes_per_token(dims: lla_dims) -> float:
    return load().lla_cache_bytes_per_token(ctypes.byref(dims))


def lla_rope_table_bytes(dims: lla_dims) -> int:
    return load().lla_rope_table_bytes(ctypes.byref(dims))


def lla_rope_table_build(dims: lla_dims, table, stream=None) -> None:
    _check("lla_rope_table_build",
           load().lla_rope_table_build(ctypes.byref(dims), _ptr(table), _stream(stream)))


def lla_encode(dims: lla_dims, codec: lla_codec, cache: lla_cache, layer: int, x_k, x_v,
               pos_start: int, n_new: int, stream=None) -> None:
    _check("lla_encode", load().lla_encode(ctypes.byref(dims), ctypes.byref(codec),
                                           ctypes.byref(cache), layer, _ptr(x_k), _ptr(x_v),
                                           pos_start, n_new, _stream(stream)))


def make_proj(w_k, w_v, d_model: int) -> lla_proj:
    return lla_proj(_ptr(w_k), _ptr(w_v), d_model)


def lla_encode_fused_acc_bytes(dims: lla_dims, n_new: int) -> int:
    return load().lla_encode_fused_acc_bytes(ctypes.byref(dims), n_new)


def lla_encode_fused(dims, codec, proj, cache, layer, loop, h, pos_start, n_new, acc, acc_bytes,
                     stream=None) -> None:
    _check("lla_encode_fused", lla_encode_fused_status(dims, codec, proj, cache, layer, loop, h,
                                                       pos_start, n_new, acc, acc_bytes,
                                                       _stream(stream)))


def lla_encode_fused_status(dims, codec, proj, cache, layer, loop, h, pos_start, n_new, acc,
                            acc_bytes, stream=0) -> int:
    return load().lla_encode_fused(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(proj),
                                   ctypes.byref(cache), layer, loop, _ptr(h), pos_start, n_new,
                                   _ptr(acc), acc_bytes, stream)


def lla_decode_workspace_bytes(dims: lla_dims, n_ctx: int, loop_count: int, opts=None) -> int:
    return load().lla_decode_workspace_bytes(ctypes.byref(dims), n_ctx, loop_count,
                                             ctypes.byref(opts) if opts is not None else None)


def lla_decode_num_splits(dims: lla_dims, n_ctx: int, loop_count: int, opts=None) -> int:
    return load().lla_decode_num_splits(ctypes.byref(dims), n_ctx, loop_count,
                                        ctypes.byref(opts) if opts is not None else None)


def lla_decode_attn(dims: lla_dims, codec: lla_codec, cache: lla_cache, layer: int, n_ctx: int,
                    ctx_lens, q, loop_begin: int, loop_count: int, out, workspace,
                    workspace_bytes: int, opts=None, stream=None) -> None:
    _check("lla_decode_attn", load().lla_decode_attn(
        ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache), layer, n_ctx,
        _ptr(ctx_lens), _ptr(q), loop_begin, loop_count, _ptr(out), _ptr(workspace),
        workspace_bytes, ctypes.byref(opts) if opts is not None else None, _stream(stream)))


def lla_decode_attn_noalloc(dims: lla_dims, codec: lla_codec, cache: lla_cache, layer: int,
                            n_ctx: int, ctx_lens, q, loop_begin: int, loop_count: int, out,
                            opts=None, stream=None) -> None:
    """lla_decode_attn with the split partials in the library's fixed device array."""
    _check("lla_decode_attn_noalloc", load().lla_decode_attn_noalloc(
        ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache), layer, n_ctx,
        _ptr(ctx_lens), _ptr(q), loop_begin, loop_count, _ptr(out),
        ctypes.byref(opts) if opts is not None else None, _stream(stream)))


def lla_stream_ceiling(mode: int, src, dst, n_vectors: int, workgroups: int, stream=None) -> None:
    """Measurement helper (include/lla_stream.h): a plain streaming pass, mode 0 read-only,
    1 copy, 2 four reads per write, 3 four writes per read; 4-6 read-only with every wave
    streaming its own chunk through direct-to-LDS loads (4), registers (5) or both (6);
    7 the narrow fold's latent-row pattern (per wave a key and a value row plane)."""
    st = load().lla_stream_ceiling(mode, _ptr(src), _ptr(dst), n_vectors, workgroups, _stream(stream))
    if st != 0:
        raise RuntimeError(f"lla_stream_ceiling failed: {st}")


def lla_decode_absorbed_workspace_bytes(dims: lla_dims, d_rope: int, n_ctx: int, loop_count: int,
                                        opts=None) -> int:
    return load().lla_decode_absorbed_workspace_bytes(
        ctypes.byref(dims), d_rope, n_ctx, loop_count,
        ctypes.byref(opts) if opts is not None else None)


def lla_decode_absorbed_supported(dims: lla_dims, d_rope: int) -> bool:
    return bool(load().lla_decode_absorbed_supported(ctypes.byref(dims), d_rope))


def lla_decode_attn_absorbed(dims: lla_dims, codec: lla_codec, cache: lla_cache, k_rope,
                             d_rope: int, layer: int, n_ctx: int, ctx_lens, q, loop_begin: int,
                             loop_count: int, out, workspace, workspace_bytes: int, opts=None,
                             stream=None) -> None:
    _check("lla_decode_attn_absorbed", lla_decode_attn_absorbed_status(
        dims, codec, cache, k_rope, d_rope, layer, n_ctx, ctx_lens, q, loop_begin, loop_count,
        out, workspace, workspace_bytes, opts, _stream(stream)))


def lla_decode_attn_absorbed_status(dims, codec, cache, k_rope, d_rope, layer, n_ctx, ctx_lens, q,
                                    loop_begin, loop_count, out, workspace, workspace_bytes,
                                    opts=None, stream=0) -> int:
    return load().lla_decode_attn_absorbed(
        ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache), _ptr(k_rope), d_rope, layer,
        n_ctx, _ptr(ctx_lens), _ptr(q), loop_begin, loop_count, _ptr(out), _ptr(workspace),
        workspace_bytes, ctypes.byref(opts) if opts is not None else None, stream)


def lla_decode_absorbed_paged_workspace_bytes(dims: lla_dims, d_rope: int, n_ctx: int,
                                              loop_count: int, opts=None) -> int:
    return load().lla_decode_absorbed_paged_workspace_bytes(
        ctypes.byref(dims), d_rope, n_ctx, loop_count,
        ctypes.byref(opts) if opts is not None else None)


def lla_decode_attn_absorbed_paged(dims, codec, cache, pages, k_rope, d_rope: int, layer: int,
                                   n_ctx: int, ctx_lens, q, loop_begin: int, loop_count: int, out,
                                   workspace, workspace_bytes: int, opts=None, stream=None) -> None:
    _check("lla_decode_attn_absorbed_paged", lla_decode_attn_absorbed_paged_status(
        dims, codec, cache, pages, k_rope, d_rope, layer, n_ctx, ctx_lens, q, loop_begin,
        loop_count, out, workspace, workspace_bytes, opts, _stream(stream)))


def lla_decode_attn_absorbed_paged_status(dims, codec, cache, pages, k_rope, d_rope, layer, n_ctx,
                                          ctx_lens, q, loop_begin, loop_count, out, workspace,
                                          workspace_bytes, opts=None, stream=0) -> int:
    return load().lla_decode_attn_absorbed_paged(
        ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
        ctypes.byref(pages) if pages is not None else None, _ptr(k_rope), d_rope, layer, n_ctx,
        _ptr(ctx_lens), _ptr(q), loop_begin, loop_count, _ptr(out), _ptr(workspace),
        workspace_bytes, ctypes.byref(opts) if opts is not None else None, stream)


def lla_decode_attn_status(dims, codec, cache, layer, n_ctx, ctx_lens, q, loop_begin, loop_count,
                           out, workspace, workspace_bytes, opts=None, stream=0) -> int:
    """Same call, returning the raw status instead of raising (for argument tests)."""
    return load().lla_decode_attn(
        ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache), layer, n_ctx,
        _ptr(ctx_lens), _ptr(q), loop_begin, loop_count, _ptr(out), _ptr(workspace),
        workspace_bytes, ctypes.byref(opts) if opts is not None else None, stream)


def lla_encode_status(dims, codec, cache, layer, x_k, x_v, pos_start, n_new, stream=0) -> int:
    return load().lla_encode(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache), layer,
                             _ptr(x_k), _ptr(x_v), pos_start, n_new, stream)


def lla_decode_teacher_workspace_bytes(dims: lla_dims, n_ctx: int, loop_count: int,
                                       opts=None) -> int:
    return load().lla_decode_teacher_workspace_bytes(
        ctypes.byref(dims), n_ctx, loop_count, ctypes.byref(opts) if opts is not None else None)


def lla_decode_teacher_supported(dims: lla_dims) -> bool:
    return bool(load().lla_decode_teacher_supported(ctypes.byref(dims)))


def lla_decode_teacher_num_splits(dims: lla_dims, n_ctx: int, loop_count: int, opts=None) -> int:
    return load().lla_decode_teacher_num_splits(
        ctypes.byref(dims), n_ctx, loop_count, ctypes.byref(opts) if opts is not None else None)


def lla_decode_paged_num_splits(dims: lla_dims, n_ctx: int, loop_count: int, opts=None) -> int:
    return load().lla_decode_paged_num_splits(
        ctypes.byref(dims), n_ctx, loop_count, ctypes.byref(opts) if opts is not None else None)


def lla_decode_attn_teacher(dims: lla_dims, k_cache, v_cache, layer: int, n_ctx: int, ctx_lens, q,
                            loop_begin: int, loop_count: int, out, workspace, workspace_bytes: int,
                            opts=None, stream=None) -> None:
    _check("lla_decode_attn_teacher", lla_decode_attn_teacher_status(
        dims, k_cache, v_cache, layer, n_ctx, ctx_lens, q, loop_begin, loop_count, out, workspace,
        workspace_bytes, opts, _stream(stream)))


def lla_decode_attn_teacher_status(dims, k_cache, v_cache, layer, n_ctx, ctx_lens, q, loop_begin,
                                   loop_count, out, workspace, workspace_bytes, opts=None,
                                   stream=0) -> int:
    return load().lla_decode_attn_teacher(
        ctypes.byref(dims), _ptr(k_cache), _ptr(v_cache), layer, n_ctx, _ptr(ctx_lens), _ptr(q),
        loop_begin, loop_count, _ptr(out), _ptr(workspace), workspace_bytes,
        ctypes.byref(opts) if opts is not None else None, stream)


def lla_reconstruct(dims: lla_dims, codec: lla_codec, cache: lla_cache, layer: int,
                    loop_begin: int, loop_count: int, pos_start: int, n_tok: int, k_out, v_out,
                    stream=None) -> None:
    _check("lla_reconstruct", lla_reconstruct_status(dims, codec, cache, layer, loop_begin,
                                                     loop_count, pos_start, n_tok, k_out, v_out,
                                                     _stream(stream)))


def lla_reconstruct_status(dims, codec, cache, layer, loop_begin, loop_count, pos_start, n_tok,
                           k_out, v_out, stream=0) -> int:
    return load().lla_reconstruct(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                  layer, loop_begin, loop_count, pos_start, n_tok, _ptr(k_out),
                                  _ptr(v_out), stream)


def make_pages(block_table, max_blocks: int, num_pages: int) -> lla_pages:
    return lla_pages(_ptr(block_table), max_blocks, num_pages)


def lla_encode_paged(dims, codec, cache, pages, layer, x_k, x_v, pos_start, n_new, stream=None):
    _check("lla_encode_paged", lla_encode_paged_status(dims, codec, cache, pages, layer, x_k, x_v,
                                                       pos_start, n_new, _stream(stream)))


def lla_encode_paged_status(dims, codec, cache, pages, layer, x_k, x_v, pos_start, n_new,
                            stream=0) -> int:
    return load().lla_encode_paged(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                   ctypes.byref(pages), layer, _ptr(x_k), _ptr(x_v), pos_start,
                                   n_new, stream)


def lla_decode_paged_workspace_bytes(dims, n_ctx, loop_count, opts=None) -> int:
    return load().lla_decode_paged_workspace_bytes(
        ctypes.byref(dims), n_ctx, loop_count, ctypes.byref(opts) if opts is not None else None)


def lla_decode_attn_paged(dims, codec, cache, pages, layer, n_ctx, ctx_lens, q, loop_begin,
                          loop_count, out, workspace, workspace_bytes, opts=None, stream=None):
    _check("lla_decode_attn_paged", lla_decode_attn_paged_status(
        dims, codec, cache, pages, layer, n_ctx, ctx_lens, q, loop_begin, loop_count, out,
        workspace, workspace_bytes, opts, _stream(stream)))


def lla_decode_attn_paged_status(dims, codec, cache, pages, layer, n_ctx, ctx_lens, q, loop_begin,
                                 loop_count, out, workspace, workspace_bytes, opts=None,
                                 stream=0) -> int:
    return load().lla_decode_attn_paged(
        ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache), ctypes.byref(pages), layer,
        n_ctx, _ptr(ctx_lens), _ptr(q), loop_begin, loop_count, _ptr(out), _ptr(workspace),
        workspace_bytes, ctypes.byref(opts) if opts is not None else None, stream)
