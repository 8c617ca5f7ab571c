"""Python binding of liborthros.so, the gfx950 Orthros attention hot path.

Argument marshalling only: every function below checks that the tensors are
dense and on the GPU, derives the sizes from their shapes, and calls the C
entry point of the same name with raw device pointers and the current HIP
stream. All arithmetic happens in the library's HIP kernels. There is no CPU
fallback: if the library is missing or fails to load, the functions raise.

Layouts (see include/orthros.h for the full contract):
  q_pre / o            [B, T, Hq, D]     qx_pre / o_x   [B, T_out, Hq, D]
  k_cache / v_cache    [B, Hkv, cap, D]  k_new / v_new  [B, n, Hkv, D]
  alpha, beta, ...     fp32 [Hq*D]       cache_len      int32 [B] (device)
"""
import ctypes
import os

import torch

__all__ = [
    "ORTHROS_F32", "ORTHROS_BF16", "ORTHROS_OP_GLOBAL_XATTN",
    "ORTHROS_OP_DECODE_PAIR", "OrthrosError", "lib", "library_path",
    "orthros_kv_append", "orthros_swa_prefill", "orthros_global_xattn",
    "orthros_decode_pair", "orthros_decode_pair_noalloc",
    "orthros_kv_append_paged", "ORTHROS_NOALLOC_SCRATCH_BYTES",
    "orthros_decode_pair_paged", "orthros_workspace_bytes",
    "orthros_workspace_counter_bytes", "ORTHROS_NOALLOC_COUNTER_BYTES",
    "orthros_check_device_errors", "orthros_abi_version",
    "orthros_strerror", "orthros_last_error", "workspace",
]

ORTHROS_F32 = 0
ORTHROS_BF16 = 1
ORTHROS_OP_GLOBAL_XATTN = 1
ORTHROS_OP_DECODE_PAIR = 2
ORTHROS_NOALLOC_SCRATCH_BYTES = 64 << 20
ORTHROS_NOALLOC_COUNTER_BYTES = 64 << 10

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "liborthros.so")
_lib = None


class OrthrosError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"orthros error {code}: {message}")
        self.code = code


def lib():
    """The loaded liborthros.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise OrthrosError(-5, f"{library_path} is missing: build it with "
                               "`python -m long_context_prefill_swa_amd.build`")
    L = ctypes.CDLL(library_path)
    vp, i32, i64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                        ctypes.c_size_t)
    L.orthros_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                    i64, i32, vp]
    L.orthros_swa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                      i32, i32, i64, i32, vp, i32, vp]
    L.orthros_global_xattn.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                       i32, i32, i32, i64, vp, i32, vp, sz, vp]
    L.orthros_decode_pair.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, i32, i32, i32, i32, i64,
                                      i64, i32, vp, i32, vp, sz, vp]
    L.orthros_decode_pair_noalloc.argtypes = [vp] * 13 + [i32] * 4 + [
        i64, i64, i32, vp, i32, vp]
    L.orthros_kv_append_paged.argtypes = [vp, vp, i64, i32, vp, i32, vp, vp,
                                          vp, i32, i32, i32, i32, i32, vp]
    L.orthros_decode_pair_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, vp, i64, i32, vp, i32, vp,
                                            vp, vp, i32, i32, i32, i32, i64,
                                            i32, vp, i32, vp, sz, vp]
    L.orthros_layer_forward.argtypes = [vp] * 13 + [i32] * 7 + [i64, i32, vp,
                                                                sz, vp]
    L.orthros_attn_backward.argtypes = [vp] * 20 + [i32] * 6 + [i64, i32, vp,
                                                               i32, vp, sz, vp]
    L.orthros_backward_workspace_bytes.argtypes = [i32] * 6
    L.orthros_backward_workspace_bytes.restype = sz
    L.orthros_layer_workspace_bytes.argtypes = [i32] * 7
    L.orthros_layer_workspace_bytes.restype = sz
    L.orthros_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i64,
                                          vp]
    L.orthros_workspace_bytes.restype = sz
    L.orthros_workspace_counter_bytes.argtypes = [i32, i32, i32, i32, i32,
                                                  i32, i64, vp]
    L.orthros_workspace_counter_bytes.restype = sz
    L.orthros_strerror.argtypes = [i32]
    L.orthros_strerror.restype = ctypes.c_char_p
    L.orthros_last_error.argtypes = []
    L.orthros_last_error.restype = ctypes.c_char_p
    L.orthros_check_device_errors.argtypes = [vp]
    L.orthros_abi_version.argtypes = []
    for name in ("orthros_kv_append", "orthros_swa_prefill",
                 "orthros_global_xattn", "orthros_decode_pair",
                 "orthros_decode_pair_noalloc",
                 "orthros_kv_append_paged", "orthros_decode_pair_paged",
                 "orthros_check_device_errors", "orthros_abi_version"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def _check(rc):
    if rc != 0:
        msg = lib().orthros_last_error().decode(errors="replace")
        raise OrthrosError(rc, msg or orthros_strerror(rc))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ORTHROS_BF16
    if t.dtype == torch.float32:
        return ORTHROS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None):
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
    return ctypes.c_void_p(t.data_ptr())


def _vecs(n, *named):
    """fp32 vectors of n entries (alpha/beta: Hq*D) on the GPU, given as
    (tensor, name) pairs; every size is checked before any device check."""
    for t, name in named:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} elements (Hq*D), got "
                             f"{t.numel()}")
    return [_dev(t, name, torch.float32) for t, name in named]


def _lens(t, B, name="cache_len"):
    """Checks the int32 [B] cache lengths' size (before any device check)
    and returns the tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.int32 or t.numel() != B:
        raise ValueError(f"{name} must be int32 with B={B} entries, got "
                         f"{t.dtype} with {t.numel()}")
    return t


def _stream(stream, like):
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _scratch(nbytes, device, stream, zero_bytes=0):
    """Scratch allocated here for one call, its first zero_bytes cleared.
    Both happen on the stream the call runs on: the clearing is then ordered
    before the call, and the caching allocator, which ties a block to the
    stream current at allocation, does not hand the block out again before
    that stream's work is done."""
    def make():
        ws = torch.empty(max(int(nbytes), 16), dtype=torch.uint8,
                         device=device)
        if zero_bytes:
            ws[:int(zero_bytes)].zero_()
        return ws
    if stream is None:
        return make()
    with torch.cuda.stream(stream):
        return make()


def _split_scratch(op, B, Hq, Hkv, D, T_out, max_len, head_map, device,
                   stream):
    """Per-call workspace of a split-KV call (None when it needs none)."""
    need = orthros_workspace_bytes(op, B, Hq, Hkv, D, T_out, max_len, head_map)
    if not need:
        return None
    return _scratch(need, device, stream, orthros_workspace_counter_bytes(
        op, B, Hq, Hkv, D, T_out, max_len, head_map))


def _map(head_map, Hq=None):
    """Host int32 copy of the head map (the library reads Hq entries)."""
    if head_map is None:
        return None, None
    if Hq is not None and len(head_map) != Hq:
        raise ValueError(f"head_map must have Hq={Hq} entries, got "
                         f"{len(head_map)}")
    arr = (ctypes.c_int32 * len(head_map))(*[int(x) for x in head_map])
    return ctypes.cast(arr, ctypes.c_void_p), arr


def orthros_strerror(code):
    return lib().orthros_strerror(int(code)).decode()


def orthros_last_error():
    return lib().orthros_last_error().decode(errors="replace")


def orthros_abi_version():
    return int(lib().orthros_abi_version())


def orthros_workspace_bytes(op, B, Hq, Hkv, D, T_out, max_len, head_map=None):
    hm, _keep = _map(head_map, Hq)
    return int(lib().orthros_workspace_bytes(op, B, Hq, Hkv, D, T_out,
                                             int(max_len), hm))


def orthros_workspace_counter_bytes(op, B, Hq, Hkv, D, T_out, max_len,
                                    head_map=None):
    hm, _keep = _map(head_map, Hq)
    return int(lib().orthros_workspace_counter_bytes(op, B, Hq, Hkv, D, T_out,
                                                     int(max_len), hm))


def workspace(nbytes, device):
    """Caller-owned workspace (16-byte aligned) for the split-KV calls,
    zero-filled on the current stream: its leading arrival counters must be
    zero before the first call, and every call leaves them zero. Zero it
    again (ws.zero_()) before a call with more (batch entry, head group)
    pairs than the calls it has served."""
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def orthros_kv_append(k_cache, v_cache, cache_len, k_new, v_new, stream=None):
    B, Hkv, cap, D = k_cache.shape
    n_new = k_new.shape[1]
    if tuple(k_new.shape) != (B, n_new, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, n, Hkv, D]")
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    dt = k_cache.dtype
    cl_p = _dev(_lens(cache_len, B), "cache_len", torch.int32)
    _check(lib().orthros_kv_append(
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        cl_p, _dev(k_new, "k_new", dt),
        _dev(v_new, "v_new", dt), B, n_new, Hkv, D, cap, _dtype_code(k_cache),
        _stream(stream, k_cache)))


def orthros_swa_prefill(q_pre, alpha, beta, k_cache, v_cache, o, W,
                        head_map=None, stream=None):
    B, T, Hq, D = q_pre.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, Hkv, cap, D]")
    if o.shape != q_pre.shape:
        raise ValueError("o must have q_pre's shape")
    dt = q_pre.dtype
    a_p, b_p = _vecs(Hq * D, (alpha, "alpha"), (beta, "beta"))
    hm, _keep = _map(head_map, Hq)
    _check(lib().orthros_swa_prefill(
        _dev(q_pre, "q_pre", dt), a_p, b_p, _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), _dev(o, "o", dt), B, T, Hq, Hkv, D, cap,
        int(W), hm, _dtype_code(q_pre), _stream(stream, q_pre)))


def orthros_global_xattn(qx_pre, alpha_x, beta_x, k_cache, v_cache, o_x, T_in,
                         head_map=None, ws=None, stream=None):
    B, T_out, Hq, D = qx_pre.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, Hkv, cap, D]")
    if o_x.shape != qx_pre.shape:
        raise ValueError("o_x must have qx_pre's shape")
    dt = qx_pre.dtype
    ax_p, bx_p = _vecs(Hq * D, (alpha_x, "alpha_x"), (beta_x, "beta_x"))
    if ws is None:
        ws = _split_scratch(ORTHROS_OP_GLOBAL_XATTN, B, Hq, Hkv, D, T_out,
                            int(T_in) + T_out, head_map, qx_pre.device, stream)
    hm, _keep = _map(head_map, Hq)
    _check(lib().orthros_global_xattn(
        _dev(qx_pre, "qx_pre", dt), ax_p, bx_p, _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), _dev(o_x, "o_x", dt), B, int(T_in),
        T_out, Hq, Hkv, D, cap, hm, _dtype_code(qx_pre), _dev(ws, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream, qx_pre)))


def orthros_decode_pair(q_pre, qx_pre, alpha, beta, alpha_x, beta_x, k_new,
                        v_new, k_cache, v_cache, cache_len, o, o_x,
                        max_len_after, W, head_map=None, ws=None, stream=None):
    B, Hq, D = q_pre.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, Hkv, cap, D]")
    if tuple(k_new.shape) != (B, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, Hkv, D]")
    if qx_pre.shape != q_pre.shape or o.shape != q_pre.shape or o_x.shape != q_pre.shape:
        raise ValueError("q_pre, qx_pre, o, o_x must all be [B, Hq, D]")
    dt = q_pre.dtype
    _lens(cache_len, B)
    aff = _vecs(Hq * D, (alpha, "alpha"), (beta, "beta"),
                (alpha_x, "alpha_x"), (beta_x, "beta_x"))
    cl_p = _dev(cache_len, "cache_len", torch.int32)
    if ws is None:
        ws = _split_scratch(ORTHROS_OP_DECODE_PAIR, B, Hq, Hkv, D, 1,
                            int(max_len_after), head_map, q_pre.device, stream)
    hm, _keep = _map(head_map, Hq)
    _check(lib().orthros_decode_pair(
        _dev(q_pre, "q_pre", dt), _dev(qx_pre, "qx_pre", dt), *aff,
        _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt),
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        cl_p, _dev(o, "o", dt),
        _dev(o_x, "o_x", dt), B, Hq, Hkv, D, cap, int(max_len_after), int(W),
        hm, _dtype_code(q_pre), _dev(ws, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream, q_pre)))


def orthros_decode_pair_noalloc(q_pre, qx_pre, alpha, beta, alpha_x, beta_x,
                                k_new, v_new, k_cache, v_cache, cache_len, o,
                                o_x, max_len_after, W, head_map=None,
                                stream=None):
    """orthros_decode_pair with no workspace and no allocation: the library's
    static per-device scratch (ORTHROS_NOALLOC_SCRATCH_BYTES) holds the
    partials. Calls overlapping in time on one device race."""
    B, Hq, D = q_pre.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, Hkv, cap, D]")
    if tuple(k_new.shape) != (B, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, Hkv, D]")
    if qx_pre.shape != q_pre.shape or o.shape != q_pre.shape or o_x.shape != q_pre.shape:
        raise ValueError("q_pre, qx_pre, o, o_x must all be [B, Hq, D]")
    dt = q_pre.dtype
    _lens(cache_len, B)
    aff = _vecs(Hq * D, (alpha, "alpha"), (beta, "beta"),
                (alpha_x, "alpha_x"), (beta_x, "beta_x"))
    cl_p = _dev(cache_len, "cache_len", torch.int32)
    hm, _keep = _map(head_map, Hq)
    _check(lib().orthros_decode_pair_noalloc(
        _dev(q_pre, "q_pre", dt), _dev(qx_pre, "qx_pre", dt), *aff,
        _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt),
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        cl_p, _dev(o, "o", dt), _dev(o_x, "o_x", dt), B, Hq, Hkv, D, cap,
        int(max_len_after), int(W), hm, _dtype_code(q_pre),
        _stream(stream, q_pre)))


def _paged(k_pool, v_pool, block_table):
    n_pages, Hkv, page_size, D = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table must be a [B, max_pages] tensor")
    if block_table.dtype != torch.int32:
        raise ValueError(f"block_table must be int32, got {block_table.dtype}")
    return n_pages, Hkv, page_size, D, block_table.shape[1]


def orthros_kv_append_paged(k_pool, v_pool, block_table, cache_len, k_new,
                            v_new, stream=None):
    """Paged cache append. k_pool, v_pool [n_pages, Hkv, page_size, D];
    block_table int32 [B, max_pages]; k_new, v_new [B, n, Hkv, D]."""
    n_pages, Hkv, page_size, D, max_pages = _paged(k_pool, v_pool, block_table)
    B, n_new = k_new.shape[0], k_new.shape[1]
    if tuple(k_new.shape) != (B, n_new, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, n, Hkv, D]")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B rows")
    dt = k_pool.dtype
    cl_p = _dev(_lens(cache_len, B), "cache_len", torch.int32)
    _check(lib().orthros_kv_append_paged(
        _dev(k_pool, "k_pool", dt), _dev(v_pool, "v_pool", dt), n_pages,
        page_size, _dev(block_table, "block_table", torch.int32), max_pages,
        cl_p, _dev(k_new, "k_new", dt),
        _dev(v_new, "v_new", dt), B, n_new, Hkv, D, _dtype_code(k_pool),
        _stream(stream, k_pool)))


def orthros_decode_pair_paged(q_pre, qx_pre, alpha, beta, alpha_x, beta_x,
                              k_new, v_new, k_pool, v_pool, block_table,
                              cache_len, o, o_x, max_len_after, W,
                              head_map=None, ws=None, stream=None):
    """Decode pair step on a paged cache (see orthros_kv_append_paged)."""
    n_pages, Hkv, page_size, D, max_pages = _paged(k_pool, v_pool, block_table)
    B, Hq = q_pre.shape[0], q_pre.shape[1]
    if tuple(q_pre.shape) != (B, Hq, D):
        raise ValueError("q_pre must be [B, Hq, D]")
    if tuple(k_new.shape) != (B, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, Hkv, D]")
    if qx_pre.shape != q_pre.shape or o.shape != q_pre.shape or o_x.shape != q_pre.shape:
        raise ValueError("q_pre, qx_pre, o, o_x must all be [B, Hq, D]")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B rows")
    dt = q_pre.dtype
    _lens(cache_len, B)
    aff = _vecs(Hq * D, (alpha, "alpha"), (beta, "beta"),
                (alpha_x, "alpha_x"), (beta_x, "beta_x"))
    cl_p = _dev(cache_len, "cache_len", torch.int32)
    if ws is None:
        ws = _split_scratch(ORTHROS_OP_DECODE_PAIR, B, Hq, Hkv, D, 1,
                            int(max_len_after), head_map, q_pre.device, stream)
    hm, _keep = _map(head_map, Hq)
    _check(lib().orthros_decode_pair_paged(
        _dev(q_pre, "q_pre", dt), _dev(qx_pre, "qx_pre", dt), *aff,
        _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt),
        _dev(k_pool, "k_pool", dt), _dev(v_pool, "v_pool", dt), n_pages,
        page_size, _dev(block_table, "block_table", torch.int32), max_pages,
        cl_p, _dev(o, "o", dt),
        _dev(o_x, "o_x", dt), B, Hq, Hkv, D, int(max_len_after), int(W), hm,
        _dtype_code(q_pre), _dev(ws, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream, q_pre)))


def orthros_backward_workspace_bytes(B, T, T_out, Hq, Hkv, D):
    return int(lib().orthros_backward_workspace_bytes(B, T, T_out, Hq, Hkv, D))


def orthros_attn_backward(q_pre, qx_pre, alpha, beta, alpha_x, beta_x,
                          k_cache, v_cache, o, o_x, d_o, d_ox, W,
                          head_map=None, out=None, ws=None, stream=None):
    """Gradients of both streams. q_pre, o, d_o [B, T, Hq, D]; qx_pre, o_x,
    d_ox [B, T_out, Hq, D] (or None with T_out = 0); caches [B, Hkv, cap, D].
    Returns a dict: dq_pre, dqx_pre, dk, dv ([B, T, Hkv, D]), d_alpha,
    d_beta, d_alpha_x, d_beta_x ([Hq*D] fp32). `out` may supply them."""
    B, T, Hq, D = q_pre.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    T_out = 0 if qx_pre is None else qx_pre.shape[1]
    if tuple(k_cache.shape) != (B, Hkv, cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, Hkv, cap, D]")
    for name, t in (("o", o), ("d_o", d_o)):
        if t.shape != q_pre.shape:
            raise ValueError(f"{name} must have q_pre's shape")
    if T_out:
        for name, t in (("o_x", o_x), ("d_ox", d_ox)):
            if t.shape != qx_pre.shape:
                raise ValueError(f"{name} must have qx_pre's shape")
    dev, bf, f32 = q_pre.device, torch.bfloat16, torch.float32
    g = dict(out or {})
    g.setdefault("dq_pre", torch.empty_like(q_pre))
    g.setdefault("dqx_pre", None if not T_out else torch.empty_like(qx_pre))
    g.setdefault("dk", torch.empty((B, T, Hkv, D), dtype=bf, device=dev))
    g.setdefault("dv", torch.empty((B, T, Hkv, D), dtype=bf, device=dev))
    for name in ("d_alpha", "d_beta", "d_alpha_x", "d_beta_x"):
        g.setdefault(name, torch.empty(Hq * D, dtype=f32, device=dev))
    aff = (_vecs(Hq * D, (alpha, "alpha"), (beta, "beta"),
                 (alpha_x, "alpha_x"), (beta_x, "beta_x")) if T_out else
           _vecs(Hq * D, (alpha, "alpha"), (beta, "beta")) +
           [_dev(alpha_x, "alpha_x", f32), _dev(beta_x, "beta_x", f32)])
    if ws is None:
        ws = _scratch(orthros_backward_workspace_bytes(B, T, T_out, Hq, Hkv, D),
                      dev, stream)
    hm, _keep = _map(head_map, Hq)
    _check(lib().orthros_attn_backward(
        _dev(q_pre, "q_pre", bf), _dev(qx_pre, "qx_pre", bf), *aff,
        _dev(k_cache, "k_cache", bf), _dev(v_cache, "v_cache", bf),
        _dev(o, "o", bf), _dev(o_x, "o_x", bf), _dev(d_o, "d_o", bf),
        _dev(d_ox, "d_ox", bf), _dev(g["dq_pre"], "dq_pre", bf),
        _dev(g["dqx_pre"], "dqx_pre", bf), _dev(g["dk"], "dk", bf),
        _dev(g["dv"], "dv", bf), _dev(g["d_alpha"], "d_alpha", f32),
        _dev(g["d_beta"], "d_beta", f32), _dev(g["d_alpha_x"], "d_alpha_x", f32),
        _dev(g["d_beta_x"], "d_beta_x", f32), B, T, T_out, Hq, Hkv, D, cap,
        int(W), hm, ORTHROS_BF16, _dev(ws, "ws"),
        0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream, q_pre)))
    return g


def orthros_layer_workspace_bytes(B, T, T_out, d_model, Hq, Hkv, D):
    return int(lib().orthros_layer_workspace_bytes(B, T, T_out, d_model, Hq,
                                                   Hkv, D))


def orthros_layer_forward(x, w_q, w_k, w_v, w_o, alpha, beta, alpha_x,
                          beta_x, k_cache, v_cache, cache_len, y, T_out, W,
                          ws=None, stream=None):
    """x, y [B, T+T_out, d_model]; weights stored out x in (a linear
    layer's weight): w_q [Hq*D, d_model], w_k, w_v [Hkv*D, d_model],
    w_o [d_model, Hq*D]; caches [B, Hkv, cap, D]."""
    B, M, d_model = x.shape
    T = M - int(T_out)
    Hkv, cap, D = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    Hq = w_q.shape[0] // D
    if tuple(k_cache.shape) != (B, Hkv, cap, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, Hkv, cap, D]")
    if (tuple(w_q.shape) != (Hq * D, d_model) or
            tuple(w_k.shape) != (Hkv * D, d_model) or w_v.shape != w_k.shape or
            tuple(w_o.shape) != (d_model, Hq * D)):
        raise ValueError("weights must be [Hq*D, d_model], [Hkv*D, d_model] "
                         "x2 and [d_model, Hq*D]")
    if y.shape != x.shape:
        raise ValueError("y must have x's shape")
    bf = torch.bfloat16
    f32 = torch.float32
    aff = (_vecs(Hq * D, (alpha, "alpha"), (beta, "beta"),
                 (alpha_x, "alpha_x"), (beta_x, "beta_x")) if int(T_out) else
           _vecs(Hq * D, (alpha, "alpha"), (beta, "beta")) +
           [_dev(alpha_x, "alpha_x", f32), _dev(beta_x, "beta_x", f32)])
    cl_p = _dev(_lens(cache_len, B), "cache_len", torch.int32)
    if ws is None:
        ws = _scratch(orthros_layer_workspace_bytes(B, T, int(T_out), d_model,
                                                    Hq, Hkv, D), x.device,
                      stream)
    _check(lib().orthros_layer_forward(
        _dev(x, "x", bf), _dev(w_q, "w_q", bf), _dev(w_k, "w_k", bf),
        _dev(w_v, "w_v", bf), _dev(w_o, "w_o", bf), *aff,
        _dev(k_cache, "k_cache", bf), _dev(v_cache, "v_cache", bf), cl_p,
        _dev(y, "y", bf), B, T, int(T_out), d_model, Hq, Hkv, D, cap, int(W),
        _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream, x)))


def orthros_check_device_errors(stream=None, device=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    _check(lib().orthros_check_device_errors(ctypes.c_void_p(stream.cuda_stream)))
