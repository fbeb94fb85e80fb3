"""Python binding of libsala: argument marshalling only.

Every step of the hot path runs in libsala's HIP kernels; this module only turns torch tensors
into pointers and sizes, allocates workspace through torch, passes torch's current stream and
raises on a non-OK status. It fails loudly (SalaError at import of the library) when
libsala.so is missing: there is no CPU fallback.

Entry points mirror include/sala.h: linear_prefill, linear_decode_step, kv_append, kv_pool,
block_select, sparse_attn, dense_attn, the backward calls, the packed variable-length (varlen)
calls (+ workspace_bytes, abi_version).
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SALA_LIBRARY may name another build of the library (the sanitizer-instrumented one in the tests)
LIB_PATH = os.environ.get("SALA_LIBRARY") or os.path.join(_PKG, "libsala.so")

SALA_F32, SALA_BF16 = 0, 1
OP_LINEAR_PREFILL, OP_BLOCK_SELECT, OP_SPARSE_ATTN, OP_DENSE_ATTN, OP_LINEAR_BACKWARD = 1, 2, 3, 4, 5
OP_SPARSE_ATTN_BACKWARD, OP_KV_NORM_BACKWARD, OP_SPARSE_DECODE_STEP = 6, 7, 8
STATUS = {0: "ok", 1: "null pointer", 2: "invalid", 3: "unsupported", 4: "workspace", 5: "hip"}


class SalaError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"libsala {what}: status {status} ({STATUS.get(status, '?')})")


class LinearDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("pos0", ctypes.c_int64), ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("chunk", ctypes.c_int32), ("reserved_", ctypes.c_int32)]


class SparseDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("n_local", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("scale", ctypes.c_float), ("reserved_", ctypes.c_int32),
                ("kv_len", ctypes.c_int64), ("kv_capacity", ctypes.c_int64)]


_VP = ctypes.c_void_p
_lib = None


def lib():
    """Load libsala.so once (raises SalaError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SalaError(-1, f"library not built: {LIB_PATH} missing (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.sala_linear_prefill.argtypes = [ctypes.POINTER(LinearDesc)] + [_VP] * 10 + [ctypes.c_size_t, _VP]
        L.sala_linear_decode_step.argtypes = [ctypes.POINTER(LinearDesc)] + [_VP] * 9
        L.sala_linear_decode_step_at.argtypes = [ctypes.POINTER(LinearDesc)] + [_VP] * 10
        L.sala_sparse_decode_step.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 13 + [ctypes.c_size_t, _VP]
        L.sala_sparse_decode_step_noalloc.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 13
        L.sala_linear_backward.argtypes = [ctypes.POINTER(LinearDesc)] + [_VP] * 17 + [ctypes.c_size_t, _VP]
        L.sala_sparse_attn_backward.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 15 + [ctypes.c_size_t, _VP]
        L.sala_kv_norm_backward.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 6 + [ctypes.c_size_t, _VP]
        L.sala_kv_append.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 7
        L.sala_kv_pool.argtypes = [ctypes.POINTER(SparseDesc), _VP, _VP, ctypes.c_int64, ctypes.c_int64, _VP]
        L.sala_block_select.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 6 + [ctypes.c_size_t, _VP]
        L.sala_sparse_attn.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 9 + [ctypes.c_size_t, _VP]
        L.sala_dense_attn.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 7 + [ctypes.c_size_t, _VP]
        L.sala_sparse_layer_uses_dense.argtypes = [ctypes.POINTER(SparseDesc)]
        L.sala_linear_prefill_varlen.argtypes = [ctypes.POINTER(LinearDesc)] + [_VP] * 12 + [ctypes.c_size_t, _VP]
        L.sala_kv_append_varlen.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 9
        L.sala_block_select_varlen.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 7 + [ctypes.c_size_t, _VP]
        L.sala_sparse_attn_varlen.argtypes = [ctypes.POINTER(SparseDesc)] + [_VP] * 10
        L.sala_varlen_query_blocks.argtypes = [ctypes.c_int32, _VP]
        L.sala_varlen_query_blocks.restype = ctypes.c_int64
        L.sala_varlen_workspace_bytes.argtypes = [ctypes.c_int, _VP, _VP, _VP]
        L.sala_varlen_workspace_bytes.restype = ctypes.c_size_t
        L.sala_workspace_bytes.argtypes = [ctypes.c_int, _VP]
        L.sala_workspace_bytes.restype = ctypes.c_size_t
        L.sala_status_str.argtypes = [ctypes.c_int]
        L.sala_status_str.restype = ctypes.c_char_p
        for name in ("sala_linear_prefill", "sala_linear_decode_step", "sala_linear_backward",
                     "sala_sparse_attn_backward", "sala_kv_norm_backward",
                     "sala_kv_append", "sala_kv_pool",
                     "sala_block_select", "sala_sparse_attn", "sala_dense_attn",
                     "sala_sparse_layer_uses_dense", "sala_abi_version", "sala_last_hip_error",
                     "sala_linear_prefill_varlen", "sala_kv_append_varlen", "sala_block_select_varlen",
                     "sala_sparse_attn_varlen", "sala_linear_decode_step_at", "sala_sparse_decode_step",
                     "sala_sparse_decode_step_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def abi_version():
    return lib().sala_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SALA_BF16
    if t.dtype == torch.float32:
        return SALA_F32
    raise SalaError(2, f"dtype {t.dtype} (need bfloat16 or float32)")


def _check(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise SalaError(2, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise SalaError(2, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SalaError(2, f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _call(fn, *args, what=""):
    st = fn(*args)
    if st != 0:
        raise SalaError(st, what)


def workspace_bytes(op, desc):
    n = lib().sala_workspace_bytes(op, ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise SalaError(2, "workspace_bytes: invalid descriptor")
    return n


def _workspace(op, desc, device, workspace):
    need = workspace_bytes(op, desc)
    if need == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(need, dtype=torch.uint8, device=device), need


def linear_desc(q, pos0, rope_base, eps, n_kv_heads=None, chunk=64):
    B, N, H, d = q.shape
    return LinearDesc(B, N, H, n_kv_heads or H, d, _dtype_code(q), int(pos0), float(rope_base), float(eps),
                      int(chunk), 0)


def linear_prefill(q, k, v, g, *, pos0=0, rope_base=10000.0, eps=1e-6, state_in=None,
                   state_out=None, q_norm_w=None, k_norm_w=None, out=None, workspace=None, chunk=64,
                   stream=None):
    """q, g: [B, N, H, d]; k, v: [B, N, Hkv, d] (bf16 or f32, Hkv dividing H); returns
    (out, state_out [B, Hkv, d, d] f32)."""
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _check(t, n, q.dtype)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    for n, t, hh in (("k", k, Hkv), ("v", v, Hkv), ("g", g, H)):
        if tuple(t.shape) != (B, N, hh, d):
            raise SalaError(2, f"{n} shape {tuple(t.shape)} != {(B, N, hh, d)}")
    if out is None:
        out = torch.empty_like(q)
    if state_out is None:
        state_out = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=q.device)
    for n, t in (("state_in", state_in), ("state_out", state_out), ("q_norm_w", q_norm_w),
                 ("k_norm_w", k_norm_w)):
        _check(t, n, torch.float32)
    desc = linear_desc(q, pos0, rope_base, eps, Hkv, chunk)
    ws, ws_bytes = _workspace(OP_LINEAR_PREFILL, desc, q.device, workspace)
    _call(lib().sala_linear_prefill, ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
          _ptr(q_norm_w), _ptr(k_norm_w), _ptr(state_in), _ptr(state_out), _ptr(out), _ptr(ws),
          ws_bytes, _stream(stream), what="linear_prefill")
    return out, state_out


def linear_backward(q, k, v, g, dout, *, pos0=0, rope_base=10000.0, eps=1e-6, state_in=None,
                    dstate_out=None, q_norm_w=None, k_norm_w=None, need_norm_w_grads=False,
                    need_dstate_in=True, workspace=None, stream=None):
    """Gradients of the linear layer (bf16 inputs [B, N, H, d], d = 128). Returns a dict with
    dq, dk, dv, dg [B, N, H, d] f32, dstate_in [B, H, d, d] f32 (or None) and, when
    need_norm_w_grads, dq_norm_w, dk_norm_w [d] f32."""
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g), ("dout", dout)):
        _check(t, n, torch.bfloat16)
    B, N, H, d = q.shape
    for n, t in (("k", k), ("v", v), ("g", g), ("dout", dout)):
        if tuple(t.shape) != (B, N, H, d):
            raise SalaError(2, f"{n} shape {tuple(t.shape)} != {(B, N, H, d)}")
    for n, t in (("state_in", state_in), ("dstate_out", dstate_out), ("q_norm_w", q_norm_w),
                 ("k_norm_w", k_norm_w)):
        _check(t, n, torch.float32)
    f32 = dict(dtype=torch.float32, device=q.device)
    grads = {n: torch.empty((B, N, H, d), **f32) for n in ("dq", "dk", "dv", "dg")}
    grads["dstate_in"] = torch.empty((B, H, d, d), **f32) if need_dstate_in else None
    grads["dq_norm_w"] = torch.empty(d, **f32) if need_norm_w_grads else None
    grads["dk_norm_w"] = torch.empty(d, **f32) if need_norm_w_grads else None
    desc = linear_desc(q, pos0, rope_base, eps)
    ws, ws_bytes = _workspace(OP_LINEAR_BACKWARD, desc, q.device, workspace)
    _call(lib().sala_linear_backward, ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
          _ptr(q_norm_w), _ptr(k_norm_w), _ptr(state_in), _ptr(dout), _ptr(dstate_out),
          *(_ptr(grads[n]) for n in ("dq", "dk", "dv", "dg", "dq_norm_w", "dk_norm_w", "dstate_in")),
          _ptr(ws), ws_bytes, _stream(stream), what="linear_backward")
    return grads


def linear_decode_step(q, k, v, g, state, pos, *, rope_base=10000.0, eps=1e-6, q_norm_w=None,
                       k_norm_w=None, out=None, stream=None):
    """q, g: [B, H, d]; k, v: [B, Hkv, d]; state [B, Hkv, d, d] f32 updated in place; returns
    out [B, H, d]."""
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _check(t, n, q.dtype)
    _check(state, "state", torch.float32)
    B, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    desc = LinearDesc(B, 1, H, k.shape[1], d, _dtype_code(q), int(pos), float(rope_base), float(eps), 64, 0)
    _call(lib().sala_linear_decode_step, ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
          _ptr(q_norm_w), _ptr(k_norm_w), _ptr(state), _ptr(out), _stream(stream),
          what="linear_decode_step")
    return out


def linear_decode_step_at(q, k, v, g, state, pos, *, rope_base=10000.0, eps=1e-6, q_norm_w=None, k_norm_w=None,
                          out=None, stream=None):
    """As linear_decode_step with token b at position pos[b] (pos: device int64 tensor [B])."""
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _check(t, n, q.dtype)
    _check(state, "state", torch.float32)
    _check(pos, "pos", torch.int64)
    B, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    desc = LinearDesc(B, 1, H, k.shape[1], d, _dtype_code(q), 0, float(rope_base), float(eps), 64, 0)
    _call(lib().sala_linear_decode_step_at, ctypes.byref(desc), _ptr(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
          _ptr(q_norm_w), _ptr(k_norm_w), _ptr(state), _ptr(out), _stream(stream), what="linear_decode_step_at")
    return out


def sparse_decode_step(q, k_new, v_new, g, k_cache, v_cache, k_pool, kv_lens, kv_max, *, topk=64, n_local=2,
                       eps=1e-6, scale=0.0, q_norm_w=None, k_norm_w=None, sel=None, out=None, workspace=None,
                       stream=None):
    """Sparse-layer decode step with sequence b's cache holding kv_lens[b] tokens once its new
    token is in (kv_lens: device int64 [B], each <= kv_max). q, g [B, Hq, d]; k_new, v_new
    [B, Hkv, d] bf16. Appends, selects (sel [B, Hkv, topk]) and attends; returns (out, sel)."""
    for n, t in (("q", q), ("g", g), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                 ("v_cache", v_cache)):
        _check(t, n, torch.bfloat16)
    _check(k_pool, "k_pool", torch.float32)
    _check(kv_lens, "kv_lens", torch.int64)
    B, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    desc = sparse_desc(batch=B, n_q=1, n_heads=Hq, n_kv_heads=Hkv, head_dim=d, dtype=q.dtype, kv_len=kv_max,
                       kv_capacity=cap, topk=topk, n_local=n_local, eps=eps, scale=scale)
    if sel is None:
        sel = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    ws, ws_bytes = _workspace(OP_SPARSE_DECODE_STEP, desc, q.device, workspace)
    _call(lib().sala_sparse_decode_step, ctypes.byref(desc), _ptr(kv_lens), _ptr(q), _ptr(q_norm_w), _ptr(k_new),
          _ptr(v_new), _ptr(k_norm_w), _ptr(g), _ptr(k_cache), _ptr(v_cache), _ptr(k_pool), _ptr(sel), _ptr(out),
          _ptr(ws), ws_bytes, _stream(stream), what="sparse_decode_step")
    return out, sel


def sparse_decode_step_noalloc(q, k_new, v_new, g, k_cache, v_cache, k_pool, kv_lens, kv_max, *, topk=64,
                               n_local=2, eps=1e-6, scale=0.0, q_norm_w=None, k_norm_w=None, sel=None, out=None,
                               stream=None):
    """sparse_decode_step with the library's static scratch array instead of a workspace (nothing
    is allocated by the library; sel and out are allocated here only when not given)."""
    for n, t in (("q", q), ("g", g), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                 ("v_cache", v_cache)):
        _check(t, n, torch.bfloat16)
    _check(k_pool, "k_pool", torch.float32)
    _check(kv_lens, "kv_lens", torch.int64)
    B, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    desc = sparse_desc(batch=B, n_q=1, n_heads=Hq, n_kv_heads=Hkv, head_dim=d, dtype=q.dtype, kv_len=kv_max,
                       kv_capacity=cap, topk=topk, n_local=n_local, eps=eps, scale=scale)
    if sel is None:
        sel = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _call(lib().sala_sparse_decode_step_noalloc, ctypes.byref(desc), _ptr(kv_lens), _ptr(q), _ptr(q_norm_w),
          _ptr(k_new), _ptr(v_new), _ptr(k_norm_w), _ptr(g), _ptr(k_cache), _ptr(v_cache), _ptr(k_pool), _ptr(sel),
          _ptr(out), _stream(stream), what="sparse_decode_step_noalloc")
    return out, sel


def sparse_desc(*, batch, n_q, n_heads, n_kv_heads, head_dim, dtype, kv_len, kv_capacity, topk=64,
                n_local=2, eps=1e-6, scale=0.0, block=64):
    code = dtype if isinstance(dtype, int) else (SALA_BF16 if dtype == torch.bfloat16 else SALA_F32)
    return SparseDesc(batch, n_q, n_heads, n_kv_heads, head_dim, code, block, topk, n_local,
                      float(eps), float(scale), 0, int(kv_len), int(kv_capacity))


def kv_append(k_new, v_new, k_cache, v_cache, k_pool, kv_len, *, eps=1e-6, k_norm_w=None,
              n_heads=None, stream=None):
    """k_new, v_new [B, n_q, Hkv, d]; caches [B, Hkv, cap, d]; k_pool [B, Hkv, cap/64, d] f32.
    kv_len = tokens in the cache after the append."""
    B, nq, Hkv, d = k_new.shape
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, n, k_new.dtype)
    _check(k_pool, "k_pool", torch.float32)
    desc = sparse_desc(batch=B, n_q=nq, n_heads=n_heads or Hkv, n_kv_heads=Hkv, head_dim=d,
                       dtype=k_new.dtype, kv_len=kv_len, kv_capacity=k_cache.shape[2], topk=3,
                       n_local=2, eps=eps)
    _call(lib().sala_kv_append, ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_norm_w),
          _ptr(k_cache), _ptr(v_cache), _ptr(k_pool), _stream(stream), what="kv_append")


def kv_pool(k_cache, k_pool, kv_len, blk_begin, blk_end, *, stream=None):
    B, Hkv, cap, d = k_cache.shape
    _check(k_cache, "k_cache")
    _check(k_pool, "k_pool", torch.float32)
    desc = sparse_desc(batch=B, n_q=1, n_heads=Hkv, n_kv_heads=Hkv, head_dim=d, dtype=k_cache.dtype,
                       kv_len=kv_len, kv_capacity=cap, topk=3, n_local=2)
    _call(lib().sala_kv_pool, ctypes.byref(desc), _ptr(k_cache), _ptr(k_pool), int(blk_begin),
          int(blk_end), _stream(stream), what="kv_pool")


def block_select(q, k_pool, kv_len, kv_capacity, *, n_kv_heads, topk=64, n_local=2, eps=1e-6,
                 q_norm_w=None, sel=None, sel_scores=None, workspace=None, stream=None):
    """q [B, n_q, Hq, d]; returns sel [B, Hkv, nqb, topk] int32. sel_scores: optional f32 tensor
    of sel's shape receiving each entry's block score (+inf forced, -inf padding)."""
    _check(q, "q")
    _check(k_pool, "k_pool", torch.float32)
    B, nq, Hq, d = q.shape
    desc = sparse_desc(batch=B, n_q=nq, n_heads=Hq, n_kv_heads=n_kv_heads, head_dim=d, dtype=q.dtype,
                       kv_len=kv_len, kv_capacity=kv_capacity, topk=topk, n_local=n_local, eps=eps)
    q0 = kv_len - nq
    nqb = (kv_len - 1) // 64 - q0 // 64 + 1
    if sel is None:
        sel = torch.empty((B, n_kv_heads, nqb, topk), dtype=torch.int32, device=q.device)
    ws, ws_bytes = _workspace(OP_BLOCK_SELECT, desc, q.device, workspace)
    _check(sel_scores, "sel_scores", torch.float32)
    _call(lib().sala_block_select, ctypes.byref(desc), _ptr(q), _ptr(q_norm_w), _ptr(k_pool),
          _ptr(sel), _ptr(sel_scores), _ptr(ws), ws_bytes, _stream(stream), what="block_select")
    return sel


def sparse_attn(q, k_cache, v_cache, g, sel, kv_len, *, topk=None, n_local=2, eps=1e-6, scale=0.0,
                q_norm_w=None, out=None, lse=None, workspace=None, stream=None):
    """q, g [B, n_q, Hq, d]; caches [B, Hkv, cap, d]; sel from block_select. Returns out.
    lse: optional [B, n_q, Hq] f32 tensor that receives each row's log2-sum-exp2 (bf16 prefill)."""
    for n, t in (("q", q), ("g", g), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, n, q.dtype)
    _check(sel, "sel", torch.int32)
    B, nq, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    desc = sparse_desc(batch=B, n_q=nq, n_heads=Hq, n_kv_heads=Hkv, head_dim=d, dtype=q.dtype,
                       kv_len=kv_len, kv_capacity=cap, topk=topk or sel.shape[-1], n_local=n_local,
                       eps=eps, scale=scale)
    if out is None:
        out = torch.empty_like(q)
    ws, ws_bytes = _workspace(OP_SPARSE_ATTN, desc, q.device, workspace)
    _check(lse, "lse", torch.float32)
    _call(lib().sala_sparse_attn, ctypes.byref(desc), _ptr(q), _ptr(q_norm_w), _ptr(k_cache),
          _ptr(v_cache), _ptr(g), _ptr(sel), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream),
          what="sparse_attn")
    return out


def sparse_attn_backward(q, k_cache, v_cache, g, sel, kv_len, dout, *, topk=None, n_local=2, eps=1e-6,
                         scale=0.0, q_norm_w=None, need_norm_w_grad=False, out=None, lse=None, workspace=None,
                         stream=None):
    """Gradients of sparse_attn (bf16, prefill, fixed selection). Returns a dict with dq, dg
    [B, n_q, Hq, d], dk_cache, dv_cache [B, Hkv, cap, d] (all f32) and dq_norm_w [d] f32 when
    need_norm_w_grad (else None). out, lse: the forward's output and lse (both or neither);
    given, the forward is not rerun."""
    for n, t in (("q", q), ("g", g), ("k_cache", k_cache), ("v_cache", v_cache), ("dout", dout), ("out", out)):
        _check(t, n, torch.bfloat16)
    _check(lse, "lse", torch.float32)
    _check(sel, "sel", torch.int32)
    B, nq, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    desc = sparse_desc(batch=B, n_q=nq, n_heads=Hq, n_kv_heads=Hkv, head_dim=d, dtype=q.dtype,
                       kv_len=kv_len, kv_capacity=cap, topk=topk or sel.shape[-1], n_local=n_local,
                       eps=eps, scale=scale)
    f32 = dict(dtype=torch.float32, device=q.device)
    r = dict(dq=torch.empty((B, nq, Hq, d), **f32), dg=torch.empty((B, nq, Hq, d), **f32),
             dk_cache=torch.empty((B, Hkv, cap, d), **f32), dv_cache=torch.empty((B, Hkv, cap, d), **f32),
             dq_norm_w=torch.empty(d, **f32) if need_norm_w_grad else None)
    ws, ws_bytes = _workspace(OP_SPARSE_ATTN_BACKWARD, desc, q.device, workspace)
    _call(lib().sala_sparse_attn_backward, ctypes.byref(desc), _ptr(q), _ptr(q_norm_w), _ptr(k_cache),
          _ptr(v_cache), _ptr(g), _ptr(sel), _ptr(dout), _ptr(out), _ptr(lse), _ptr(r["dq"]), _ptr(r["dk_cache"]),
          _ptr(r["dv_cache"]), _ptr(r["dg"]), _ptr(r["dq_norm_w"]), _ptr(ws), ws_bytes, _stream(stream),
          what="sparse_attn_backward")
    return r


def kv_norm_backward(k_new, dk_cache, kv_len, *, n_heads, eps=1e-6, k_norm_w=None, need_norm_w_grad=False,
                     workspace=None, stream=None):
    """Backward of the key normalisation of kv_append for the appended tokens. k_new bf16
    [B, n_q, Hkv, d]; dk_cache f32 [B, Hkv, cap, d]. Returns (dk_new f32, dk_norm_w f32 or None)."""
    _check(k_new, "k_new", torch.bfloat16)
    _check(dk_cache, "dk_cache", torch.float32)
    B, nq, Hkv, d = k_new.shape
    cap = dk_cache.shape[2]
    desc = sparse_desc(batch=B, n_q=nq, n_heads=n_heads, n_kv_heads=Hkv, head_dim=d, dtype=k_new.dtype,
                       kv_len=kv_len, kv_capacity=cap, topk=3, n_local=2, eps=eps)
    dk = torch.empty((B, nq, Hkv, d), dtype=torch.float32, device=k_new.device)
    dw = torch.empty(d, dtype=torch.float32, device=k_new.device) if need_norm_w_grad else None
    ws, ws_bytes = _workspace(OP_KV_NORM_BACKWARD, desc, k_new.device, workspace)
    _call(lib().sala_kv_norm_backward, ctypes.byref(desc), _ptr(k_new), _ptr(k_norm_w), _ptr(dk_cache), _ptr(dk),
          _ptr(dw), _ptr(ws), ws_bytes, _stream(stream), what="kv_norm_backward")
    return dk, dw


def dense_attn(q, k_cache, v_cache, g, kv_len, *, eps=1e-6, scale=0.0, q_norm_w=None, out=None,
               workspace=None, stream=None):
    """Dense mode of the sparse layer: causal attention over every cached block up to each
    query's own. q, g [B, n_q, Hq, d]; caches [B, Hkv, cap, d]. Returns out."""
    for n, t in (("q", q), ("g", g), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, n, q.dtype)
    B, nq, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    desc = sparse_desc(batch=B, n_q=nq, n_heads=Hq, n_kv_heads=Hkv, head_dim=d, dtype=q.dtype,
                       kv_len=kv_len, kv_capacity=cap, topk=3, n_local=2, eps=eps, scale=scale)
    if out is None:
        out = torch.empty_like(q)
    ws, ws_bytes = _workspace(OP_DENSE_ATTN, desc, q.device, workspace)
    _call(lib().sala_dense_attn, ctypes.byref(desc), _ptr(q), _ptr(q_norm_w), _ptr(k_cache),
          _ptr(v_cache), _ptr(g), _ptr(out), _ptr(ws), ws_bytes, _stream(stream), what="dense_attn")
    return out


def sparse_layer_uses_dense(*, batch, n_q, n_heads, n_kv_heads, head_dim, dtype, kv_len, kv_capacity,
                            topk=64, n_local=2):
    """The library's dense/sparse switch for a sparse-layer call (1 dense, 0 sparse)."""
    desc = sparse_desc(batch=batch, n_q=n_q, n_heads=n_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                       dtype=dtype, kv_len=kv_len, kv_capacity=kv_capacity, topk=topk, n_local=n_local)
    r = lib().sala_sparse_layer_uses_dense(ctypes.byref(desc))
    if r < 0:
        raise SalaError(2, "sparse_layer_uses_dense: invalid descriptor")
    return bool(r)


# ---------------------------------------------------------------- packed variable-length batches


class Varlen:
    """Host arrays of a packed batch: seqlens (token counts of this call) and pos0 (position of
    each sequence's first token of this call). cu_seqlens / pos0 are kept as ctypes arrays, which
    the library reads during each call."""

    def __init__(self, seqlens, pos0=None):
        seqlens = [int(n) for n in seqlens]
        self.nseq = len(seqlens)
        cu = [0]
        for n in seqlens:
            cu.append(cu[-1] + n)
        self.seqlens, self.cu = seqlens, cu
        self.pos0 = [0] * self.nseq if pos0 is None else [int(p) for p in pos0]
        self._cu = (ctypes.c_int32 * (self.nseq + 1))(*cu)
        self._pos0 = (ctypes.c_int64 * max(1, self.nseq))(*self.pos0)

    @property
    def total(self):
        return self.cu[-1]

    def query_blocks(self):
        n = lib().sala_varlen_query_blocks(self.nseq, self._cu)
        if n < 0:
            raise SalaError(2, "varlen_query_blocks")
        return n

    def args(self):
        return self._cu, self._pos0


def varlen_workspace_bytes(op, desc, vl):
    n = lib().sala_varlen_workspace_bytes(op, ctypes.byref(desc), *vl.args())
    if n == ctypes.c_size_t(-1).value:
        raise SalaError(2, "varlen_workspace_bytes: invalid arguments")
    return n


def _varlen_workspace(op, desc, vl, device, workspace):
    need = varlen_workspace_bytes(op, desc, vl)
    if need == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(need, dtype=torch.uint8, device=device), need


def linear_prefill_varlen(q, k, v, g, vl, *, rope_base=10000.0, eps=1e-6, state_in=None, state_out=None,
                          q_norm_w=None, k_norm_w=None, out=None, workspace=None, stream=None):
    """q, k, v, g: [T, H, d] bf16 packed by vl (Varlen); states [nseq, H, d, d] f32. Returns
    (out [T, H, d], state_out)."""
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _check(t, n, torch.bfloat16)
    T, H, d = q.shape
    if T != vl.total:
        raise SalaError(2, f"packed tokens {T} != sum of seqlens {vl.total}")
    if out is None:
        out = torch.empty_like(q)
    if state_out is None:
        state_out = torch.empty((vl.nseq, k.shape[1], d, d), dtype=torch.float32, device=q.device)
    for n, t in (("state_in", state_in), ("state_out", state_out), ("q_norm_w", q_norm_w),
                 ("k_norm_w", k_norm_w)):
        _check(t, n, torch.float32)
    desc = LinearDesc(vl.nseq, T, H, k.shape[1], d, SALA_BF16, 0, float(rope_base), float(eps), 64, 0)
    ws, ws_bytes = _varlen_workspace(OP_LINEAR_PREFILL, desc, vl, q.device, workspace)
    _call(lib().sala_linear_prefill_varlen, ctypes.byref(desc), *vl.args(), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
          _ptr(q_norm_w), _ptr(k_norm_w), _ptr(state_in), _ptr(state_out), _ptr(out), _ptr(ws), ws_bytes,
          _stream(stream), what="linear_prefill_varlen")
    return out, state_out


def _sparse_varlen_desc(vl, Hq, Hkv, d, cap, topk, n_local, eps, scale=0.0):
    return sparse_desc(batch=vl.nseq, n_q=vl.total, n_heads=Hq, n_kv_heads=Hkv, head_dim=d, dtype=torch.bfloat16,
                       kv_len=0, kv_capacity=cap, topk=topk, n_local=n_local, eps=eps, scale=scale)


def kv_append_varlen(k_new, v_new, k_cache, v_cache, k_pool, vl, *, n_heads=None, eps=1e-6, k_norm_w=None,
                     stream=None):
    """k_new, v_new [T, Hkv, d] bf16 packed by vl; caches [nseq, Hkv, cap, d]; k_pool
    [nseq, Hkv, cap/64, d] f32. Sequence s's tokens go to positions pos0[s] .."""
    T, Hkv, d = k_new.shape
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, n, torch.bfloat16)
    _check(k_pool, "k_pool", torch.float32)
    desc = _sparse_varlen_desc(vl, n_heads or Hkv, Hkv, d, k_cache.shape[2], 3, 2, eps)
    _call(lib().sala_kv_append_varlen, ctypes.byref(desc), *vl.args(), _ptr(k_new), _ptr(v_new), _ptr(k_norm_w),
          _ptr(k_cache), _ptr(v_cache), _ptr(k_pool), _stream(stream), what="kv_append_varlen")


def block_select_varlen(q, k_pool, vl, kv_capacity, *, n_kv_heads, topk=64, n_local=2, eps=1e-6, q_norm_w=None,
                        sel=None, workspace=None, stream=None):
    """q [T, Hq, d] bf16 packed by vl; returns sel [query_blocks * Hkv, topk] int32: the
    per-sequence [Hkv, nqb_s, topk] blocks one after another."""
    _check(q, "q", torch.bfloat16)
    _check(k_pool, "k_pool", torch.float32)
    T, Hq, d = q.shape
    desc = _sparse_varlen_desc(vl, Hq, n_kv_heads, d, kv_capacity, topk, n_local, eps)
    if sel is None:
        sel = torch.empty((vl.query_blocks() * n_kv_heads, topk), dtype=torch.int32, device=q.device)
    ws, ws_bytes = _varlen_workspace(OP_BLOCK_SELECT, desc, vl, q.device, workspace)
    _call(lib().sala_block_select_varlen, ctypes.byref(desc), *vl.args(), _ptr(q), _ptr(q_norm_w), _ptr(k_pool),
          _ptr(sel), _ptr(ws), ws_bytes, _stream(stream), what="block_select_varlen")
    return sel


def sparse_attn_varlen(q, k_cache, v_cache, g, sel, vl, *, topk=None, n_local=2, eps=1e-6, scale=0.0,
                       q_norm_w=None, out=None, stream=None):
    """q, g [T, Hq, d] bf16 packed by vl; caches [nseq, Hkv, cap, d]; sel from
    block_select_varlen. Returns out [T, Hq, d]."""
    for n, t in (("q", q), ("g", g), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, n, torch.bfloat16)
    _check(sel, "sel", torch.int32)
    T, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    desc = _sparse_varlen_desc(vl, Hq, Hkv, d, cap, topk or sel.shape[-1], n_local, eps, scale)
    if out is None:
        out = torch.empty_like(q)
    _call(lib().sala_sparse_attn_varlen, ctypes.byref(desc), *vl.args(), _ptr(q), _ptr(q_norm_w), _ptr(k_cache),
          _ptr(v_cache), _ptr(g), _ptr(sel), _ptr(out), _stream(stream), what="sparse_attn_varlen")
    return out
