"""Python binding of libpa, the paged KV-cache hot path for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libpa.so`` behind the C ABI declared in ``include/pa.h``.  There is no CPU
fallback -- if the library is missing or fails to load, every call raises.

Pools: K is [NB][Hkv][D/x][bs][x] with x = 16 / element size (16-byte
granules, token-minor), V is [NB][Hkv][bs][D] (see include/pa.h).

Tensors are torch tensors on the current HIP device; element types are
``torch.bfloat16`` or ``torch.float32`` for K/V/Q, ``torch.int32`` for block
tables, context lengths, positions and block mappings, ``torch.int64`` for
slots.  Calls are asynchronous on torch's current stream (or ``stream=``).
"""

from __future__ import annotations

import ctypes
import os

# PA_LIBRARY may name another build of the same library (the host-sanitized
# one of build.py --sanitize); by default the in-tree libpa.so is loaded.
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F32 = 0
PA_BF16 = 1
PA_DECODE_VECTOR_ONLY = 1
PA_NOALLOC_MAX_WORKSPACE = 34 << 20  # bytes (include/pa.h)

STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_DTYPE",
          4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_HIP", 7: "PA_ERR_CAPACITY"}

# name -> (restype, argtypes); mirrors include/pa.h and include/pa_block_manager.h
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class BMStats(ctypes.Structure):
    """pa_bm_stats (include/pa_block_manager.h)."""
    _fields_ = [("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("used_blocks", ctypes.c_int32), ("shared_blocks", ctypes.c_int32),
                ("live_sequences", ctypes.c_int32), ("logical_blocks", ctypes.c_int64),
                ("logical_tokens", ctypes.c_int64), ("stored_tokens", ctypes.c_int64),
                ("physical_slots", ctypes.c_int64), ("swapped_sequences", ctypes.c_int32),
                ("num_host_blocks", ctypes.c_int32), ("free_host_blocks", ctypes.c_int32)]


SIGNATURES = {
    "pa_abi_version": (_I32, []),
    "pa_bm_create": (ctypes.c_int, [_I32, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_void_p)]),
    "pa_bm_create_with_host": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32,
                                              ctypes.POINTER(ctypes.c_void_p)]),
    "pa_bm_destroy": (None, [_P]),
    "pa_bm_swap_out": (ctypes.c_int, [_P, _P, _I32, _P, _P]),
    "pa_bm_swap_in": (ctypes.c_int, [_P, _P, _I32, _P, _P]),
    "pa_bm_add_sequence": (ctypes.c_int, [_P, _P]),
    "pa_bm_fork": (ctypes.c_int, [_P, _I32, _P]),
    "pa_bm_free_sequence": (ctypes.c_int, [_P, _I32]),
    "pa_bm_append": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _P]),
    "pa_bm_tables": (ctypes.c_int, [_P, _P, _I32, _P, _P]),
    "pa_bm_get_stats": (ctypes.c_int, [_P, ctypes.POINTER(BMStats)]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_probe_read": (ctypes.c_int, [_P, _I64, _P, _I32, _P]),
    "pa_probe_gather": (ctypes.c_int, [_P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32,
                                       ctypes.c_int, _P, _I32, _P]),
    "pa_compute_slots": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P, _I32, _I32, _I32, _P]),
    "pa_write_kv": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32,
                                   ctypes.c_int, _P]),
    "pa_write_kv_at": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _P, _P, _I32, _I64, _I32,
                                      _I32, _I32, _I32, ctypes.c_int, _P, _P]),
    "pa_copy_blocks": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, ctypes.c_int, _P]),
    "pa_swap_blocks": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                      ctypes.c_int, _P]),
    "pa_decode_partition_size": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "pa_decode_streamk_workers": (_I32, [_I32, _I32, _I32, _I32, ctypes.c_int, ctypes.c_uint32]),
    "pa_decode_workspace_size": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                    ctypes.c_int, ctypes.c_uint32]),
    "pa_decode_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                           _I32, _I32, _I32, ctypes.c_float, _I32, _P,
                                           ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32, _P]),
    "pa_decode_attention_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I32,
                                                  _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                  ctypes.c_float, _I32, _P, ctypes.c_size_t,
                                                  ctypes.c_int, ctypes.c_uint32, _P]),
    "pa_decode_attention_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I32,
                                                   _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                   ctypes.c_float, _I32, ctypes.c_int,
                                                   ctypes.c_uint32, _P]),
    "pa_decode_shared_workspace_size": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, ctypes.c_int]),
    "pa_decode_attention_shared": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P,
                                                  _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                  _I32, ctypes.c_float, _P, ctypes.c_size_t,
                                                  ctypes.c_int, _P]),
    "pa_prefill_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                            _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                                            ctypes.c_int, _P]),
}


class PAError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")


_lib = None


def lib():
    """The loaded libpa (ctypes.CDLL).  torch is imported first so that libpa
    binds to the HIP runtime torch already loaded (same soname), and streams
    and device pointers from torch are valid in the library."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (loads torch's HIP runtime)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m paged_kv_cache_188_amd.build` "
                "(there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn, code):
    if code != 0:
        raise PAError(fn, code)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported element type {t.dtype}")


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _pools(k_cache, v_cache):
    """(NB, Hkv, bs, D) from the K [NB][Hkv][D/x][bs][x] and V [NB][Hkv][bs][D]
    pools; checks that they agree and that x is the 16-byte granule."""
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("K pool must be [NB][Hkv][D/x][bs][x] and V pool [NB][Hkv][bs][D]")
    nb, hkv, dx, bs, x = k_cache.shape
    if x * k_cache.element_size() != 16:
        raise ValueError("K pool granule must be 16 bytes")
    if tuple(v_cache.shape) != (nb, hkv, bs, dx * x):
        raise ValueError("K and V pools disagree")
    _need(k_cache, k_cache.dtype, "k_cache")
    _need(v_cache, k_cache.dtype, "v_cache")
    return nb, hkv, bs, dx * x


def _shape(t, shape, name):
    """ValueError unless tensor t (if given) has exactly `shape`: a buffer of
    the wrong size would make a kernel read or write past its end."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")


class PreparedCall:
    """One library call whose arguments were validated and marshalled once.

    Calling it issues the same launch(es) again on the same stream, with the
    same device buffers (their contents may change between calls): the
    per-call host work is one foreign-function call.  The tensors the call
    reads and writes are kept alive by the object.  ``result`` is what the
    unprepared call returns (the output tensor)."""

    __slots__ = ("_fn", "_name", "_args", "_keep", "result")

    def __init__(self, name, args, keep, result):
        self._fn = getattr(lib(), name)
        self._name = name
        self._args = tuple(args)
        self._keep = keep
        self.result = result

    def __call__(self):
        code = self._fn(*self._args)
        if code != 0:
            raise PAError(self._name, code)
        return self.result


# ---------------------------------------------------------------------------
# operations
# ---------------------------------------------------------------------------

def compute_slots(block_tables, positions, block_size, num_blocks, seq_ids=None, out=None,
                  stream=None):
    """slot[j] = table[seq][pos // bs] * bs + pos % bs (int64), -1 for padding
    or invalid tokens.  ``seq_ids=None``: token j belongs to sequence j."""
    import torch
    if block_tables.dim() != 2 or positions.dim() != 1:
        raise ValueError("block_tables must be [S][MB] and positions [T]")
    n = positions.numel()
    _shape(seq_ids, (n,), "seq_ids")
    _shape(out, (n,), "out")
    _need(block_tables, torch.int32, "block_tables")
    _need(positions, torch.int32, "positions")
    if seq_ids is not None:
        _need(seq_ids, torch.int32, "seq_ids")
    if out is None:
        out = torch.empty(n, dtype=torch.int64, device=positions.device)
    _need(out, torch.int64, "out")
    s, mb = block_tables.shape
    _check("pa_compute_slots", lib().pa_compute_slots(
        _ptr(out), _ptr(block_tables), s, mb, _ptr(seq_ids), _ptr(positions), n, block_size,
        num_blocks, _stream(stream)))
    return out


def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None):
    """Store k_new/v_new [T][Hkv][D] in the pools at their slots."""
    import torch
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    _need(slot_mapping, torch.int64, "slot_mapping")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("new K/V must have the pool's element type")
    t = slot_mapping.numel()
    if k_new.shape[0] != t or v_new.shape != k_new.shape or tuple(k_new.shape[1:]) != (hkv, d):
        raise ValueError("k_new/v_new must be [T][Hkv][D] matching slot_mapping")
    if t and (k_new.stride(2) != 1 or k_new.stride(1) != d or v_new.stride() != k_new.stride()):
        raise ValueError("k_new/v_new rows must be contiguous [Hkv][D] with one token stride")
    _check("pa_write_kv", lib().pa_write_kv(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), t,
        k_new.stride(0) if t else 0, nb, bs, hkv, d, _dtype_code(k_cache), _stream(stream)))


def write_kv_at(k_cache, v_cache, k_new, v_new, block_tables, positions, seq_ids=None,
                slots_out=None, stream=None, prepare=False):
    """compute_slots + write_kv in one launch: token j goes to the slot of
    (seq_ids[j] or j, positions[j]); the slots are also written to
    ``slots_out`` when given.  With ``prepare=True`` the validated call is
    returned as a PreparedCall instead of being issued."""
    import torch
    if block_tables.dim() != 2 or positions.dim() != 1:
        raise ValueError("block_tables must be [S][MB] and positions [T]")
    _shape(seq_ids, positions.shape, "seq_ids")
    _shape(slots_out, positions.shape, "slots_out")
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    _need(block_tables, torch.int32, "block_tables")
    _need(positions, torch.int32, "positions")
    if seq_ids is not None:
        _need(seq_ids, torch.int32, "seq_ids")
    if slots_out is not None:
        _need(slots_out, torch.int64, "slots_out")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("new K/V must have the pool's element type")
    t = positions.numel()
    if k_new.shape[0] != t or v_new.shape != k_new.shape or tuple(k_new.shape[1:]) != (hkv, d):
        raise ValueError("k_new/v_new must be [T][Hkv][D] matching positions")
    if t and (k_new.stride(2) != 1 or k_new.stride(1) != d or v_new.stride() != k_new.stride()):
        raise ValueError("k_new/v_new rows must be contiguous [Hkv][D] with one token stride")
    s, mb = block_tables.shape
    call = PreparedCall("pa_write_kv_at", (
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_tables), s, mb,
        _ptr(seq_ids), _ptr(positions), t, k_new.stride(0) if t else 0, nb, bs, hkv, d,
        _dtype_code(k_cache), _ptr(slots_out), _stream(stream)),
        (k_cache, v_cache, k_new, v_new, block_tables, positions, seq_ids, slots_out), None)
    return call if prepare else call()


def copy_blocks(k_cache, v_cache, block_mapping, stream=None, prepare=False):
    """For each (src, dst) row of block_mapping [n][2]: block dst := block src.
    With ``prepare=True`` the validated call is returned as a PreparedCall
    instead of being issued."""
    import torch
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [n][2] (src, dst)")
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    _need(block_mapping, torch.int32, "block_mapping")
    n = block_mapping.shape[0]
    call = PreparedCall("pa_copy_blocks", (
        _ptr(k_cache), _ptr(v_cache), _ptr(block_mapping), n, nb, bs, hkv, d,
        _dtype_code(k_cache), _stream(stream)), (k_cache, v_cache, block_mapping), None)
    return call if prepare else call()


def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping, stream=None):
    """For each (src, dst) row of block_mapping [n][2] (a device int32
    tensor): block dst of (dst_k, dst_v) := block src of (src_k, src_v).
    Either pool pair may be pinned host tensors (pin_memory=True)."""
    import torch
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [n][2] (src, dst)")
    dnb, hkv, bs, d = _host_or_device_pools(dst_k, dst_v)
    snb, hkv2, bs2, d2 = _host_or_device_pools(src_k, src_v)
    if (hkv, bs, d) != (hkv2, bs2, d2) or dst_k.dtype != src_k.dtype:
        raise ValueError("the two pool pairs disagree in block shape or element type")
    _need(block_mapping, torch.int32, "block_mapping")
    n = block_mapping.shape[0]
    _check("pa_swap_blocks", lib().pa_swap_blocks(
        _ptr(dst_k), _ptr(dst_v), _ptr(src_k), _ptr(src_v), _ptr(block_mapping), n, snb, dnb,
        bs, hkv, d, _dtype_code(src_k), _stream(stream)))


def _host_or_device_pools(k_cache, v_cache):
    """_pools for a pool pair in device memory or in pinned host memory."""
    if not (k_cache.is_cuda and v_cache.is_cuda):
        if not (k_cache.is_pinned() and v_cache.is_pinned()):
            raise TypeError("host pools must be pinned (pin_memory=True)")
        if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
            raise TypeError("pools must be contiguous")
        if k_cache.dim() != 5 or v_cache.dim() != 4:
            raise ValueError("K pool must be [NB][Hkv][D/x][bs][x] and V pool [NB][Hkv][bs][D]")
        nb, hkv, dx, bs, x = k_cache.shape
        if x * k_cache.element_size() != 16 or tuple(v_cache.shape) != (nb, hkv, bs, dx * x):
            raise ValueError("K and V pools disagree")
        return nb, hkv, bs, dx * x
    return _pools(k_cache, v_cache)


def decode_partition_size(num_seqs, num_kv_heads, block_size, max_context_len, partition_size=0):
    return int(lib().pa_decode_partition_size(num_seqs, num_kv_heads, block_size,
                                              max_context_len, partition_size))


def decode_streamk_workers(num_seqs, head_dim, block_size, partition_size=0, dtype=None,
                           vector_only=False):
    """Waves the stream-K path launches (0: the call takes fixed partitions)."""
    import torch
    code = PA_F32 if dtype == torch.float32 else PA_BF16
    return int(lib().pa_decode_streamk_workers(num_seqs, head_dim, block_size, partition_size,
                                               code, PA_DECODE_VECTOR_ONLY if vector_only else 0))


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_context_len, partition_size=0, dtype=None, vector_only=False):
    """Workspace bytes for decode_attention with the same arguments; dtype is
    a torch dtype (default bfloat16)."""
    import torch
    code = PA_F32 if dtype == torch.float32 else PA_BF16
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len, partition_size, code,
                                              PA_DECODE_VECTOR_ONLY if vector_only else 0))


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                     partition_size=0, workspace=None, out=None, vector_only=False, stream=None,
                     k_new=None, v_new=None, prepare=False):
    """Paged decode attention; returns float32 [S][Hq][D].  ``workspace`` (a
    uint8 device tensor) is allocated here when not given.  With ``k_new`` /
    ``v_new`` ([S][Hkv][D]) each sequence's new token (position ctx-1) is
    stored in the pools and attended in the same call
    (pa_decode_attention_append).  With ``prepare=True`` nothing is launched:
    the validated call is returned as a PreparedCall, to be issued later (as
    often as wanted) with the same buffers."""
    import torch
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [S][Hq][D] and block_tables [S][MB]")
    s, hq, d = q.shape
    mb = block_tables.shape[1]
    _shape(block_tables, (s, mb), "block_tables")
    _shape(context_lens, (s,), "context_lens")
    _shape(out, (s, hq, d), "out")
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("q and the pools disagree in head_dim")
    _need(q, k_cache.dtype, "q")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    need = decode_workspace_size(s, hq, hkv, d, bs, max_context_len, partition_size,
                                 k_cache.dtype, vector_only)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    ws = (_ptr(workspace) if workspace is not None else None,
          workspace.numel() if workspace is not None else 0)
    tail = (_dtype_code(k_cache), PA_DECODE_VECTOR_ONLY if vector_only else 0, _stream(stream))
    keep = (q, k_cache, v_cache, block_tables, context_lens, workspace, out, k_new, v_new)
    if k_new is not None:
        if v_new is None or k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
            raise TypeError("k_new and v_new must both be given, with the pool's element type")
        if k_new.shape != (s, hkv, d) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [S][Hkv][D]")
        if k_new.stride(2) != 1 or k_new.stride(1) != d or v_new.stride() != k_new.stride():
            raise ValueError("k_new/v_new rows must be contiguous [Hkv][D] with one token stride")
        name = "pa_decode_attention_append"
        args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                k_new.stride(0), _ptr(block_tables), _ptr(context_lens), s, hq, hkv, d, bs, nb,
                mb, int(max_context_len), float(scale), int(partition_size)) + ws + tail
    else:
        name = "pa_decode_attention"
        args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                _ptr(context_lens), s, hq, hkv, d, bs, nb, mb, int(max_context_len),
                float(scale), int(partition_size)) + ws + tail
    call = PreparedCall(name, args, keep, out)
    return call if prepare else call()


def decode_attention_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale,
                             max_context_len, partition_size=0, out=None, vector_only=False,
                             stream=None, k_new=None, v_new=None):
    """decode_attention (k_new/v_new None) or its append form, through
    pa_decode_attention_noalloc: no workspace argument and nothing allocated
    by the library (``out`` is allocated here when not given).  Calls on one
    GPU share the library's static workspace and must not overlap."""
    import torch
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [S][Hq][D] and block_tables [S][MB]")
    s, hq, d = q.shape
    mb = block_tables.shape[1]
    _shape(context_lens, (s,), "context_lens")
    _shape(out, (s, hq, d), "out")
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("q and the pools disagree in head_dim")
    _need(q, k_cache.dtype, "q")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if (k_new is None) != (v_new is None):
        raise TypeError("give both k_new and v_new, or neither")
    stride = 0
    if k_new is not None:
        if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
            raise TypeError("k_new and v_new must have the pool's element type")
        if k_new.shape != (s, hkv, d) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [S][Hkv][D]")
        if k_new.stride(2) != 1 or k_new.stride(1) != d or v_new.stride() != k_new.stride():
            raise ValueError("k_new/v_new rows must be contiguous [Hkv][D] with one token stride")
        stride = k_new.stride(0)
    if out is None:
        out = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    _check("pa_decode_attention_noalloc", lib().pa_decode_attention_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), stride,
        _ptr(block_tables), _ptr(context_lens), s, hq, hkv, d, bs, nb, mb, int(max_context_len),
        float(scale), int(partition_size), _dtype_code(k_cache),
        PA_DECODE_VECTOR_ONLY if vector_only else 0, _stream(stream)))
    return out


def shared_prefix_groups(block_tables, context_lens, block_size, group):
    """Host-side grouping for decode_attention_shared: (group_start,
    shared_len) as int32 numpy arrays, from host copies of the block tables
    [S][MB] and context lengths [S].

    Consecutive sequences are grouped while they share leading physical
    blocks with the group's first member, at most 16 // group of them (the
    sequences whose query heads fill one matrix-core tile; group = query
    heads per KV head), and only while a new member does not lower the
    group's saving, (members - 1) x shared blocks.  shared_len is the shared
    block count times block_size (0 for a lone sequence); the library trims
    it further."""
    import numpy as np
    bt = np.asarray(block_tables)
    ctx = np.asarray(context_lens).astype(np.int64)
    S = ctx.shape[0]
    cap = max(1, 16 // int(group))

    def used(i):
        n = int(-(-max(int(ctx[i]), 0) // block_size))
        return bt[i, :min(n, bt.shape[1])]

    def common(a, b):
        m = min(a.shape[0], b.shape[0])
        neq = np.nonzero((a[:m] != b[:m]) | (a[:m] < 0))[0]
        return int(neq[0]) if neq.size else m

    starts, lens = [0], []
    i = 0
    while i < S:
        first = used(i)
        members, blocks = 1, 0
        while i + members < S and members < cap:
            c = common(first, used(i + members))
            new = c if members == 1 else min(blocks, c)
            if new == 0 or members * new < (members - 1) * blocks:
                break
            blocks = new
            members += 1
        i += members
        starts.append(i)
        lens.append(blocks * block_size if members > 1 else 0)
    return np.asarray(starts, dtype=np.int32), np.asarray(lens, dtype=np.int32)


def decode_shared_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype=None):
    """Workspace bytes for decode_attention_shared (bf16 only; 0 = unsupported)."""
    import torch
    code = PA_F32 if dtype == torch.float32 else PA_BF16
    return int(lib().pa_decode_shared_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                     head_dim, code))


def decode_attention_shared(q, k_cache, v_cache, block_tables, context_lens, group_start,
                            shared_len, scale, max_context_len, workspace=None, out=None,
                            stream=None, k_new=None, v_new=None, prepare=False):
    """decode_attention (or its append form, with k_new / v_new) for groups
    of consecutive sequences whose first shared_len[g] tokens map to the same
    physical blocks (group g = sequences group_start[g] .. group_start[g+1]-1;
    int32 device tensors of G+1 and G entries): each shared block is read
    once per group (pa_decode_attention_shared)."""
    import torch
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [S][Hq][D] and block_tables [S][MB]")
    s, hq, d = q.shape
    mb = block_tables.shape[1]
    _shape(block_tables, (s, mb), "block_tables")
    _shape(context_lens, (s,), "context_lens")
    _shape(out, (s, hq, d), "out")
    if group_start.dim() != 1 or group_start.numel() < 2:
        raise ValueError("group_start must be [num_groups + 1]")
    ng = group_start.numel() - 1
    _shape(shared_len, (ng,), "shared_len")
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("q and the pools disagree in head_dim")
    _need(q, k_cache.dtype, "q")
    for t, name in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                    (group_start, "group_start"), (shared_len, "shared_len")):
        _need(t, torch.int32, name)
    need = decode_shared_workspace_size(s, hq, hkv, d, k_cache.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    if (k_new is None) != (v_new is None):
        raise TypeError("give both k_new and v_new, or neither")
    stride = 0
    if k_new is not None:
        if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
            raise TypeError("k_new and v_new must have the pool's element type")
        if k_new.shape != (s, hkv, d) or v_new.shape != k_new.shape:
            raise ValueError("k_new/v_new must be [S][Hkv][D]")
        if k_new.stride(2) != 1 or k_new.stride(1) != d or v_new.stride() != k_new.stride():
            raise ValueError("k_new/v_new rows must be contiguous [Hkv][D] with one token stride")
        stride = k_new.stride(0)
    args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), stride,
            _ptr(block_tables), _ptr(context_lens), _ptr(group_start), _ptr(shared_len), ng, s,
            hq, hkv, d, bs, nb, mb, int(max_context_len), float(scale),
            _ptr(workspace) if workspace is not None else None,
            workspace.numel() if workspace is not None else 0, _dtype_code(k_cache),
            _stream(stream))
    keep = (q, k_cache, v_cache, block_tables, context_lens, group_start, shared_len, workspace,
            out, k_new, v_new)
    call = PreparedCall("pa_decode_attention_shared", args, keep, out)
    return call if prepare else call()


def prefill_attention(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                      max_query_len, out=None, stream=None):
    """Multi-query (chunked prefill) paged attention, bf16; returns float32
    [T][Hq][D] for q [T][Hq][D].  Sequence i owns rows query_start[i] ..
    query_start[i+1]-1 (int32 [S+1]); its chunk ends its context
    context_lens[i] and attends causally (pa_prefill_attention)."""
    import torch
    if q.dim() != 3 or context_lens.dim() != 1 or block_tables.dim() != 2:
        raise ValueError("q must be [T][Hq][D], context_lens [S] and block_tables [S][MB]")
    t, hq, d = q.shape
    s = context_lens.shape[0]
    if query_start.shape != (s + 1,) or block_tables.shape[0] != s:
        raise ValueError("query_start must be [S+1] and block_tables [S][MB]")
    _shape(out, (t, hq, d), "out")
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("q and the pools disagree in head_dim")
    _need(q, k_cache.dtype, "q")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    _need(query_start, torch.int32, "query_start")
    if out is None:
        out = torch.empty((t, hq, d), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    _check("pa_prefill_attention", lib().pa_prefill_attention(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), s, t, hq, hkv, d, bs, nb, block_tables.shape[1],
        int(max_query_len), float(scale), _dtype_code(k_cache), _stream(stream)))
    return out


def probe_read(buf, sink_len=2048, stream=None):
    """Bandwidth probe (include/pa_probe.h): read every byte of the device
    tensor ``buf`` once with sink_len workgroups; returns the uint32 sink
    (as int32), whose XOR is the XOR of all 32-bit words of ``buf``."""
    import torch
    if not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous device tensor")
    sink = torch.empty(sink_len, dtype=torch.int32, device=buf.device)
    _check("pa_probe_read", lib().pa_probe_read(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink_len, _stream(stream)))
    return sink


def probe_gather(k_cache, v_cache, block_tables, context_lens, sink_len=2048, stream=None):
    """Bandwidth probe (include/pa_probe.h): read the K/V chunks a decode
    call over the same pools, tables and context lengths reads, and nothing
    else; returns the uint32 sink (as int32)."""
    import torch
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    s, mb = block_tables.shape
    if context_lens.shape != (s,):
        raise ValueError("context_lens must be [S] for block_tables [S][MB]")
    sink = torch.empty(sink_len, dtype=torch.int32, device=k_cache.device)
    _check("pa_probe_gather", lib().pa_probe_gather(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), mb, _ptr(context_lens), s, hkv, d, bs,
        nb, _dtype_code(k_cache), _ptr(sink), sink_len, _stream(stream)))
    return sink


class BlockManager:
    """Host block manager of include/pa_block_manager.h (numpy in and out).

    Hands out physical block ids of a pool of ``num_blocks`` blocks, keeps the
    block tables, reference counts and copy-on-write; its slots, copy pairs
    and tables feed write_kv, copy_blocks and decode_attention."""

    def __init__(self, num_blocks, block_size, max_seqs, max_blocks_per_seq, num_host_blocks=0):
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        h = ctypes.c_void_p()
        _check("pa_bm_create_with_host", lib().pa_bm_create_with_host(
            num_blocks, num_host_blocks, block_size, max_seqs, max_blocks_per_seq,
            ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    def add_sequence(self):
        out = ctypes.c_int32()
        _check("pa_bm_add_sequence", lib().pa_bm_add_sequence(self._h, ctypes.byref(out)))
        return out.value

    def fork(self, parent):
        out = ctypes.c_int32()
        _check("pa_bm_fork", lib().pa_bm_fork(self._h, int(parent), ctypes.byref(out)))
        return out.value

    def free_sequence(self, seq):
        _check("pa_bm_free_sequence", lib().pa_bm_free_sequence(self._h, int(seq)))

    def append(self, seq_ids, counts):
        """Slots (int64, all new tokens in order) and copy-on-write pairs
        (int32 [k][2]) for counts[i] new tokens of seq_ids[i]."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        cnt = np.ascontiguousarray(counts, dtype=np.int32)
        if ids.shape != cnt.shape or ids.ndim != 1:
            raise ValueError("seq_ids and counts must be 1-D of one length")
        slots = np.empty(int(cnt.sum()) if cnt.size else 0, dtype=np.int64)
        pairs = np.empty((max(1, ids.size), 2), dtype=np.int32)
        ncopy = ctypes.c_int32()
        _check("pa_bm_append", lib().pa_bm_append(
            self._h, ids.ctypes.data, cnt.ctypes.data, ids.size, slots.ctypes.data,
            pairs.ctypes.data, ctypes.byref(ncopy)))
        return slots, pairs[:ncopy.value].copy()

    def _move(self, fn, seq_ids):
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        pairs = np.empty((max(1, ids.size * self.max_blocks_per_seq), 2), dtype=np.int32)
        n = ctypes.c_int32()
        _check(fn, getattr(lib(), fn)(self._h, ids.ctypes.data, ids.size, pairs.ctypes.data,
                                      ctypes.byref(n)))
        return pairs[:n.value].copy()

    def swap_out(self, seq_ids):
        """Swap the sequences out; (GPU block, host block) pairs int32 [k][2]."""
        return self._move("pa_bm_swap_out", seq_ids)

    def swap_in(self, seq_ids):
        """Swap the sequences back in; (host block, GPU block) pairs."""
        return self._move("pa_bm_swap_in", seq_ids)

    def tables(self, seq_ids):
        """(tables int32 [n][max_blocks_per_seq] padded with -1, lengths int32 [n])."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        t = np.empty((ids.size, self.max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _check("pa_bm_tables", lib().pa_bm_tables(self._h, ids.ctypes.data, ids.size,
                                                  t.ctypes.data, lens.ctypes.data))
        return t, lens

    def stats(self):
        st = BMStats()
        _check("pa_bm_get_stats", lib().pa_bm_get_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in BMStats._fields_}
