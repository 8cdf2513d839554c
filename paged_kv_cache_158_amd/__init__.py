"""Paged KV-cache attention on AMD Instinct MI355X (gfx950).

Thin Python binding over `libpa.so` (C ABI in `include/pa.h`): argument
marshalling only.  Every step of the path runs in the library — the HIP
kernels for cache writes, block copies and attention, and the C++ block
manager for the logical-to-physical mapping.  PyTorch serves only as the
owner of device memory and streams.

Importing this package loads `libpa.so` from the package directory and
fails loudly when it has not been built (`python
paged_kv_cache_158_amd/build.py`).  There is no fallback.  The environment
variable PA_LIBRARY names another library file of the package directory to
load instead (`libpa_timeline.so`, the same kernels recording per-wave
timestamps, used by `timeline.py`).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, os.path.basename(os.environ.get("PA_LIBRARY") or "libpa.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python {os.path.join(_HERE, 'build.py')}`")

# PyTorch owns device memory and streams, so libpa must run on the HIP
# runtime torch loaded.  torch's bundled libamdhip64 carries the same soname
# libpa.so needs, so loading torch first makes libpa bind to it; loading libpa
# first would map a second runtime whose stream handles torch cannot share.
import torch as _torch_mod  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are mapped in this process "
                      f"({_hip_runtimes()}); import torch before loading libpa")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4
PA_ERR_OUT_OF_BLOCKS = -5
PA_ERR_NO_SEQUENCE = -6

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_FP8_E4M3 = 2

# KV head order inside a slot (pa_layout): plain, or rotated by the in-block
# position (pa_cache_head_index gives a head's index under either)
LAYOUT_PLAIN = 0
LAYOUT_ROTATED = 1

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)


class CacheDims(ctypes.Structure):
    _fields_ = [("num_blocks", _i32), ("block_size", _i32), ("num_heads", _i32),
                ("num_kv_heads", _i32), ("head_dim", _i32), ("dtype", _i32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("layout", _i32)]


_pdims = ctypes.POINTER(CacheDims)


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib_version = _sig("pa_version", ctypes.c_int, [])
_cache_head_index = _sig("pa_cache_head_index", _i32, [_i32, _i32, _i32, _i32])
_status_string = _sig("pa_status_string", ctypes.c_char_p, [ctypes.c_int])
_cache_write = _sig("pa_cache_write", ctypes.c_int,
                    [_vp, _vp, _vp, _i32, _vp, _vp, _pdims, _vp])
_copy_blocks = _sig("pa_copy_blocks", ctypes.c_int, [_vp, _vp, _vp, _i32, _pdims, _vp])
_swap_blocks = _sig("pa_swap_blocks", ctypes.c_int,
                    [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _pdims, _vp])
_decode_partition_size = _sig("pa_decode_partition_size", _i32, [_pdims, _i32, _i32, _i32])
_decode_ws = _sig("pa_decode_workspace_bytes", ctypes.c_size_t, [_pdims, _i32, _i32, _i32])
_DECODE_ARGS = [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, ctypes.c_float, _vp, _pdims, _i32,
                _vp, ctypes.c_size_t, _vp]
_decode = _sig("pa_decode", ctypes.c_int, _DECODE_ARGS)
_decode_partials = _sig("pa_decode_partials", ctypes.c_int, _DECODE_ARGS)
_decode_noalloc = _sig("pa_decode_noalloc", ctypes.c_int, _DECODE_ARGS[:12] + [_vp])
# bytes of the fixed device scratch pa_decode_noalloc uses (PA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20
_decode_append = _sig("pa_decode_append", ctypes.c_int,
                      [_vp, _vp, _vp, _vp] + _DECODE_ARGS[1:])
_decode_append_partials = _sig("pa_decode_append_partials", ctypes.c_int,
                               [_vp, _vp, _vp, _vp] + _DECODE_ARGS[1:])
_decode_merge = _sig("pa_decode_merge", ctypes.c_int,
                     [_vp, _i32, _i32, _i32, _vp, _pdims, _i32, _vp, ctypes.c_size_t, _vp])
_varlen_ws = _sig("pa_varlen_workspace_bytes", ctypes.c_size_t, [_pdims, _i32, _i32, _i32, _i32])
_varlen = _sig("pa_varlen", ctypes.c_int,
               [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, ctypes.c_float, _vp,
                _pdims, _vp, ctypes.c_size_t, _vp])
_bm_create = _sig("pa_bm_create", ctypes.c_int, [_i32, _i32, _pi32, ctypes.POINTER(_vp)])
_bm_destroy = _sig("pa_bm_destroy", None, [_vp])
_bm_new = _sig("pa_bm_new", ctypes.c_int, [_vp, _i64])
_bm_new_prefix = _sig("pa_bm_new_prefix", ctypes.c_int, [_vp, _i64, _pi32, _i32, _pi32])
_bm_fork = _sig("pa_bm_fork", ctypes.c_int, [_vp, _i64, _i64])
_bm_free = _sig("pa_bm_free", ctypes.c_int, [_vp, _i64])
_bm_append = _sig("pa_bm_append", ctypes.c_int, [_vp, _i64, _i32, _pi32, _pi32, _pi32])
_bm_num_tokens = _sig("pa_bm_num_tokens", ctypes.c_int, [_vp, _i64, _pi32])
_bm_block_table = _sig("pa_bm_block_table", ctypes.c_int, [_vp, _i64, _pi32, _i32, _pi32])
_bm_ref_count = _sig("pa_bm_ref_count", ctypes.c_int, [_vp, _i32, _pi32])
_bm_num_free = _sig("pa_bm_num_free", _i32, [_vp])
_bm_block_cached = _sig("pa_bm_block_cached", ctypes.c_int, [_vp, _i32, _pi32])
_bm_batch_tables = _sig("pa_bm_batch_tables", ctypes.c_int,
                        [_vp, ctypes.POINTER(_i64), _i32, _pi32, _i32, _pi32])


class PAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class OutOfBlocks(PAError):
    pass


def status_string(status: int) -> str:
    return _status_string(status).decode()


def version() -> int:
    return _lib_version()


def cache_head_index(kv_head: int, pos_in_block: int, num_kv_heads: int,
                     layout: int = LAYOUT_PLAIN) -> int:
    """pa_cache_head_index: head index of KV head kv_head inside the slot of
    in-block position pos_in_block under `layout` (-1 for bad arguments)."""
    return int(_cache_head_index(kv_head, pos_in_block, num_kv_heads, layout))


def _check(st: int, what: str) -> None:
    if st == PA_ERR_OUT_OF_BLOCKS:
        raise OutOfBlocks(st, what)
    if st != PA_OK:
        raise PAError(st, what)


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.float8_e4m3fn:
        return DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float8_e4m3fn caches)")


def _io_dtype(k_cache):
    """dtype of q, k, v and out for a cache: bf16 for FP8 caches, else the cache's."""
    torch = _torch()
    return torch.bfloat16 if k_cache.dtype == torch.float8_e4m3fn else k_cache.dtype


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _dev_or_pinned(t, name, dtype=None):
    """Pointer of a GPU tensor or of a pinned host tensor (pin_memory)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream_obj(stream):
    return _torch().cuda.current_stream() if stream is None else stream


def _stream(stream):
    return ctypes.c_void_p(_stream_obj(stream).cuda_stream)


def cache_dims(k_cache, num_heads: int, kv_scales=None, layout: int = LAYOUT_PLAIN) -> CacheDims:
    """Dims of a cache tensor [num_blocks][block_size][num_kv_heads][head_dim].
    kv_scales: (k_scale, v_scale), float32 GPU tensors [num_kv_heads], for
    float8_e4m3fn caches (a code c of KV head h stands for c * scale[h]).
    layout: LAYOUT_PLAIN or LAYOUT_ROTATED, the KV head order inside a slot."""
    nb, bs, hkv, d = k_cache.shape
    dims = CacheDims(nb, bs, num_heads, hkv, d, _dtype_code(k_cache))
    dims.layout = int(layout)
    if kv_scales is not None:
        torch = _torch()
        ks, vs = kv_scales
        for t, name in ((ks, "k_scale"), (vs, "v_scale")):
            if tuple(t.shape) != (hkv,):
                raise ValueError(f"{name} must be [num_kv_heads]")
        dims.k_scale = _dev(ks, "k_scale", torch.float32)
        dims.v_scale = _dev(vs, "v_scale", torch.float32)
    return dims


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI, without the pa_ prefix)
# ---------------------------------------------------------------------------

def cache_write(k, v, slot_mapping, k_cache, v_cache, stream=None, kv_scales=None,
                layout=LAYOUT_PLAIN) -> None:
    """pa_cache_write: k_cache/v_cache rows slot_mapping[i] <- k[i]/v[i]
    (float8_e4m3fn caches: their codes under kv_scales)."""
    torch = _torch()
    n = int(slot_mapping.shape[0])
    dims = cache_dims(k_cache, k_cache.shape[2], kv_scales, layout)
    for name, t in (("k", k), ("v", v)):
        if t.dtype != _io_dtype(k_cache) or tuple(t.shape) != (n, k_cache.shape[2], k_cache.shape[3]):
            raise ValueError(f"{name} must be [{n}][num_kv_heads][head_dim] of the cache dtype "
                             "(bf16 for float8_e4m3fn caches)")
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    st = _cache_write(_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping", torch.int32),
                      n, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                      ctypes.byref(dims), _stream(stream))
    _check(st, "pa_cache_write")


def copy_blocks(k_cache, v_cache, block_pairs, stream=None) -> None:
    """pa_copy_blocks: whole physical blocks src -> dst ([n][2] int32 pairs)."""
    torch = _torch()
    n = int(block_pairs.shape[0])
    if n and tuple(block_pairs.shape) != (n, 2):
        raise ValueError("block_pairs must be [n][2]")
    dims = cache_dims(k_cache, k_cache.shape[2])
    st = _copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                      _dev(block_pairs, "block_pairs", torch.int32) if n else None, n,
                      ctypes.byref(dims), _stream(stream))
    _check(st, "pa_copy_blocks")


def swap_blocks(src_k, src_v, dst_k, dst_v, block_pairs, stream=None) -> None:
    """pa_swap_blocks: whole blocks from one pool to another ([n][2] int32
    (src, dst) pairs), e.g. GPU caches to a pinned host pool (swap out) or
    back (swap in).  Pools and pairs are GPU tensors or pinned host tensors;
    the copy is complete once `stream` is synchronised."""
    torch = _torch()
    n = int(block_pairs.shape[0])
    if n and tuple(block_pairs.shape) != (n, 2):
        raise ValueError("block_pairs must be [n][2]")
    if tuple(src_k.shape[1:]) != tuple(dst_k.shape[1:]) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools must share block shape and dtype")
    if src_v.shape != src_k.shape or dst_v.shape != dst_k.shape:
        raise ValueError("K and V pools must have the same shape")
    if n == 0:
        return
    dims = cache_dims(src_k, src_k.shape[2])
    st = _swap_blocks(_dev_or_pinned(src_k, "src_k"), _dev_or_pinned(src_v, "src_v"),
                      int(src_k.shape[0]), _dev_or_pinned(dst_k, "dst_k"),
                      _dev_or_pinned(dst_v, "dst_v"), int(dst_k.shape[0]),
                      _dev_or_pinned(block_pairs, "block_pairs", torch.int32), n,
                      ctypes.byref(dims), _stream(stream))
    _check(st, "pa_swap_blocks")


def decode_partition_size(dims: CacheDims, num_seqs: int, max_context_len: int,
                          partition_size: int = 0) -> int:
    """Effective split-K partition size for `partition_size` (0: library
    choice).  A result of 0 means the balanced split: per KV head all rows'
    chunks are laid end to end and cut into equal ranges, one per wave, so
    every wave gets the same number of tokens up to one chunk."""
    p = _decode_partition_size(ctypes.byref(dims), num_seqs, max_context_len, partition_size)
    if p < 0:
        raise PAError(PA_ERR_INVALID_ARG, "pa_decode_partition_size")
    return p


def decode_workspace_bytes(dims: CacheDims, num_seqs: int, max_context_len: int,
                           partition_size: int = 0) -> int:
    return int(_decode_ws(ctypes.byref(dims), num_seqs, max_context_len, partition_size))


def _decode_call(fn, name, q, k_cache, v_cache, block_tables, context_lens, scale, out,
                 max_context_len, partition_size, workspace, stream, kv_scales=None,
                 layout=LAYOUT_PLAIN):
    torch = _torch()
    n, H, D = q.shape
    dims = cache_dims(k_cache, H, kv_scales, layout)
    if q.dtype != _io_dtype(k_cache) or out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must have the caches' dtype (bf16 for float8_e4m3fn caches); "
                         "out must match q's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != n or context_lens.shape[0] != n:
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    s = _stream_obj(stream)
    ws_ptr, ws_bytes, _keep = _workspace(dims, n, max_context_len, partition_size, workspace,
                                         q.device, s)
    st = fn(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
            _dev(context_lens, "context_lens", torch.int32), n, int(max_context_len),
            float(scale), _dev(out, "out"), ctypes.byref(dims), int(partition_size),
            ws_ptr, ws_bytes, ctypes.c_void_p(s.cuda_stream))
    _check(st, name)


def _scratch(need, device, s):
    """A workspace of `need` bytes for one call enqueued on stream s.  torch's
    caching allocator may hand a freed block to other work once the stream
    that allocated it moves on, so the block is taken from s's own pool
    (allocated while s is current): it is reused only by later work on s,
    which runs after the kernels of this call."""
    torch = _torch()
    with torch.cuda.stream(s):
        return torch.empty(need, dtype=torch.uint8, device=device)


def _workspace(dims, n, max_context_len, partition_size, workspace, device, s):
    """(pointer, bytes, tensor) of the decode scratch.  Without a caller
    workspace, torch allocates one for this call (the C ABI itself never
    allocates); pass a persistent one to keep allocations out of a loop."""
    need = decode_workspace_bytes(dims, n, max_context_len, partition_size)
    if not need:
        return None, 0, None
    if workspace is None:
        workspace = _scratch(need, device, s)
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), workspace


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
           max_context_len: int, partition_size: int = 0, workspace=None, stream=None,
           kv_scales=None, layout=LAYOUT_PLAIN) -> None:
    """pa_decode: out[s][h] = attention of q[s][h] over context_lens[s] paged tokens
    (float8_e4m3fn caches: kv_scales = (k_scale, v_scale))."""
    _decode_call(_decode, "pa_decode", q, k_cache, v_cache, block_tables, context_lens, scale,
                 out, max_context_len, partition_size, workspace, stream, kv_scales, layout)


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
                   max_context_len: int, partition_size: int = 0, stream=None,
                   kv_scales=None, layout=LAYOUT_PLAIN) -> None:
    """pa_decode_noalloc: pa_decode with the library's fixed per-GPU scratch
    instead of a workspace (nothing is allocated; calls that overlap on one
    GPU race).  Raises PAError (PA_ERR_WORKSPACE) when the batch needs more
    than NOALLOC_SCRATCH_BYTES of scratch."""
    torch = _torch()
    n, H, D = q.shape
    dims = cache_dims(k_cache, H, kv_scales, layout)
    if q.dtype != _io_dtype(k_cache) or out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must have the caches' dtype (bf16 for float8_e4m3fn caches); "
                         "out must match q's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != n or context_lens.shape[0] != n:
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    st = _decode_noalloc(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                         _dev(block_tables, "block_tables", torch.int32),
                         int(block_tables.shape[1]),
                         _dev(context_lens, "context_lens", torch.int32), n,
                         int(max_context_len), float(scale), _dev(out, "out"),
                         ctypes.byref(dims), int(partition_size), _stream(stream))
    _check(st, "pa_decode_noalloc")


def decode_append(q, k, v, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                  scale: float, out, max_context_len: int, partition_size: int = 0,
                  workspace=None, stream=None, kv_scales=None, partials_only=False,
                  layout=LAYOUT_PLAIN) -> None:
    """pa_decode_append: cache_write of one new token per sequence (row s's
    token to slot_mapping[s], position context_lens[s] - 1) and decode, in
    one launch (partials_only: pa_decode_append_partials, its partition
    phase; pa_decode_merge completes it)."""
    torch = _torch()
    entry = _decode_append_partials if partials_only else _decode_append
    name = "pa_decode_append_partials" if partials_only else "pa_decode_append"
    n, H, D = q.shape
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or tuple(t.shape) != (n, k_cache.shape[2], k_cache.shape[3]):
            raise ValueError(f"{name} must be [num_seqs][num_kv_heads][head_dim] of q's dtype")
    if int(slot_mapping.shape[0]) != n:
        raise ValueError("slot_mapping must have one slot per sequence")
    kp, vp, sp = _dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping", torch.int32)

    def fn(q_, kc, vc, *rest):
        return entry(q_, kp, vp, sp, kc, vc, *rest)

    _decode_call(fn, name, q, k_cache, v_cache, block_tables, context_lens, scale,
                 out, max_context_len, partition_size, workspace, stream, kv_scales, layout)


class PreparedCall:
    """One C-ABI call with its arguments checked and marshalled once (device
    pointers, sizes, dims, stream).  Calling it issues the call again with
    the same arguments, so a loop that repeats a step over the same buffers
    pays only the C call itself.  The tensors it was made from are kept
    alive by it; their contents may change between calls, their storage
    must not."""

    def __init__(self, fn, name, args, keep):
        self._fn, self._name, self._args, self._keep = fn, name, args, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st, self._name)


def prepare_decode_append(q, k, v, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                          scale: float, out, max_context_len: int, partition_size: int = 0,
                          workspace=None, stream=None, kv_scales=None, partials_only=False,
                          layout=LAYOUT_PLAIN) -> PreparedCall:
    """decode_append with every argument checked now: returns a PreparedCall
    that enqueues pa_decode_append (or its partition phase) on `stream` (the
    current stream now when None).  A workspace is required when the call
    needs one."""
    torch = _torch()
    n, H, D = q.shape
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or tuple(t.shape) != (n, k_cache.shape[2], k_cache.shape[3]):
            raise ValueError(f"{name} must be [num_seqs][num_kv_heads][head_dim] of q's dtype")
    if int(slot_mapping.shape[0]) != n:
        raise ValueError("slot_mapping must have one slot per sequence")
    dims = cache_dims(k_cache, H, kv_scales, layout)
    if q.dtype != _io_dtype(k_cache) or out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must have the caches' dtype (bf16 for float8_e4m3fn caches); "
                         "out must match q's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != n or context_lens.shape[0] != n:
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    need = decode_workspace_bytes(dims, n, max_context_len, partition_size)
    if need and workspace is None:
        raise ValueError("a prepared call needs a persistent workspace")
    ws_ptr = _dev(workspace, "workspace") if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if need else 0
    fn = _decode_append_partials if partials_only else _decode_append
    args = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
            _dev(slot_mapping, "slot_mapping", torch.int32), _dev(k_cache, "k_cache"),
            _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables", torch.int32),
            int(block_tables.shape[1]), _dev(context_lens, "context_lens", torch.int32), n,
            int(max_context_len), float(scale), _dev(out, "out"), ctypes.byref(dims),
            int(partition_size), ws_ptr, ws_bytes, _stream(stream))
    keep = (q, k, v, slot_mapping, k_cache, v_cache, block_tables, context_lens, out, workspace,
            kv_scales, dims)
    return PreparedCall(fn, "pa_decode_append_partials" if partials_only else "pa_decode_append",
                        args, keep)


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
                    max_context_len: int, partition_size: int = 0, workspace=None,
                    stream=None, kv_scales=None, layout=LAYOUT_PLAIN) -> None:
    """pa_decode_partials: the partition phase of pa_decode."""
    _decode_call(_decode_partials, "pa_decode_partials", q, k_cache, v_cache, block_tables,
                 context_lens, scale, out, max_context_len, partition_size, workspace, stream,
                 kv_scales, layout)


def decode_merge(context_lens, out, k_cache, max_context_len: int, max_blocks_per_seq: int,
                 partition_size: int = 0, workspace=None, stream=None) -> None:
    """pa_decode_merge: the log-sum-exp merge phase of pa_decode."""
    torch = _torch()
    n, H, D = out.shape
    dims = cache_dims(k_cache, H)
    if workspace is None and decode_workspace_bytes(dims, n, max_context_len, partition_size):
        raise ValueError("pa_decode_merge needs the workspace pa_decode_partials wrote")
    s = _stream_obj(stream)
    ws_ptr, ws_bytes, _keep = _workspace(dims, n, max_context_len, partition_size, workspace,
                                         out.device, s)
    st = _decode_merge(_dev(context_lens, "context_lens", torch.int32), n, int(max_context_len),
                       int(max_blocks_per_seq), _dev(out, "out"), ctypes.byref(dims),
                       int(partition_size), ws_ptr, ws_bytes, ctypes.c_void_p(s.cuda_stream))
    _check(st, "pa_decode_merge")


def varlen_workspace_bytes(dims: CacheDims, num_seqs: int, total_q: int, max_query_len: int,
                           max_seq_len: int) -> int:
    return int(_varlen_ws(ctypes.byref(dims), num_seqs, total_q, max_query_len, max_seq_len))


def varlen(q, query_start_loc, seq_lens, k_cache, v_cache, block_tables, scale: float, out,
           max_query_len: int, max_seq_len: int, workspace=None, stream=None,
           kv_scales=None, layout=LAYOUT_PLAIN) -> None:
    """pa_varlen: chunked-prefill and decode rows of one batch, segments by query_start_loc."""
    torch = _torch()
    T, H, D = q.shape
    n = int(seq_lens.shape[0])
    dims = cache_dims(k_cache, H, kv_scales, layout)
    if q.dtype != _io_dtype(k_cache) or out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must have the caches' dtype (bf16 for float8_e4m3fn caches); "
                         "out must match q's shape")
    if int(query_start_loc.shape[0]) != n + 1 or block_tables.dim() != 2 or \
            int(block_tables.shape[0]) != n:
        raise ValueError("query_start_loc must be [num_seqs+1], block_tables [num_seqs][max_blocks]")
    need = varlen_workspace_bytes(dims, n, T, max_query_len, max_seq_len)
    s = _stream_obj(stream)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:  # torch allocates the scratch for this call, on s
            workspace = _scratch(need, q.device, s)
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _varlen(_dev(q, "q"), _dev(query_start_loc, "query_start_loc", torch.int32),
                 _dev(seq_lens, "seq_lens", torch.int32), n, T, int(max_query_len),
                 int(max_seq_len), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                 _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
                 float(scale), _dev(out, "out"), ctypes.byref(dims), ws_ptr, ws_bytes,
                 ctypes.c_void_p(s.cuda_stream))
    _check(st, "pa_varlen")


# ---------------------------------------------------------------------------
# host block manager
# ---------------------------------------------------------------------------

class BlockManager:
    """pa_bm_*: logical blocks of each sequence mapped onto a pool of physical blocks."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        h = _vp()
        arr = None
        if free_order is not None:
            if len(free_order) != num_blocks:
                raise ValueError("free_order must list every block once")
            arr = (_i32 * num_blocks)(*[int(b) for b in free_order])
        _check(_bm_create(num_blocks, block_size, arr, ctypes.byref(h)), "pa_bm_create")
        self._h = h

    def close(self) -> None:
        # at interpreter exit the module's globals may already be gone
        if getattr(self, "_h", None) and _bm_destroy is not None:
            _bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def new(self, sid: int) -> None:
        _check(_bm_new(self._h, sid), "pa_bm_new")

    def new_prefix(self, sid: int, tokens) -> int:
        """Start sid with its prompt's token ids; returns the prompt tokens
        covered by cached blocks (append the rest next)."""
        import numpy as np
        arr = np.ascontiguousarray(tokens, dtype=np.int32)
        hit = _i32(0)
        _check(_bm_new_prefix(self._h, sid, arr.ctypes.data_as(_pi32), int(arr.size),
                              ctypes.byref(hit)), "pa_bm_new_prefix")
        return hit.value

    def fork(self, parent: int, child: int) -> None:
        _check(_bm_fork(self._h, parent, child), "pa_bm_fork")

    def free(self, sid: int) -> None:
        _check(_bm_free(self._h, sid), "pa_bm_free")

    def append(self, sid: int, n: int) -> Tuple[list, Optional[Tuple[int, int]]]:
        """Slots of n new tokens, and the (src, dst) copy-on-write pair or None."""
        slots = (_i32 * max(n, 1))()
        src, dst = _i32(-1), _i32(-1)
        _check(_bm_append(self._h, sid, n, slots, ctypes.byref(src), ctypes.byref(dst)),
               "pa_bm_append")
        cp = None if src.value < 0 else (src.value, dst.value)
        return list(slots[:n]), cp

    def append_into(self, sid: int, n: int, out_slots) -> Optional[Tuple[int, int]]:
        """As append, writing the slots into a host int32 numpy array (no list)."""
        src, dst = _i32(-1), _i32(-1)
        ptr = out_slots.ctypes.data_as(_pi32)
        _check(_bm_append(self._h, sid, n, ptr, ctypes.byref(src), ctypes.byref(dst)),
               "pa_bm_append")
        return None if src.value < 0 else (src.value, dst.value)

    def num_tokens(self, sid: int) -> int:
        x = _i32()
        _check(_bm_num_tokens(self._h, sid, ctypes.byref(x)), "pa_bm_num_tokens")
        return x.value

    def block_table(self, sid: int) -> list:
        n = _i32()
        _bm_block_table(self._h, sid, None, 0, ctypes.byref(n))
        buf = (_i32 * max(n.value, 1))()
        _check(_bm_block_table(self._h, sid, buf, n.value, ctypes.byref(n)), "pa_bm_block_table")
        return list(buf[: n.value])

    def ref_count(self, block: int) -> int:
        x = _i32()
        _check(_bm_ref_count(self._h, block, ctypes.byref(x)), "pa_bm_ref_count")
        return x.value

    def num_free(self) -> int:
        return int(_bm_num_free(self._h))

    def block_cached(self, block: int) -> bool:
        x = _i32(0)
        _check(_bm_block_cached(self._h, block, ctypes.byref(x)), "pa_bm_block_cached")
        return bool(x.value)

    def batch_tables(self, seq_ids: Sequence[int], width: int):
        """Host numpy (tables [n][width] -1 padded, context_lens [n]) for a batch."""
        import numpy as np
        n = len(seq_ids)
        ids = (_i64 * max(n, 1))(*[int(s) for s in seq_ids])
        tables = np.empty((n, width), dtype=np.int32)
        lens = np.empty((n,), dtype=np.int32)
        _check(_bm_batch_tables(self._h, ids, n, tables.ctypes.data_as(_pi32), width,
                                lens.ctypes.data_as(_pi32)), "pa_bm_batch_tables")
        return tables, lens


__all__ = ["BlockManager", "CacheDims", "DTYPE_BF16", "DTYPE_F32", "DTYPE_FP8_E4M3",
           "LAYOUT_PLAIN", "LAYOUT_ROTATED", "OutOfBlocks",
           "PAError", "PreparedCall", "cache_dims", "cache_head_index", "cache_write",
           "prepare_decode_append", "decode_noalloc", "NOALLOC_SCRATCH_BYTES",
           "copy_blocks", "decode", "decode_append", "decode_merge", "decode_partials", "decode_partition_size", "decode_workspace_bytes",
           "status_string", "swap_blocks", "varlen", "varlen_workspace_bytes", "version", "LIB_PATH"]
