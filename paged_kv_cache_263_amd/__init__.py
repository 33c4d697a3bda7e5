"""Paged KV-cache attention for AMD MI355X (gfx950) - Python binding.

A thin ctypes layer over ``libpagedkv.so`` (C ABI in ``include/pagedkv.h``).
Functions keep the C names; this module only marshals arguments.  torch is
used for device memory and streams; every step of the computation runs in the
library's host allocator or its HIP kernels.  There is no fallback: if the
library is missing, importing this package fails.

Build the library with ``python paged_kv_cache_263_amd/build.py``.
"""

from __future__ import annotations

import ctypes
import os

import torch  # imported first: the library then binds to the HIP runtime torch loaded

__all__ = [
    "PagedKVError", "Pool", "KVCache", "LIB_PATH",
    "kv_pool_create", "kv_pool_destroy", "kv_pool_alloc", "kv_pool_incref", "kv_pool_free",
    "kv_pool_refcount", "kv_pool_stats", "kv_pool_free_list", "kv_pool_evictable_list",
    "seq_create", "seq_append", "seq_append_batch", "seq_fork", "seq_share_prefix", "seq_free",
    "seq_len", "seq_num_blocks", "seq_swap_out", "seq_swap_in", "seq_create_cached", "seq_cache_tokens",
    "block_table_build",
    "paged_attn_workspace_size", "paged_attn_decode", "paged_attn_decode_noalloc", "paged_attn_prefill_chunk",
    "kv_cache_write", "kv_copy_blocks", "kv_swap_block_bytes", "kv_swap_out", "kv_swap_in",
    "pkv_strerror", "pkv_last_error", "pkv_version",
]

# PKV_LIBRARY names another build of the same library (the sanitized host
# build that tests the allocator under ASan/UBSan); by default the in-tree one.
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_F32, PKV_BF16, PKV_FP8_E4M3, PKV_INT8 = 0, 1, 2, 3
BLOCK_SIZE = 16
HEAD_DIM = 128
_STATUS = {0: "OK", -1: "INVALID", -2: "OOM", -3: "STATE", -4: "UNSUPPORTED", -5: "HIP", -6: "WORKSPACE"}


class PagedKVError(RuntimeError):
    """A non-zero status from the library; ``code`` is its PKV_ERR_* name."""

    def __init__(self, status: int, message: str):
        self.status = status
        self.code = _STATUS.get(status, str(status))
        super().__init__(f"{self.code}: {message}")


class pkv_copy(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("dst", ctypes.c_int32), ("valid_tokens", ctypes.c_int32)]


class pkv_stats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("used_blocks", ctypes.c_int32), ("shared_blocks", ctypes.c_int32),
                ("refcount_sum", ctypes.c_int64), ("cow_count", ctypes.c_int64),
                ("num_seqs", ctypes.c_int64), ("tokens", ctypes.c_int64), ("waste_tokens", ctypes.c_int64),
                ("swapped_seqs", ctypes.c_int64), ("swapped_tokens", ctypes.c_int64),
                ("cached_blocks", ctypes.c_int64), ("evictable_blocks", ctypes.c_int64),
                ("matched_tokens", ctypes.c_int64)]


class pkv_cache(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int32), ("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class pkv_attn_args(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("q", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("kv_lens", ctypes.c_void_p), ("max_kv_len", ctypes.c_int32),
                ("cu_q", ctypes.c_void_p), ("num_decode", ctypes.c_int32),
                ("max_decode_kv_len", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
                ("total_q", ctypes.c_int32), ("decode_parts", ctypes.c_int32),
                ("prefill_parts", ctypes.c_int32),
                ("shared_prefix_blocks", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("events", ctypes.c_void_p * 4)]


_i32, _p, _pi32 = ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
_SIGNATURES = {
    "kv_pool_create": (ctypes.c_int, [_i32, _i32, _pi32, ctypes.POINTER(_p)]),
    "kv_pool_destroy": (None, [_p]),
    "kv_pool_alloc": (ctypes.c_int, [_p, _i32, _pi32]),
    "kv_pool_incref": (ctypes.c_int, [_p, _pi32, _i32]),
    "kv_pool_free": (ctypes.c_int, [_p, _pi32, _i32]),
    "kv_pool_refcount": (ctypes.c_int, [_p, _i32, _pi32]),
    "kv_pool_stats": (ctypes.c_int, [_p, ctypes.POINTER(pkv_stats)]),
    "kv_pool_free_list": (ctypes.c_int, [_p, _pi32, _i32, _pi32]),
    "kv_pool_evictable_list": (ctypes.c_int, [_p, _pi32, _i32, _pi32]),
    "seq_create": (ctypes.c_int, [_p, _pi32]),
    "seq_append": (ctypes.c_int, [_p, _i32, _i32, _pi32, ctypes.POINTER(pkv_copy), _pi32]),
    "seq_append_batch": (ctypes.c_int, [_p, _pi32, _pi32, _i32, _pi32, ctypes.POINTER(pkv_copy), _pi32]),
    "seq_fork": (ctypes.c_int, [_p, _i32, _pi32]),
    "seq_share_prefix": (ctypes.c_int, [_p, _i32, _i32, _pi32]),
    "seq_free": (ctypes.c_int, [_p, _i32]),
    "seq_len": (ctypes.c_int, [_p, _i32, _pi32]),
    "seq_num_blocks": (ctypes.c_int, [_p, _i32, _pi32]),
    "seq_swap_out": (ctypes.c_int, [_p, _i32, _pi32, _i32, _pi32]),
    "seq_swap_in": (ctypes.c_int, [_p, _i32, _pi32, _i32, _pi32]),
    "seq_create_cached": (ctypes.c_int, [_p, _i32, _pi32, _i32, _pi32, _pi32]),
    "seq_cache_tokens": (ctypes.c_int, [_p, _i32, _i32, _pi32, _i32, _pi32]),
    "block_table_build": (ctypes.c_int, [_p, _pi32, _i32, _i32, _pi32, _pi32]),
    "paged_attn_workspace_size": (ctypes.c_int, [ctypes.POINTER(pkv_cache), ctypes.POINTER(pkv_attn_args),
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "paged_attn_decode": (ctypes.c_int, [ctypes.POINTER(pkv_cache), ctypes.POINTER(pkv_attn_args), _p]),
    "paged_attn_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(pkv_cache), ctypes.POINTER(pkv_attn_args), _p]),
    "paged_attn_prefill_chunk": (ctypes.c_int, [ctypes.POINTER(pkv_cache), ctypes.POINTER(pkv_attn_args), _p]),
    "kv_cache_write": (ctypes.c_int, [ctypes.POINTER(pkv_cache), _i32, _i32, _i32, _p, _p, _p, _p, _p, _i32,
                                      _p, _i32, _p, _p]),
    "kv_copy_blocks": (ctypes.c_int, [ctypes.POINTER(pkv_cache), ctypes.POINTER(pkv_copy), _i32, _p]),
    "kv_swap_block_bytes": (ctypes.c_int, [ctypes.POINTER(pkv_cache), ctypes.POINTER(ctypes.c_size_t)]),
    "kv_swap_out": (ctypes.c_int, [ctypes.POINTER(pkv_cache), _pi32, _i32, _p, _p]),
    "kv_swap_in": (ctypes.c_int, [ctypes.POINTER(pkv_cache), _p, _pi32, _i32, _p]),
    "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_int, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run: python paged_kv_cache_263_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise PagedKVError(status, _lib.pkv_last_error().decode())


def pkv_strerror(status: int) -> str:
    return _lib.pkv_strerror(status).decode()


def pkv_last_error() -> str:
    return _lib.pkv_last_error().decode()


def pkv_version() -> int:
    return _lib.pkv_version()


def _i32_array(values):
    values = [int(v) for v in values]
    return (ctypes.c_int32 * max(1, len(values)))(*values), len(values)


# ---------------------------------------------------------------------------
# host allocator


class Pool:
    """Handle of a host block pool (metadata only); freed on garbage collection."""

    def __init__(self, handle):
        self._h = handle

    @property
    def handle(self):
        if self._h is None:
            raise PagedKVError(-1, "pool destroyed")
        return self._h

    def destroy(self):
        if self._h is not None:
            _lib.kv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def kv_pool_create(num_blocks: int, order=None, block_size: int = BLOCK_SIZE) -> Pool:
    h = ctypes.c_void_p()
    arr = None
    if order is not None:
        arr, n = _i32_array(order)
        if n != num_blocks:
            raise PagedKVError(-1, "order must list every block once")
    _check(_lib.kv_pool_create(num_blocks, block_size, arr, ctypes.byref(h)))
    return Pool(h)


def kv_pool_destroy(pool: Pool) -> None:
    pool.destroy()


def kv_pool_alloc(pool: Pool, n: int) -> list:
    out = (ctypes.c_int32 * max(1, n))()
    _check(_lib.kv_pool_alloc(pool.handle, n, out))
    return list(out[:n])


def kv_pool_incref(pool: Pool, ids) -> None:
    arr, n = _i32_array(ids)
    _check(_lib.kv_pool_incref(pool.handle, arr, n))


def kv_pool_free(pool: Pool, ids) -> None:
    arr, n = _i32_array(ids)
    _check(_lib.kv_pool_free(pool.handle, arr, n))


def kv_pool_refcount(pool: Pool, block: int) -> int:
    out = ctypes.c_int32()
    _check(_lib.kv_pool_refcount(pool.handle, block, ctypes.byref(out)))
    return out.value


def kv_pool_stats(pool: Pool) -> dict:
    s = pkv_stats()
    _check(_lib.kv_pool_stats(pool.handle, ctypes.byref(s)))
    return {name: getattr(s, name) for name, _ in pkv_stats._fields_}


def kv_pool_free_list(pool: Pool) -> list:
    n = ctypes.c_int32()
    cap = kv_pool_stats(pool)["num_blocks"]
    out = (ctypes.c_int32 * max(1, cap))()
    _check(_lib.kv_pool_free_list(pool.handle, out, cap, ctypes.byref(n)))
    return list(out[: n.value])


def kv_pool_evictable_list(pool: Pool) -> list:
    """Retained prefix-cache blocks with no reference, least recently used first."""
    n = ctypes.c_int32()
    cap = kv_pool_stats(pool)["num_blocks"]
    out = (ctypes.c_int32 * max(1, cap))()
    _check(_lib.kv_pool_evictable_list(pool.handle, out, cap, ctypes.byref(n)))
    return list(out[: n.value])


def seq_create_cached(pool: Pool, tenant: int, tokens) -> tuple:
    """New sequence holding the cached leading full blocks of ``tokens``;
    returns (seq, tokens matched)."""
    arr, n = _i32_array(tokens)
    s, m = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.seq_create_cached(pool.handle, tenant, arr, n, ctypes.byref(s), ctypes.byref(m)))
    return s.value, m.value


def seq_cache_tokens(pool: Pool, seq: int, start: int, tokens) -> int:
    """Register seq's full blocks holding positions start.. (token ids
    ``tokens``); returns how many blocks were keyed."""
    arr, n = _i32_array(tokens)
    k = ctypes.c_int32()
    _check(_lib.seq_cache_tokens(pool.handle, seq, start, arr, n, ctypes.byref(k)))
    return k.value


def seq_create(pool: Pool) -> int:
    s = ctypes.c_int32()
    _check(_lib.seq_create(pool.handle, ctypes.byref(s)))
    return s.value


def seq_append(pool: Pool, seq: int, n_tokens: int):
    """Returns (slots, copies); copies is a list of (src, dst, valid_tokens)."""
    slots = (ctypes.c_int32 * max(1, n_tokens))()
    cp = pkv_copy()
    nc = ctypes.c_int32()
    _check(_lib.seq_append(pool.handle, seq, n_tokens, slots, ctypes.byref(cp), ctypes.byref(nc)))
    return list(slots[:n_tokens]), [(cp.src, cp.dst, cp.valid_tokens)] if nc.value else []


def seq_append_batch(pool: Pool, seqs, n_tokens, out_slots=None):
    """Append n_tokens[i] tokens to seqs[i] for all i (all or nothing).

    Returns (slots, copies).  ``out_slots`` may be a preallocated ctypes int32
    array (or a CPU int32 tensor) of sum(n_tokens) entries, filled in place."""
    sa, n = _i32_array(seqs)
    na, _ = _i32_array(n_tokens)
    total = sum(int(x) for x in n_tokens)
    if out_slots is None:
        buf = (ctypes.c_int32 * max(1, total))()
        ptr = buf
    elif isinstance(out_slots, torch.Tensor):
        buf = out_slots
        ptr = ctypes.cast(out_slots.data_ptr(), _pi32)
    else:
        buf = out_slots
        ptr = out_slots
    copies = (pkv_copy * max(1, n))()
    nc = ctypes.c_int32()
    _check(_lib.seq_append_batch(pool.handle, sa, na, n, ptr, copies, ctypes.byref(nc)))
    cps = [(copies[i].src, copies[i].dst, copies[i].valid_tokens) for i in range(nc.value)]
    if out_slots is None:
        return list(buf[:total]), cps
    return buf, cps


def seq_fork(pool: Pool, parent: int) -> int:
    c = ctypes.c_int32()
    _check(_lib.seq_fork(pool.handle, parent, ctypes.byref(c)))
    return c.value


def seq_share_prefix(pool: Pool, src: int, n_tokens: int) -> int:
    c = ctypes.c_int32()
    _check(_lib.seq_share_prefix(pool.handle, src, n_tokens, ctypes.byref(c)))
    return c.value


def seq_free(pool: Pool, seq: int) -> None:
    _check(_lib.seq_free(pool.handle, seq))


def _swap_ids(fn, pool: Pool, seq: int) -> list:
    n = ctypes.c_int32()
    cap = max(1, -(-seq_len(pool, seq) // BLOCK_SIZE))
    out = (ctypes.c_int32 * cap)()
    _check(fn(pool.handle, seq, out, cap, ctypes.byref(n)))
    return list(out[: n.value])


def seq_swap_out(pool: Pool, seq: int) -> list:
    """Swap seq out: its block ids in logical order (copy them to host memory
    with kv_swap_out before reusing them); seq then holds no blocks."""
    return _swap_ids(_lib.seq_swap_out, pool, seq)


def seq_swap_in(pool: Pool, seq: int) -> list:
    """Swap seq back in: its fresh block ids in logical order (copy the host
    copy into them with kv_swap_in)."""
    return _swap_ids(_lib.seq_swap_in, pool, seq)


def seq_len(pool: Pool, seq: int) -> int:
    n = ctypes.c_int32()
    _check(_lib.seq_len(pool.handle, seq, ctypes.byref(n)))
    return n.value


def seq_num_blocks(pool: Pool, seq: int) -> int:
    n = ctypes.c_int32()
    _check(_lib.seq_num_blocks(pool.handle, seq, ctypes.byref(n)))
    return n.value


def block_table_build(pool: Pool, seqs, max_blocks: int):
    """Returns (table, lens) as CPU int32 tensors [n, max_blocks] and [n]."""
    sa, n = _i32_array(seqs)
    table = torch.empty((n, max_blocks), dtype=torch.int32)
    lens = torch.empty((n,), dtype=torch.int32)
    _check(_lib.block_table_build(pool.handle, sa, n, max_blocks, ctypes.cast(table.data_ptr(), _pi32),
                                  ctypes.cast(lens.data_ptr(), _pi32)))
    return table, lens


# ---------------------------------------------------------------------------
# device cache and kernels

_DT = {PKV_F32: torch.float32, PKV_BF16: torch.bfloat16, PKV_FP8_E4M3: torch.uint8, PKV_INT8: torch.int8}
_QDT = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}
_NAMES = {"f32": PKV_F32, "bf16": PKV_BF16, "fp8": PKV_FP8_E4M3, "int8": PKV_INT8}


class KVCache:
    """Device K/V pools (torch tensors owned by this object).

    k_pool: [layers, num_blocks, kv_heads, 16, 128]; v_pool: [layers, num_blocks,
    kv_heads, 128, 16] (token-minor inside a block); fp8 pools hold E4M3 codes
    as uint8 and int8 pools signed codes as int8, each with fp32 scales
    [layers, kv_heads] for K and V."""

    def __init__(self, kv_dtype, num_layers: int, num_blocks: int, num_kv_heads: int, device="cuda",
                 k_scale=None, v_scale=None, zero: bool = True):
        self.kv_dtype = _NAMES.get(kv_dtype, kv_dtype)
        self.num_layers, self.num_blocks, self.num_kv_heads = num_layers, num_blocks, num_kv_heads
        dt = _DT[self.kv_dtype]
        alloc = torch.zeros if zero else torch.empty
        self.k_pool = alloc((num_layers, num_blocks, num_kv_heads, BLOCK_SIZE, HEAD_DIM), dtype=dt, device=device)
        self.v_pool = alloc((num_layers, num_blocks, num_kv_heads, HEAD_DIM, BLOCK_SIZE), dtype=dt, device=device)
        self.k_scale = self.v_scale = None
        if self.kv_dtype in (PKV_FP8_E4M3, PKV_INT8):
            if k_scale is None or v_scale is None:
                raise PagedKVError(-1, "fp8 and int8 caches need k_scale and v_scale")
            self.k_scale = torch.as_tensor(k_scale, dtype=torch.float32).reshape(num_layers, num_kv_heads).to(device)
            self.v_scale = torch.as_tensor(v_scale, dtype=torch.float32).reshape(num_layers, num_kv_heads).to(device)
        self._desc = pkv_cache(self.kv_dtype, num_layers, num_blocks, num_kv_heads, HEAD_DIM, BLOCK_SIZE,
                               self.k_pool.data_ptr(), self.v_pool.data_ptr(),
                               self.k_scale.data_ptr() if self.k_scale is not None else None,
                               self.v_scale.data_ptr() if self.v_scale is not None else None)

    @property
    def desc(self) -> pkv_cache:
        return self._desc

    @property
    def value_dtype(self) -> torch.dtype:
        return torch.float32 if self.kv_dtype == PKV_F32 else torch.bfloat16


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _torch_stream(stream, device):
    """The torch stream object a call's kernels are enqueued on (the current
    stream, the given one, or a raw hipStream_t handle wrapped)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _hip_fn(name, res, args):
    # the HIP runtime the library is linked against (looked up through the library's own handle)
    fn = getattr(_lib, name)
    fn.restype, fn.argtypes = res, args
    return fn


def _dev_ptr(t):
    """Device address of a device tensor, or of a pinned host tensor (which the
    kernels then read over the host link, with no staging copy)."""
    if t is None:
        return None
    if t.is_cuda:
        return ctypes.c_void_p(t.data_ptr())
    if not t.is_pinned():
        raise PagedKVError(-1, "a host tensor passed to a device call must be pinned")
    dev = ctypes.c_void_p()
    st = _hip_fn("hipHostGetDevicePointer", ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                            ctypes.c_uint])(ctypes.byref(dev), t.data_ptr(), 0)
    if st != 0 or not dev.value:
        raise PagedKVError(-5, f"hipHostGetDevicePointer failed ({st})")
    return dev


def _args(cache: KVCache, q, out, block_table, kv_lens, max_kv_len, layer, decode_parts, workspace,
          cu_q=None, num_decode=0, max_decode_kv_len=0, max_q_len=0, total_q=0) -> pkv_attn_args:
    if q.dtype not in _QDT:
        raise PagedKVError(-4, f"query dtype {q.dtype}")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or out.shape != q.shape or out.dtype != q.dtype:
        raise PagedKVError(-1, "q and out must be [rows, heads, 128] of one dtype")
    if cu_q is None and q.shape[0] != block_table.shape[0]:
        raise PagedKVError(-1, "decode needs one query row per block-table row")
    if kv_lens.numel() != block_table.shape[0]:
        raise PagedKVError(-1, "kv_lens needs one entry per block-table row")
    for t in (q, out, block_table, kv_lens):
        if not t.is_contiguous():
            raise PagedKVError(-1, "tensors must be contiguous")
    if block_table.dtype != torch.int32 or kv_lens.dtype != torch.int32:
        raise PagedKVError(-1, "block_table and kv_lens must be int32")
    a = pkv_attn_args()
    a.layer = layer
    a.q_dtype = _QDT[q.dtype]
    a.num_seqs = block_table.shape[0]
    a.num_q_heads = q.shape[1]
    a.q = q.data_ptr()
    a.out = out.data_ptr()
    a.block_table = block_table.data_ptr()
    a.max_blocks = block_table.shape[1]
    a.kv_lens = kv_lens.data_ptr()
    a.max_kv_len = int(max_kv_len)
    a.cu_q = cu_q.data_ptr() if cu_q is not None else None
    a.num_decode = num_decode
    a.max_decode_kv_len = int(max_decode_kv_len)
    a.max_q_len = int(max_q_len)
    a.total_q = int(total_q)
    a.decode_parts = decode_parts
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def paged_attn_workspace_size(cache: KVCache, args: pkv_attn_args) -> int:
    n = ctypes.c_size_t()
    _check(_lib.paged_attn_workspace_size(ctypes.byref(cache.desc), ctypes.byref(args), ctypes.byref(n)))
    return n.value


def _with_workspace(cache, a, workspace, device, ts):
    """Workspace for the call: the caller's, or one allocated here under the
    call's own stream ``ts``, so that the caching allocator hands its memory
    to nothing else before the kernels on ``ts`` that use it have run."""
    if workspace is None:
        need = paged_attn_workspace_size(cache, a)
        if need:
            with torch.cuda.stream(ts):
                workspace = torch.empty(need, dtype=torch.uint8, device=device)
            a.workspace = workspace.data_ptr()
            a.workspace_bytes = need
    return workspace


def _new_out(q, ts):
    # allocated on the call's stream for the same reason as the workspace
    with torch.cuda.stream(ts):
        return torch.empty_like(q)


def _set_events(a, events):
    if events is not None:
        for i, e in enumerate(events):
            a.events[i] = e


def paged_attn_decode(cache: KVCache, q, block_table, kv_lens, max_kv_len: int, out=None, layer: int = 0,
                      decode_parts: int = 0, workspace=None, stream=None, events=None,
                      shared_prefix_blocks: int = 0):
    """q [rows, Hq, 128] -> out [rows, Hq, 128] (q's dtype).  ``events``: up to
    four hipEvent_t handles (ints) recorded around the kernels (see the header).
    ``shared_prefix_blocks``: the caller's promise that every row's table starts
    with the same that many block ids (attention over them is computed once)."""
    ts = _torch_stream(stream, q.device)
    if out is None:
        out = _new_out(q, ts)
    a = _args(cache, q, out, block_table, kv_lens, max_kv_len, layer, decode_parts, workspace)
    a.shared_prefix_blocks = shared_prefix_blocks
    _set_events(a, events)
    keep = _with_workspace(cache, a, workspace, q.device, ts)  # noqa: F841 (stream-ordered reuse)
    _check(_lib.paged_attn_decode(ctypes.byref(cache.desc), ctypes.byref(a), _stream(ts)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def paged_attn_decode_noalloc(cache: KVCache, q, block_table, kv_lens, max_kv_len: int, out, layer: int = 0,
                              decode_parts: int = 0, stream=None, events=None, shared_prefix_blocks: int = 0):
    """paged_attn_decode with no allocation anywhere (nor here): ``out`` is the
    caller's, and the workspace is the library's fixed per-GPU array of
    NOALLOC_SCRATCH_BYTES (calls that overlap on one GPU race on it)."""
    if out is None:
        raise PagedKVError(-1, "paged_attn_decode_noalloc needs the caller's out tensor")
    a = _args(cache, q, out, block_table, kv_lens, max_kv_len, layer, decode_parts, None)
    a.shared_prefix_blocks = shared_prefix_blocks
    _set_events(a, events)
    _check(_lib.paged_attn_decode_noalloc(ctypes.byref(cache.desc), ctypes.byref(a), _stream(stream)))
    return out


def paged_attn_prefill_chunk(cache: KVCache, q, cu_q, block_table, kv_lens, max_kv_len: int, num_decode: int,
                             max_q_len: int, out=None, layer: int = 0, max_decode_kv_len: int = 0,
                             decode_parts: int = 0, workspace=None, stream=None, events=None,
                             prefill_parts: int = 0):
    """q [total_q, Hq, 128]; rows 0..num_decode-1 are decode rows (cu_q[i] = i)."""
    ts = _torch_stream(stream, q.device)
    if out is None:
        out = _new_out(q, ts)
    a = _args(cache, q, out, block_table, kv_lens, max_kv_len, layer, decode_parts, workspace, cu_q=cu_q,
              num_decode=num_decode, max_decode_kv_len=max_decode_kv_len, max_q_len=max_q_len,
              total_q=q.shape[0])
    a.prefill_parts = prefill_parts
    _set_events(a, events)
    keep = _with_workspace(cache, a, workspace, q.device, ts)  # noqa: F841 (stream-ordered reuse)
    _check(_lib.paged_attn_prefill_chunk(ctypes.byref(cache.desc), ctypes.byref(a), _stream(ts)))
    return out


def kv_cache_write(cache: KVCache, k_new, v_new, slots, layer: int = 0, rows=None, positions=None,
                   block_table=None, kv_lens=None, stream=None) -> None:
    """Write [n, Hkv, 128] K/V values to their slots (int32 [n]).  slots, rows
    and positions may be device tensors or pinned host tensors."""
    if k_new.dtype != cache.value_dtype or v_new.dtype != cache.value_dtype:
        raise PagedKVError(-4, f"values must be {cache.value_dtype}")
    for t in (k_new, v_new, slots):
        if not t.is_contiguous():
            raise PagedKVError(-1, "tensors must be contiguous")
    n = int(slots.numel())
    want = (n, cache.num_kv_heads, HEAD_DIM)
    if tuple(k_new.shape) != want or tuple(v_new.shape) != want or slots.dtype != torch.int32:
        raise PagedKVError(-1, f"k_new/v_new must be {want} and slots int32 [n]")
    for t in (rows, positions):
        if t is not None and (t.dtype != torch.int32 or t.numel() != n):
            raise PagedKVError(-1, "rows/positions must be int32 [n]")
    num_rows = int(block_table.shape[0]) if block_table is not None else 0
    max_blocks = int(block_table.shape[1]) if block_table is not None else 0
    _check(_lib.kv_cache_write(ctypes.byref(cache.desc), layer, n,
                               PKV_F32 if cache.value_dtype == torch.float32 else PKV_BF16,
                               _ptr(k_new), _ptr(v_new), _dev_ptr(slots), _dev_ptr(rows), _dev_ptr(positions),
                               num_rows,
                               _ptr(block_table), max_blocks, _ptr(kv_lens), _stream(stream)))


def kv_swap_block_bytes(cache: KVCache) -> int:
    n = ctypes.c_size_t()
    _check(_lib.kv_swap_block_bytes(ctypes.byref(cache.desc), ctypes.byref(n)))
    return n.value


def _swap_args(cache: KVCache, ids, host):
    ids = [int(b) for b in ids]
    need = len(ids) * kv_swap_block_bytes(cache)
    if host.is_cuda or not host.is_contiguous() or host.numel() * host.element_size() < need:
        raise PagedKVError(-1, f"host swap buffer must be a contiguous host tensor of at least {need} bytes")
    return (ctypes.c_int32 * max(1, len(ids)))(*ids), len(ids)


def kv_swap_out(cache: KVCache, ids, host, stream=None) -> None:
    """Copy blocks ids[i] (all layers, K and V) to slot i of the pinned host
    tensor ``host`` (at least len(ids) * kv_swap_block_bytes bytes)."""
    arr, n = _swap_args(cache, ids, host)
    _check(_lib.kv_swap_out(ctypes.byref(cache.desc), arr, n, ctypes.c_void_p(host.data_ptr()), _stream(stream)))


def kv_swap_in(cache: KVCache, host, ids, stream=None) -> None:
    """Copy slot i of the pinned host tensor ``host`` into block ids[i]."""
    arr, n = _swap_args(cache, ids, host)
    _check(_lib.kv_swap_in(ctypes.byref(cache.desc), ctypes.c_void_p(host.data_ptr()), arr, n, _stream(stream)))


def kv_copy_blocks(cache: KVCache, copies, stream=None) -> None:
    """copies: iterable of (src, dst, valid_tokens)."""
    copies = list(copies)
    arr = (pkv_copy * max(1, len(copies)))(*[pkv_copy(*c) for c in copies])
    _check(_lib.kv_copy_blocks(ctypes.byref(cache.desc), arr, len(copies), _stream(stream)))
