"""Python binding of libpagedkv.so (ctypes).

Argument marshalling only: every step of the cache write and of decode
attention runs in the library's HIP kernels.  Torch provides device memory
and the current stream; the functions check device, dtype, shape and
contiguity, then pass raw pointers to the C ABI declared in
``include/pagedkv.h``.  There is no fallback: if the library is not built,
or a call fails, a ``RuntimeError`` is raised.

Pool layout (see the header): ``k_cache [num_blocks, Hkv, D/x, 16, x]`` with
``x = 16 / element_size`` and ``v_cache [num_blocks, Hkv, D, 16]``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")
BLOCK_SIZE = 16

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
FP8_POOL_DTYPES = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}

_lib = None

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_u32 = ctypes.c_uint32

DECODE_SHARED_BLOCKS = 1   # decode flag: sequences share blocks, read K/V through the caches

_SIGNATURES = {
    "pkv_abi_version": (_i32, []),
    "pkv_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attention_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                                          _i32, _i32, _i32, _vp, _sz, _i32, _i32, _u32, _vp]),
    "pkv_paged_attention_decode_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32,
                                                     _i64, _i32, _i32, _i32, _vp, _sz, _i32, _i32, _u32, _vp]),
    "pkv_paged_attention_decode_reduce": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _sz,
                                                 _i32, _i32, _vp]),
    "pkv_paged_attention_decode_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32,
                                                 _i32, _i64, _i32, _i32, _i32, _vp, _sz, _i32, _i32, _u32, _vp]),
    "pkv_paged_attention_decode_append_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32,
                                                            _i32, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _sz, _i32,
                                                            _i32, _u32, _vp]),
    "pkv_paged_attention_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32,
                                                  _i64, _i32, _i32, _i32, _i32, _i32, _u32, _vp]),
    "pkv_reshape_and_cache_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pkv_paged_attention_decode_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32,
                                              _i64, _i32, _i32, _i32, _vp, _sz, _i32, _u32, _vp]),
    "pkv_paged_attention_decode_partitions_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32,
                                                         _i32, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _sz, _i32,
                                                         _u32, _vp]),
    "pkv_paged_attention_decode_append_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32,
                                                     _i32, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _sz, _i32, _u32,
                                                     _vp]),
    "pkv_paged_attention_decode_append_partitions_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp,
                                                                _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                                                _vp, _sz, _i32, _u32, _vp]),
    "pkv_copy_blocks": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp]),
    "pkv_paged_attention_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                           _i64, _i32, _i32, _i32, _i32, _vp]),
    "pkv_paged_attention_prefill_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32,
                                               _i32, _i32, _i32, _i64, _i32, _i32, _i32, _vp]),
    "pkv_paged_attention_decode_vector_alu": (_i32, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32,
                                                     _i32, _i64, _i32, _i32, _i32, _vp, _sz, _i32, _vp]),
    "pkv_hbm_read_bench": (_i32, [_vp, _i64, _vp, _i64, _i32, _i32, _vp, _vp]),
    "pkv_issue_rate_bench": (_i32, [_i32, _i32, _i32, _vp, _vp]),
    "pkv_status_string": (ctypes.c_char_p, [_i32]),
    "pkv_last_error": (ctypes.c_char_p, []),
}


def load_library(path: str = LIB_PATH):
    """Load libpagedkv.so (after torch, so it binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m paged_kv_cache_372_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.pkv_last_error().decode(errors="replace")
        raise RuntimeError(f"{what} failed: {_STATUS.get(status, status)}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_tensor(t: torch.Tensor, name: str, device: torch.device) -> None:
    _require(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _require(t.device == device, f"{name} is on {t.device}, expected {device}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def pool_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype) -> Tuple[tuple, tuple]:
    """Shapes of the K and V pools for this library's layout."""
    x = 16 // torch.empty((), dtype=dtype).element_size()
    return ((num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x), (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE))


def _pool_dims(k_cache: torch.Tensor, v_cache: torch.Tensor) -> Tuple[int, int, int]:
    _require(k_cache.dim() == 5 and v_cache.dim() == 4, "k_cache must be 5-D and v_cache 4-D (see pool_shapes)")
    nb, hkv, nch, bs, x = k_cache.shape
    D = nch * x
    _require(bs == BLOCK_SIZE, f"block_size must be {BLOCK_SIZE}")
    _require(x * k_cache.element_size() == 16, "k_cache last dim must span 16 bytes")
    _require(tuple(v_cache.shape) == (nb, hkv, D, bs), f"v_cache shape {tuple(v_cache.shape)} != {(nb, hkv, D, bs)}")
    _require(k_cache.dtype == v_cache.dtype, "k_cache and v_cache dtypes differ")
    return nb, hkv, D


def reshape_and_cache(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Write k_new/v_new ``[T, Hkv, D]`` into the pools at ``slot_mapping`` (int64 ``[T]``)."""
    lib = load_library()
    dev = k_cache.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (slot_mapping, "slot_mapping"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _check_tensor(t, n, dev)
    nb, hkv, D = _pool_dims(k_cache, v_cache)
    _require(k_new.dim() == 3 and tuple(k_new.shape[1:]) == (hkv, D), f"k_new must be [T, {hkv}, {D}]")
    _require(v_new.shape == k_new.shape, "v_new shape must match k_new")
    _require(k_new.dtype == k_cache.dtype and v_new.dtype == k_cache.dtype, "new K/V dtype must match the pools")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (k_new.shape[0],),
             "slot_mapping must be int64 [T]")
    st = lib.pkv_reshape_and_cache(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                                   k_new.shape[0], hkv, D, BLOCK_SIZE, nb, _dtype_code(k_cache), _stream(dev))
    _check(st, "reshape_and_cache")


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_context_len: int, partition_size: int = 0, kv_dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes a decode of these sizes needs on the current device."""
    code = PKV_BF16 if kv_dtype == torch.bfloat16 else (PKV_FP8_E4M3 if kv_dtype in FP8_POOL_DTYPES else PKV_F32)
    return int(load_library().pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                         max_context_len, partition_size, code))


class _DecodeArgs:
    """Validated decode arguments, reused by the one-call and two-phase entry points.

    A plan holds references to every tensor it points at, so none of them is
    freed (and its memory handed to another tensor) while the plan lives.
    Fixed when the plan is built: the stream (the device's current stream at
    that moment) and ``max_context_len``, which bounds the context lengths
    the kernels read (longer ones are clamped to it).  Build a new plan when
    either changes, e.g. when contexts grow past the bound.
    """

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, out, partition_size,
                 max_context_len, workspace, shared_blocks=False, k_scale=None, v_scale=None, k_new=None,
                 v_new=None):
        dev = q.device
        self._keep = (q, k_cache, v_cache, block_tables, context_lens, out, k_scale, v_scale, k_new, v_new)
        self.fp8 = k_cache.dtype in FP8_POOL_DTYPES
        self.append = k_new is not None or v_new is not None
        for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                     (context_lens, "context_lens"), (out, "out")):
            _check_tensor(t, n, dev)
        nb, hkv, D = _pool_dims(k_cache, v_cache)
        _require(q.dim() == 3 and q.shape[2] == D, f"q must be [B, Hq, {D}]")
        B, hq = q.shape[0], q.shape[1]
        if self.fp8:
            _require(q.dtype == torch.bfloat16, "q must be bf16 over an fp8 cache")
            _require(k_scale is not None and v_scale is not None, "an fp8 cache needs k_scale and v_scale")
            _check_scales(k_scale, v_scale, hkv, dev)
        else:
            _require(q.dtype == k_cache.dtype, "q dtype must match the pools")
        _require(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
        _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
                 "block_tables must be int32 [B, max_blocks_per_seq]")
        _require(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (B,), "context_lens must be int32 [B]")
        if max_context_len is None:  # costs a device->host synchronisation
            max_context_len = int(context_lens.max().item()) if B else 0
        self.max_context_len = int(max_context_len)
        self.B, self.hq, self.hkv, self.D, self.nb = B, hq, hkv, D, nb
        self.partition_size = int(partition_size)
        need = decode_workspace_bytes(B, hq, hkv, D, self.max_context_len, self.partition_size, k_cache.dtype)
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace is not None:
            _check_tensor(workspace, "workspace", dev)
        self.workspace = workspace
        self.ws_ptr = _ptr(workspace) if workspace is not None else None
        self.ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        flags = DECODE_SHARED_BLOCKS if shared_blocks else 0
        if self.append:
            _require(self.fp8 or k_cache.dtype == torch.bfloat16, "the fused append takes bf16 or fp8 pools")
            _require(k_new is not None and v_new is not None, "the fused append needs both k_new and v_new")
            _check_tensor(k_new, "k_new", dev)
            _check_tensor(v_new, "v_new", dev)
            _require(tuple(k_new.shape) == (B, hkv, D) and tuple(v_new.shape) == (B, hkv, D),
                     f"k_new and v_new must be [B, {hkv}, {D}]")
            _require(k_new.dtype == torch.bfloat16 and v_new.dtype == torch.bfloat16, "new K/V rows must be bf16")
            if self.fp8:
                self.args = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                             _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), float(scale), _ptr(out), B, hq,
                             hkv, D, BLOCK_SIZE, nb, block_tables.shape[1], self.max_context_len,
                             self.partition_size, self.ws_ptr, self.ws_bytes, _dtype_code(out), flags, _stream(dev))
            else:
                self.args = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                             _ptr(context_lens), float(scale), _ptr(out), B, hq, hkv, D, BLOCK_SIZE, nb,
                             block_tables.shape[1], self.max_context_len, self.partition_size, self.ws_ptr,
                             self.ws_bytes, _dtype_code(k_cache), _dtype_code(out), flags, _stream(dev))
        elif self.fp8:
            self.args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                         _ptr(context_lens), float(scale), _ptr(out), B, hq, hkv, D, BLOCK_SIZE, nb,
                         block_tables.shape[1], self.max_context_len, self.partition_size, self.ws_ptr,
                         self.ws_bytes, _dtype_code(out), flags, _stream(dev))
        else:
            self.args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                         float(scale), _ptr(out), B, hq, hkv, D, BLOCK_SIZE, nb, block_tables.shape[1],
                         self.max_context_len, self.partition_size, self.ws_ptr, self.ws_bytes,
                         _dtype_code(k_cache), _dtype_code(out), flags, _stream(dev))
        self.reduce_args = (_ptr(context_lens), _ptr(out), B, hq, hkv, D, BLOCK_SIZE, block_tables.shape[1],
                            self.max_context_len, self.partition_size, self.ws_ptr, self.ws_bytes,
                            PKV_FP8_E4M3 if self.fp8 else _dtype_code(k_cache), _dtype_code(out), _stream(dev))


def paged_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           out: torch.Tensor, *, partition_size: int = 0, max_context_len: Optional[int] = None,
                           workspace: Optional[torch.Tensor] = None, shared_blocks: bool = False) -> None:
    """Decode attention of ``q [B, Hq, D]`` over the paged cache into ``out``.

    ``max_context_len`` (host-known bound of ``context_lens``) avoids a
    device-to-host sync; ``workspace`` (uint8, >= ``decode_workspace_bytes``,
    reusable) avoids an allocation.  ``shared_blocks``: several sequences
    point at the same physical blocks (a common prefix); K/V are then read
    through the caches instead of streamed.  It never changes the result.
    """
    a = _DecodeArgs(q, k_cache, v_cache, block_tables, context_lens, scale, out, partition_size, max_context_len,
                    workspace, shared_blocks)
    _check(load_library().pkv_paged_attention_decode(*a.args), "paged_attention_decode")


def paged_attention_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float, out: torch.Tensor, *,
                                  partition_size: int = 0, max_context_len: Optional[int] = None,
                                  workspace: Optional[torch.Tensor] = None, shared_blocks: bool = False) -> None:
    """One decode step in one launch pair: store ``k_new``/``v_new [B, Hkv, D]`` (bf16) at position
    ``context_lens[s] - 1`` of each sequence, then attend as ``paged_attention_decode``.

    Pool and output equal ``reshape_and_cache`` with the slots of those positions followed by
    ``paged_attention_decode``, bit for bit; at most 16 query heads per KV head.
    """
    a = _DecodeArgs(q, k_cache, v_cache, block_tables, context_lens, scale, out, partition_size, max_context_len,
                    workspace, shared_blocks, k_new=k_new, v_new=v_new)
    _check(load_library().pkv_paged_attention_decode_append(*a.args), "paged_attention_decode_append")


def paged_attention_decode_append_fp8(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                      k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                                      v_scale: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                                      scale: float, out: torch.Tensor, *, partition_size: int = 0,
                                      max_context_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                                      shared_blocks: bool = False) -> None:
    """``paged_attention_decode_append`` over fp8 (E4M3) pools: the bf16 rows ``k_new``/``v_new``
    ``[B, Hkv, D]`` are stored as the codes ``reshape_and_cache_fp8`` would store (per-KV-head
    ``k_scale``/``v_scale``), then the step attends as ``paged_attention_decode_fp8``; pools and output
    equal those two calls, bit for bit."""
    a = _DecodeArgs(q, k_cache, v_cache, block_tables, context_lens, scale, out, partition_size, max_context_len,
                    workspace, shared_blocks, k_scale, v_scale, k_new=k_new, v_new=v_new)
    _check(load_library().pkv_paged_attention_decode_append_fp8(*a.args), "paged_attention_decode_append_fp8")


NOALLOC_SCRATCH_BYTES = 64 << 20   # the library's fixed decode scratch (PKV_NOALLOC_SCRATCH_BYTES)


def paged_attention_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                   out: torch.Tensor, *, max_context_len: int, partition_size: int = 0,
                                   shared_blocks: bool = False) -> None:
    """``paged_attention_decode`` with no workspace and no allocation, for callers that cannot allocate
    (graph capture, tight serving loops).  The library's fixed per-device scratch
    (``NOALLOC_SCRATCH_BYTES``) stands in for the workspace; sizes that need more raise.  Calls that
    overlap on one device (other streams, other threads) race on that scratch.  ``max_context_len`` is
    required: finding it on the device would need a synchronisation and an allocation.  bf16 or f32 pools.
    """
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens"), (out, "out")):
        _check_tensor(t, n, dev)
    nb, hkv, D = _pool_dims(k_cache, v_cache)
    _require(q.dim() == 3 and q.shape[2] == D and q.dtype == k_cache.dtype, f"q must be [B, Hq, {D}] of the pools' dtype")
    B, hq = q.shape[0], q.shape[1]
    _require(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
             "block_tables must be int32 [B, max_blocks_per_seq]")
    _require(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (B,), "context_lens must be int32 [B]")
    _require(max_context_len is not None, "max_context_len is required")
    st = lib.pkv_paged_attention_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                                _ptr(context_lens), float(scale), _ptr(out), B, hq, hkv, D,
                                                BLOCK_SIZE, nb, block_tables.shape[1], int(max_context_len),
                                                int(partition_size), _dtype_code(k_cache), _dtype_code(out),
                                                DECODE_SHARED_BLOCKS if shared_blocks else 0, _stream(dev))
    _check(st, "paged_attention_decode_noalloc")


def prepare_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, *, partition_size=0,
                   max_context_len=None, workspace=None, shared_blocks=False, k_scale=None,
                   v_scale=None, k_new=None, v_new=None) -> _DecodeArgs:
    """Validate once; the returned plan drives ``run_decode`` / ``run_partitions`` / ``run_reduce``
    repeatedly on the same tensors (their contents may change between runs).  The plan keeps those
    tensors alive, and fixes the stream (the current one now) and ``max_context_len`` (contexts longer
    than it are clamped): build a new plan when either must change.  fp8 pools (uint8 /
    float8_e4m3fn) take ``k_scale`` / ``v_scale``; ``k_new`` / ``v_new`` select the fused append
    (``paged_attention_decode_append``)."""
    return _DecodeArgs(q, k_cache, v_cache, block_tables, context_lens, scale, out, partition_size, max_context_len,
                       workspace, shared_blocks, k_scale, v_scale, k_new, v_new)


def run_decode(a: _DecodeArgs) -> None:
    lib = load_library()
    if a.append and a.fp8:
        _check(lib.pkv_paged_attention_decode_append_fp8(*a.args), "paged_attention_decode_append_fp8")
    elif a.append:
        _check(lib.pkv_paged_attention_decode_append(*a.args), "paged_attention_decode_append")
    elif a.fp8:
        _check(lib.pkv_paged_attention_decode_fp8(*a.args), "paged_attention_decode_fp8")
    else:
        _check(lib.pkv_paged_attention_decode(*a.args), "paged_attention_decode")


def run_partitions(a: _DecodeArgs) -> None:
    lib = load_library()
    if a.append and a.fp8:
        _check(lib.pkv_paged_attention_decode_append_partitions_fp8(*a.args),
               "paged_attention_decode_append_partitions_fp8")
    elif a.append:
        _check(lib.pkv_paged_attention_decode_append_partitions(*a.args), "paged_attention_decode_append_partitions")
    elif a.fp8:
        _check(lib.pkv_paged_attention_decode_partitions_fp8(*a.args), "paged_attention_decode_partitions_fp8")
    else:
        _check(lib.pkv_paged_attention_decode_partitions(*a.args), "paged_attention_decode_partitions")


def run_reduce(a: _DecodeArgs) -> None:
    _check(load_library().pkv_paged_attention_decode_reduce(*a.reduce_args), "paged_attention_decode_reduce")


def _prefill_args(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, out, max_context_len, fp8):
    """Validated shapes of a prefill call: (B, T, Hq, Hkv, D, num_blocks, max_context_len)."""
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens"), (query_start_loc, "query_start_loc"), (out, "out")):
        _check_tensor(t, n, dev)
    nb, hkv, D = _pool_dims(k_cache, v_cache)
    if fp8:
        _require(k_cache.dtype in FP8_POOL_DTYPES and v_cache.dtype == k_cache.dtype,
                 "fp8 pools must be uint8 or float8_e4m3fn")
    else:
        _require(k_cache.dtype == torch.bfloat16, "prefill takes bf16 pools (fp8: paged_attention_prefill_fp8)")
    _require(q.dim() == 3 and q.shape[2] == D and q.dtype == torch.bfloat16, f"q must be bf16 [T, Hq, {D}]")
    T, hq = q.shape[0], q.shape[1]
    B = context_lens.shape[0] if context_lens.dim() == 1 else -1
    _require(context_lens.dtype == torch.int32 and B >= 0, "context_lens must be int32 [B]")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
             "block_tables must be int32 [B, max_blocks_per_seq]")
    _require(query_start_loc.dtype == torch.int32 and tuple(query_start_loc.shape) == (B + 1,),
             "query_start_loc must be int32 [B + 1]")
    _require(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    if max_context_len is None:  # costs a device->host synchronisation
        max_context_len = int(context_lens.max().item()) if B else 0
    return B, T, hq, hkv, D, nb, int(max_context_len)


def paged_attention_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                            scale: float, out: torch.Tensor, *, max_context_len: Optional[int] = None) -> None:
    """Multi-token-query (chunked prefill) attention of ``q [T, Hq, D]`` into ``out``.

    Request ``s`` owns rows ``query_start_loc[s] .. query_start_loc[s+1]-1``:
    the last ``n_s`` of its ``context_lens[s]`` cached tokens, each attending
    causally over its sequence.  bf16 pools (fp8: ``paged_attention_prefill_fp8``).
    """
    lib = load_library()
    B, T, hq, hkv, D, nb, mcl = _prefill_args(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                                              out, max_context_len, False)
    st = lib.pkv_paged_attention_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                         _ptr(context_lens), _ptr(query_start_loc), float(scale), _ptr(out), B, T,
                                         hq, hkv, D, BLOCK_SIZE, nb, block_tables.shape[1], mcl,
                                         _dtype_code(k_cache), _dtype_code(out), _stream(q.device))
    _check(st, "paged_attention_prefill")


def paged_attention_prefill_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                k_scale: torch.Tensor, v_scale: torch.Tensor, block_tables: torch.Tensor,
                                context_lens: torch.Tensor, query_start_loc: torch.Tensor, scale: float,
                                out: torch.Tensor, *, max_context_len: Optional[int] = None) -> None:
    """Chunked-prefill attention of bf16 ``q [T, Hq, D]`` over fp8 (E4M3) pools with per-KV-head scales."""
    lib = load_library()
    B, T, hq, hkv, D, nb, mcl = _prefill_args(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                                              out, max_context_len, True)
    _check_scales(k_scale, v_scale, hkv, q.device)
    st = lib.pkv_paged_attention_prefill_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                             _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc),
                                             float(scale), _ptr(out), B, T, hq, hkv, D, BLOCK_SIZE, nb,
                                             block_tables.shape[1], mcl, _dtype_code(out), _stream(q.device))
    _check(st, "paged_attention_prefill_fp8")


def _check_scales(k_scale: torch.Tensor, v_scale: torch.Tensor, hkv: int, device) -> None:
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _check_tensor(t, n, device)
        _require(t.dtype == torch.float32 and tuple(t.shape) == (hkv,), f"{n} must be float32 [{hkv}]")


def reshape_and_cache_fp8(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                          k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                          v_scale: torch.Tensor) -> None:
    """Quantise k_new/v_new ``[T, Hkv, D]`` (f32 or bf16) into fp8 (E4M3) pools with per-KV-head scales."""
    lib = load_library()
    dev = k_cache.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (slot_mapping, "slot_mapping"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _check_tensor(t, n, dev)
    _require(k_cache.dtype in FP8_POOL_DTYPES and v_cache.dtype == k_cache.dtype, "fp8 pools must be uint8 or float8_e4m3fn")
    nb, hkv, D = _pool_dims(k_cache, v_cache)
    _require(k_new.dim() == 3 and tuple(k_new.shape[1:]) == (hkv, D), f"k_new must be [T, {hkv}, {D}]")
    _require(v_new.shape == k_new.shape and v_new.dtype == k_new.dtype, "v_new must match k_new")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (k_new.shape[0],),
             "slot_mapping must be int64 [T]")
    _check_scales(k_scale, v_scale, hkv, dev)
    st = lib.pkv_reshape_and_cache_fp8(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(k_scale), _ptr(v_scale), k_new.shape[0], hkv, D, BLOCK_SIZE, nb,
                                       _dtype_code(k_new), _stream(dev))
    _check(st, "reshape_and_cache_fp8")


def paged_attention_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                               v_scale: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                               scale: float, out: torch.Tensor, *, partition_size: int = 0,
                               max_context_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                               shared_blocks: bool = False) -> None:
    """Decode attention of bf16 ``q [B, Hq, D]`` over fp8 (E4M3) pools with per-KV-head scales."""
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens"), (out, "out")):
        _check_tensor(t, n, dev)
    _require(k_cache.dtype in FP8_POOL_DTYPES and v_cache.dtype == k_cache.dtype, "fp8 pools must be uint8 or float8_e4m3fn")
    nb, hkv, D = _pool_dims(k_cache, v_cache)
    _require(q.dim() == 3 and q.shape[2] == D and q.dtype == torch.bfloat16, f"q must be bf16 [B, Hq, {D}]")
    B, hq = q.shape[0], q.shape[1]
    _require(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
             "block_tables must be int32 [B, max_blocks_per_seq]")
    _require(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (B,), "context_lens must be int32 [B]")
    _check_scales(k_scale, v_scale, hkv, dev)
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    need = decode_workspace_bytes(B, hq, hkv, D, int(max_context_len), int(partition_size), torch.uint8)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.pkv_paged_attention_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                            _ptr(block_tables), _ptr(context_lens), float(scale), _ptr(out), B, hq,
                                            hkv, D, BLOCK_SIZE, nb, block_tables.shape[1], int(max_context_len),
                                            int(partition_size), ws_ptr, ws_bytes, _dtype_code(out),
                                            DECODE_SHARED_BLOCKS if shared_blocks else 0, _stream(dev))
    _check(st, "paged_attention_decode_fp8")


def _pool_code(t: torch.Tensor) -> int:
    return PKV_FP8_E4M3 if t.dtype in FP8_POOL_DTYPES else _dtype_code(t)


def swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor, dst_v: torch.Tensor,
                pairs: torch.Tensor) -> None:
    """Copy whole blocks ``pairs[i] = (src, dst)`` from the source pools to the destination pools.

    Pools may be device tensors or pinned host tensors (``pin_memory=True``);
    ``pairs`` is int64 ``[n, 2]`` on the device or pinned.  The launch goes on
    the current stream of the device that holds a device-side pool.
    """
    lib = load_library()
    dev_t = next((t for t in (src_k, dst_k) if t.is_cuda), None)
    _require(dev_t is not None, "at least one side must be a device pool")
    for t, n in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v"), (pairs, "pairs")):
        _require(isinstance(t, torch.Tensor) and t.is_contiguous(), f"{n} must be a contiguous tensor")
        _require(t.is_cuda or t.is_pinned(), f"{n} must be on the device or in pinned host memory")
    nbs, hkv, D = _pool_dims(src_k, src_v)
    nbd, hkv2, D2 = _pool_dims(dst_k, dst_v)
    _require((hkv, D) == (hkv2, D2) and src_k.dtype == dst_k.dtype, "source and destination pools differ in shape")
    _require(pairs.dtype == torch.int64 and pairs.dim() == 2 and pairs.shape[1] == 2, "pairs must be int64 [n, 2]")
    st = lib.pkv_copy_blocks(_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(pairs), pairs.shape[0], nbs,
                             nbd, hkv, D, BLOCK_SIZE, _pool_code(src_k), _stream(dev_t.device))
    _check(st, "copy_blocks")


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs: torch.Tensor) -> None:
    """Copy-on-write inside one pool: block ``src`` to block ``dst`` for every pair of ``pairs`` (int64 ``[n, 2]``)."""
    swap_blocks(k_cache, v_cache, k_cache, v_cache, pairs)


def hbm_read_bench(src: torch.Tensor, sink: torch.Tensor, tiles: Optional[torch.Tensor] = None,
                   tile_bytes: int = 4096, streaming: bool = True) -> None:
    """Measurement aid: read ``src`` (contiguous, device) front to back, or the tiles ``tiles`` (int32,
    device) of ``tile_bytes`` each, with nothing else done; ``sink`` is a device uint32 ``[1024]``."""
    lib = load_library()
    dev = src.device
    _check_tensor(src, "src", dev)
    _check_tensor(sink, "sink", dev)
    _require(sink.dtype in (torch.int32, torch.uint32) and sink.numel() >= 1024, "sink must be 32-bit [1024]")
    if tiles is not None:
        _check_tensor(tiles, "tiles", dev)
        _require(tiles.dtype == torch.int32 and tiles.dim() == 1, "tiles must be int32 [n]")
    nbytes = src.numel() * src.element_size()
    st = lib.pkv_hbm_read_bench(_ptr(src), nbytes, _ptr(tiles) if tiles is not None else None,
                                tiles.numel() if tiles is not None else 0, int(tile_bytes), 1 if streaming else 0,
                                _ptr(sink), _stream(dev))
    _check(st, "hbm_read_bench")


ISSUE_RATE_PATTERNS = ("mfma_16x16x32_bf16_1acc", "mfma_16x16x32_bf16_4acc", "mfma_32x32x16_bf16_1acc",
                       "mfma_32x32x16_bf16_4acc", "v_fma_f32", "v_exp_f32+v_add_f32", "ds_read_b128")


def issue_rate_bench(pattern: int, waves_per_simd: int, iters: int, sink: torch.Tensor) -> None:
    """Measurement aid: one launch of ``iters`` x 16 instructions of pattern ``pattern``
    (``ISSUE_RATE_PATTERNS``) per wave, one workgroup of 256 x ``waves_per_simd`` threads per
    compute unit; ``sink`` is a device 32-bit tensor of at least 512 elements."""
    lib = load_library()
    dev = sink.device
    _check_tensor(sink, "sink", dev)
    _require(sink.dtype in (torch.int32, torch.uint32) and sink.numel() >= 512, "sink must be 32-bit [>= 512]")
    _check(lib.pkv_issue_rate_bench(int(pattern), int(waves_per_simd), int(iters), _ptr(sink), _stream(dev)),
           "issue_rate_bench")


def paged_attention_decode_vector_alu(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                      out: torch.Tensor, *, partition_size: int = 0,
                                      max_context_len: Optional[int] = None,
                                      workspace: Optional[torch.Tensor] = None) -> None:
    """Measurement aid: bf16 decode with every product an fp32 FMA on the vector ALU (the fp32 path's
    kernel); agrees with ``paged_attention_decode`` within the bf16 bar."""
    lib = load_library()
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens"), (out, "out")):
        _check_tensor(t, n, dev)
    nb, hkv, D = _pool_dims(k_cache, v_cache)
    _require(k_cache.dtype == torch.bfloat16 and q.dtype == torch.bfloat16, "bf16 q and pools")
    _require(q.dim() == 3 and q.shape[2] == D, f"q must be [B, Hq, {D}]")
    B, hq = q.shape[0], q.shape[1]
    _require(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
             "block_tables must be int32 [B, max_blocks_per_seq]")
    _require(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (B,), "context_lens must be int32 [B]")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    need = decode_workspace_bytes(B, hq, hkv, D, int(max_context_len), int(partition_size), torch.float32)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.pkv_paged_attention_decode_vector_alu(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                                   _ptr(context_lens), float(scale), _ptr(out), B, hq, hkv, D,
                                                   BLOCK_SIZE, nb, block_tables.shape[1], int(max_context_len),
                                                   int(partition_size), ws_ptr, ws_bytes, _dtype_code(out),
                                                   _stream(dev))
    _check(st, "paged_attention_decode_vector_alu")

