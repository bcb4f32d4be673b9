"""MI355X-native paged decode attention - Python binding of libpagedkv.so.

Thin marshalling over the C ABI in ``include/pagedkv.h``: every function
checks tensor dtypes/shapes/devices, passes raw device pointers and torch's
current HIP stream, and raises on a non-zero status.  All arithmetic runs in
the HIP kernels; nothing here falls back to PyTorch or the CPU.  If the
library is not built, :func:`lib` raises.

Sources: [ITH] iThome ithelp article 10405755 on PagedAttention; [PU] Fanyi Pu,
"Infra: PagedAttention" (sections cited per function).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

from .block_manager import BlockManager, PoolExhaustedError, block_key, slot_mapping_for
from .scheduler import Batcher, Request

__all__ = [
    "lib", "paged_attention_decode", "paged_attention_decode_append",
    "paged_attention_decode_noalloc", "reshape_and_cache",
    "copy_blocks", "cascade_decode", "cascade_workspace_size", "cascade_plan_kernel",
    "paged_prefill", "swap_out",
    "swap_in", "swap_buffer",
    "merge_attention_states", "decode_workspace_size", "DecodeWorkspace", "new_kv_cache",
    "BlockManager", "Batcher", "Request", "block_key",
    "PoolExhaustedError", "slot_mapping_for", "PagedKVError", "LIB_PATH",
    "check_decode_inputs", "check_slot_mapping", "check_block_pairs",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_OK, PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP = 0, -1, -2, -3, -4
_DTYPES = {torch.bfloat16: 0, torch.float32: 1}
_KERNELS = {"auto": 0, "mfma": 1, "generic": 2, "stream": 3, "stream_wg": 4}


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().pkv_status_string(status).decode()} ({status})")


class DecodeDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("partition_size", ctypes.c_int32),
        ("out_dtype", ctypes.c_int),
        ("kernel", ctypes.c_int),
        ("waves_per_group", ctypes.c_int32),
        ("balance_partitions", ctypes.c_int32),
        ("stream_waves", ctypes.c_int32),
        ("no_shared_blocks", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_373_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        dims_p = ctypes.POINTER(DecodeDims)
        L.pkv_decode_workspace_size.argtypes = [dims_p, i32]
        L.pkv_decode_workspace_size.restype = sz
        L.pkv_decode_workspace_zeroed_bytes.argtypes = [dims_p, i32]
        L.pkv_decode_workspace_zeroed_bytes.restype = sz
        L.pkv_decode_plan_kernel.argtypes = [dims_p, i32]
        L.pkv_decode_plan_kernel.restype = i32
        L.pkv_paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, i32, ctypes.c_float, vp,
                                                 dims_p, vp, sz, vp]
        L.pkv_paged_attention_decode.restype = ctypes.c_int
        L.pkv_paged_attention_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32,
                                                        ctypes.c_float, vp, dims_p, vp, sz, vp]
        L.pkv_paged_attention_decode_append.restype = ctypes.c_int
        L.pkv_paged_attention_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, ctypes.c_float,
                                                         vp, dims_p, vp]
        L.pkv_paged_attention_decode_noalloc.restype = ctypes.c_int
        L.pkv_reshape_and_cache.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, i32, i32, vp]
        L.pkv_reshape_and_cache.restype = ctypes.c_int
        L.pkv_copy_blocks.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i32, i64,
                                      vp]
        L.pkv_copy_blocks.restype = ctypes.c_int
        L.pkv_merge_attention_states.argtypes = [vp, vp, i32, i32, i32, vp, ctypes.c_int, vp]
        L.pkv_merge_attention_states.restype = ctypes.c_int
        L.pkv_cascade_workspace_size.argtypes = [dims_p, i32, i32, i32]
        L.pkv_cascade_workspace_size.restype = sz
        L.pkv_cascade_plan_kernel.argtypes = [dims_p, i32, i32, i32]
        L.pkv_cascade_plan_kernel.restype = i32
        L.pkv_cascade_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                         ctypes.c_float, vp, dims_p, vp, sz, vp]
        L.pkv_cascade_decode.restype = ctypes.c_int
        L.pkv_paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_float,
                                        vp, dims_p, vp]
        L.pkv_paged_prefill.restype = ctypes.c_int
        for name in ("pkv_swap_out", "pkv_swap_in"):
            getattr(L, name).argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i32, i64,
                                         vp, vp]
            getattr(L, name).restype = ctypes.c_int
        L.pkv_check_decode_inputs.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp]
        L.pkv_check_decode_inputs.restype = ctypes.c_int
        L.pkv_check_slot_mapping.argtypes = [vp, i32, i32, i32, vp, vp]
        L.pkv_check_slot_mapping.restype = ctypes.c_int
        L.pkv_check_block_pairs.argtypes = [vp, i32, i32, vp, vp]
        L.pkv_check_block_pairs.restype = ctypes.c_int
        L.pkv_status_string.argtypes = [i32]
        L.pkv_status_string.restype = ctypes.c_char_p
        L.pkv_abi_version.restype = i32
        _lib = L
    return _lib


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def new_kv_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 device="cuda", fill: Optional[float] = None):
    """Allocate (k_cache [P,Hkv,B,D], v_cache [P,Hkv,D,B]) in bf16."""
    k = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=torch.bfloat16,
                    device=device)
    v = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=torch.bfloat16,
                    device=device)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return k, v


def _dims(q, k_cache, block_tables, max_seq_len, partition_size, out_dtype, kernel,
          waves_per_group, balance_partitions, stream_waves=0,
          no_shared_blocks=False) -> DecodeDims:
    s, hq, d = q.shape
    p, hkv, bs, _ = k_cache.shape
    mb = block_tables.shape[1]
    return DecodeDims(s, hq, hkv, d, p, mb, mb * bs if max_seq_len is None else int(max_seq_len),
                      int(partition_size), _DTYPES[out_dtype], _KERNELS[kernel],
                      int(waves_per_group), int(bool(balance_partitions)), int(stream_waves),
                      int(bool(no_shared_blocks)))


def decode_workspace_size(q, k_cache, block_tables, *, max_seq_len=None, partition_size=0,
                          out_dtype=torch.bfloat16, kernel="auto", waves_per_group=0,
                          balance_partitions=False, stream_waves=0,
                          no_shared_blocks=False) -> int:
    dims = _dims(q, k_cache, block_tables, max_seq_len, partition_size, out_dtype, kernel,
                 waves_per_group, balance_partitions, stream_waves, no_shared_blocks)
    n = lib().pkv_decode_workspace_size(ctypes.byref(dims), k_cache.shape[2])
    if n == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID, "pkv_decode_workspace_size")
    return int(n)


def decode_plan_kernel(q, k_cache, block_tables, *, max_seq_len=None, partition_size=0,
                       out_dtype=torch.bfloat16, kernel="auto", waves_per_group=0,
                       balance_partitions=False, stream_waves=0,
                       no_shared_blocks=False) -> str:
    """Name of the kernel family a decode call with these arguments runs
    (what ``kernel="auto"`` resolves to)."""
    dims = _dims(q, k_cache, block_tables, max_seq_len, partition_size, out_dtype, kernel,
                 waves_per_group, balance_partitions, stream_waves, no_shared_blocks)
    k = lib().pkv_decode_plan_kernel(ctypes.byref(dims), k_cache.shape[2])
    names = {v: n for n, v in _KERNELS.items()}
    if k not in names or k == 0:
        raise PagedKVError(PKV_ERR_INVALID, "pkv_decode_plan_kernel")
    return names[k]


def _torch_stream(stream):
    """The torch stream object for a call's ``stream`` argument (torch's
    current stream when None)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(_stream(stream))


def _zero_prefix(buf: torch.Tensor, n: int, stream) -> None:
    """Clear buf[:n] with a fill kernel on ``stream`` (torch's current stream
    when None), so the clearing is ordered before the call that follows on
    that stream."""
    with torch.cuda.stream(_torch_stream(stream)):
        buf[:n].zero_()


class DecodeWorkspace:
    """Device scratch for :func:`paged_attention_decode` that keeps the C
    ABI's workspace contract: its leading counter region must be zero when a
    call starts (each call leaves it zero), and the bytes after it may hold a
    previous call's partial results.  The object remembers how many leading
    bytes are known to be zero and clears more (with a fill kernel on the
    call's stream) only when a call needs a larger counter region.

    One workspace serves calls on one stream at a time (the C ABI's rule:
    calls that may overlap need different workspaces).  A grown buffer is
    allocated and zeroed on the stream of the call that needs it, and every
    stream that uses the buffer is recorded with the allocator, so a buffer
    that is replaced is not reused while work queued on such a stream may
    still touch it.

    ``buffer`` may wrap an existing uint8 device tensor of any contents; by
    default the workspace allocates and grows its own zero-filled buffer."""

    def __init__(self, buffer: Optional[torch.Tensor] = None, device=None):
        if buffer is not None:
            if buffer.dtype != torch.uint8 or not buffer.is_cuda or buffer.dim() != 1:
                raise ValueError("workspace buffer must be a 1-d uint8 device tensor")
        self.buffer = buffer
        self.device = buffer.device if buffer is not None else device
        self.zeroed = 0  # leading bytes known to be zero
        self.growable = buffer is None
        self._streams = set()  # streams (by handle) recorded on the current buffer

    def prepare(self, nbytes: int, zeroed_bytes: int, device, stream=None) -> torch.Tensor:
        st = _torch_stream(stream)
        if self.buffer is None or self.buffer.numel() < nbytes:
            if not self.growable:
                raise ValueError(f"workspace holds {self.buffer.numel()} bytes, call needs {nbytes}")
            with torch.cuda.stream(st):
                self.buffer = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            self.zeroed = self.buffer.numel()
            self._streams = {st.cuda_stream}
        elif zeroed_bytes > self.zeroed:
            _zero_prefix(self.buffer, zeroed_bytes, st)
        if st.cuda_stream not in self._streams and not torch.cuda.is_current_stream_capturing():
            # (under graph capture the graph's replays are ordered by the
            # caller; the buffer stays referenced by this object meanwhile)
            self.buffer.record_stream(st)
            self._streams.add(st.cuda_stream)
        # after the call: the counter region is zero again, the partial
        # results behind it are not
        if nbytes > 0:
            self.zeroed = zeroed_bytes
        return self.buffer


_ws_cache = {}


def _default_workspace(device: torch.device, stream) -> DecodeWorkspace:
    """The workspace a call without one uses: one per (device, stream), so
    calls on different streams never share counters."""
    key = (device.type, device.index, _torch_stream(stream).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None:
        ws = DecodeWorkspace(device=device)
        _ws_cache[key] = ws
    return ws


_plan_cache = {}


def _decode_sizes(dims: DecodeDims, bs: int):
    """(workspace bytes, zeroed bytes) of a decode call, cached per dims."""
    key = (bytes(dims), bs)
    hit = _plan_cache.get(key)
    if hit is None:
        L = lib()
        need = L.pkv_decode_workspace_size(ctypes.byref(dims), bs)
        if need == ctypes.c_size_t(-1).value:
            raise PagedKVError(PKV_ERR_INVALID, "pkv_paged_attention_decode")
        hit = (int(need), int(L.pkv_decode_workspace_zeroed_bytes(ctypes.byref(dims), bs)))
        if len(_plan_cache) > 4096:
            _plan_cache.clear()
        _plan_cache[key] = hit
    return hit


def _decode(q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, block_size, scale, out,
            max_seq_len, partition_size, kernel, waves_per_group, balance_partitions,
            stream_waves, no_shared_blocks, workspace, stream) -> torch.Tensor:
    _check(q, "q", torch.bfloat16, 3)
    _check(k_cache, "k_cache", torch.bfloat16, 4)
    _check(v_cache, "v_cache", torch.bfloat16, 4)
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(seq_lens, "seq_lens", torch.int32, 1)
    if out.dtype not in _DTYPES:
        raise TypeError("out must be bf16 or fp32")
    _check(out, "out", out.dtype, 3)
    s, hq, d = q.shape
    p, hkv, bs, d2 = k_cache.shape
    if bs != block_size or d2 != d or tuple(v_cache.shape) != (p, hkv, d, bs):
        raise ValueError("cache shapes must be k [P,Hkv,B,D] and v [P,Hkv,D,B] matching q")
    if tuple(out.shape) != (s, hq, d) or block_tables.shape[0] != s or seq_lens.shape[0] != s:
        raise ValueError("q, out, block_tables and seq_lens disagree on the batch")
    if k_new is not None:
        _check(k_new, "k_new", torch.bfloat16, 3)
        _check(v_new, "v_new", torch.bfloat16, 3)
        if tuple(k_new.shape) != (s, hkv, d) or tuple(v_new.shape) != (s, hkv, d):
            raise ValueError("k_new and v_new must be [S, Hkv, D]")
    dims = _dims(q, k_cache, block_tables, max_seq_len, partition_size, out.dtype, kernel,
                 waves_per_group, balance_partitions, stream_waves, no_shared_blocks)
    L = lib()
    need, zeroed = _decode_sizes(dims, bs)
    ws_ptr, ws_len = None, 0
    if need:
        if workspace is None:
            workspace = _default_workspace(q.device, stream)
        if isinstance(workspace, DecodeWorkspace):
            buf = workspace.prepare(need, zeroed, q.device, stream)
        else:
            if workspace.dtype != torch.uint8 or not workspace.is_cuda:
                raise ValueError("workspace must be a uint8 device tensor or a DecodeWorkspace")
            buf = workspace
            if buf.numel() < need:
                raise ValueError(f"workspace holds {buf.numel()} bytes, call needs {need}")
            if zeroed:
                _zero_prefix(buf, zeroed, stream)
        ws_ptr, ws_len = buf.data_ptr(), buf.numel()
    if k_new is None:
        st = L.pkv_paged_attention_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                          block_tables.data_ptr(), seq_lens.data_ptr(), bs,
                                          float(scale), out.data_ptr(), ctypes.byref(dims),
                                          ws_ptr, ws_len, _stream(stream))
        what = "pkv_paged_attention_decode"
    else:
        st = L.pkv_paged_attention_decode_append(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), block_tables.data_ptr(), seq_lens.data_ptr(), bs, float(scale),
            out.data_ptr(), ctypes.byref(dims), ws_ptr, ws_len, _stream(stream))
        what = "pkv_paged_attention_decode_append"
    if st != PKV_OK:
        raise PagedKVError(st, what)
    return out


def paged_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                           scale: float, out: torch.Tensor, *, max_seq_len: Optional[int] = None,
                           partition_size: int = 0, kernel: str = "auto",
                           waves_per_group: int = 0, balance_partitions: bool = False,
                           stream_waves: int = 0, no_shared_blocks: bool = False,
                           workspace=None, stream=None) -> torch.Tensor:
    """Single-query paged decode attention ([ITH §PagedAttention 的核心想法];
    [PU §按 Block 分配]).  Writes ``out`` [S, Hq, D] (bf16 or fp32) and returns
    it.  ``max_seq_len`` defaults to the table capacity (max_blocks * B).
    ``no_shared_blocks=True`` declares that no physical block is read by two
    of the call's sequences (a speed hint; see ``pkv_decode_dims``).
    ``workspace`` is a :class:`DecodeWorkspace` (reused across calls; the
    default is one per device and stream) or a raw uint8 device tensor, whose
    counter region is then cleared before every call."""
    return _decode(q, None, None, k_cache, v_cache, block_tables, seq_lens, block_size, scale,
                   out, max_seq_len, partition_size, kernel, waves_per_group,
                   balance_partitions, stream_waves, no_shared_blocks, workspace, stream)


NOALLOC_SCRATCH_BYTES = 16 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def paged_attention_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, block_tables: torch.Tensor,
                                   seq_lens: torch.Tensor, block_size: int, scale: float,
                                   out: torch.Tensor, *, max_seq_len: Optional[int] = None,
                                   partition_size: int = 0, kernel: str = "auto",
                                   waves_per_group: int = 0, balance_partitions: bool = False,
                                   stream_waves: int = 0, no_shared_blocks: bool = False,
                                   stream=None) -> torch.Tensor:
    """:func:`paged_attention_decode` for callers that cannot allocate: the
    split-KV scratch is the library's fixed per-device array (at most
    ``NOALLOC_SCRATCH_BYTES``), so nothing is allocated here or in the
    library.  Calls that may overlap on one device race on that array."""
    _check(q, "q", torch.bfloat16, 3)
    _check(k_cache, "k_cache", torch.bfloat16, 4)
    _check(v_cache, "v_cache", torch.bfloat16, 4)
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(seq_lens, "seq_lens", torch.int32, 1)
    if out.dtype not in _DTYPES:
        raise TypeError("out must be bf16 or fp32")
    _check(out, "out", out.dtype, 3)
    s, hq, d = q.shape
    p, hkv, bs, d2 = k_cache.shape
    if bs != block_size or d2 != d or tuple(v_cache.shape) != (p, hkv, d, bs):
        raise ValueError("cache shapes must be k [P,Hkv,B,D] and v [P,Hkv,D,B] matching q")
    if tuple(out.shape) != (s, hq, d) or block_tables.shape[0] != s or seq_lens.shape[0] != s:
        raise ValueError("q, out, block_tables and seq_lens disagree on the batch")
    dims = _dims(q, k_cache, block_tables, max_seq_len, partition_size, out.dtype, kernel,
                 waves_per_group, balance_partitions, stream_waves, no_shared_blocks)
    st = lib().pkv_paged_attention_decode_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        seq_lens.data_ptr(), bs, float(scale), out.data_ptr(), ctypes.byref(dims),
        _stream(stream))
    if st != PKV_OK:
        raise PagedKVError(st, "pkv_paged_attention_decode_noalloc")
    return out


def paged_attention_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                  block_size: int, scale: float, out: torch.Tensor, *,
                                  max_seq_len: Optional[int] = None, partition_size: int = 0,
                                  kernel: str = "auto", waves_per_group: int = 0,
                                  balance_partitions: bool = False, stream_waves: int = 0,
                                  no_shared_blocks: bool = False,
                                  workspace=None, stream=None) -> torch.Tensor:
    """One decode step: writes k_new/v_new [S, Hkv, D] (the token at position
    T_b - 1 of each sequence) into the slot its block table gives, then
    attends over the T_b tokens ([ITH §手動畫一次 block table]; [PU §按 Block
    分配]).  With the stream kernel both happen in one launch."""
    return _decode(q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, block_size, scale,
                   out, max_seq_len, partition_size, kernel, waves_per_group,
                   balance_partitions, stream_waves, no_shared_blocks, workspace, stream)


def cascade_workspace_size(q, k_cache, block_tables, num_groups: int, max_prefix_len: int, *,
                           max_seq_len=None, out_dtype=torch.bfloat16) -> int:
    dims = _dims(q, k_cache, block_tables, max_seq_len, 0, out_dtype, "auto", 0, False)
    n = lib().pkv_cascade_workspace_size(ctypes.byref(dims), int(num_groups),
                                         int(max_prefix_len), k_cache.shape[2])
    if n == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID, "pkv_cascade_workspace_size")
    return int(n)


def cascade_plan_kernel(q, k_cache, block_tables, num_groups: int, max_prefix_len: int, *,
                        max_seq_len=None, out_dtype=torch.bfloat16, kernel: str = "auto") -> str:
    """The form :func:`cascade_decode` runs: "stream_wg" (one launch) or
    "mfma" (two launches)."""
    dims = _dims(q, k_cache, block_tables, max_seq_len, 0, out_dtype, kernel, 0, False)
    k = lib().pkv_cascade_plan_kernel(ctypes.byref(dims), int(num_groups), int(max_prefix_len),
                                      k_cache.shape[2])
    if k not in (_KERNELS["stream_wg"], _KERNELS["mfma"]):
        raise PagedKVError(PKV_ERR_INVALID, "pkv_cascade_plan_kernel")
    return "stream_wg" if k == _KERNELS["stream_wg"] else "mfma"


_cascade_ws = {}


def cascade_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, seq_lens: torch.Tensor,
                   group_starts: torch.Tensor, prefix_lens: torch.Tensor, block_size: int,
                   scale: float, out: torch.Tensor, *, max_prefix_len: int,
                   max_seq_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                   kernel: str = "auto", stream=None) -> torch.Tensor:
    """Shared-prefix decode ([PU §共享前缀，分叉时 Copy-on-write]; [PU §按 Block
    分配]): the same result as :func:`paged_attention_decode`, with the blocks
    a group of sequences shares read once per group.  Group g is the
    sequences ``group_starts[g] .. group_starts[g+1]-1`` (int32 [NG+1] on the
    device), sharing their first ``prefix_lens[g]`` tokens (int32 [NG], whole
    blocks); :meth:`BlockManager.shared_prefix_groups` derives both from the
    tables.  ``workspace`` is a uint8 device tensor (default: one per device,
    grown as needed); it needs no initialisation.  ``kernel``: "stream_wg"
    (one launch, a workgroup per group, KV head and block of members),
    "mfma" (two launches: segments, then their merge) or "auto" (the first
    when a task fits its LDS records)."""
    _check(q, "q", torch.bfloat16, 3)
    _check(k_cache, "k_cache", torch.bfloat16, 4)
    _check(v_cache, "v_cache", torch.bfloat16, 4)
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(seq_lens, "seq_lens", torch.int32, 1)
    _check(group_starts, "group_starts", torch.int32, 1)
    _check(prefix_lens, "prefix_lens", torch.int32, 1)
    if out.dtype not in _DTYPES:
        raise TypeError("out must be bf16 or fp32")
    _check(out, "out", out.dtype, 3)
    s, hq, d = q.shape
    p, hkv, bs, d2 = k_cache.shape
    if bs != block_size or d2 != d or tuple(v_cache.shape) != (p, hkv, d, bs):
        raise ValueError("cache shapes must be k [P,Hkv,B,D] and v [P,Hkv,D,B] matching q")
    if tuple(out.shape) != (s, hq, d) or block_tables.shape[0] != s or seq_lens.shape[0] != s:
        raise ValueError("q, out, block_tables and seq_lens disagree on the batch")
    ng = prefix_lens.shape[0]
    if group_starts.shape[0] != ng + 1:
        raise ValueError("group_starts must hold num_groups + 1 entries")
    if kernel not in ("auto", "stream_wg", "mfma"):
        raise ValueError("cascade kernel must be 'auto', 'stream_wg' or 'mfma'")
    dims = _dims(q, k_cache, block_tables, max_seq_len, 0, out.dtype, kernel, 0, False)
    L = lib()
    need = L.pkv_cascade_workspace_size(ctypes.byref(dims), ng, int(max_prefix_len), bs)
    if need == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID, "pkv_cascade_decode")
    if workspace is None:
        key = (q.device.type, q.device.index)
        workspace = _cascade_ws.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device=q.device)
            _cascade_ws[key] = workspace
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 device tensor of at least {need} bytes")
    st = L.pkv_cascade_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                              block_tables.data_ptr(), seq_lens.data_ptr(),
                              group_starts.data_ptr(), prefix_lens.data_ptr(), ng,
                              int(max_prefix_len), bs, float(scale), out.data_ptr(),
                              ctypes.byref(dims), workspace.data_ptr(), workspace.numel(),
                              _stream(stream))
    if st != PKV_OK:
        raise PagedKVError(st, "pkv_cascade_decode")
    return out


def paged_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_tables: torch.Tensor, seq_lens: torch.Tensor, cu_q_lens: torch.Tensor,
                  block_size: int, scale: float, out: torch.Tensor, *, max_q_len: int,
                  max_seq_len: Optional[int] = None, stream=None) -> torch.Tensor:
    """Causal multi-query attention of each sequence's new tokens over its
    cached tokens ([PU §KV Cache 为什么会浪费显存]; [PU §Continuous Batching];
    [PU §按 Block 分配]).  ``q``/``out`` [N, Hq, D] hold the new tokens
    sequence by sequence (rows cu_q_lens[b] .. cu_q_lens[b+1]-1, int32 [S+1]
    on the device); they are the last q_len_b of the seq_lens[b] cached
    tokens, whose K/V are already in the cache."""
    _check(q, "q", torch.bfloat16, 3)
    _check(k_cache, "k_cache", torch.bfloat16, 4)
    _check(v_cache, "v_cache", torch.bfloat16, 4)
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(seq_lens, "seq_lens", torch.int32, 1)
    _check(cu_q_lens, "cu_q_lens", torch.int32, 1)
    if out.dtype not in _DTYPES:
        raise TypeError("out must be bf16 or fp32")
    _check(out, "out", out.dtype, 3)
    n, hq, d = q.shape
    p, hkv, bs, d2 = k_cache.shape
    s = seq_lens.shape[0]
    if bs != block_size or d2 != d or tuple(v_cache.shape) != (p, hkv, d, bs):
        raise ValueError("cache shapes must be k [P,Hkv,B,D] and v [P,Hkv,D,B] matching q")
    if tuple(out.shape) != (n, hq, d) or block_tables.shape[0] != s or cu_q_lens.shape[0] != s + 1:
        raise ValueError("q, out, block_tables, seq_lens and cu_q_lens disagree")
    mb = block_tables.shape[1]
    dims = DecodeDims(s, hq, hkv, d, p, mb, mb * bs if max_seq_len is None else int(max_seq_len),
                      0, _DTYPES[out.dtype], 0, 0, 0, 0)
    st = lib().pkv_paged_prefill(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 block_tables.data_ptr(), seq_lens.data_ptr(),
                                 cu_q_lens.data_ptr(), n, int(max_q_len), bs, float(scale),
                                 out.data_ptr(), ctypes.byref(dims), _stream(stream))
    if st != PKV_OK:
        raise PagedKVError(st, "pkv_paged_prefill")
    return out


def reshape_and_cache(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Write token n's K,V rows into slot slot_mapping[n] (< 0: skipped)
    ([ITH §手動畫一次 block table]; [PU §按 Block 分配])."""
    _check(k, "k", torch.bfloat16, 3)
    _check(v, "v", torch.bfloat16, 3)
    _check(slot_mapping, "slot_mapping", torch.int64, 1)
    _check(k_cache, "k_cache", torch.bfloat16, 4)
    _check(v_cache, "v_cache", torch.bfloat16, 4)
    n, hkv, d = k.shape
    p, hkv2, bs, d2 = k_cache.shape
    if tuple(v.shape) != (n, hkv, d) or slot_mapping.shape[0] != n or (hkv2, d2) != (hkv, d) \
            or tuple(v_cache.shape) != (p, hkv, d, bs):
        raise ValueError("reshape_and_cache: inconsistent shapes")
    st = lib().pkv_reshape_and_cache(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), n, hkv,
                                     d, k_cache.data_ptr(), v_cache.data_ptr(), p, bs,
                                     _stream(stream))
    if st != PKV_OK:
        raise PagedKVError(st, "pkv_reshape_and_cache")


def copy_blocks(k_caches: Sequence[torch.Tensor], v_caches: Sequence[torch.Tensor],
                block_pairs: torch.Tensor, stream=None) -> None:
    """cache[dst] = cache[src] in every layer for each (src, dst) row of
    ``block_pairs`` (int32 [N, 2], on the device) ([PU §共享前缀，分叉时
    Copy-on-write])."""
    if len(k_caches) != len(v_caches) or not k_caches:
        raise ValueError("need one k and one v cache per layer")
    _check(block_pairs, "block_pairs", torch.int32, 2)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [N, 2]")
    shape = tuple(k_caches[0].shape)
    for kc, vc in zip(k_caches, v_caches):
        _check(kc, "k_cache", torch.bfloat16, 4)
        _check(vc, "v_cache", torch.bfloat16, 4)
        if tuple(kc.shape) != shape or vc.shape[0] != shape[0] or vc.numel() != kc.numel():
            raise ValueError("all layers must share one cache shape")
    n_layers = len(k_caches)
    karr = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in k_caches])
    varr = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in v_caches])
    block_bytes = k_caches[0][0].numel() * 2
    st = lib().pkv_copy_blocks(karr, varr, n_layers, block_pairs.data_ptr(),
                               block_pairs.shape[0], block_bytes, _stream(stream))
    if st != PKV_OK:
        raise PagedKVError(st, "pkv_copy_blocks")


def _swap(name, k_caches, v_caches, block_ids, host_buffer, stream):
    if len(k_caches) != len(v_caches) or not k_caches:
        raise ValueError("need one k and one v cache per layer")
    _check(block_ids, "block_ids", torch.int32, 1)
    shape = tuple(k_caches[0].shape)
    for kc, vc in zip(k_caches, v_caches):
        _check(kc, "k_cache", torch.bfloat16, 4)
        _check(vc, "v_cache", torch.bfloat16, 4)
        if tuple(kc.shape) != shape or vc.shape[0] != shape[0] or vc.numel() != kc.numel():
            raise ValueError("all layers must share one cache shape")
    n_layers, n = len(k_caches), block_ids.shape[0]
    block_bytes = k_caches[0][0].numel() * 2
    if host_buffer.is_cuda or not host_buffer.is_pinned() or not host_buffer.is_contiguous():
        raise ValueError("host_buffer must be a contiguous pinned host tensor")
    if host_buffer.numel() * host_buffer.element_size() < n_layers * 2 * n * block_bytes:
        raise ValueError("host_buffer is smaller than layers x 2 x blocks x block bytes")
    karr = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in k_caches])
    varr = (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in v_caches])
    st = getattr(lib(), name)(karr, varr, n_layers, block_ids.data_ptr(), n, block_bytes,
                              host_buffer.data_ptr(), _stream(stream))
    if st != PKV_OK:
        raise PagedKVError(st, name)


def swap_buffer(k_caches: Sequence[torch.Tensor], num_ids: int) -> torch.Tensor:
    """A pinned host buffer for swapping ``num_ids`` blocks of these layers:
    uint16 [layers, 2, num_ids, Hkv*B*D] (the layout pkv_swap_out writes)."""
    return torch.empty((len(k_caches), 2, num_ids, k_caches[0][0].numel()), dtype=torch.int16,
                       pin_memory=True)


def swap_out(k_caches: Sequence[torch.Tensor], v_caches: Sequence[torch.Tensor],
             block_ids: torch.Tensor, host_buffer: torch.Tensor, stream=None) -> None:
    """Copy blocks ``block_ids`` (int32, on the device) of every layer's K and
    V cache to the pinned ``host_buffer`` ([AK §故事沒有說完的部分]: pages
    swapped out under memory pressure).  Asynchronous on the stream."""
    _swap("pkv_swap_out", k_caches, v_caches, block_ids, host_buffer, stream)


def swap_in(k_caches: Sequence[torch.Tensor], v_caches: Sequence[torch.Tensor],
            block_ids: torch.Tensor, host_buffer: torch.Tensor, stream=None) -> None:
    """The way back: block i of ``host_buffer`` becomes block block_ids[i] of
    every layer (which may differ from where it was swapped out from; the
    table follows it)."""
    _swap("pkv_swap_in", k_caches, v_caches, block_ids, host_buffer, stream)


def merge_attention_states(part_out: torch.Tensor, part_lse: torch.Tensor,
                           out: torch.Tensor, stream=None) -> torch.Tensor:
    """o = sum_r Z_r o_r / sum_r Z_r over segments r, with part_lse = ln Z_r
    ([PU §按 Block 分配]).  part_out fp32 [R, N, D], part_lse fp32 [R, N],
    out [R, D] bf16 or fp32."""
    _check(part_out, "part_out", torch.float32, 3)
    _check(part_lse, "part_lse", torch.float32, 2)
    if out.dtype not in _DTYPES:
        raise TypeError("out must be bf16 or fp32")
    _check(out, "out", out.dtype, 2)
    r, n, d = part_out.shape
    if tuple(part_lse.shape) != (r, n) or tuple(out.shape) != (r, d):
        raise ValueError("merge_attention_states: inconsistent shapes")
    st = lib().pkv_merge_attention_states(part_out.data_ptr(), part_lse.data_ptr(), r, n, d,
                                          out.data_ptr(), _DTYPES[out.dtype], _stream(stream))
    if st != PKV_OK:
        raise PagedKVError(st, "pkv_merge_attention_states")
    return out


# Checkers of device-resident inputs: each returns the C ABI's violation
# bit mask (0 when the inputs are consistent), synchronising with the stream.

def _flags_result(st, name, flags, stream) -> int:
    if st != PKV_OK:
        raise PagedKVError(st, name)
    return int(flags.item())


def check_decode_inputs(block_tables: torch.Tensor, seq_lens: torch.Tensor, num_blocks: int,
                        block_size: int, max_seq_len: int, stream=None) -> int:
    """Bit 0: a used table entry outside [0, num_blocks); bit 1: a length
    outside [0, min(max_seq_len, max_blocks_per_seq * block_size)]."""
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.shape[0] != block_tables.shape[0]:
        raise ValueError("seq_lens and block_tables disagree on the number of sequences")
    flags = torch.empty(1, dtype=torch.int32, device=seq_lens.device)
    st = lib().pkv_check_decode_inputs(block_tables.data_ptr(), seq_lens.data_ptr(),
                                       seq_lens.shape[0], block_tables.shape[1], num_blocks,
                                       block_size, max_seq_len, flags.data_ptr(), _stream(stream))
    return _flags_result(st, "pkv_check_decode_inputs", flags, stream)


def check_slot_mapping(slot_mapping: torch.Tensor, num_blocks: int, block_size: int,
                       stream=None) -> int:
    """Bit 0: a slot >= num_blocks * block_size; bit 1: a non-negative slot
    that appears twice."""
    _check(slot_mapping, "slot_mapping", torch.int64, 1)
    flags = torch.empty(1, dtype=torch.int32, device=slot_mapping.device)
    st = lib().pkv_check_slot_mapping(slot_mapping.data_ptr(), slot_mapping.shape[0], num_blocks,
                                      block_size, flags.data_ptr(), _stream(stream))
    return _flags_result(st, "pkv_check_slot_mapping", flags, stream)


def check_block_pairs(block_pairs: torch.Tensor, num_blocks: int, stream=None) -> int:
    """Bit 0: a src or dst outside [0, num_blocks); bit 1: a dst that appears
    twice; bit 2: a dst that is also some pair's src."""
    _check(block_pairs, "block_pairs", torch.int32, 2)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [N, 2]")
    flags = torch.empty(1, dtype=torch.int32, device=block_pairs.device)
    st = lib().pkv_check_block_pairs(block_pairs.data_ptr(), block_pairs.shape[0], num_blocks,
                                     flags.data_ptr(), _stream(stream))
    return _flags_result(st, "pkv_check_block_pairs", flags, stream)
