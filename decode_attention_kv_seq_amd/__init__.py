"""decode_attention_kv_seq_amd -- fp16 single-query decode attention on MI355X.

A thin Python binding over ``libattn_decode.so`` (declared in
``include/attn_decode.h``).  This module only checks and marshals
arguments: every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and the stream; each call runs with its
tensors' device current and enqueues on that device's
``torch.cuda.current_stream()`` unless a stream is given.

The operation (page "Developing Apple Metal Kernels in Rust - A Deep Dive
Through Attention", section "The MSL, briefly"): per head,
``softmax(q . K^T / sqrt(head_dim))`` over positions ``0..current_pos``,
then the weighted sum of V; K and V laid out ``[seq_len, n_heads, head_dim]``,
q and the output ``[n_heads, head_dim]``.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_decode.so")

ATTN_OK = 0
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_DIM", 3: "ATTN_ERR_ALIGN",
                4: "ATTN_ERR_WORKSPACE", 5: "ATTN_ERR_HIP"}
MAX_HEAD_DIM = 256


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), detail))
        self.status = status
        self.detail = detail


_lib = None


class PlanInfo(ctypes.Structure):
    """attn_plan_info of include/attn_decode.h."""
    _fields_ = [("balanced", ctypes.c_uint32), ("heads_per_workgroup", ctypes.c_uint32),
                ("workgroups", ctypes.c_uint64), ("chunk", ctypes.c_uint32),
                ("chunks", ctypes.c_uint32), ("launches", ctypes.c_uint32),
                ("partial_slots", ctypes.c_uint64), ("workspace_slots", ctypes.c_uint64),
                ("unroll", ctypes.c_uint32), ("max_waves", ctypes.c_uint32)]


PLAN_DEVICE_POS, PLAN_PAGED, PLAN_STEP, PLAN_FROM_SCORES = 1, 2, 4, 8


def load_library(path: str = LIB_PATH):
    """Load the HIP library.  There is no fallback: a missing library is an error."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libattn_decode.so is not built (%s); run "
                          "`python -m decode_attention_kv_seq_amd._build`" % path)
    lib = ctypes.CDLL(path)
    vp, sz, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32
    lib.attn_decode_workspace_bytes.argtypes = [u32, u32, u32, u32]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode_f16.argtypes = [vp, vp, vp, vp, u32, u32, u32, u32, vp, vp, sz, vp]
    lib.attn_decode_f16.restype = ctypes.c_int
    lib.attn_decode_f16_batched.argtypes = [vp, vp, vp, vp, vp, u32, u32, u32, u32, vp, vp, sz, vp]
    lib.attn_decode_f16_batched.restype = ctypes.c_int
    lib.attn_decode_f16_batched_noalloc.argtypes = [vp, vp, vp, vp, vp, u32, u32, u32, u32, vp, vp]
    lib.attn_decode_f16_batched_noalloc.restype = ctypes.c_int
    lib.attn_decode_f16_split.argtypes = [vp, vp, vp, vp, u32, u32, u32, u32, u32, vp, vp, sz, vp]
    lib.attn_decode_f16_split.restype = ctypes.c_int
    lib.attn_decode_f16_combine.argtypes = [vp, vp, u32, u32, u32, u32, u32, vp, sz, vp]
    lib.attn_decode_f16_combine.restype = ctypes.c_int
    lib.attn_decode_f16_paged.argtypes = [vp, vp, vp, vp, vp, vp, u32, u32, u32, u32, u32, u32,
                                          vp, vp, sz, vp]
    lib.attn_decode_f16_paged.restype = ctypes.c_int
    lib.attn_decode_f16_paged_split.argtypes = [vp, vp, vp, vp, vp, u32, u32, u32, u32, u32, u32,
                                                vp, vp, sz, vp]
    lib.attn_decode_f16_paged_split.restype = ctypes.c_int
    lib.attn_paged_table_check.argtypes = [vp, vp, u32, u32, u32, u32, vp, vp]
    lib.attn_paged_table_check.restype = ctypes.c_int
    lib.attn_qk_f16.argtypes = [vp, vp, vp, u32, u32, u32, u32, vp]
    lib.attn_qk_f16.restype = ctypes.c_int
    lib.attn_pv_f16.argtypes = [vp, vp, vp, u32, u32, u32, u32, vp, sz, vp]
    lib.attn_pv_f16.restype = ctypes.c_int
    f64 = ctypes.c_double
    i32 = ctypes.c_int
    lib.attn_decode_step_f16.argtypes = [vp, vp, vp, vp, vp, vp, u32, u32, u32, u32, u32, f64, i32,
                                         vp, sz, vp]
    lib.attn_decode_step_f16.restype = ctypes.c_int
    lib.attn_decode_step_f16_batched.argtypes = [vp, vp, vp, vp, vp, vp, vp, u32, u32, u32, u32,
                                                 u32, f64, i32, vp, sz, vp]
    lib.attn_decode_step_f16_batched.restype = ctypes.c_int
    lib.attn_decode_step_f16_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, u32, u32, u32, u32,
                                               u32, u32, u32, f64, i32, vp, sz, vp]
    lib.attn_decode_step_f16_paged.restype = ctypes.c_int
    lib.attn_rope_f16.argtypes = [vp, vp, vp, u32, u32, u32, u32, f64, i32, vp]
    lib.attn_rope_f16.restype = ctypes.c_int
    lib.attn_softmax_workspace_bytes.argtypes = [u32, u32]
    lib.attn_softmax_workspace_bytes.restype = sz
    lib.attn_softmax_f32.argtypes = [vp, vp, u32, u32, vp, sz, vp]
    lib.attn_softmax_f32.restype = ctypes.c_int
    lib.attn_decode_plan.argtypes = [u32, u32, u32, u32, u32, u32, ctypes.POINTER(PlanInfo)]
    lib.attn_decode_plan.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, _lib.attn_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with ``stream=`` (when given) as the current stream.
    torch's caching allocator ties each block to the stream that is current
    when it is allocated, and reuses a freed block on that stream without
    waiting for other streams: so the workspace, ``out`` and dump that a
    wrapper allocates for work it enqueues on ``stream`` must come from
    ``stream``'s own blocks, not the current stream's."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return run


def _req(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _req_buf(t: torch.Tensor, name: str, device):
    """A caller's scratch buffer (any dtype): contiguous, on ``device``.  The
    library takes raw device pointers, so a host tensor must never reach it."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _req_dump(dump, shape, device):
    """An optional caller-provided fp32 score dump of the given shape."""
    if dump is not None:
        _req(dump, "dump", torch.float32, device)
        if tuple(dump.shape) != tuple(shape):
            raise ValueError("dump must be %s" % list(shape))


def plan(batch: int, n_heads: int, head_dim: int, seq_len: int, current_pos: int = 0,
         flags: int = 0) -> dict:
    """attn_decode_plan: how a call with these sizes runs (host only).
    flags: PLAN_* bits naming the call (0: the single-sequence decode)."""
    info = PlanInfo()
    _check(load_library().attn_decode_plan(batch, n_heads, head_dim, seq_len, current_pos, flags,
                                           ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def workspace_bytes(batch: int, n_heads: int, head_dim: int, seq_len: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(batch, n_heads, head_dim, seq_len))


def alloc_workspace(batch, n_heads, head_dim, seq_len, device) -> torch.Tensor:
    n = workspace_bytes(batch, n_heads, head_dim, seq_len)
    if n == 0:
        raise ValueError("invalid sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _cp_tensor(cp: torch.Tensor, batch: int, device) -> torch.Tensor:
    if not isinstance(cp, torch.Tensor) or cp.dtype not in (torch.int32, torch.uint32):
        raise TypeError("current_pos must be an int32/uint32 GPU tensor")
    _req(cp, "current_pos", cp.dtype, device)
    if tuple(cp.shape) != (batch,):
        raise ValueError("current_pos must have shape [%d]" % batch)
    return cp


@_on_stream
def decode(q, k, v, current_pos: int, *, out=None, dump: bool = False, workspace=None,
           stream=None):
    """One sequence: q [H, D], k/v [S, H, D] fp16 -> out [H, D] fp16.

    With ``dump=True`` also returns the fp32 score dump [H, S] (natural-log
    units, -inf after current_pos)."""
    lib = load_library()
    _req(k, "k", torch.float16)
    dev = k.device
    _req(q, "q", torch.float16, dev)
    _req(v, "v", torch.float16, dev)
    if k.dim() != 3 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [seq_len, n_heads, head_dim]")
    S, H, D = k.shape
    if tuple(q.shape) != (H, D):
        raise ValueError("q must be [n_heads, head_dim] = [%d, %d]" % (H, D))
    if not 0 <= int(current_pos) <= 0xFFFFFFFF:
        raise ValueError("current_pos must fit in uint32")
    if out is None:
        out = torch.empty((H, D), dtype=torch.float16, device=dev)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != (H, D):
        raise ValueError("out must be [n_heads, head_dim]")
    sc = torch.empty((H, S), dtype=torch.float32, device=dev) if dump else None
    if workspace is None:
        workspace = alloc_workspace(1, H, D, S, dev)
    _req_buf(workspace, "workspace", dev)
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_decode_f16(_ptr(q), _ptr(k), _ptr(v), _ptr(out), H, D, S, int(current_pos),
                                   _ptr(sc), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream_handle(stream)))
    return (out, sc) if dump else out


@_on_stream
def decode_batched(q, k, v, current_pos, *, out=None, dump: bool = False, workspace=None,
                   stream=None):
    """Ragged batch: q [B, H, D], k/v [B, S, H, D] fp16, current_pos int32 [B]
    on the GPU -> out [B, H, D] fp16 (and the dump [B, H, S] with dump=True)."""
    lib = load_library()
    _req(k, "k", torch.float16)
    dev = k.device
    _req(q, "q", torch.float16, dev)
    _req(v, "v", torch.float16, dev)
    if k.dim() != 4 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [batch, capacity, n_heads, head_dim]")
    B, S, H, D = k.shape
    if tuple(q.shape) != (B, H, D):
        raise ValueError("q must be [batch, n_heads, head_dim]")
    cp = _cp_tensor(current_pos, B, dev)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float16, device=dev)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [batch, n_heads, head_dim]")
    sc = torch.empty((B, H, S), dtype=torch.float32, device=dev) if dump else None
    if workspace is None:
        workspace = alloc_workspace(B, H, D, S, dev)
    _req_buf(workspace, "workspace", dev)
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_decode_f16_batched(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cp), B, H, D, S,
                                           _ptr(sc), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream_handle(stream)))
    return (out, sc) if dump else out


NOALLOC_SCRATCH_BYTES = 32 << 20   # ATTN_NOALLOC_SCRATCH_BYTES


@_on_stream
def decode_batched_noalloc(q, k, v, current_pos, *, out, dump=None, stream=None):
    """decode_batched through attn_decode_f16_batched_noalloc: the library's
    own per-GPU workspace, so nothing is allocated by the call (``out`` and
    ``dump`` are the caller's).  Calls that overlap on one GPU race."""
    lib = load_library()
    _req(k, "k", torch.float16)
    dev = k.device
    _req(q, "q", torch.float16, dev)
    _req(v, "v", torch.float16, dev)
    if k.dim() != 4 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [batch, capacity, n_heads, head_dim]")
    B, S, H, D = k.shape
    if tuple(q.shape) != (B, H, D):
        raise ValueError("q must be [batch, n_heads, head_dim]")
    cp = _cp_tensor(current_pos, B, dev)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [batch, n_heads, head_dim]")
    _req_dump(dump, (B, H, S), dev)
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_decode_f16_batched_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cp), B, H,
                                                   D, S, _ptr(dump), _stream_handle(stream)))
    return out


def _batch_view(q, k, v):
    """Accept single-sequence (3-D cache) or batched (4-D cache) tensors."""
    if k.dim() == 3:
        return q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
    return q, k, v


@_on_stream
def split(q, k, v, current_pos, workspace, *, dump=None, stream=None):
    """First launch of a decode: stream the cache into the workspace.

    ``current_pos`` is an int (every sequence) or an int32 GPU tensor [B]."""
    lib = load_library()
    q3, k4, v4 = _batch_view(q, k, v)
    for t, n in ((q3, "q"), (k4, "k"), (v4, "v")):
        _req(t, n, torch.float16, k.device)
    B, S, H, D = k4.shape
    if tuple(v4.shape) != tuple(k4.shape) or tuple(q3.shape) != (B, H, D):
        raise ValueError("shape mismatch")
    cp_dev, cp_host = (None, int(current_pos)) if not isinstance(current_pos, torch.Tensor) \
        else (_cp_tensor(current_pos, B, k.device), 0)
    _req_dump(dump, (B, H, S), k.device)
    _req_buf(workspace, "workspace", k.device)
    with torch.cuda.device(k.device):   # launch on the tensors' device
        _check(lib.attn_decode_f16_split(_ptr(q3), _ptr(k4), _ptr(v4), _ptr(cp_dev), cp_host, B, H, D, S,
                                         _ptr(dump), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _stream_handle(stream)))


@_on_stream
def combine(out, current_pos, batch, n_heads, head_dim, seq_len, workspace, *, stream=None):
    """Second launch: merge the workspace partials into ``out``."""
    lib = load_library()
    _req(out, "out", torch.float16)
    cp_dev, cp_host = (None, int(current_pos)) if not isinstance(current_pos, torch.Tensor) \
        else (_cp_tensor(current_pos, batch, out.device), 0)
    _req_buf(workspace, "workspace", out.device)
    with torch.cuda.device(out.device):   # launch on the tensors' device
        _check(lib.attn_decode_f16_combine(_ptr(out), _ptr(cp_dev), cp_host, batch, n_heads, head_dim,
                                           seq_len, _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream_handle(stream)))
    return out


def _paged_args(q, k_pool, v_pool, block_table, current_pos):
    _req(k_pool, "k_pool", torch.float16)
    dev = k_pool.device
    _req(q, "q", torch.float16, dev)
    _req(v_pool, "v_pool", torch.float16, dev)
    if k_pool.dim() != 4 or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool must be [num_blocks, page_size, n_heads, head_dim]")
    NB, P, H, D = k_pool.shape
    if q.dim() != 3 or tuple(q.shape[1:]) != (H, D):
        raise ValueError("q must be [batch, n_heads, head_dim]")
    B = q.shape[0]
    if not isinstance(block_table, torch.Tensor) or block_table.dtype not in (torch.int32, torch.uint32):
        raise TypeError("block_table must be an int32/uint32 GPU tensor")
    _req(block_table, "block_table", block_table.dtype, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch, max_blocks]")
    cp = _cp_tensor(current_pos, B, dev)
    return B, H, D, P, block_table.shape[1], NB, cp


@_on_stream
def decode_paged(q, k_pool, v_pool, block_table, current_pos, *, out=None, dump=False,
                 workspace=None, stream=None):
    """Paged cache: q [B, H, D]; k/v pools [num_blocks, page_size, H, D];
    block_table int32 [B, max_blocks]; current_pos int32 [B] (GPU tensors)."""
    lib = load_library()
    B, H, D, P, MB, NB, cp = _paged_args(q, k_pool, v_pool, block_table, current_pos)
    dev = k_pool.device
    cap = P * MB
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float16, device=dev)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [batch, n_heads, head_dim]")
    sc = torch.empty((B, H, cap), dtype=torch.float32, device=dev) if dump else None
    if workspace is None:
        workspace = alloc_workspace(B, H, D, cap, dev)
    _req_buf(workspace, "workspace", dev)
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_decode_f16_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out),
                                         _ptr(block_table), _ptr(cp), B, H, D, P, MB, NB, _ptr(sc),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream_handle(stream)))
    return (out, sc) if dump else out


@_on_stream
def split_paged(q, k_pool, v_pool, block_table, current_pos, workspace, *, dump=None, stream=None):
    """First launch of a paged decode; `combine(out, current_pos, B, H, D,
    max_blocks * page_size, workspace)` is the second."""
    lib = load_library()
    B, H, D, P, MB, NB, cp = _paged_args(q, k_pool, v_pool, block_table, current_pos)
    _req_dump(dump, (B, H, P * MB), k_pool.device)
    _req_buf(workspace, "workspace", k_pool.device)
    with torch.cuda.device(k_pool.device):   # launch on the tensors' device
        _check(lib.attn_decode_f16_paged_split(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                               _ptr(cp), B, H, D, P, MB, NB, _ptr(dump),
                                               _ptr(workspace),
                                               workspace.numel() * workspace.element_size(),
                                               _stream_handle(stream)))


@_on_stream
def paged_table_check(block_table, current_pos, page_size: int, num_blocks: int, *, result=None,
                      stream=None):
    """attn_paged_table_check: -> uint32 GPU tensor [2] (entries a paged call
    reads that are >= num_blocks; the first sequence holding one, or
    0xFFFFFFFF).  Asynchronous, like every call."""
    lib = load_library()
    _req(block_table, "block_table", block_table.dtype)
    if block_table.dtype not in (torch.int32, torch.uint32) or block_table.dim() != 2:
        raise TypeError("block_table must be an int32/uint32 GPU tensor [batch, max_blocks]")
    dev = block_table.device
    B, MB = block_table.shape
    cp = _cp_tensor(current_pos, B, dev)
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=dev)
    _req_buf(result, "result", dev)
    if result.numel() * result.element_size() < 8:
        raise ValueError("result must hold two uint32 words")
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_paged_table_check(_ptr(block_table), _ptr(cp), B, int(page_size), MB,
                                          int(num_blocks), _ptr(result), _stream_handle(stream)))
    return result


@_on_stream
def qk(q, k, current_pos: int, *, scores=None, stream=None):
    """First dispatch: q [H, D], k [S, H, D] -> fp16 scores [H, S]
    (scaled, -inf after current_pos)."""
    lib = load_library()
    _req(k, "k", torch.float16)
    dev = k.device
    _req(q, "q", torch.float16, dev)
    if k.dim() != 3:
        raise ValueError("k must be [seq_len, n_heads, head_dim]")
    S, H, D = k.shape
    if tuple(q.shape) != (H, D):
        raise ValueError("q must be [n_heads, head_dim]")
    if scores is None:
        scores = torch.empty((H, S), dtype=torch.float16, device=dev)
    _req(scores, "scores", torch.float16, dev)
    if tuple(scores.shape) != (H, S):
        raise ValueError("scores must be [n_heads, seq_len]")
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_qk_f16(_ptr(q), _ptr(k), _ptr(scores), H, D, S, int(current_pos),
                               _stream_handle(stream)))
    return scores


@_on_stream
def pv(scores, v, current_pos: int, *, out=None, workspace=None, stream=None):
    """Second dispatch: fp16 scores [H, S], v [S, H, D] -> out [H, D]."""
    lib = load_library()
    _req(v, "v", torch.float16)
    dev = v.device
    _req(scores, "scores", torch.float16, dev)
    if v.dim() != 3:
        raise ValueError("v must be [seq_len, n_heads, head_dim]")
    S, H, D = v.shape
    if tuple(scores.shape) != (H, S):
        raise ValueError("scores must be [n_heads, seq_len]")
    if out is None:
        out = torch.empty((H, D), dtype=torch.float16, device=dev)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != (H, D):
        raise ValueError("out must be [n_heads, head_dim]")
    if workspace is None:
        workspace = alloc_workspace(1, H, D, S, dev)
    _req_buf(workspace, "workspace", dev)
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_pv_f16(_ptr(scores), _ptr(v), _ptr(out), H, D, S, int(current_pos),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream_handle(stream)))
    return out


def _rope_params(rope_dims, head_dim, base):
    dims = head_dim if rope_dims is None else int(rope_dims)
    if not 0 <= dims <= 0xFFFFFFFF:
        raise ValueError("rope_dims out of range")
    return dims, float(base)


@_on_stream
def decode_step(q, k_new, v_new, k_cache, v_cache, current_pos, *, rope_dims=None,
                rope_base: float = 10000.0, traditional: bool = False, out=None, workspace=None,
                stream=None):
    """One decode step: rotate q and k_new at the new token's position, append
    the rotated k_new and v_new at slot current_pos of the caches (written in
    place), and attend over positions 0..current_pos.

    Single sequence: q, k_new, v_new [H, D]; caches [S, H, D]; current_pos an
    int < S.  Batch: q, k_new, v_new [B, H, D]; caches [B, S, H, D];
    current_pos an int32 GPU tensor [B] (values >= S use slot S - 1).
    ``rope_dims`` defaults to head_dim.  Returns out, shaped like q."""
    lib = load_library()
    _req(k_cache, "k_cache", torch.float16)
    dev = k_cache.device
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (v_cache, "v_cache")):
        _req(t, n, torch.float16, dev)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must have the same shape")
    batched = k_cache.dim() == 4
    if k_cache.dim() not in (3, 4):
        raise ValueError("caches must be [S, H, D] or [B, S, H, D]")
    S, H, D = k_cache.shape[-3:]
    B = k_cache.shape[0] if batched else 1
    row_shape = (B, H, D) if batched else (H, D)
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        if tuple(t.shape) != row_shape:
            raise ValueError("%s must be %s" % (n, list(row_shape)))
    if out is None:
        out = torch.empty(row_shape, dtype=torch.float16, device=dev)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != row_shape:
        raise ValueError("out must be %s" % list(row_shape))
    dims, base = _rope_params(rope_dims, D, rope_base)
    if workspace is None:
        workspace = alloc_workspace(B, H, D, S, dev)
    _req_buf(workspace, "workspace", dev)
    ws_n = workspace.numel() * workspace.element_size()
    if batched:
        cp = _cp_tensor(current_pos, B, dev)
        with torch.cuda.device(dev):   # launch on the tensors' device
            _check(lib.attn_decode_step_f16_batched(
                _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(cp),
                B, H, D, S, dims, base, 1 if traditional else 0, _ptr(workspace), ws_n,
                _stream_handle(stream)))
    else:
        if not 0 <= int(current_pos) <= 0xFFFFFFFF:
            raise ValueError("current_pos must fit in uint32")
        with torch.cuda.device(dev):   # launch on the tensors' device
            _check(lib.attn_decode_step_f16(
                _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(out), H, D, S,
                int(current_pos), dims, base, 1 if traditional else 0, _ptr(workspace), ws_n,
                _stream_handle(stream)))
    return out


@_on_stream
def decode_step_paged(q, k_new, v_new, k_pool, v_pool, block_table, current_pos, *,
                      rope_dims=None, rope_base: float = 10000.0, traditional: bool = False,
                      out=None, workspace=None, stream=None):
    """The decode step on a paged cache: q, k_new, v_new [B, H, D]; pools
    [num_blocks, page_size, H, D] (slot current_pos written in place);
    block_table int32 [B, max_blocks] and current_pos int32 [B] on the GPU."""
    lib = load_library()
    B, H, D, P, MB, NB, cp = _paged_args(q, k_pool, v_pool, block_table, current_pos)
    dev = k_pool.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _req(t, n, torch.float16, dev)
        if tuple(t.shape) != (B, H, D):
            raise ValueError("%s must be [batch, n_heads, head_dim]" % n)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float16, device=dev)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [batch, n_heads, head_dim]")
    dims, base = _rope_params(rope_dims, D, rope_base)
    if workspace is None:
        workspace = alloc_workspace(B, H, D, P * MB, dev)
    _req_buf(workspace, "workspace", dev)
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_decode_step_f16_paged(
            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(out),
            _ptr(block_table), _ptr(cp), B, H, D, P, MB, NB, dims, base, 1 if traditional else 0,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return out


@_on_stream
def rope(x, positions, *, rope_dims=None, rope_base: float = 10000.0, traditional: bool = False,
         out=None, stream=None):
    """Rotary embedding: x [B, H, D] fp16, positions int32/uint32 GPU tensor
    [B] (row (b, h) turns at positions[b]) -> fp16 [B, H, D]."""
    lib = load_library()
    _req(x, "x", torch.float16)
    dev = x.device
    if x.dim() != 3:
        raise ValueError("x must be [batch, n_heads, head_dim]")
    B, H, D = x.shape
    pos = _cp_tensor(positions, B, dev)
    if out is None:
        out = torch.empty_like(x)
    _req(out, "out", torch.float16, dev)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [batch, n_heads, head_dim]")
    dims, base = _rope_params(rope_dims, D, rope_base)
    with torch.cuda.device(dev):   # launch on the tensors' device
        _check(lib.attn_rope_f16(_ptr(x), _ptr(out), _ptr(pos), B, H, D, dims, base,
                                 1 if traditional else 0, _stream_handle(stream)))
    return out


def softmax_workspace_bytes(rows: int, cols: int) -> int:
    return int(load_library().attn_softmax_workspace_bytes(rows, cols))


@_on_stream
def softmax(x, *, out=None, workspace=None, stream=None):
    """Row softmax of an fp32 GPU tensor [rows, cols] (last dimension).
    ``out`` may be ``x`` itself."""
    lib = load_library()
    _req(x, "x", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    rows, cols = x.shape
    if out is None:
        out = torch.empty_like(x)
    _req(out, "out", torch.float32, x.device)
    if tuple(out.shape) != (rows, cols):
        raise ValueError("out must be [rows, cols]")
    if workspace is None:
        n = softmax_workspace_bytes(rows, cols)
        if n == 0:
            raise ValueError("invalid sizes")
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    _req_buf(workspace, "workspace", x.device)
    with torch.cuda.device(x.device):   # launch on the tensors' device
        _check(lib.attn_softmax_f32(_ptr(x), _ptr(out), rows, cols, _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream_handle(stream)))
    return out
