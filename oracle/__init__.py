"""CPU oracle for single-query decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never touches it.

The arithmetic lives in ``attn_oracle.c`` (fp64 scalar loops, its own
binary16 decoder); this module only marshals numpy arrays through ctypes.  It
follows the page "Developing Apple Metal Kernels in Rust - A Deep Dive
Through Attention", section "The MSL, briefly" (kernels attention_qk_f16 and
attention_pv_f16).  The decode step around it (rotary embedding of q and of
the new key, the append of the new row, then attention) follows the page
"Tutorial 16: Writing Custom Metal Kernels", section "5. Example: Fused RoPE
Kernel", for the rotation.  The row softmax on its own follows the Foundry
notes' fm_softmax (section "API Reference").
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import _build


def _bits(a) -> np.ndarray:
    """Contiguous uint16 view of an fp16/uint16 numpy array or torch tensor."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().contiguous().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 or uint16 data, got %s" % a.dtype)
    return a


def _ptr(a, ct):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ct))


class OracleLib:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        u32 = ctypes.c_uint32
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_half_to_double_array.argtypes = [u16p, ctypes.c_size_t, f64p]
        lib.oracle_half_to_double_array.restype = None
        lib.oracle_attn_decode.argtypes = [u16p, u16p, u16p, u32, u32, u32, u32, u32, u32,
                                           f64p, f64p, f64p]
        lib.oracle_attn_decode.restype = ctypes.c_int
        lib.oracle_attn_pv_from_scores.argtypes = [u16p, u16p, u32, u32, u32, u32, u32, u32, f64p]
        lib.oracle_attn_pv_from_scores.restype = ctypes.c_int
        lib.oracle_double_to_half.argtypes = [ctypes.c_double]
        lib.oracle_double_to_half.restype = ctypes.c_uint16
        lib.oracle_double_to_half_array.argtypes = [f64p, ctypes.c_size_t, u16p]
        lib.oracle_double_to_half_array.restype = None
        lib.oracle_rope.argtypes = [u16p, u32, u32, u32, ctypes.c_double, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_uint32), f64p]
        lib.oracle_rope.restype = ctypes.c_int
        lib.oracle_softmax_rows.argtypes = [ctypes.POINTER(ctypes.c_float), u32, u32, f64p]
        lib.oracle_softmax_rows.restype = ctypes.c_int
        self.path = path
        self.lib = lib

    def half_to_double(self, bits) -> np.ndarray:
        b = _bits(bits)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_half_to_double_array(_ptr(b, ctypes.c_uint16), b.size,
                                             _ptr(out, ctypes.c_double))
        return out

    def decode(self, q, k, v, current_pos: int, *, want_scores=False, want_weights=False,
               threads: int = 1):
        """One sequence.  q [H, D], k/v [S, H, D] (fp16 or uint16 bits).

        Returns ``(out [H, D], scores [H, S] or None, weights [H, S] or None)``,
        all float64.  ``threads > 1`` splits the heads over host threads
        (ctypes releases the GIL); each head is computed the same way.
        """
        shape = tuple(k.shape)
        if len(shape) != 3:
            raise ValueError("k must be [seq_len, n_heads, head_dim]")
        S, H, D = shape
        if tuple(v.shape) != shape or tuple(q.shape)[-2:] != (H, D):
            raise ValueError("shape mismatch")
        if int(current_pos) < 0:
            raise ValueError("current_pos must be >= 0")
        qb, kb, vb = _bits(q), _bits(k), _bits(v)
        out = np.zeros((H, D), dtype=np.float64)
        scores = np.empty((H, S), dtype=np.float64) if want_scores else None
        weights = np.empty((H, S), dtype=np.float64) if want_weights else None
        cp = min(int(current_pos), 0xFFFFFFFF)
        f64 = ctypes.c_double
        u16 = ctypes.c_uint16

        def run(lo_hi):
            lo, hi = lo_hi
            rc = self.lib.oracle_attn_decode(_ptr(qb, u16), _ptr(kb, u16), _ptr(vb, u16),
                                             H, D, S, cp, lo, hi, _ptr(out, f64),
                                             _ptr(scores, f64), _ptr(weights, f64))
            if rc != 0:
                raise RuntimeError("oracle_attn_decode failed")

        threads = max(1, min(int(threads), H))
        if threads == 1:
            run((0, H))
        else:
            bounds = [(H * i // threads, H * (i + 1) // threads) for i in range(threads)]
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, bounds))
        return out, scores, weights

    def pv_from_scores(self, scores, v, current_pos: int):
        """Second kernel of the page's two-dispatch form: scores [H, S] fp16
        bits, v [S, H, D] -> out [H, D] float64."""
        S, H, D = tuple(v.shape)
        if tuple(scores.shape) != (H, S):
            raise ValueError("scores must be [n_heads, seq_len]")
        sb, vb = _bits(scores), _bits(v)
        out = np.zeros((H, D), dtype=np.float64)
        rc = self.lib.oracle_attn_pv_from_scores(_ptr(sb, ctypes.c_uint16), _ptr(vb, ctypes.c_uint16),
                                                 H, D, S, min(int(current_pos), 0xFFFFFFFF), 0, H,
                                                 _ptr(out, ctypes.c_double))
        if rc != 0:
            raise RuntimeError("oracle_attn_pv_from_scores failed")
        return out

    def double_to_half(self, x) -> np.ndarray:
        """fp64 values -> IEEE binary16 bits (uint16), nearest with ties to even."""
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.oracle_double_to_half_array(_ptr(a, ctypes.c_double), a.size,
                                             _ptr(out, ctypes.c_uint16))
        return out

    def rope(self, x, positions, *, dims: int, base: float = 10000.0,
             traditional: bool = False) -> np.ndarray:
        """Rotary embedding of rows of fp16 values.

        x [..., head_dim] (fp16 or uint16 bits); positions broadcast against
        x's leading dimensions (one position per row).  Returns float64 of
        x's shape, exact up to fp64 rounding.
        """
        xb = _bits(x)
        D = xb.shape[-1]
        lead = xb.shape[:-1]
        pos = np.ascontiguousarray(np.broadcast_to(np.asarray(positions, dtype=np.int64), lead))
        if pos.size and (pos.min() < 0 or pos.max() > 0xFFFFFFFF):
            raise ValueError("positions must fit uint32")
        pos = pos.astype(np.uint32).reshape(-1)
        rows = int(np.prod(lead)) if lead else 1
        out = np.empty(xb.shape, dtype=np.float64)
        rc = self.lib.oracle_rope(_ptr(xb, ctypes.c_uint16), rows, D, int(dims), float(base),
                                  1 if traditional else 0, _ptr(pos, ctypes.c_uint32),
                                  _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle_rope rejected its arguments")
        return out

    def decode_step(self, q, k_new, v_new, k_cache, v_cache, current_pos: int, *, dims: int,
                    base: float = 10000.0, traditional: bool = False, threads: int = 1):
        """One decode step of one sequence: rotate, append, attend.

        q, k_new, v_new [H, D] fp16 (q and k_new before rotation); k_cache and
        v_cache [S, H, D] uint16 numpy arrays, whose row pos = min(current_pos,
        S - 1) is OVERWRITTEN here with the rotated, fp16-rounded k_new and
        with v_new (the append).  Rows before pos hold earlier tokens, already
        rotated.  Then attention over positions 0..pos with the rotated,
        fp16-rounded q.

        Returns a dict: out [H, D] float64; q_rot and k_rot, the exact fp64
        rotations; q16 and k16, their fp16 bits.
        """
        S = k_cache.shape[0]
        if not (isinstance(k_cache, np.ndarray) and k_cache.dtype == np.uint16
                and isinstance(v_cache, np.ndarray) and v_cache.dtype == np.uint16):
            raise TypeError("k_cache and v_cache must be uint16 numpy arrays (updated in place)")
        pos = min(int(current_pos), S - 1)
        q_rot = self.rope(q, pos, dims=dims, base=base, traditional=traditional)
        k_rot = self.rope(k_new, pos, dims=dims, base=base, traditional=traditional)
        q16 = self.double_to_half(q_rot)
        k16 = self.double_to_half(k_rot)
        k_cache[pos] = k16
        v_cache[pos] = _bits(v_new)
        out, _, _ = self.decode(q16, k_cache, v_cache, pos, threads=threads)
        return {"out": out, "q_rot": q_rot, "k_rot": k_rot, "q16": q16, "k16": k16, "pos": pos}

    def softmax_rows(self, x, threads: int = 1) -> np.ndarray:
        """Row softmax of an fp32 [rows, cols] array (numpy or torch) -> float64."""
        if hasattr(x, "detach"):
            x = x.detach().cpu().contiguous().numpy()
        a = np.ascontiguousarray(x)
        if a.dtype != np.float32 or a.ndim != 2:
            raise TypeError("x must be a float32 [rows, cols] array")
        rows, cols = a.shape
        out = np.empty((rows, cols), dtype=np.float64)
        fp = ctypes.POINTER(ctypes.c_float)

        def run(lo_hi):
            lo, hi = lo_hi
            if hi > lo:
                rc = self.lib.oracle_softmax_rows(a[lo:hi].ctypes.data_as(fp), hi - lo, cols,
                                                  out[lo:hi].ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
                if rc != 0:
                    raise ValueError("oracle_softmax_rows rejected its arguments")

        threads = max(1, min(int(threads), rows))
        bounds = [(rows * i // threads, rows * (i + 1) // threads) for i in range(threads)]
        if threads == 1:
            run(bounds[0])
        else:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, bounds))
        return out

    def decode_batched(self, q, k, v, current_pos, *, want_scores=False, threads: int = 1):
        """Independent sequences: q [B, H, D], k/v [B, S, H, D], current_pos [B].

        The batched form is a loop of single-sequence calls, each with its
        own current_pos.
        """
        outs, scs = [], []
        for b in range(k.shape[0]):
            o, s, _ = self.decode(q[b], k[b], v[b], int(current_pos[b]),
                                  want_scores=want_scores, threads=threads)
            outs.append(o)
            scs.append(s)
        return np.stack(outs), (np.stack(scs) if want_scores else None)


_default = None


def load(build_if_missing: bool = True) -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            if not build_if_missing:
                raise RuntimeError("oracle library not built: %s" % _build.LIB)
            _build.build()
        _default = OracleLib(_build.LIB)
    return _default


def half_to_double(bits) -> np.ndarray:
    return load().half_to_double(bits)


def decode(q, k, v, current_pos, **kw):
    return load().decode(q, k, v, current_pos, **kw)


def decode_batched(q, k, v, current_pos, **kw):
    return load().decode_batched(q, k, v, current_pos, **kw)


def pv_from_scores(scores, v, current_pos):
    return load().pv_from_scores(scores, v, current_pos)


def double_to_half(x):
    return load().double_to_half(x)


def rope(x, positions, **kw):
    return load().rope(x, positions, **kw)


def decode_step(q, k_new, v_new, k_cache, v_cache, current_pos, **kw):
    return load().decode_step(q, k_new, v_new, k_cache, v_cache, current_pos, **kw)


def softmax_rows(x, **kw):
    return load().softmax_rows(x, **kw)
