"""CPU fp64 oracle for block-sparse masked attention (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. The product path never does.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent
rows); this module builds it with gcc and wraps it with ctypes. Definitions and
the passages they follow are cited in ``oracle.c``:

Mask kinds: NONE, CAUSAL, SLIDING, DOCUMENT, and the variants
CAUSAL_LOWER_RIGHT, SLIDING_LOWER_RIGHT (query position shifted by S - L) and
DOCUMENT_BIDIRECTIONAL (same document, no causal part); DENSE reads a
user-supplied L x S boolean mask (True keeps the pair).

* ``attention``   -- softmax(Q K^T * scale + mask bias) V per row, optional
  per-batch key padding (a kept key range ANDed with the mask), optional
  tanh soft-cap on the scaled score, O = 0 and lse = -inf for a row with no
  live key.
* ``block_mask``  -- 128x128 block classification by brute force over every
  in-range pair: skip / partial / full, with ascending index lists padded by 0.
* ``count_live``  -- number of live (query, key) pairs of a mask.
* ``attention_backward`` -- dq, dk, dv of sum(dO * O) by the chain rule, the
  attention matrix recomputed per row.
* ``pack_mask``   -- bit-packed form of a dense boolean mask: row i is
  4 * ceil(S / 128) uint32 words, bit b of word w is M[i, 32 w + b].

Every function is pinned by ``tests/test_oracle_pins.py`` against values the
pages print, closed forms, invariances and library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")

NONE, CAUSAL, SLIDING, DOCUMENT = 0, 1, 2, 3
CAUSAL_LOWER_RIGHT, SLIDING_LOWER_RIGHT, DOCUMENT_BIDIRECTIONAL = 4, 5, 6
DENSE = 7
_DOC_KINDS = (DOCUMENT, DOCUMENT_BIDIRECTIONAL)


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source file into a shared library at ``out``."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile oracle.c into oracle/_build/liboracle.so (always rebuilds)."""
    return compile_source(SOURCE, _LIB_PATH)


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return ctypes.POINTER(ctype)()
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _doc(doc) -> Optional[np.ndarray]:
    return None if doc is None else np.ascontiguousarray(doc, dtype=np.int32)


def _dense(kind, mask, L, S) -> Optional[np.ndarray]:
    """The DENSE kind's mask as contiguous bytes [L, S] (None for other kinds)."""
    if kind != DENSE:
        return None
    if mask is None:
        raise ValueError("the DENSE kind needs a mask")
    m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    if m.shape != (L, S):
        raise ValueError(f"mask shape {m.shape} is not (L, S) = ({L}, {S})")
    return m


class Oracle:
    """ctypes front end over one compiled copy of the oracle."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        i64, i32p = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        u8p, u32p = ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_live.restype = ctypes.c_int
        lib.oracle_live.argtypes = [ctypes.c_int, i64, i32p, u8p, i64, i64, i64, i64]
        lib.oracle_count_live.restype = i64
        lib.oracle_count_live.argtypes = [ctypes.c_int, i64, i32p, u8p, i64, i64]
        lib.oracle_block_mask.restype = ctypes.c_int
        lib.oracle_block_mask.argtypes = [ctypes.c_int, i64, i32p, u8p, i64, i64, i64,
                                          i32p, i32p, i32p, i32p]
        lib.oracle_pack_mask.restype = ctypes.c_int
        lib.oracle_pack_mask.argtypes = [u8p, i64, i64, u32p]
        lib.oracle_attention.restype = ctypes.c_int
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_attention.argtypes = [f64p, f64p, f64p, i64, i64, i64, i64, i64, i64,
                                         ctypes.c_int, i64, i32p, u8p, ctypes.c_double,
                                         ctypes.c_double, i64p, i64p, i64p, i64, f64p, f64p]
        lib.oracle_attention_backward_dq_rows.restype = ctypes.c_int
        lib.oracle_attention_backward_dq_rows.argtypes = [
            f64p, f64p, f64p, f64p, i64, i64, i64, i64, i64, ctypes.c_int, i64, i32p, u8p,
            ctypes.c_double, ctypes.c_double, i64p, i64p, i64p, i64, f64p]
        lib.oracle_attention_backward.restype = ctypes.c_int
        lib.oracle_attention_backward.argtypes = [f64p, f64p, f64p, f64p, i64, i64, i64, i64, i64,
                                                  ctypes.c_int, i64, i32p, u8p, ctypes.c_double,
                                                  ctypes.c_double, i64p, i64p, f64p, f64p, f64p]
        self._lib = lib

    @staticmethod
    def _check_doc(kind, d, L, S):
        if kind in _DOC_KINDS and (d is None or len(d) < max(L, S)):
            raise ValueError("document kind needs ids for max(L, S) positions")

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def live(self, kind: int, i: int, j: int, window: int = 0, doc=None, L: int = 0,
             S: int = 0, mask=None) -> bool:
        """The predicate for query i and key j (L and S matter only to the
        lower-right kinds and DENSE)."""
        d = _doc(doc)
        m = _dense(kind, mask, L, S)
        if m is not None and not (0 <= i < L and 0 <= j < S):
            raise ValueError("pair outside the mask")
        return bool(self._lib.oracle_live(kind, window, _ptr(d, ctypes.c_int32),
                                          _ptr(m, ctypes.c_uint8), L, S, i, j))

    def count_live(self, kind: int, L: int, S: int, window: int = 0, doc=None, mask=None) -> int:
        d = _doc(doc)
        self._check_doc(kind, d, L, S)
        m = _dense(kind, mask, L, S)
        return int(self._lib.oracle_count_live(kind, window, _ptr(d, ctypes.c_int32),
                                               _ptr(m, ctypes.c_uint8), L, S))

    def pack_mask(self, mask) -> np.ndarray:
        """Bit-packed mask: uint32 [L, 4 * ceil(S / 128)], bit b of word w of
        row i = mask[i, 32 w + b] (0 past S)."""
        m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        L, S = m.shape
        bits = np.zeros((L, 4 * (-(-S // 128))), np.uint32)
        if self._lib.oracle_pack_mask(_ptr(m, ctypes.c_uint8), L, S, _ptr(bits, ctypes.c_uint32)) != 0:
            raise ValueError("oracle_pack_mask rejected its arguments")
        return bits

    def block_mask(self, kind: int, L: int, S: int, window: int = 0, doc=None, block: int = 128,
                   mask=None):
        """(kv_num_blocks [nq], kv_indices [nq,nk], full_kv_num_blocks [nq],
        full_kv_indices [nq,nk]) as int32 arrays."""
        d = _doc(doc)
        self._check_doc(kind, d, L, S)
        m = _dense(kind, mask, L, S)
        nq, nk = -(-L // block), -(-S // block)
        kv_num = np.zeros(nq, np.int32)
        kv_idx = np.zeros((nq, nk), np.int32)
        full_num = np.zeros(nq, np.int32)
        full_idx = np.zeros((nq, nk), np.int32)
        rc = self._lib.oracle_block_mask(kind, window, _ptr(d, ctypes.c_int32),
                                         _ptr(m, ctypes.c_uint8), L, S, block,
                                         _ptr(kv_num, ctypes.c_int32), _ptr(kv_idx, ctypes.c_int32),
                                         _ptr(full_num, ctypes.c_int32),
                                         _ptr(full_idx, ctypes.c_int32))
        if rc != 0:
            raise ValueError("oracle_block_mask rejected its arguments")
        return kv_num, kv_idx, full_num, full_idx

    def attention(self, q, k, v, kind: int, scale: float, window: int = 0, doc=None,
                  softcap: float = 0.0, rows=None, key_start=None, key_end=None, mask=None):
        """fp64 masked softmax attention.

        q [B,H,L,E], k [B,H,S,E], v [B,H,S,Ev] (any float dtype; converted to
        fp64 exactly). key_start, key_end: optional per-batch [B] kept key
        range [start, end) (key padding, ANDed with the mask). mask: the
        DENSE kind's boolean [L, S]. Returns
        (out, lse): for rows=None, out [B,H,L,Ev] and lse [B,H,L]; otherwise
        out [len(rows), Ev] and lse [len(rows)] for the flat row ids
        (b*H + h)*L + i.
        """
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        B, H, L, E = q.shape
        S, Ev = k.shape[2], v.shape[3]
        if k.shape != (B, H, S, E) or v.shape[:3] != (B, H, S):
            raise ValueError("q/k/v shapes disagree")
        d = _doc(doc)
        self._check_doc(kind, d, L, S)
        m = _dense(kind, mask, L, S)
        ks = None if key_start is None else np.ascontiguousarray(key_start, dtype=np.int64)
        ke = None if key_end is None else np.ascontiguousarray(key_end, dtype=np.int64)
        for a in (ks, ke):
            if a is not None and a.shape != (B,):
                raise ValueError("key_start / key_end need one entry per batch")
        if rows is None:
            n, rows_arr = B * H * L, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= B * H * L):
                raise ValueError("row id out of range")
            n = rows_arr.size
        out = np.zeros((n, Ev), np.float64)
        lse = np.zeros(n, np.float64)
        rc = self._lib.oracle_attention(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                        _ptr(v, ctypes.c_double), B, H, L, S, E, Ev, kind, window,
                                        _ptr(d, ctypes.c_int32), _ptr(m, ctypes.c_uint8),
                                        softcap, scale,
                                        _ptr(ks, ctypes.c_int64), _ptr(ke, ctypes.c_int64),
                                        _ptr(rows_arr, ctypes.c_int64), n,
                                        _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
        if rc != 0:
            raise RuntimeError("oracle_attention failed")
        if rows is None:
            return out.reshape(B, H, L, Ev), lse.reshape(B, H, L)
        return out, lse


_default: Optional[Oracle] = None


def _attention_backward(self, q, k, v, dout, kind: int, scale: float, window: int = 0, doc=None,
                        softcap: float = 0.0, key_start=None, key_end=None, mask=None):
    """fp64 gradients (dq, dk, dv) of sum(dout * O) for O = attention(q, k, v,
    ...): q, dout [B,H,L,E], k, v [B,H,S,E] (K/V heads expanded to H)."""
    q, k, v, dout = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, H, L, E = q.shape
    S = k.shape[2]
    if k.shape != (B, H, S, E) or v.shape != (B, H, S, E) or dout.shape != q.shape:
        raise ValueError("q/k/v/dout shapes disagree (the backward takes E = Ev)")
    d = _doc(doc)
    self._check_doc(kind, d, L, S)
    m = _dense(kind, mask, L, S)
    ks = None if key_start is None else np.ascontiguousarray(key_start, dtype=np.int64)
    ke = None if key_end is None else np.ascontiguousarray(key_end, dtype=np.int64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    rc = self._lib.oracle_attention_backward(
        _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
        _ptr(dout, ctypes.c_double), B, H, L, S, E, kind, window, _ptr(d, ctypes.c_int32),
        _ptr(m, ctypes.c_uint8), softcap, scale, _ptr(ks, ctypes.c_int64), _ptr(ke, ctypes.c_int64),
        _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oracle_attention_backward failed")
    return dq, dk, dv


Oracle.attention_backward = _attention_backward


def _attention_backward_dq_rows(self, q, k, v, dout, kind: int, scale: float, rows, window: int = 0,
                                doc=None, softcap: float = 0.0, mask=None):
    """dq of attention_backward for flat rows (b*H + h)*L + i only: [len(rows), E]."""
    q, k, v, dout = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, H, L, E = q.shape
    S = k.shape[2]
    d = _doc(doc)
    self._check_doc(kind, d, L, S)
    m = _dense(kind, mask, L, S)
    rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
    if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= B * H * L):
        raise ValueError("row id out of range")
    out = np.zeros((rows_arr.size, E), np.float64)
    rc = self._lib.oracle_attention_backward_dq_rows(
        _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
        _ptr(dout, ctypes.c_double), B, H, L, S, E, kind, window, _ptr(d, ctypes.c_int32),
        _ptr(m, ctypes.c_uint8), softcap, scale, None, None, _ptr(rows_arr, ctypes.c_int64),
        rows_arr.size, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oracle_attention_backward_dq_rows failed")
    return out


Oracle.attention_backward_dq_rows = _attention_backward_dq_rows


def default() -> Oracle:
    """The oracle built from oracle.c (built on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def live(kind, i, j, window=0, doc=None, L=0, S=0, mask=None):
    return default().live(kind, i, j, window, doc, L, S, mask)


def count_live(kind, L, S, window=0, doc=None, mask=None):
    return default().count_live(kind, L, S, window, doc, mask)


def pack_mask(mask):
    return default().pack_mask(mask)


def block_mask(kind, L, S, window=0, doc=None, block=128, mask=None):
    return default().block_mask(kind, L, S, window, doc, block, mask)


def attention(q, k, v, kind, scale, window=0, doc=None, softcap=0.0, rows=None, key_start=None,
              key_end=None, mask=None):
    return default().attention(q, k, v, kind, scale, window, doc, softcap, rows, key_start, key_end,
                               mask)


def attention_backward(q, k, v, dout, kind, scale, window=0, doc=None, softcap=0.0, key_start=None,
                       key_end=None, mask=None):
    return default().attention_backward(q, k, v, dout, kind, scale, window, doc, softcap, key_start,
                                        key_end, mask)


def attention_backward_dq_rows(q, k, v, dout, kind, scale, rows, window=0, doc=None, softcap=0.0,
                               mask=None):
    return default().attention_backward_dq_rows(q, k, v, dout, kind, scale, rows, window, doc, softcap,
                                                mask)
