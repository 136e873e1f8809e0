"""Block-sparse fused attention forward for AMD MI355X (gfx950).

Thin ctypes binding over ``libbsattn.so`` (C ABI in ``include/bsattn.h``).
It only marshals arguments: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is missing or a call fails, an
exception is raised.

    bm = create_block_mask("sliding_window", S, S, window=256)
    out, lse = attention(q, k, v, bm, return_lse=True)

Mask rules ("FlexAttention on Apple Silicon: block masks", sections Mask 1-3):
``"none"``, ``"causal"`` (q >= kv), ``"sliding_window"`` (q >= kv and
q - kv < window), ``"document"`` (q >= kv and same document id); the
bottom-right aligned ``"causal_lower_right"`` and
``"sliding_window_lower_right"`` (query position shifted by kv_len - q_len,
"SDPA replaces hand-written attention", section 4, pitfall 3) and
``"document_bidirectional"`` (same document id only). score_mod: ``None`` or
``"softcap"`` (c * tanh(s / c), "FlexAttention on Apple Silicon", section
"Bonus"). K/V with fewer heads than Q (a divisor) is grouped-query attention
(query head h reads K/V head h // (H // H_kv); SDPA page, section 5).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Union

import torch

__all__ = [
    "BlockMask", "BsattnError", "create_block_mask", "create_block_mask_from_dense",
    "create_block_mask_from_bits", "pack_mask", "mask_words", "attention", "attention_backward",
    "num_blocks", "schedule_len", "library_path", "attention_noalloc",
    "workspace_size",
    "MASK_NONE", "MASK_CAUSAL", "MASK_SLIDING_WINDOW", "MASK_DOCUMENT",
    "MASK_CAUSAL_LOWER_RIGHT", "MASK_SLIDING_WINDOW_LOWER_RIGHT", "MASK_DOCUMENT_BIDIRECTIONAL",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libbsattn.so")

# Values from include/bsattn.h.
ATTN_OK = 0
F32, BF16, F16 = 0, 1, 2
MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT = 0, 1, 2, 3
MASK_CAUSAL_LOWER_RIGHT, MASK_SLIDING_WINDOW_LOWER_RIGHT, MASK_DOCUMENT_BIDIRECTIONAL = 4, 5, 6
MASK_CUSTOM = 7
_WINDOWED = (MASK_SLIDING_WINDOW, MASK_SLIDING_WINDOW_LOWER_RIGHT)
_DOCUMENTS = (MASK_DOCUMENT, MASK_DOCUMENT_BIDIRECTIONAL)
SCORE_NONE, SCORE_SOFTCAP = 0, 1
BLOCK_SIZE = 128

_KINDS = {"none": MASK_NONE, "causal": MASK_CAUSAL, "sliding_window": MASK_SLIDING_WINDOW,
          "sliding": MASK_SLIDING_WINDOW, "document": MASK_DOCUMENT,
          "causal_lower_right": MASK_CAUSAL_LOWER_RIGHT,
          "sliding_window_lower_right": MASK_SLIDING_WINDOW_LOWER_RIGHT,
          "document_bidirectional": MASK_DOCUMENT_BIDIRECTIONAL}
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class BsattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"bsattn status {status}: {message}")
        self.status = status


class _BlockMaskStruct(ctypes.Structure):
    _fields_ = [
        ("kv_num_blocks", ctypes.c_void_p),
        ("kv_indices", ctypes.c_void_p),
        ("full_kv_num_blocks", ctypes.c_void_p),
        ("full_kv_indices", ctypes.c_void_p),
        ("schedule", ctypes.c_void_p),
        ("q_len", ctypes.c_int32),
        ("kv_len", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_q_blocks", ctypes.c_int32),
        ("num_kv_blocks", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("document_id", ctypes.c_void_p),
        ("mask_bits", ctypes.c_void_p),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m block_sparse_attention_35_amd.build` "
            "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.attn_num_blocks.restype = i32
    lib.attn_num_blocks.argtypes = [i32, i32]
    lib.attn_block_mask_schedule_len.restype = i32
    lib.attn_block_mask_schedule_len.argtypes = [i32, i32, i32]
    lib.attn_build_block_mask.restype = i32
    lib.attn_build_block_mask.argtypes = [i32, i32, vp, i32, i32, i32,
                                          ctypes.POINTER(_BlockMaskStruct), vp]
    lib.attn_mask_words.restype = i32
    lib.attn_mask_words.argtypes = [i32]
    lib.attn_pack_mask.restype = i32
    lib.attn_pack_mask.argtypes = [vp, ctypes.c_int64, i32, i32, vp, vp]
    lib.attn_build_block_mask_custom.restype = i32
    lib.attn_build_block_mask_custom.argtypes = [vp, i32, i32, i32, ctypes.POINTER(_BlockMaskStruct), vp]
    lib.attn_backward.restype = i32
    lib.attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                  ctypes.POINTER(_BlockMaskStruct), i32, ctypes.c_float, ctypes.c_float,
                                  vp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_backward_workspace_size.restype = i32
    lib.attn_backward_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(_BlockMaskStruct),
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_forward.restype = i32
    lib.attn_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                 i64p, i64p, i64p, i64p, ctypes.POINTER(_BlockMaskStruct),
                                 i32, ctypes.c_float, ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.attn_forward_gqa.restype = i32
    lib.attn_forward_gqa.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     i64p, i64p, i64p, i64p, ctypes.POINTER(_BlockMaskStruct),
                                     i32, ctypes.c_float, ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.attn_forward_padded.restype = i32
    lib.attn_forward_padded.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                        i64p, i64p, i64p, i64p, ctypes.POINTER(_BlockMaskStruct),
                                        i32, ctypes.c_float, ctypes.c_float, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.attn_forward_noalloc.restype = i32
    lib.attn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                         i64p, i64p, i64p, i64p, ctypes.POINTER(_BlockMaskStruct),
                                         i32, ctypes.c_float, ctypes.c_float, vp, vp, vp]
    lib.attn_forward_workspace_size.restype = i32
    lib.attn_forward_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(_BlockMaskStruct),
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i32]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        lib = _load()
        msg = lib.attn_last_error().decode() or lib.attn_status_string(status).decode()
        raise BsattnError(status, msg)


def num_blocks(length: int, block_size: int = BLOCK_SIZE) -> int:
    n = _load().attn_num_blocks(length, block_size)
    if n < 0:
        raise BsattnError(-1, f"bad length {length} or block size {block_size}")
    return n


def schedule_len(q_len: int, kv_len: int, block_size: int = BLOCK_SIZE) -> int:
    """int32 entries of a BlockMask's work-plan array (from the library)."""
    n = _load().attn_block_mask_schedule_len(q_len, kv_len, block_size)
    if n < 0:
        raise BsattnError(-1, f"bad lengths {q_len}, {kv_len} or block size {block_size}")
    return n


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class BlockMask:
    """Device-resident 128x128 BlockMask (shared by every batch and head).

    Tensors (int32, on the mask's device): ``kv_num_blocks [nq]``,
    ``kv_indices [nq, nk]`` (partial blocks), ``full_kv_num_blocks [nq]``,
    ``full_kv_indices [nq, nk]`` (full blocks), ``schedule [4 + 8 nq]`` (the
    forward's work plan: item count, then 4-int descriptors ``(qb | chunk <<
    20 | (k - 1) << 22, full blocks, partial blocks, first block)`` by
    decreasing cost).
    """

    def __init__(self, kind: int, q_len: int, kv_len: int, window: int,
                 document_id: Optional[torch.Tensor], device: torch.device,
                 mask_bits: Optional[torch.Tensor] = None):
        nq, nk = num_blocks(q_len), num_blocks(kv_len)
        opt = dict(dtype=torch.int32, device=device)
        self.kind, self.q_len, self.kv_len, self.window = kind, q_len, kv_len, window
        self.document_id = document_id
        self.mask_bits = mask_bits  # CUSTOM: int32 [q_len, 4 nk] bit-packed mask
        self.device = device
        self.kv_num_blocks = torch.empty(nq, **opt)
        self.kv_indices = torch.empty(nq, nk, **opt)
        self.full_kv_num_blocks = torch.empty(nq, **opt)
        self.full_kv_indices = torch.empty(nq, nk, **opt)
        self.schedule = torch.zeros(schedule_len(q_len, kv_len), **opt)
        self._struct = _BlockMaskStruct()
        s = self._struct
        s.kv_num_blocks = self.kv_num_blocks.data_ptr()
        s.kv_indices = self.kv_indices.data_ptr()
        s.full_kv_num_blocks = self.full_kv_num_blocks.data_ptr()
        s.full_kv_indices = self.full_kv_indices.data_ptr()
        s.schedule = self.schedule.data_ptr()

    @property
    def num_q_blocks(self) -> int:
        return self.kv_num_blocks.shape[0]

    @property
    def num_kv_blocks(self) -> int:
        return self.kv_indices.shape[1]

    def rebuild(self):
        """Enqueue the library's mask build on the current stream."""
        with torch.cuda.device(self.device):
            if self.kind == MASK_CUSTOM:
                _check(_load().attn_build_block_mask_custom(
                    self.mask_bits.data_ptr(), self.q_len, self.kv_len, BLOCK_SIZE,
                    ctypes.byref(self._struct), _stream_handle(self.device)))
            else:
                doc = self.document_id.data_ptr() if self.document_id is not None else None
                _check(_load().attn_build_block_mask(self.kind, self.window, doc, self.q_len,
                                                     self.kv_len, BLOCK_SIZE,
                                                     ctypes.byref(self._struct),
                                                     _stream_handle(self.device)))
        return self


def create_block_mask(kind: Union[str, int], q_len: int, kv_len: int, window: Optional[int] = None,
                      document_id: Optional[torch.Tensor] = None,
                      device: Union[str, torch.device] = "cuda") -> BlockMask:
    """Build a BlockMask with attn_build_block_mask (asynchronous on the
    current stream of ``device``)."""
    if kind in ("custom", MASK_CUSTOM):
        raise ValueError("custom masks: create_block_mask_from_dense or create_block_mask_from_bits")
    k = _KINDS[kind] if isinstance(kind, str) else int(kind)
    device = torch.device(device)
    if device.type != "cuda":
        raise ValueError("the BlockMask lives in GPU memory; pass a cuda device")
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    if k in _WINDOWED:
        if window is None:
            raise ValueError("sliding_window needs window=")
        w = int(window)
    else:
        w = 0
    doc = None
    if k in _DOCUMENTS:
        if document_id is None:
            raise ValueError("document mask needs document_id=")
        if document_id.numel() < max(q_len, kv_len):
            raise ValueError("document_id must cover max(q_len, kv_len) positions")
        doc = document_id.to(device=device, dtype=torch.int32).contiguous()
    return BlockMask(k, q_len, kv_len, w, doc, device).rebuild()


def mask_words(kv_len: int) -> int:
    """uint32 words per row of a bit-packed mask: 4 * ceil(kv_len / 128)."""
    n = _load().attn_mask_words(kv_len)
    if n < 0:
        raise BsattnError(-1, f"bad kv_len {kv_len}")
    return n


def pack_mask(mask: torch.Tensor) -> torch.Tensor:
    """Bit-pack a dense boolean mask [q_len, kv_len] (True keeps the pair) on
    its GPU with attn_pack_mask: int32 [q_len, mask_words(kv_len)], bit b of
    word w of row i = mask[i, 32 w + b]."""
    if mask.dim() != 2 or mask.device.type != "cuda":
        raise ValueError("mask must be a 2-D tensor on a cuda device")
    if mask.dtype not in (torch.bool, torch.uint8):
        raise ValueError("mask must be torch.bool or torch.uint8")
    L, S = mask.shape
    if S > 0 and mask.stride(1) != 1:
        mask = mask.contiguous()
    stride = mask.stride(0) if L > 1 else S
    bits = torch.empty(L, mask_words(S), dtype=torch.int32, device=mask.device)
    with torch.cuda.device(mask.device):
        _check(_load().attn_pack_mask(mask.data_ptr() if mask.numel() else None, stride, L, S,
                                      bits.data_ptr() if bits.numel() else None,
                                      _stream_handle(mask.device)))
    return bits


def create_block_mask_from_bits(bits: torch.Tensor, q_len: int, kv_len: int) -> BlockMask:
    """BlockMask of kind CUSTOM from a bit-packed mask (int32 [q_len,
    mask_words(kv_len)] on a cuda device, kept by the BlockMask)."""
    if bits.device.type != "cuda" or bits.dtype != torch.int32:
        raise ValueError("bits must be an int32 tensor on a cuda device")
    if tuple(bits.shape) != (q_len, mask_words(kv_len)) or not bits.is_contiguous():
        raise ValueError(f"bits must be contiguous [{q_len}, {mask_words(kv_len)}]")
    return BlockMask(MASK_CUSTOM, q_len, kv_len, 0, None, bits.device, mask_bits=bits).rebuild()


def create_block_mask_from_dense(mask: torch.Tensor) -> BlockMask:
    """BlockMask of kind CUSTOM from a dense boolean mask [q_len, kv_len] on a
    cuda device (True keeps the pair): the mask is bit-packed on the GPU, and
    only the packed form is kept."""
    L, S = mask.shape
    return create_block_mask_from_bits(pack_mask(mask), L, S)


_workspaces = {}


def _workspace(nbytes: int, device: torch.device, stream: int, role: str = "forward") -> torch.Tensor:
    """A zero-filled workspace of at least nbytes, one per (device, stream,
    role), kept for later calls (the library leaves its counters at zero
    again; the forward and the backward lay theirs out differently, so each
    has its own)."""
    key = (device.index, stream, role)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def workspace_size(q: torch.Tensor, block_mask: BlockMask) -> int:
    """Bytes of workspace attention() needs for q's batch, heads and dtype
    (a function of those and the mask's lengths, cached on the mask)."""
    key = (_DTYPES[q.dtype], q.shape[0], q.shape[1])
    cache = block_mask.__dict__.setdefault("_ws_sizes", {})
    if key not in cache:
        n = ctypes.c_size_t(0)
        _check(_load().attn_forward_workspace_size(key[0], key[1], key[2],
                                                   ctypes.byref(block_mask._struct), ctypes.byref(n)))
        cache[key] = n.value
    return cache[key]


def _strides(t: torch.Tensor):
    """Element strides for the library, or None (the contiguous layout)."""
    if t.is_contiguous():
        return None
    return (ctypes.c_int64 * 4)(*t.stride())


def _check_forward_args(q, k, v, out, lse, workspace, key_start, key_end):
    """Host-side checks of attention()'s tensors (every tensor on q's device;
    the library writes B*H*L*E elements through out's strides and B*H*L floats
    of lse, so both must have exactly those shapes). Returns (B, H, H_kv, L,
    S, E); raises ValueError."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, seq, E]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one dtype among float32, bfloat16, float16")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    B, H, L, E = q.shape
    H_kv, S = k.shape[1], k.shape[2]
    if k.shape != (B, H_kv, S, E) or v.shape != (B, H_kv, S, E) or H_kv < 1 or H % H_kv:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is not None and (tuple(out.shape) != (B, H, L, E) or out.dtype != q.dtype
                            or out.device != q.device or (out.numel() and out.stride(-1) != 1)):
        raise ValueError(f"out must be a {q.dtype} tensor of shape {(B, H, L, E)} on {q.device} "
                         "with a contiguous head dim")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H, L) or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, L] tensor on q's device")
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != q.device
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    for t in (key_start, key_end):
        if t is not None and (t.dtype != torch.int32 or t.device != q.device
                              or tuple(t.shape) != (B,) or not t.is_contiguous()):
            raise ValueError("key_start / key_end must be contiguous int32 tensors [B] on q's device")
    return B, H, H_kv, L, S, E


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: BlockMask,
              score_mod: Optional[str] = None, softcap: float = 30.0,
              scale: Optional[float] = None, return_lse: bool = False,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, key_start: Optional[torch.Tensor] = None,
              key_end: Optional[torch.Tensor] = None):
    """Fused block-sparse attention forward (attn_forward, or attn_forward_gqa
    when k and v have fewer heads than q).

    q [B,H,L,E], k/v [B,H_kv,S,E] (H a multiple of H_kv) on the GPU, one dtype
    among fp32/bf16/fp16,
    head dim contiguous. ``scale`` defaults to 1/sqrt(E) ("SDPA replaces
    hand-written attention", section 1). Returns O [B,H,L,E] (and the fp32
    natural-log logsumexp [B,H,L] when ``return_lse``). ``key_start`` /
    ``key_end``: optional int32 GPU tensors [B], the kept key range of each
    batch entry (key padding, ANDed with the mask; attn_forward_padded).
    ``workspace``: a
    zero-filled uint8 GPU tensor of at least ``workspace_size(q, block_mask)``
    bytes; by default one cached per device and stream is used.
    """
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    B, H, H_kv, L, S, E = _check_forward_args(q, k, v, out, lse, workspace, key_start, key_end)
    if scale is None:
        scale = 1.0 / math.sqrt(E)
    sm = {None: SCORE_NONE, "none": SCORE_NONE, "softcap": SCORE_SOFTCAP}[score_mod]
    if out is None:
        out = torch.empty(B, H, L, E, dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty(B, H, L, dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = _stream_handle(q.device)
        need = workspace_size(q, block_mask)
        if workspace is None and need > 0:
            workspace = _workspace(need, q.device, stream)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        lse_ptr = lse.data_ptr() if lse is not None else None
        pads = [t.data_ptr() if t is not None else None for t in (key_start, key_end)]
        if key_start is not None or key_end is not None:
            _check(_load().attn_forward_padded(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                _DTYPES[q.dtype], B, H, H_kv, L, S, E,
                _strides(q), _strides(k), _strides(v), _strides(out),
                ctypes.byref(block_mask._struct), sm, float(softcap), float(scale),
                pads[0], pads[1], ws_ptr, ws_bytes, stream))
        elif H_kv == H:
            _check(_load().attn_forward(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                _DTYPES[q.dtype], B, H, L, S, E,
                _strides(q), _strides(k), _strides(v), _strides(out),
                ctypes.byref(block_mask._struct), sm, float(softcap), float(scale),
                ws_ptr, ws_bytes, stream))
        else:
            _check(_load().attn_forward_gqa(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                _DTYPES[q.dtype], B, H, H_kv, L, S, E,
                _strides(q), _strides(k), _strides(v), _strides(out),
                ctypes.byref(block_mask._struct), sm, float(softcap), float(scale),
                ws_ptr, ws_bytes, stream))
    return (out, lse) if return_lse else out


def _check_backward_args(q, k, v, out, lse, dout, key_start, key_end):
    """Host-side checks of attention_backward()'s tensors (one dtype and device;
    k and v [B, H_kv, S, E] with H_kv dividing H; the library reads and writes
    contiguous tensors of exactly these shapes). Returns (B, H, H_kv, L, S, E);
    raises ValueError."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (k, v, out, dout):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, out and dout must share dtype and device")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, seq, E]")
    B, H, L, E = q.shape
    Hk, S = k.shape[1], k.shape[2]
    if (out.shape != q.shape or dout.shape != q.shape or tuple(k.shape) != (B, Hk, S, E)
            or v.shape != k.shape or Hk < 1 or H % Hk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)} "
                         f"out{tuple(out.shape)} dout{tuple(dout.shape)}")
    if tuple(lse.shape) != (B, H, L) or lse.dtype != torch.float32 or lse.device != q.device:
        raise ValueError("lse must be float32 [B, H, L] on q's device")
    for t in (key_start, key_end):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (B,) or t.device != q.device
                              or not t.is_contiguous()):
            raise ValueError("key_start / key_end must be contiguous int32 [B] on the tensors' device")
    return B, H, Hk, L, S, E


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor, dout: torch.Tensor, block_mask: BlockMask,
                       score_mod: Optional[str] = None, softcap: float = 30.0,
                       scale: Optional[float] = None, key_start: Optional[torch.Tensor] = None,
                       key_end: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(dout * out) through ``attention`` (fp32,
    bf16 or fp16), with the attention matrix recomputed from ``lse`` (the forward's
    logsumexp) by attn_backward. ``out`` and ``lse`` are the forward's outputs
    for the same arguments; k and v may have fewer heads (grouped-query
    attention), and dk, dv then sum over the query heads that share a K/V head.
    Tensors are made contiguous; the call is asynchronous on the current
    stream."""
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a cuda device")
    B, H, Hk, L, S, E = _check_backward_args(q, k, v, out, lse, dout, key_start, key_end)
    q, k, v, out, dout, lse = (t.contiguous() for t in (q, k, v, out, dout, lse))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lib = _load()
    nbytes = ctypes.c_size_t(0)
    _check(lib.attn_backward_workspace_size(B, H, Hk, ctypes.byref(block_mask._struct), ctypes.byref(nbytes)))
    stream = _stream_handle(q.device)
    ws = _workspace(nbytes.value, q.device, stream, role="backward")
    sm = SCORE_SOFTCAP if score_mod == "softcap" else SCORE_NONE
    if score_mod not in (None, "softcap"):
        raise ValueError(f"unknown score_mod {score_mod!r}")
    sc = 1.0 / math.sqrt(E) if scale is None else float(scale)
    ptr = lambda t: t.data_ptr() if t is not None and t.numel() else None
    with torch.cuda.device(q.device):
        _check(lib.attn_backward(ptr(q), ptr(k), ptr(v), ptr(out), ptr(lse), ptr(dout), ptr(dq), ptr(dk),
                                 ptr(dv), _DTYPES[q.dtype], B, H, Hk, L, S, E,
                                 ctypes.byref(block_mask._struct), sm, float(softcap), sc,
                                 ptr(key_start), ptr(key_end), ws.data_ptr(), ws.numel(), stream))
    return dq, dk, dv


def attention_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: BlockMask,
                      out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                      score_mod: Optional[str] = None, softcap: float = 30.0,
                      scale: Optional[float] = None, key_start: Optional[torch.Tensor] = None,
                      key_end: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``attention`` through attn_forward_noalloc: the library allocates no
    device memory (its split items use a fixed per-GPU scratch array) and the
    caller passes ``out`` (and ``lse``). Calls that overlap in time on one GPU
    race on that scratch."""
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if out is None:
        raise ValueError("attention_noalloc needs out")
    B, H, H_kv, L, S, E = _check_forward_args(q, k, v, out, lse, None, key_start, key_end)
    sc = 1.0 / math.sqrt(E) if scale is None else float(scale)
    sm = {None: SCORE_NONE, "none": SCORE_NONE, "softcap": SCORE_SOFTCAP}[score_mod]
    ptr = lambda t: t.data_ptr() if t is not None else None
    with torch.cuda.device(q.device):
        _check(_load().attn_forward_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), ptr(lse),
            _DTYPES[q.dtype], B, H, H_kv, L, S, E,
            _strides(q), _strides(k), _strides(v), _strides(out),
            ctypes.byref(block_mask._struct), sm, float(softcap), sc,
            ptr(key_start), ptr(key_end), _stream_handle(q.device)))
    return out
