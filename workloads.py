"""Seeded synthetic workloads shared by the tests, the benchmark and smoke().

This module holds only input generation: shapes, dtypes, mask recipes and
seeded random tensors. It contains none of the attention arithmetic, so both
the HIP path and the CPU oracle may take their inputs from here.

Workloads (all B=1, E=64, layout [B, H, seq, E] contiguous, i.i.d. N(0,1)):

* ``causal_256_f32`` -- H=2, L=S=256, fp32, causal (the small case).
* ``causal_8192_bf16`` -- H=8, L=S=8192, bf16, causal. The FlexAttention
  benchmark on Apple M1 Max ("FlexAttention on MPS vs SDPA", results table,
  causal row) uses this shape: batch 1, 8 heads, head dim 64, bf16.
* ``sliding_8192_w{64,256,1024,4096}_bf16`` -- the same shape with a
  sliding-window causal mask, one workload per window of that table.
* ``sliding_32768_w256_bf16`` -- H=8, L=S=32768, window 256 (the table's
  last row).
* ``document_8192_f16_softcap`` -- H=16, L=S=8192, fp16, document-packed
  causal mask with ids 0 on [0,2048), 1 on [2048,5000), 2 on [5000,8192), and
  a tanh soft-cap of 30 ("FlexAttention on Apple Silicon: block masks",
  sections "Mask 3: document-packed" and "Bonus: a score_mod for soft-capping").

Variant workloads (the mask and head-sharing variants of the same kernel):

* ``causal_lower_right_2048x8192_bf16`` -- H=8, L=2048 queries at the end of
  S=8192 keys, bottom-right aligned causal mask (chunked inference against a
  cache: "SDPA replaces hand-written attention", section 4, pitfall 3).
* ``gqa_causal_8192_h32_kv8_bf16`` -- 32 query heads sharing 8 K/V heads
  (same page, section 5), L=S=8192, causal.
* ``document_bidirectional_8192_f16_softcap`` -- the document workload's
  shape and ids with the bidirectional (block-diagonal) document mask.
* ``decode_gqa_b8_h32_kv8_s8192_bf16`` -- decode: one new query per sequence
  (L=1) against S=8192 cached keys, B=8 sequences, 32 query heads sharing 8
  K/V heads, bottom-right causal (the query sees every key: SDPA page,
  section 4, pitfall 3, KV-cache inference; section 5, GQA).
* ``causal_8192_keypad_b2_bf16`` -- B=2, H=8, L=S=8192 causal with key
  padding: batch entry 0 keeps every key, entry 1 keys [2048, 7168) (left
  and right padding ANDed with the causal mask; SDPA page, section 4,
  pitfall 1 and section 5).
* ``custom_blocks_8192_bf16`` -- H=8, L=S=8192 with a user-supplied dense
  boolean mask (the form SDPA takes masks in: "FlexAttention on MPS vs SDPA",
  setup notes; True keeps the pair: SDPA page, section 4, pitfall 1): each
  128 x 128 block is all True with probability 0.08, holds i.i.d. pairs kept
  with probability 0.5 with probability 0.06, and is all False otherwise
  (about 14% of the blocks live, like the table's W=1024 row), seed 11.

User masks (``block_structured_mask``): per 128 x 128 block one uniform draw
picks full / partial / empty, then the partial blocks' pairs are drawn
i.i.d.; both from ``numpy.random.default_rng(seed)``.

Generation: ``numpy.random.default_rng(seed).standard_normal(shape, float32)``
drawn for q, then k, then v, then rounded to the workload dtype with
round-to-nearest-even (torch's CPU cast). Both sides read the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Mask kinds, numbered as in include/bsattn.h.
MASK_NONE = 0
MASK_CAUSAL = 1
MASK_SLIDING_WINDOW = 2
MASK_DOCUMENT = 3
MASK_CAUSAL_LOWER_RIGHT = 4
MASK_SLIDING_WINDOW_LOWER_RIGHT = 5
MASK_DOCUMENT_BIDIRECTIONAL = 6
MASK_CUSTOM = 7
DOCUMENT_KINDS = (MASK_DOCUMENT, MASK_DOCUMENT_BIDIRECTIONAL)

BLOCK = 128

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    S: int
    E: int
    dtype: str            # "f32" | "bf16" | "f16"
    kind: int             # MASK_*
    window: int = 0       # sliding-window size W (the two sliding-window kinds)
    doc_bounds: tuple = ()  # document start offsets after the first (document kinds)
    softcap: float = 0.0  # 0 = no score_mod, else c in c*tanh(s/c)
    H_kv: int = 0         # K/V heads (grouped-query attention); 0 = H
    key_ranges: tuple = ()  # per batch entry (start, end) kept keys; () = no padding
    mask_recipe: tuple = ()  # CUSTOM: (p_full, p_partial, density, seed) of block_structured_mask

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.E)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("causal_256_f32", 1, 2, 256, 256, 64, "f32", MASK_CAUSAL),
        Workload("causal_8192_bf16", 1, 8, 8192, 8192, 64, "bf16", MASK_CAUSAL),
        Workload("sliding_8192_w64_bf16", 1, 8, 8192, 8192, 64, "bf16", MASK_SLIDING_WINDOW, 64),
        Workload("sliding_8192_w256_bf16", 1, 8, 8192, 8192, 64, "bf16", MASK_SLIDING_WINDOW, 256),
        Workload("sliding_8192_w1024_bf16", 1, 8, 8192, 8192, 64, "bf16", MASK_SLIDING_WINDOW, 1024),
        Workload("sliding_8192_w4096_bf16", 1, 8, 8192, 8192, 64, "bf16", MASK_SLIDING_WINDOW, 4096),
        Workload("sliding_32768_w256_bf16", 1, 8, 32768, 32768, 64, "bf16", MASK_SLIDING_WINDOW, 256),
        Workload("document_8192_f16_softcap", 1, 16, 8192, 8192, 64, "f16", MASK_DOCUMENT, 0,
                 (2048, 5000), 30.0),
        Workload("causal_lower_right_2048x8192_bf16", 1, 8, 2048, 8192, 64, "bf16",
                 MASK_CAUSAL_LOWER_RIGHT),
        Workload("gqa_causal_8192_h32_kv8_bf16", 1, 32, 8192, 8192, 64, "bf16", MASK_CAUSAL,
                 H_kv=8),
        Workload("document_bidirectional_8192_f16_softcap", 1, 16, 8192, 8192, 64, "f16",
                 MASK_DOCUMENT_BIDIRECTIONAL, 0, (2048, 5000), 30.0),
        Workload("causal_8192_keypad_b2_bf16", 2, 8, 8192, 8192, 64, "bf16", MASK_CAUSAL,
                 key_ranges=((0, 8192), (2048, 7168))),
        Workload("decode_gqa_b8_h32_kv8_s8192_bf16", 8, 32, 1, 8192, 64, "bf16",
                 MASK_CAUSAL_LOWER_RIGHT, H_kv=8),
        Workload("custom_blocks_8192_bf16", 1, 8, 8192, 8192, 64, "bf16", MASK_CUSTOM,
                 mask_recipe=(0.08, 0.06, 0.5, 11)),
    ]
}


def document_ids(length: int, bounds: tuple) -> np.ndarray:
    """int32 ids: 0 before bounds[0], 1 from bounds[0], 2 from bounds[1], ..."""
    ids = np.zeros(length, dtype=np.int32)
    for d, start in enumerate(bounds, start=1):
        ids[start:] = d
    return ids


def make_qkv(w: Workload, seed: int = 0):
    """Seeded q, k, v as CPU torch tensors of the workload dtype: q [B,H,L,E],
    k and v [B,H_kv,S,E]."""
    rng = np.random.default_rng(seed)
    hk = w.kv_heads
    shapes = [(w.B, w.H, w.L, w.E), (w.B, hk, w.S, w.E), (w.B, hk, w.S, w.E)]
    out = []
    for shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32)
        out.append(torch.from_numpy(x).to(w.torch_dtype))
    return tuple(out)


def block_structured_mask(L: int, S: int, seed: int, p_full: float = 0.1, p_partial: float = 0.1,
                          density: float = 0.5) -> np.ndarray:
    """Seeded boolean [L, S]: each 128 x 128 block (ragged at the ends) is all
    True with probability p_full, i.i.d. pairs kept with probability
    `density` with probability p_partial, all False otherwise."""
    rng = np.random.default_rng(seed)
    nq, nk = -(-L // BLOCK), -(-S // BLOCK)
    u = rng.random((nq, nk))
    full = np.repeat(np.repeat(u < p_full, BLOCK, 0), BLOCK, 1)[:L, :S]
    part = np.repeat(np.repeat((u >= p_full) & (u < p_full + p_partial), BLOCK, 0), BLOCK, 1)[:L, :S]
    return full | (part & (rng.random((L, S), dtype=np.float32) < density))


def make_mask(w: Workload) -> Optional[np.ndarray]:
    """The user mask of a CUSTOM workload (None for the rule kinds)."""
    if w.kind != MASK_CUSTOM:
        return None
    p_full, p_partial, density, seed = w.mask_recipe
    return block_structured_mask(w.L, w.S, seed, p_full, p_partial, density)


def make_doc(w: Workload) -> Optional[np.ndarray]:
    if w.kind not in DOCUMENT_KINDS:
        return None
    return document_ids(max(w.L, w.S), w.doc_bounds)


def sample_rows(w: Workload, count: int, seed: int = 1234) -> np.ndarray:
    """Flat row ids (b*H*L + h*L + i) for spot checks at full size.

    Always includes the first and last row of every head plus the rows at
    each 128-block boundary of head 0; the rest are drawn uniformly.
    """
    rng = np.random.default_rng(seed)
    n = w.B * w.H * w.L
    fixed = []
    for bh in range(w.B * w.H):
        fixed += [bh * w.L, bh * w.L + w.L - 1]
    fixed += [min(i, w.L - 1) for i in range(0, w.L, BLOCK)]
    fixed += [min(i + BLOCK - 1, w.L - 1) for i in range(0, w.L, BLOCK)]
    extra = rng.integers(0, n, size=max(0, count - len(fixed)))
    return np.unique(np.concatenate([np.asarray(fixed, dtype=np.int64), extra.astype(np.int64)]))
