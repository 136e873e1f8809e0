"""GPU parity: the HIP path against the fp64 oracle, through the C ABI.

* BlockMask arrays bit-exact (counts, index lists, zero padding) and the
  schedule equal to the unique descending-cost order.
* Forward O within the stated tolerance: max-abs 1e-2 and mean-abs 1e-3 for
  bf16/fp16, 1e-5 for fp32 (max and mean). The logsumexp is the log of the
  normaliser the kernel divides by, a sum of probabilities rounded to the
  input type (relative error u = 2^-8 for bf16, 2^-11 for fp16 per term), so
  |lse error| <= -ln(1 - u) + fp32 terms: 3.9e-3 for bf16 (bound 4e-3); for
  fp16 4.9e-4 plus at most 8192 subnormal terms of absolute error 2^-25
  (2.4e-4), bound 1e-3; fp32 1e-5. Every case compares every element of O
  and every row's logsumexp, the full workloads (the shapes and launch
  configuration the benchmark times) included; only the 524,800-token band
  (whose oracle would take minutes) compares sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_35_amd as bsa
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

# (O max-abs, O mean-abs, lse max-abs)
TOL = {"f32": (1e-5, 1e-5, 1e-5), "bf16": (1e-2, 1e-3, 4e-3), "f16": (1e-2, 1e-3, 1e-3)}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def expected_plan(n):
    """The forward's work plan from the live block counts n[qb]: with
    C = max(16, ceil(max n / 2)), a query block with n > C blocks becomes two
    items (its first C blocks, then the rest); items by decreasing cost, ties
    by 2 qb + chunk. Returns (C, [qb | chunk << 20 | (k - 1) << 22, ...])."""
    n = [int(x) for x in n]
    split_len = max(16, -(-max(n, default=0) // 2))
    items = []
    for qb, c in enumerate(n):
        if c > split_len:
            items.append((split_len, 2 * qb, qb | (1 << 22)))
            items.append((c - split_len, 2 * qb + 1, qb | (1 << 20) | (1 << 22)))
        else:
            items.append((c, 2 * qb, qb))
    items.sort(key=lambda it: (-it[0], it[1]))
    return split_len, [code for _, _, code in items]


def _mask_on_gpu(w: wl.Workload, dev, doc=None):
    doc = wl.make_doc(w) if doc is None else doc
    dt = torch.from_numpy(doc).to(dev) if doc is not None else None
    bm = bsa.create_block_mask(w.kind, w.L, w.S, window=w.window or None, document_id=dt, device=dev)
    return bm, doc


def _check_mask(bm, w: wl.Workload, doc, want=None):
    torch.cuda.synchronize()
    if want is None:
        want = oracle.block_mask(w.kind, w.L, w.S, w.window, doc)
    got = (bm.kv_num_blocks, bm.kv_indices, bm.full_kv_num_blocks, bm.full_kv_indices)
    for name, g, e in zip(("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                           "full_kv_indices"), got, want):
        g = g.cpu().numpy()
        assert g.shape == e.shape and np.array_equal(g, e), f"{w.name}: {name} differs"
    split_len, codes = expected_plan(want[0] + want[2])
    got = bm.schedule.cpu().numpy()
    count = int(got[0])
    assert count == len(codes) and got[1:4].tolist() == [split_len, 0, 0], f"{w.name}: plan header"
    desc = got[4:].reshape(-1, 4)
    assert desc[:count, 0].tolist() == codes, f"{w.name}: work plan order"
    assert (desc[count:] == -1).all(), f"{w.name}: unused plan entries"
    for code, nf, npart, first in desc[:count].tolist():
        qb, chunk, k = code & 0xFFFFF, (code >> 20) & 3, ((code >> 22) & 3) + 1
        assert (nf, npart) == (int(want[2][qb]), int(want[0][qb])), f"{w.name}: counts of {qb}"
        m0 = split_len if chunk == 1 else 0
        lists = list(want[3][qb][:nf]) + list(want[1][qb][:npart])
        if m0 < nf + npart:
            assert first == lists[m0], f"{w.name}: first block of item {code}"


def _odd(name, dtype, H, L, S, kind, window=0, bounds=(), softcap=0.0, B=1):
    return wl.Workload(name, B, H, L, S, 64, dtype, kind, window, bounds, softcap)


# (user-supplied masks have their own tests: test_custom_mask_gpu.py)
MASK_CASES = [w for w in wl.WORKLOADS.values() if w.kind != wl.MASK_CUSTOM] + [
    _odd("none_300x200", "bf16", 1, 300, 200, wl.MASK_NONE),
    _odd("causal_1000", "bf16", 1, 1000, 1000, wl.MASK_CAUSAL),
    _odd("causal_L200_S700", "bf16", 1, 200, 700, wl.MASK_CAUSAL),
    _odd("causal_L700_S200", "bf16", 1, 700, 200, wl.MASK_CAUSAL),
    _odd("sliding_w1", "bf16", 1, 1000, 1000, wl.MASK_SLIDING_WINDOW, 1),
    _odd("sliding_w_gt_S", "bf16", 1, 1000, 1000, wl.MASK_SLIDING_WINDOW, 5000),
    _odd("sliding_empty_rows", "bf16", 1, 400, 130, wl.MASK_SLIDING_WINDOW, 20),
    _odd("document_ragged", "f16", 1, 1000, 1000, wl.MASK_DOCUMENT, 0, (300, 777)),
    _odd("document_L_ne_S", "f16", 1, 600, 900, wl.MASK_DOCUMENT, 0, (130, 500)),
    _odd("none_zero_kv", "bf16", 1, 256, 0, wl.MASK_NONE),
    _odd("causal_lr_1000", "bf16", 1, 1000, 1000, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("causal_lr_L200_S700", "bf16", 1, 200, 700, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("causal_lr_L700_S200", "bf16", 1, 700, 200, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("causal_lr_L1_S1000", "bf16", 1, 1, 1000, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("sliding_lr_L300_S1000_w100", "bf16", 1, 300, 1000, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 100),
    _odd("sliding_lr_L1000_S300_w50", "bf16", 1, 1000, 300, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 50),
    _odd("document_bidir_ragged", "f16", 1, 1000, 1000, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (300, 777)),
    _odd("document_bidir_L_ne_S", "f16", 1, 600, 900, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (130, 500)),
    _odd("document_bidir_aligned", "f16", 1, 1024, 1024, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (256, 768)),
]


@pytest.mark.parametrize("w", MASK_CASES, ids=[w.name for w in MASK_CASES])
def test_block_mask_bit_exact(dev, w):
    bm, doc = _mask_on_gpu(w, dev)
    _check_mask(bm, w, doc)


@pytest.mark.parametrize("kind", [wl.MASK_DOCUMENT, wl.MASK_DOCUMENT_BIDIRECTIONAL])
def test_block_mask_unsorted_document_ids(dev, kind):
    w = _odd("document_random_ids", "bf16", 1, 777, 777, kind)
    doc = np.random.default_rng(4).integers(0, 3, size=777).astype(np.int32)
    bm, _ = _mask_on_gpu(w, dev, doc)
    _check_mask(bm, w, doc)


def _expand_kv(w: wl.Workload, x: torch.Tensor) -> torch.Tensor:
    """K or V with each K/V head repeated for its H / H_kv query heads: the
    definition of grouped-query attention, for the oracle."""
    return x.repeat_interleave(w.H // w.kv_heads, dim=1) if w.kv_heads != w.H else x


def _run(w: wl.Workload, dev, seed=0, doc=None, qkv=None):
    q, k, v = wl.make_qkv(w, seed) if qkv is None else qkv
    bm, doc = _mask_on_gpu(w, dev, doc)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o, lse = bsa.attention(qd, kd, vd, bm, score_mod="softcap" if w.softcap else None,
                           softcap=w.softcap or 30.0, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    return (q, k, v), doc, o, lse


def _compare(w, got_o, got_lse, want_o, want_lse, what):
    tmax, tmean, tlse = TOL[w.dtype]
    got_o = got_o.astype(np.float64)
    err = np.abs(got_o - want_o)
    assert np.isfinite(got_o).all(), f"{what}: non-finite output"
    assert err.max() <= tmax, f"{what}: max-abs {err.max():.3g} > {tmax}"
    assert err.mean() <= tmean, f"{what}: mean-abs {err.mean():.3g} > {tmean}"
    empty = np.isneginf(want_lse)
    assert np.array_equal(np.isneginf(got_lse), empty), f"{what}: empty-row pattern"
    if (~empty).any():
        lerr = np.abs(got_lse[~empty] - want_lse[~empty])
        assert lerr.max() <= tlse, f"{what}: lse max-abs {lerr.max():.3g} > {tlse}"
    assert np.all(got_o[empty] == 0.0), f"{what}: empty rows must be zero"


SMALL = [
    wl.WORKLOADS["causal_256_f32"],
    _odd("causal_1024_bf16", "bf16", 2, 1024, 1024, wl.MASK_CAUSAL),
    _odd("causal_1024_f16", "f16", 2, 1024, 1024, wl.MASK_CAUSAL),
    _odd("sliding_w64_1024_bf16", "bf16", 2, 1024, 1024, wl.MASK_SLIDING_WINDOW, 64),
    _odd("sliding_w256_2048_bf16", "bf16", 1, 2048, 2048, wl.MASK_SLIDING_WINDOW, 256),
    _odd("sliding_w200_1000_f16", "f16", 2, 1000, 1000, wl.MASK_SLIDING_WINDOW, 200),
    _odd("document_softcap_1000_f16", "f16", 2, 1000, 1000, wl.MASK_DOCUMENT, 0, (300, 777), 30.0),
    _odd("document_softcap_1024_bf16", "bf16", 1, 1024, 1024, wl.MASK_DOCUMENT, 0, (256, 700), 30.0),
    _odd("none_300x200_bf16", "bf16", 2, 300, 200, wl.MASK_NONE),
    _odd("none_300x200_f32_softcap", "f32", 1, 300, 200, wl.MASK_NONE, 0, (), 5.0),
    _odd("causal_L700_S200_f16", "f16", 1, 700, 200, wl.MASK_CAUSAL),
    _odd("causal_L200_S700_bf16", "bf16", 1, 200, 700, wl.MASK_CAUSAL),
    _odd("sliding_empty_rows_bf16", "bf16", 1, 400, 130, wl.MASK_SLIDING_WINDOW, 20),
    _odd("sliding_w7_f32", "f32", 2, 333, 333, wl.MASK_SLIDING_WINDOW, 7),
    _odd("document_f32", "f32", 1, 512, 512, wl.MASK_DOCUMENT, 0, (100, 300)),
    _odd("causal_B2H3_bf16", "bf16", 3, 256, 256, wl.MASK_CAUSAL, B=2),
    _odd("none_zero_kv_bf16", "bf16", 1, 256, 0, wl.MASK_NONE),
    # 34 query blocks: blocks with more than 17 live kv blocks run as two
    # chunks merged through the workspace
    _odd("causal_4352_bf16_split", "bf16", 1, 4352, 4352, wl.MASK_CAUSAL),
    _odd("document_4400_f16_split", "f16", 1, 4400, 4400, wl.MASK_DOCUMENT, 0, (600, 2500), 30.0),
    _odd("none_3000x4300_bf16_split", "bf16", 1, 3000, 4300, wl.MASK_NONE),
    # 34 query blocks x 16 heads: the plan's two-way split (fewer heads split
    # the kv range instead, below)
    _odd("causal_4352_h16_bf16_plan_split", "bf16", 16, 4352, 4352, wl.MASK_CAUSAL),
    # decode and other few-query-block shapes: split-KV chunks and their merge
    _odd("decode_L1_S8192_lr_bf16", "bf16", 8, 1, 8192, wl.MASK_CAUSAL_LOWER_RIGHT, B=2),
    _odd("decode_L16_S5000_lr_f16", "f16", 4, 16, 5000, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("decode_L64_S3000_none_bf16", "bf16", 2, 64, 3000, wl.MASK_NONE, B=3),
    _odd("decode_L1_S9000_window_bf16", "bf16", 4, 1, 9000, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 1000),
    _odd("decode_L3_S4000_doc_softcap_f16", "f16", 2, 3, 4000, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0,
         (1000, 3500), 30.0),
    _odd("decode_gqa_L1_S6000_bf16", "bf16", 16, 1, 6000, wl.MASK_CAUSAL_LOWER_RIGHT, B=2).with_(H_kv=4),
    _odd("causal_2000_h1_bf16_kv_split", "bf16", 1, 2000, 2000, wl.MASK_CAUSAL),
    # packed rows (L x G <= 32 query rows per K/V head in one tile): exactly
    # 32 rows, a group of 5, one chunk per item (many K/V heads; few kv
    # blocks), top-left causal at L = 1, no keys at all, document masks
    _odd("packed_L4_G8_R32_lr_bf16", "bf16", 16, 4, 3000, wl.MASK_CAUSAL_LOWER_RIGHT, B=2).with_(H_kv=2),
    _odd("packed_L6_G5_R30_window_f16", "f16", 10, 6, 2500, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT,
         300).with_(H_kv=2),
    _odd("packed_L32_G1_none_bf16", "bf16", 2, 32, 1500, wl.MASK_NONE, B=2),
    _odd("packed_direct_1024_heads_bf16", "bf16", 128, 1, 700, wl.MASK_CAUSAL_LOWER_RIGHT, B=8),
    _odd("packed_direct_S200_softcap_f16", "f16", 8, 2, 200, wl.MASK_NONE, 0, (), 20.0).with_(H_kv=2),
    _odd("packed_causal_top_left_L1_S700_bf16", "bf16", 4, 1, 700, wl.MASK_CAUSAL, B=2),
    _odd("packed_L1_S0_bf16", "bf16", 4, 1, 0, wl.MASK_NONE),
    # 64 chunks, the most either merge takes: packed rows, and split-KV
    _odd("packed_64_chunks_L1_S17000_bf16", "bf16", 1, 1, 17000, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("kv_split_64_chunks_L100_S17000_f16", "f16", 1, 100, 17000, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("packed_doc_L8_S2000_f16", "f16", 4, 8, 2000, wl.MASK_DOCUMENT, 0, (5, 700, 1500)).with_(H_kv=1),
    _odd("packed_doc_bidir_L2_S3000_softcap_bf16", "bf16", 8, 2, 3000, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0,
         (1, 1200), 30.0).with_(H_kv=4),
    # chained items (sliding windows with >= 1024 work items): query blocks
    # with no key at all, B*H not dividing the 512-workgroup grid, B*H above
    # it, fp16 with the soft-cap and a ragged last block
    _odd("chain_sliding_lr_empty_blocks_bf16", "bf16", 64, 2176, 1000, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 100),
    _odd("chain_sliding_h12_ragged_softcap_f16", "f16", 12, 11000, 11000, wl.MASK_SLIDING_WINDOW, 300, (),
         20.0),
    _odd("chain_sliding_bh520_bf16", "bf16", 130, 256, 256, wl.MASK_SLIDING_WINDOW, 64, B=4),
    _odd("chain_sliding_w1920_bf16", "bf16", 8, 16384, 16384, wl.MASK_SLIDING_WINDOW, 1920),
    # mask variants and grouped-query attention
    _odd("causal_lr_L200_S700_bf16", "bf16", 2, 200, 700, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("causal_lr_L700_S200_f16", "f16", 1, 700, 200, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("causal_lr_L1_S900_bf16", "bf16", 2, 1, 900, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("causal_lr_L333_S999_f32", "f32", 1, 333, 999, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("causal_lr_2048x4352_bf16_split", "bf16", 1, 2048, 4352, wl.MASK_CAUSAL_LOWER_RIGHT),
    _odd("sliding_lr_L300_S1000_w100_bf16", "bf16", 2, 300, 1000,
         wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 100),
    _odd("sliding_lr_L1000_S300_w50_f16", "f16", 1, 1000, 300, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 50),
    _odd("sliding_lr_f32", "f32", 1, 200, 500, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 33),
    _odd("document_bidir_softcap_1000_f16", "f16", 2, 1000, 1000, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0,
         (300, 777), 30.0),
    _odd("document_bidir_600x900_bf16", "bf16", 1, 600, 900, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0,
         (130, 500)),
    _odd("document_bidir_f32", "f32", 1, 512, 512, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (100, 300)),
    _odd("document_bidir_4400_f16_split", "f16", 1, 4400, 4400, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0,
         (600, 2500), 30.0),
    _odd("gqa_causal_h4_kv2_bf16", "bf16", 4, 640, 640, wl.MASK_CAUSAL).with_(H_kv=2),
    _odd("gqa_sliding_h6_kv1_f16", "f16", 6, 700, 700, wl.MASK_SLIDING_WINDOW, 90).with_(H_kv=1),
    _odd("gqa_document_h4_kv4_bf16", "bf16", 4, 500, 500, wl.MASK_DOCUMENT, 0, (200,)).with_(H_kv=4),
    _odd("gqa_none_h4_kv2_f32", "f32", 4, 300, 200, wl.MASK_NONE).with_(H_kv=2),
    _odd("gqa_causal_lr_B2_h8_kv2_bf16", "bf16", 8, 256, 768, wl.MASK_CAUSAL_LOWER_RIGHT,
         B=2).with_(H_kv=2),
    # B*H a multiple of 8 with grouped heads (the XCD head order) and split
    # query blocks merging by their (batch, head) slot
    _odd("gqa_causal_split_B2_h8_kv2_2304_bf16", "bf16", 8, 2304, 2304, wl.MASK_CAUSAL, B=2).with_(H_kv=2),
    # fp32 at the decode and many-block shapes (fp32 never splits, packs or
    # chains: one item per query block), and with no keys
    _odd("decode_gqa_L1_S3000_lr_f32", "f32", 8, 1, 3000, wl.MASK_CAUSAL_LOWER_RIGHT).with_(H_kv=2),
    _odd("sliding_w100_2500_h4_ragged_f32", "f32", 4, 2500, 2500, wl.MASK_SLIDING_WINDOW, 100),
    _odd("none_zero_kv_f32", "f32", 1, 130, 0, wl.MASK_NONE),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_forward_small_full_compare(dev, w):
    (q, k, v), doc, o, lse = _run(w, dev)
    k, v = _expand_kv(w, k), _expand_kv(w, v)
    want_o, want_lse = oracle.attention(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), w.kind, w.scale, w.window, doc,
                                        w.softcap)
    _compare(w, o.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), want_o, want_lse,
             w.name)


FULL = [wl.WORKLOADS[n] for n in ("causal_8192_bf16", "sliding_8192_w64_bf16",
                                  "sliding_8192_w256_bf16", "sliding_8192_w1024_bf16",
                                  "sliding_8192_w4096_bf16", "sliding_32768_w256_bf16",
                                  "document_8192_f16_softcap", "causal_lower_right_2048x8192_bf16",
                                  "gqa_causal_8192_h32_kv8_bf16",
                                  "document_bidirectional_8192_f16_softcap",
                                  "decode_gqa_b8_h32_kv8_s8192_bf16")]


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_forward_full_size_every_row(dev, w):
    """The benchmark's workloads at full size, in the launch configuration
    the benchmark times, compared with the oracle on every element of O and
    every row's logsumexp (the oracle takes seconds: 2-17 s on 16 threads)."""
    print(f"full-size parity: {w.name} B={w.B} H={w.H} L={w.L} S={w.S} {w.dtype}", flush=True)
    (q, k, v), doc, o, lse = _run(w, dev)
    k, v = _expand_kv(w, k), _expand_kv(w, v)
    got_o = o.float().cpu().numpy()
    got_lse = lse.cpu().numpy().astype(np.float64)
    want_o, want_lse = oracle.attention(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), w.kind, w.scale, w.window, doc,
                                        w.softcap)
    err = np.abs(got_o.astype(np.float64) - want_o)
    live = ~np.isneginf(want_lse)
    lerr = np.abs(got_lse[live] - want_lse[live])
    print(f"full-size parity: {w.name} rows {want_lse.size} O max-abs {err.max():.3g} "
          f"mean-abs {err.mean():.3g} lse max-abs {lerr.max():.3g}", flush=True)
    _compare(w, got_o, got_lse, want_o, want_lse, w.name)
    assert live.all()  # no empty rows in these workloads


# Key padding: (workload, per-batch kept key ranges [start, end); None = 0 / S)
PADDED = [
    (_odd("pad_causal_700_bf16", "bf16", 2, 700, 700, wl.MASK_CAUSAL, B=3),
     ([0, 100, 300], [700, 650, 300])),                 # none, both ends, empty
    (_odd("pad_sliding_900_f16_right", "f16", 2, 900, 900, wl.MASK_SLIDING_WINDOW, 150, B=2),
     (None, [900, 517])),
    (_odd("pad_document_softcap_800_bf16_left", "bf16", 1, 800, 800, wl.MASK_DOCUMENT, 0, (250, 600),
          30.0, B=2), ([3, 129], None)),
    (_odd("pad_none_300x500_f32", "f32", 2, 300, 500, wl.MASK_NONE, B=2), ([10, 0], [400, 128])),
    (_odd("pad_causal_4352_bf16_split", "bf16", 1, 4352, 4352, wl.MASK_CAUSAL, B=2),
     ([0, 1000], [3000, 4352])),
    (_odd("pad_gqa_causal_lr_bf16", "bf16", 4, 256, 900, wl.MASK_CAUSAL_LOWER_RIGHT, B=2).with_(H_kv=2),
     ([128, 0], [900, 700])),
    (_odd("pad_bidir_doc_f16", "f16", 2, 640, 640, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (200, 500), B=2),
     ([64, 0], [640, 300])),
    (_odd("pad_decode_L1_S7000_bf16", "bf16", 4, 1, 7000, wl.MASK_CAUSAL_LOWER_RIGHT, B=3),
     ([0, 2500, 0], [7000, 6000, 900])),
    (_odd("pad_packed_gqa_L2_S5000_bf16", "bf16", 8, 2, 5000, wl.MASK_CAUSAL_LOWER_RIGHT, B=3).with_(H_kv=2),
     ([0, 1000, 4999], [5000, 3333, 5000])),
    (_odd("pad_packed_window_L1_f16", "f16", 4, 1, 4000, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 700, B=2),
     ([3500, 0], [4000, 2000])),
]


def _run_padded(w, ranges, dev):
    starts, ends = ranges
    q, k, v = wl.make_qkv(w, 8)
    bm, doc = _mask_on_gpu(w, dev)
    ks = None if starts is None else torch.tensor(starts, dtype=torch.int32, device=dev)
    ke = None if ends is None else torch.tensor(ends, dtype=torch.int32, device=dev)
    o, lse = bsa.attention(q.to(dev), k.to(dev), v.to(dev), bm,
                           score_mod="softcap" if w.softcap else None, softcap=w.softcap or 30.0,
                           scale=w.scale, return_lse=True, key_start=ks, key_end=ke)
    torch.cuda.synchronize()
    return (q, k, v), doc, o, lse


@pytest.mark.parametrize("w,ranges", PADDED, ids=[c[0].name for c in PADDED])
def test_forward_key_padding(dev, w, ranges):
    (q, k, v), doc, o, lse = _run_padded(w, ranges, dev)
    starts, ends = ranges
    want_o, want_lse = oracle.attention(q.double().numpy(), _expand_kv(w, k).double().numpy(),
                                        _expand_kv(w, v).double().numpy(), w.kind, w.scale,
                                        w.window, doc, w.softcap, key_start=starts, key_end=ends)
    _compare(w, o.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), want_o, want_lse,
             w.name)


def test_key_padding_full_size_every_row(dev):
    """The benchmark's padded workload (B=2, H=8, causal 8192, entry 1 keeps
    keys [2048, 7168)), in its launch configuration, on every row."""
    w = wl.WORKLOADS["causal_8192_keypad_b2_bf16"]
    ranges = ([a for a, _ in w.key_ranges], [b for _, b in w.key_ranges])
    (q, k, v), doc, o, lse = _run_padded(w, ranges, dev)
    want_o, want_lse = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                        w.kind, w.scale, key_start=ranges[0], key_end=ranges[1])
    _compare(w, o.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), want_o, want_lse,
             w.name)


def _half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output type at |x| (normal range)."""
    bits = {"bf16": 8, "f16": 11, "f32": 24}[dtype]
    ax = np.maximum(np.abs(x), np.finfo(np.float64).tiny)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(int) - bits)


FEW_KEYS = [
    # rows that keep one to three keys: O is a mix of one or two V rows and
    # can exceed 4 in magnitude, where half an ulp of bf16 (2^-6) is above
    # the 1e-2 bound that holds for rows averaging many keys
    (_odd("few_keys_S4_pad_bf16", "bf16", 4, 485, 4, wl.MASK_NONE, B=3), ([3, 2, 0], [4, 4, 1])),
    (_odd("few_keys_window2_bf16", "bf16", 8, 900, 900, wl.MASK_SLIDING_WINDOW, 2), None),
    (_odd("few_keys_window3_f16", "f16", 8, 900, 900, wl.MASK_SLIDING_WINDOW, 3), None),
]


@pytest.mark.parametrize("w,ranges", FEW_KEYS, ids=[c[0].name for c in FEW_KEYS])
def test_few_key_rows_within_output_rounding(dev, w, ranges):
    """Rows with one to three live keys: every element of O within 1e-2 plus
    half an ulp of the output type at the reference value (the rounding of O
    itself), the mean error within 1e-3 plus the mean of that half ulp, the
    logsumexp within the usual bound."""
    if ranges is None:
        (q, k, v), doc, o, lse = _run(w, dev, seed=5)
        starts = ends = None
    else:
        (q, k, v), doc, o, lse = _run_padded(w, ranges, dev)
        starts, ends = ranges
    want_o, want_lse = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                        w.kind, w.scale, w.window, doc, w.softcap,
                                        key_start=starts, key_end=ends)
    got_o = o.float().cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    err = np.abs(got_o - want_o)
    bound = TOL[w.dtype][0] + _half_ulp(want_o, w.dtype)
    print(f"{w.name}: max |O| {np.abs(want_o).max():.3g} max-abs {err.max():.3g} "
          f"worst err - bound {(err - bound).max():.3g}", flush=True)
    assert np.all(err <= bound), f"{w.name}: error above 1e-2 + half an ulp"
    assert err.mean() <= TOL[w.dtype][1] + _half_ulp(want_o, w.dtype).mean()
    empty = np.isneginf(want_lse)
    assert np.array_equal(np.isneginf(got_lse), empty)
    assert np.all(got_o[empty] == 0.0)
    if (~empty).any():
        assert np.abs(got_lse[~empty] - want_lse[~empty]).max() <= TOL[w.dtype][2]


def test_key_padding_whole_range_matches_unpadded(dev):
    """Ranges covering every key run the padded kernel with nothing to drop:
    bit-identical to the unpadded kernel."""
    w = _odd("pad_full_range_bf16", "bf16", 2, 1000, 1000, wl.MASK_SLIDING_WINDOW, 300, B=2)
    (q, k, v), _, o_pad, l_pad = _run_padded(w, ([0, 0], [1000, 1000]), dev)
    bm, _ = _mask_on_gpu(w, dev)
    o, l = bsa.attention(q.to(dev), k.to(dev), v.to(dev), bm, scale=w.scale, return_lse=True)
    assert torch.equal(o, o_pad) and torch.equal(l, l_pad)


def test_window_one_is_identity_bit_exact(dev):
    w = _odd("sliding_w1_bf16", "bf16", 2, 1000, 1000, wl.MASK_SLIDING_WINDOW, 1)
    (q, k, v), _, o, lse = _run(w, dev)
    assert torch.equal(o.cpu(), v)
    want = (q.double() * k.double()).sum(-1) * w.scale
    assert (lse.cpu().double() - want).abs().max().item() <= 1e-5


def test_uniform_v_gives_that_row(dev):
    w = _odd("doc_uniform_v_f16", "f16", 2, 1000, 1000, wl.MASK_DOCUMENT, 0, (300, 777), 30.0)
    q, k, v = wl.make_qkv(w, 1)
    v = v[:, :, :1, :].expand_as(v).contiguous()
    _, _, o, _ = _run(w, dev, qkv=(q, k, v))
    err = (o.cpu().float() - v.float()).abs().max().item()
    assert err <= 1e-2


def test_deterministic_repeat(dev):
    w = wl.WORKLOADS["causal_8192_bf16"]
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 2))
    bm = bsa.create_block_mask(w.kind, w.L, w.S, device=dev)
    o1, l1 = bsa.attention(q, k, v, bm, return_lse=True)
    for _ in range(3):
        o2, l2 = bsa.attention(q, k, v, bm, return_lse=True)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_workspace_is_left_clean(dev):
    """Split items leave the workspace's ticket counters at zero, so an
    explicit zero-filled workspace, reused, gives the cached one's results."""
    w = wl.WORKLOADS["causal_8192_bf16"]
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 5))
    bm = bsa.create_block_mask(w.kind, w.L, w.S, device=dev)
    need = bsa.workspace_size(q, bm)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    ref = bsa.attention(q, k, v, bm)
    for _ in range(3):
        got = bsa.attention(q, k, v, bm, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert int(ws[:2048 * 4].count_nonzero()) == 0  # the ticket counters


def test_workspace_shared_by_calls_of_different_shapes(dev):
    """One zero-filled workspace serves split calls whose (B*H, query blocks)
    differ: a call with more heads than the one before must not read the
    earlier call's partial results as its ticket counters."""
    small = _odd("causal_4352_h4_bf16", "bf16", 4, 4352, 4352, wl.MASK_CAUSAL)
    big = _odd("causal_4352_h32_bf16", "bf16", 32, 4352, 4352, wl.MASK_CAUSAL)
    bm = bsa.create_block_mask(wl.MASK_CAUSAL, 4352, 4352, device=dev)
    qs, ks, vs = (x.to(dev) for x in wl.make_qkv(small, 6))
    qb, kb, vb = (x.to(dev) for x in wl.make_qkv(big, 7))
    need = max(bsa.workspace_size(qs, bm), bsa.workspace_size(qb, bm))
    fresh = torch.zeros(bsa.workspace_size(qb, bm), dtype=torch.uint8, device=dev)
    ref = bsa.attention(qb, kb, vb, bm, workspace=fresh)
    shared = torch.zeros(need, dtype=torch.uint8, device=dev)
    for _ in range(2):
        bsa.attention(qs, ks, vs, bm, workspace=shared)
        got = bsa.attention(qb, kb, vb, bm, workspace=shared)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert int(shared[:2048 * 4].count_nonzero()) == 0


def test_packed_merge_deterministic_and_clean(dev):
    """Packed decode items cut into chunks (4 and 32 chunks here) and merged:
    the same bits on every call, the workspace's ticket counters left at
    zero, and one workspace shared by shapes with other chunk counts gives
    each call's own results."""
    dec = wl.WORKLOADS["decode_gqa_b8_h32_kv8_s8192_bf16"]
    long = _odd("decode_b1_h32_kv8_s65536_bf16", "bf16", 32, 1, 65536, wl.MASK_CAUSAL_LOWER_RIGHT).with_(H_kv=8)
    runs = []
    for w, seed in ((dec, 8), (long, 9)):
        q, k, v = (x.to(dev) for x in wl.make_qkv(w, seed))
        bm = bsa.create_block_mask(w.kind, w.L, w.S, device=dev)
        runs.append((q, k, v, bm, bsa.workspace_size(q, bm)))
    refs = [bsa.attention(q, k, v, bm, workspace=torch.zeros(n, dtype=torch.uint8, device=dev), return_lse=True)
            for q, k, v, bm, n in runs]
    shared = torch.zeros(max(r[4] for r in runs), dtype=torch.uint8, device=dev)
    for _ in range(3):
        for (q, k, v, bm, _), (o_ref, l_ref) in zip(runs, refs):
            o, lse = bsa.attention(q, k, v, bm, workspace=shared, return_lse=True)
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
            assert int(shared[:2048 * 4].count_nonzero()) == 0


def test_more_query_blocks_than_the_lds_plan_holds(dev):
    """4100 query blocks (L = S = 524800, window 256): past the 4096 rows the
    parallel plan keeps in LDS, the plan is ranked by the fallback kernel.
    A causal window's block lists are the same in every row past the first
    few, shifted by the row index, so each row is checked against the
    oracle's lists of a 16-block case (rows up to 15 as they are, later rows
    as row 15 shifted); then the plan, and sampled rows of O."""
    nq = 4100
    w = _odd("sliding_w256_524800_bf16", "bf16", 1, nq * 128, nq * 128, wl.MASK_SLIDING_WINDOW, 256)
    small = oracle.block_mask(w.kind, 16 * 128, 16 * 128, w.window, None)
    want = [np.zeros((nq,), np.int32), np.zeros((nq, nq), np.int32),
            np.zeros((nq,), np.int32), np.zeros((nq, nq), np.int32)]
    for qb in range(nq):
        r = min(qb, 15)
        for cnt, lst in ((0, 1), (2, 3)):
            n = int(small[cnt][r])
            want[cnt][qb] = n
            want[lst][qb, :n] = small[lst][r, :n] + (qb - r)
    bm, _ = _mask_on_gpu(w, dev)
    _check_mask(bm, w, None, want=want)
    (q, k, v), _, o, lse = _run(w, dev, qkv=wl.make_qkv(w, 3))
    # the first and last rows, the rows around the 4096th query block, and
    # rows drawn uniformly (a few seconds of the oracle)
    rows = np.unique(np.concatenate([[0, 127, 128, w.L - 1], 4096 * 128 + np.arange(-2, 2),
                                     np.random.default_rng(5).integers(0, w.L, 40)])).astype(np.int64)
    want_o, want_lse = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                        w.kind, w.scale, w.window, None, 0.0, rows=rows)
    got = o.float().reshape(-1, w.E)[torch.from_numpy(rows).to(dev)].cpu().numpy()
    got_lse = lse.reshape(-1)[torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
    _compare(w, got, got_lse, want_o, want_lse, w.name)


def test_many_heads_without_split_every_row(dev):
    """B*H*nq above 2048: long query blocks are not split."""
    w = _odd("causal_8192_h33_bf16", "bf16", 33, 8192, 8192, wl.MASK_CAUSAL)
    (q, k, v), doc, o, lse = _run(w, dev)
    want_o, want_lse = oracle.attention(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), w.kind, w.scale, w.window, doc,
                                        w.softcap)
    _compare(w, o.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), want_o, want_lse,
             w.name)


def test_strided_inputs_match_contiguous(dev):
    """q/k/v as [B, H, S, E] views of [B, S, H, E] storage."""
    w = _odd("causal_strided", "bf16", 4, 640, 640, wl.MASK_CAUSAL, B=2)
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 3))
    bm = bsa.create_block_mask(w.kind, w.L, w.S, device=dev)
    ref = bsa.attention(q, k, v, bm)
    qs, ks, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    assert qs.stride(2) != 64
    out = torch.empty(2, 640, 4, 64, dtype=torch.bfloat16, device=dev).transpose(1, 2)
    got = bsa.attention(qs, ks, vs, bm, out=out)
    assert torch.equal(got, ref)


def test_lse_optional_and_mask_reuse(dev):
    w = _odd("reuse", "bf16", 2, 512, 512, wl.MASK_SLIDING_WINDOW, 100)
    bm = bsa.create_block_mask(w.kind, w.L, w.S, window=w.window, device=dev)
    for seed in (0, 1):
        q, k, v = (x.to(dev) for x in wl.make_qkv(w, seed))
        o1 = bsa.attention(q, k, v, bm)
        o2, _ = bsa.attention(q, k, v, bm, return_lse=True)
        assert torch.equal(o1, o2)


def test_errors_raise(dev):
    q = torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16, device=dev)
    bm = bsa.create_block_mask("causal", 128, 128, device=dev)
    with pytest.raises(bsa.BsattnError):
        bsa.attention(q, q, q, bm)  # mask built for other lengths
    q128 = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(bsa.BsattnError):
        bsa.attention(q128, q128, q128, bm)  # head dim 128 has no kernel


def _force_all_partial(bm):
    """Rewrite a built BlockMask so that every live block (full or partial)
    is listed as partial, ascending, with the work plan rebuilt in the same
    format (same split length, same order rule). Full blocks then run the
    partial-block path: per-tile classes and, where a tile is not known to
    be all live, the per-pair test."""
    torch.cuda.synchronize()
    nf = bm.full_kv_num_blocks.cpu().numpy()
    npart = bm.kv_num_blocks.cpu().numpy()
    fi = bm.full_kv_indices.cpu().numpy()
    pi = bm.kv_indices.cpu().numpy()
    nq, nk = pi.shape
    lists = [sorted(list(fi[qb, :nf[qb]]) + list(pi[qb, :npart[qb]])) for qb in range(nq)]
    n = np.array([len(x) for x in lists], dtype=np.int32)
    idx = np.zeros((nq, nk), dtype=np.int32)
    for qb, x in enumerate(lists):
        idx[qb, :len(x)] = x
    split_len, codes = expected_plan(n)
    sched = np.full(bm.schedule.numel(), -1, dtype=np.int32)
    sched[:4] = [len(codes), split_len, 0, 0]
    for r, code in enumerate(codes):
        qb, chunk = code & 0xFFFFF, (code >> 20) & 3
        m0 = split_len if chunk == 1 else 0
        sched[4 + 4 * r: 8 + 4 * r] = [code, 0, n[qb], lists[qb][m0] if m0 < n[qb] else 0]
    bm.kv_num_blocks.copy_(torch.from_numpy(n))
    bm.kv_indices.copy_(torch.from_numpy(idx))
    bm.full_kv_num_blocks.zero_()
    bm.full_kv_indices.zero_()
    bm.schedule.copy_(torch.from_numpy(sched))
    torch.cuda.synchronize()
    return bm


FORCED = [_odd("forced_causal_4352_bf16", "bf16", 2, 4352, 4352, wl.MASK_CAUSAL),
          _odd("forced_causal_2048_f16", "f16", 3, 2048, 2048, wl.MASK_CAUSAL),
          wl.WORKLOADS["causal_8192_bf16"]]


@pytest.mark.parametrize("w", FORCED, ids=[w.name for w in FORCED])
def test_forced_partial_path_bit_identical(dev, w):
    """An always-true pair test through the partial-block path gives the full
    path's bits ("FlexAttention on Apple Silicon: block masks", closing
    section: only the handling of partly live blocks differs, not the
    values). With every block forced partial, the same causal attention runs
    three ways beside the normal BlockMask: a single document (the document
    rule evaluates every pair of every tile it cannot rule out, and each such
    pair of a below-diagonal block is live), the causal mask as user bits
    (tiles whose words are all ones), and the causal rule itself (below the
    diagonal every tile classifies as live). The visit order (ascending kv
    blocks) and the split points are those of the causal plan, so every
    floating-point operation on a live score is the same."""
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 4))
    bm = bsa.create_block_mask("causal", w.L, w.S, device=dev)
    o_ref, l_ref = bsa.attention(q, k, v, bm, scale=w.scale, return_lse=True)
    one_doc = torch.zeros(w.S, dtype=torch.int32, device=dev)
    masks = {
        "document": bsa.create_block_mask("document", w.L, w.S, document_id=one_doc, device=dev),
        "custom": bsa.create_block_mask_from_dense(
            torch.ones(w.L, w.S, dtype=torch.bool, device=dev).tril_()),
        "causal": bsa.create_block_mask("causal", w.L, w.S, device=dev),
    }
    for name, m in masks.items():
        _force_all_partial(m)
        assert int(m.full_kv_num_blocks.sum()) == 0
        o, l = bsa.attention(q, k, v, m, scale=w.scale, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"{w.name}: O through the forced partial path ({name})"
        assert torch.equal(l, l_ref), f"{w.name}: lse through the forced partial path ({name})"
