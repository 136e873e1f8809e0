"""GPU parity for user-supplied masks (BlockMask kind CUSTOM), through the C ABI.

* The GPU bit packing and the BlockMask built from the bits are bit-exact
  against the oracle's packing and brute-force block classification.
* The forward under a dense mask is within the rule kinds' tolerances of the
  fp64 oracle (bf16/fp16/fp32; soft-cap, grouped heads, key padding, empty
  rows, the packed-row decode path, split-KV and the plan's split items).
* A rule written out as a dense mask runs bit-identically to the rule's own
  kind (only the pair test differs, never the arithmetic).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_35_amd as bsa
import oracle
import workloads as wl
from test_parity_gpu import TOL, _compare, _expand_kv, expected_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _band(L, S, lo, hi):
    """Input mask: True where lo <= i - j <= hi."""
    d = np.arange(L)[:, None] - np.arange(S)[None, :]
    return (d >= lo) & (d <= hi)


def _random(L, S, p, seed):
    return np.random.default_rng(seed).random((L, S)) < p


def _with_empty_rows(m, rows):
    m = m.copy()
    m[rows] = False
    return m


PACK_SHAPES = [(1, 1), (3, 127), (5, 128), (7, 129), (33, 1000), (200, 4100), (2, 0), (0, 5)]


@pytest.mark.parametrize("L,S", PACK_SHAPES, ids=[f"{a}x{b}" for a, b in PACK_SHAPES])
def test_pack_mask_bit_exact(dev, L, S):
    m = _random(L, S, 0.37, L * 1000 + S)
    got = bsa.pack_mask(torch.from_numpy(m).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), oracle.pack_mask(m))


def test_pack_mask_strided_rows(dev):
    big = _random(50, 700, 0.5, 3)
    view = torch.from_numpy(big).to(dev)[:, 13:613]  # row stride 700 bytes, offset 13
    got = bsa.pack_mask(view)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), oracle.pack_mask(big[:, 13:613]))


MASKS = [
    ("blocks_1000", wl.block_structured_mask(1000, 1000, 1, 0.2, 0.3, 0.5)),
    ("blocks_ragged_700x1300", wl.block_structured_mask(700, 1300, 2, 0.3, 0.3, 0.2)),
    ("random_5pct_300x500", _random(300, 500, 0.05, 4)),
    ("all_true_640x384", np.ones((640, 384), bool)),
    ("all_true_ragged_200x300", np.ones((200, 300), bool)),
    ("all_false_256x256", np.zeros((256, 256), bool)),
    ("causal_dense_4352", _band(4352, 4352, 0, 4352)),
    ("one_row_1x900", _random(1, 900, 0.3, 5)),
]


def _check_bm(bm, m):
    torch.cuda.synchronize()
    L, S = m.shape
    want = oracle.block_mask(oracle.DENSE, L, S, mask=m)
    got = (bm.kv_num_blocks, bm.kv_indices, bm.full_kv_num_blocks, bm.full_kv_indices)
    for name, g, e in zip(("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices"),
                          got, want):
        g = g.cpu().numpy()
        assert g.shape == e.shape and np.array_equal(g, e), name
    split_len, codes = expected_plan(want[0] + want[2])
    plan = bm.schedule.cpu().numpy()
    assert plan[0] == len(codes) and plan[1] == split_len
    assert np.array_equal(plan[4:4 + 4 * len(codes):4], np.array(codes, np.int32))


@pytest.mark.parametrize("name,m", MASKS, ids=[n for n, _ in MASKS])
def test_block_mask_from_dense_bit_exact(dev, name, m):
    _check_bm(bsa.create_block_mask_from_dense(torch.from_numpy(m).to(dev)), m)


def _run(w, m, dev, seed=0, ranges=None):
    q, k, v = wl.make_qkv(w, seed)
    bm = bsa.create_block_mask_from_dense(torch.from_numpy(m).to(dev))
    ks = ke = None
    if ranges is not None:
        ks = torch.tensor(ranges[0], dtype=torch.int32, device=dev)
        ke = torch.tensor(ranges[1], dtype=torch.int32, device=dev)
    o, lse = bsa.attention(q.to(dev), k.to(dev), v.to(dev), bm,
                           score_mod="softcap" if w.softcap else None, softcap=w.softcap or 30.0,
                           scale=w.scale, return_lse=True, key_start=ks, key_end=ke)
    torch.cuda.synchronize()
    return (q, k, v), o, lse


def _w(name, dtype, B, H, L, S, softcap=0.0, H_kv=0):
    return wl.Workload(name, B, H, L, S, 64, dtype, wl.MASK_CUSTOM, softcap=softcap, H_kv=H_kv)


FORWARD = [
    (_w("blocks_1000_bf16", "bf16", 2, 3, 1000, 1000), MASKS[0][1], None),
    (_w("ragged_gqa_softcap_f16", "f16", 1, 4, 700, 1300, 30.0, H_kv=2), MASKS[1][1], None),
    (_w("random_5pct_f32", "f32", 1, 2, 300, 500), MASKS[2][1], None),
    (_w("empty_rows_bf16", "bf16", 1, 2, 640, 384),
     _with_empty_rows(wl.block_structured_mask(640, 384, 6, 0.3, 0.4, 0.3), [0, 5, 200, 639]), None),
    (_w("decode_packed_gqa_bf16", "bf16", 3, 8, 2, 3000, H_kv=2), _random(2, 3000, 0.2, 7), None),
    (_w("decode_packed_mha_f16", "f16", 1, 4, 1, 5000), _random(1, 5000, 0.02, 8), None),
    (_w("kv_split_L100_bf16", "bf16", 1, 1, 100, 9000), wl.block_structured_mask(100, 9000, 9, 0.3, 0.3, 0.5),
     None),
    # 2 x 8 heads x 32 query blocks: the plan's two-way split of query
    # blocks with more than 16 of the 18 kv blocks live
    (_w("plan_split_bf16", "bf16", 2, 8, 4096, 2304), wl.block_structured_mask(4096, 2304, 10, 0.6, 0.35, 0.5),
     None),
    (_w("padded_bf16", "bf16", 2, 2, 600, 900), wl.block_structured_mask(600, 900, 12, 0.3, 0.4, 0.5),
     ([0, 130], [900, 517])),
    (_w("padded_decode_f16", "f16", 2, 4, 1, 4000, H_kv=1), _random(1, 4000, 0.3, 13), ([100, 0], [4000, 1000])),
]


@pytest.mark.parametrize("w,m,ranges", FORWARD, ids=[f[0].name for f in FORWARD])
def test_forward_dense_mask(dev, w, m, ranges):
    (q, k, v), o, lse = _run(w, m, dev, ranges=ranges)
    want_o, want_lse = oracle.attention(q.double().numpy(), _expand_kv(w, k).double().numpy(),
                                        _expand_kv(w, v).double().numpy(), oracle.DENSE, w.scale,
                                        softcap=w.softcap, mask=m,
                                        key_start=None if ranges is None else ranges[0],
                                        key_end=None if ranges is None else ranges[1])
    _compare(w, o.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), want_o, want_lse, w.name)


def test_bits_past_kv_len_are_ignored(dev):
    """Bits set past kv_len change neither the BlockMask nor the output."""
    w = _w("tail_bits_bf16", "bf16", 1, 2, 150, 200)
    m = wl.block_structured_mask(150, 200, 14, 0.3, 0.4, 0.5)
    bits = bsa.pack_mask(torch.from_numpy(m).to(dev))
    dirty = bits.clone()
    dirty[:, 6] |= torch.tensor(-256, dtype=torch.int32)  # keys 200..223 of word 6 (bits 8..31)
    dirty[:, 7] = -1                                      # keys 224..255
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 1))
    outs = []
    for b in (bits, dirty):
        bm = bsa.create_block_mask_from_bits(b, 150, 200)
        outs.append(bsa.attention(q, k, v, bm, scale=w.scale, return_lse=True))
        torch.cuda.synchronize()
        _check_bm(bm, m)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


RULES = [
    ("causal_4352", wl.MASK_CAUSAL, 0, 4352, 4352, _band(4352, 4352, 0, 4352)),
    ("sliding_w300_2000", wl.MASK_SLIDING_WINDOW, 300, 2000, 2000, _band(2000, 2000, 0, 299)),
    ("causal_lr_decode_L3", wl.MASK_CAUSAL_LOWER_RIGHT, 0, 3, 5000, _band(3, 5000, -4997, 5000)),
]


@pytest.mark.parametrize("name,kind,win,L,S,m", RULES, ids=[r[0] for r in RULES])
def test_rule_as_dense_mask_is_bit_identical(dev, name, kind, win, L, S, m):
    w = wl.Workload(name, 1, 2, L, S, 64, "bf16", kind, win)
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 2))
    bm_rule = bsa.create_block_mask(kind, L, S, window=win or None, device=dev)
    bm_dense = bsa.create_block_mask_from_dense(torch.from_numpy(m).to(dev))
    o1, l1 = bsa.attention(q, k, v, bm_rule, scale=w.scale, return_lse=True)
    o2, l2 = bsa.attention(q, k, v, bm_dense, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_custom_workload_full_size_every_row(dev):
    """The benchmark's user-mask workload at full size: every row against
    the oracle."""
    w = wl.WORKLOADS["custom_blocks_8192_bf16"]
    m = wl.make_mask(w)
    (q, k, v), o, lse = _run(w, m, dev)
    want_o, want_lse = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                        oracle.DENSE, w.scale, mask=m)
    _compare(w, o.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64), want_o, want_lse,
             w.name)
