"""GPU parity of the backward (attn_backward), through the C ABI.

dq, dk, dv of sum(dO * O) against the fp64 oracle on the same inputs (the
forward's O and logsumexp come from the GPU forward, as in training). Every
product term passes through one rounding to the input type (P for dV, dS for
dK and dQ, and O in D = dO . O), relative error u = 2^-9 (bf16) or 2^-12
(fp16), and the result is rounded once more to the input type, so the error
of each output is a few u times the magnitude of its terms: the test bounds
the max-abs error by 8 u and the mean-abs error by 2 u, relative to the
reference's max-abs (resp. mean-abs) value (measured: at most 2.7 u and
1.3 u over the cases below). In fp32 nothing is rounded to a narrower type;
the error comes from fp32 sums over up to S terms (about sqrt(S) 2^-24
relative for sums of mixed sign, at most 2^-18 for S <= 4096) and the
1-ulp exp2, so u = 2^-18 there. At full size (the benchmark's
shapes) dq is compared on sampled rows, and dk, dv through identities that
hold exactly: sum_j dV_j = sum_i dO_i over the rows with a live key, and
sum_j dK_j = 0 without the soft-cap (each row of dS sums to zero).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_35_amd as bsa
import oracle
import workloads as wl
from test_parity_gpu import _expand_kv

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -9, "f16": 2.0 ** -12, "f32": 2.0 ** -18}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _odd(name, dtype, H, L, S, kind, window=0, bounds=(), softcap=0.0, B=1, H_kv=0):
    return wl.Workload(name, B, H, L, S, 64, dtype, kind, window, bounds, softcap, H_kv=H_kv)


def _mask(w, dev, m=None):
    if w.kind == wl.MASK_CUSTOM:
        return bsa.create_block_mask_from_dense(torch.from_numpy(m).to(dev)), None
    doc = wl.make_doc(w)
    return bsa.create_block_mask(w.kind, w.L, w.S, window=w.window or None,
                                 document_id=None if doc is None else torch.from_numpy(doc).to(dev),
                                 device=dev), doc


def _run(w, dev, m=None, ranges=None, seed=0):
    q, k, v = wl.make_qkv(w, seed)
    dout = torch.from_numpy(np.random.default_rng(seed + 99).standard_normal(
        (w.B, w.H, w.L, w.E), dtype=np.float32)).to(w.torch_dtype)
    bm, doc = _mask(w, dev, m)
    ks = ke = None
    if ranges is not None:
        ks = torch.tensor(ranges[0], dtype=torch.int32, device=dev)
        ke = torch.tensor(ranges[1], dtype=torch.int32, device=dev)
    qd, kd, vd, dd = (x.to(dev) for x in (q, k, v, dout))
    sm = "softcap" if w.softcap else None
    o, lse = bsa.attention(qd, kd, vd, bm, score_mod=sm, softcap=w.softcap or 30.0, scale=w.scale,
                           return_lse=True, key_start=ks, key_end=ke)
    dq, dk, dv = bsa.attention_backward(qd, kd, vd, o, lse, dd, bm, score_mod=sm,
                                        softcap=w.softcap or 30.0, scale=w.scale, key_start=ks,
                                        key_end=ke)
    torch.cuda.synchronize()
    return (q, k, v, dout), doc, (dq, dk, dv)


def _reduce_kv(w, g):
    """Gradient of a shared K/V head: the sum over its query heads."""
    G = w.H // w.kv_heads
    return g.reshape(w.B, w.kv_heads, G, w.S, w.E).sum(2) if G > 1 else g


def _compare(w, got, want, what):
    u = U[w.dtype]
    got = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    err = np.abs(got - want)
    scale_max, scale_mean = max(np.abs(want).max(), 1e-6), max(np.abs(want).mean(), 1e-6)
    assert err.max() <= 8 * u * scale_max, f"{what}: max-abs {err.max():.3g} vs {8 * u * scale_max:.3g}"
    assert err.mean() <= 2 * u * scale_mean, f"{what}: mean-abs {err.mean():.3g} vs {2 * u * scale_mean:.3g}"


CASES = [
    (_odd("causal_1000_bf16", "bf16", 2, 1000, 1000, wl.MASK_CAUSAL), None, None),
    (_odd("sliding_w200_1000_f16", "f16", 2, 1000, 1000, wl.MASK_SLIDING_WINDOW, 200), None, None),
    (_odd("document_softcap_1000_f16", "f16", 2, 1000, 1000, wl.MASK_DOCUMENT, 0, (300, 777), 30.0), None, None),
    (_odd("none_300x200_bf16", "bf16", 2, 300, 200, wl.MASK_NONE), None, None),
    (_odd("causal_lr_gqa_200x700_bf16", "bf16", 4, 200, 700, wl.MASK_CAUSAL_LOWER_RIGHT, H_kv=2), None, None),
    (_odd("bidir_document_gqa_softcap_bf16", "bf16", 6, 640, 640, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (200, 500),
          20.0, H_kv=2), None, None),
    (_odd("sliding_empty_rows_bf16", "bf16", 1, 400, 130, wl.MASK_SLIDING_WINDOW, 20), None, None),
    (_odd("ragged_causal_333x555_f16", "f16", 3, 333, 555, wl.MASK_CAUSAL, B=2), None, None),
    (_odd("decode_lr_L1_S3000_bf16", "bf16", 8, 1, 3000, wl.MASK_CAUSAL_LOWER_RIGHT, H_kv=2), None, None),
    (_odd("custom_blocks_700_bf16", "bf16", 2, 700, 900, wl.MASK_CUSTOM),
     wl.block_structured_mask(700, 900, 21, 0.3, 0.3, 0.4), None),
    (_odd("padded_causal_600_bf16", "bf16", 2, 600, 600, wl.MASK_CAUSAL, B=3), None, ([0, 100, 300], [600, 450, 300])),
    (_odd("custom_gqa_softcap_f16", "f16", 4, 500, 800, wl.MASK_CUSTOM, 0, (), 15.0, H_kv=1),
     wl.block_structured_mask(500, 800, 22, 0.25, 0.35, 0.3), None),
    (_odd("document_L600_S900_bf16", "bf16", 2, 600, 900, wl.MASK_DOCUMENT, 0, (130, 500)), None, None),
    (_odd("padded_empty_range_bidir_f16", "f16", 2, 384, 384, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (100,), B=2),
     None, ([50, 200], [384, 200])),
    # more than 16 live blocks per row: dQ and dK/dV items split in two and merge
    (_odd("split_causal_4352_bf16", "bf16", 1, 4352, 4352, wl.MASK_CAUSAL), None, None),
    (_odd("split_gqa_causal_2304_f16", "f16", 4, 2304, 2304, wl.MASK_CAUSAL, H_kv=2), None, None),
    # B*H a multiple of 8 with grouped heads: the dQ items take the XCD head
    # order, with split items merging by their (batch, head) slot
    (_odd("split_gqa_xcd_order_B2_h8_kv2_2304_bf16", "bf16", 8, 2304, 2304, wl.MASK_CAUSAL, B=2, H_kv=2),
     None, None),
    (_odd("split_padded_none_2560_bf16", "bf16", 1, 2560, 2560, wl.MASK_NONE, B=2), None, ([100, 0], [2560, 2200])),
    # sliding windows skip the query tiles (dK/dV) and key tiles (dQ) of a
    # partial block that no pair reaches: with a query offset, with key
    # ranges, and with windows not a multiple of the tile
    (_odd("sliding_lr_L300_S1000_w100_bf16", "bf16", 2, 300, 1000, wl.MASK_SLIDING_WINDOW_LOWER_RIGHT, 100),
     None, None),
    (_odd("sliding_padded_w150_f16", "f16", 2, 900, 900, wl.MASK_SLIDING_WINDOW, 150, B=2), None,
     ([0, 300], [900, 517])),
    (_odd("sliding_w256_2304_gqa_bf16", "bf16", 4, 2304, 2304, wl.MASK_SLIDING_WINDOW, 256, H_kv=2), None, None),
    # fp32 (fp32 MFMA, probabilities and dS unrounded)
    (wl.WORKLOADS["causal_256_f32"], None, None),
    (_odd("sliding_softcap_700_f32", "f32", 2, 700, 700, wl.MASK_SLIDING_WINDOW, 150, (), 30.0), None, None),
    (_odd("document_gqa_600_f32", "f32", 4, 600, 600, wl.MASK_DOCUMENT, 0, (100, 350), H_kv=2), None, None),
    (_odd("custom_400x520_f32", "f32", 2, 400, 520, wl.MASK_CUSTOM),
     wl.block_structured_mask(400, 520, 23, 0.3, 0.3, 0.4), None),
    (_odd("padded_bidir_f32", "f32", 2, 384, 384, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (100,), B=2),
     None, ([50, 0], [384, 300])),
    (_odd("decode_lr_L1_S3000_f32", "f32", 8, 1, 3000, wl.MASK_CAUSAL_LOWER_RIGHT, H_kv=2), None, None),
    (_odd("split_gqa_causal_2304_f32", "f32", 4, 2304, 2304, wl.MASK_CAUSAL, H_kv=2), None, None),
]


@pytest.mark.parametrize("w,m,ranges", CASES, ids=[c[0].name for c in CASES])
def test_backward_against_oracle(dev, w, m, ranges):
    (q, k, v, dout), doc, (dq, dk, dv) = _run(w, dev, m, ranges)
    want = oracle.attention_backward(q.double().numpy(), _expand_kv(w, k).double().numpy(),
                                     _expand_kv(w, v).double().numpy(), dout.double().numpy(), w.kind,
                                     w.scale, w.window, doc, w.softcap,
                                     key_start=None if ranges is None else ranges[0],
                                     key_end=None if ranges is None else ranges[1], mask=m)
    _compare(w, dq, want[0], w.name + " dq")
    _compare(w, dk, _reduce_kv(w, want[1]), w.name + " dk")
    _compare(w, dv, _reduce_kv(w, want[2]), w.name + " dv")


@pytest.mark.parametrize("L,S", [(0, 300), (300, 0)])
def test_backward_empty_sequences(dev, L, S):
    """No queries: dk = dv = 0; no keys: dq = 0 (and nothing else to write)."""
    w = _odd(f"empty_{L}x{S}_bf16", "bf16", 2, L, S, wl.MASK_NONE)
    _, _, (dq, dk, dv) = _run(w, dev)
    assert dq.shape == (1, 2, L, 64) and dk.shape == (1, 2, S, 64)
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_is_deterministic(dev, dtype):
    w = _odd(f"det_causal_gqa_{dtype}", dtype, 4, 2304, 2304, wl.MASK_CAUSAL, H_kv=2)
    _, _, g1 = _run(w, dev)
    _, _, g2 = _run(w, dev)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_backward_workspace_shared_by_shapes(dev):
    """One cached workspace serves calls of different shapes in turn (split
    and unsplit items): every call gives the bits of a call on its own."""
    ws = [_odd("ws_a_causal_2304_bf16", "bf16", 2, 2304, 2304, wl.MASK_CAUSAL),
          _odd("ws_b_sliding_700_bf16", "bf16", 3, 700, 700, wl.MASK_SLIDING_WINDOW, 90),
          _odd("ws_c_gqa_4352_bf16", "bf16", 4, 640, 4352, wl.MASK_CAUSAL_LOWER_RIGHT, H_kv=1)]
    first = [_run(w, dev)[2] for w in ws]
    again = [_run(w, dev)[2] for w in reversed(ws)][::-1]
    for w, g1, g2 in zip(ws, first, again):
        assert all(torch.equal(a, b) for a, b in zip(g1, g2)), w.name


FULL_SIZE = ["causal_8192_bf16", "sliding_32768_w256_bf16", "document_8192_f16_softcap"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_backward_full_size(dev, name):
    """The benchmark's shapes: dq on sampled rows against the oracle; dk and
    dv through exact identities (every row of these workloads has a live
    key); everything finite."""
    w = wl.WORKLOADS[name]
    (q, k, v, dout), doc, (dq, dk, dv) = _run(w, dev)
    rows = wl.sample_rows(w, 48)
    want = oracle.attention_backward_dq_rows(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                             dout.double().numpy(), w.kind, w.scale, rows, w.window, doc,
                                             w.softcap)
    got = dq.reshape(-1, w.E)[torch.from_numpy(rows).to(dev)]
    _compare(w, got, want, "dq rows")
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    u = U[w.dtype]
    # sum over keys of dV = sum over rows of dO
    sv = dv.double().sum(2).cpu().numpy()
    so = dout.double().sum(2).numpy()
    assert np.abs(sv - so).max() <= 16 * u * np.abs(dout.double().numpy()).sum(2).max()
    # sum over keys of dK = scale sum_i q_i sum_j dS_ij = 0 without the
    # soft-cap (each row of dS sums to zero; the cap weights it by 1 - t^2)
    if not w.softcap:
        sk = dk.double().sum(2).cpu().numpy()
        assert np.abs(sk).max() <= 16 * u * dk.double().abs().sum(2).max().item()


def _term_scales(w, q, k, v, dout, o, lse, live):
    """Magnitude of the terms each gradient element sums (no cancellation):
    scale sum_j |dS_ij| |k_j| for dq, scale sum_i |dS_ij| |q_i| for dk and
    sum_i P_ij |dO_i| for dv, with P = exp(s' - lse) from the oracle's
    logsumexp and dS = P (dP - D) (1 - t^2), D = dO . O from the oracle's O.
    A scale for the error bound, not a reference value."""
    G = w.H // w.kv_heads
    q, k, v, dout = (x.double().numpy() for x in (q, k, v, dout))
    k, v = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    s = np.einsum("bhie,bhje->bhij", q, k) * w.scale
    t = np.tanh(s / w.softcap) if w.softcap else np.zeros_like(s)
    sp = w.softcap * t if w.softcap else s
    p = np.where(live, np.exp(sp - np.where(np.isneginf(lse), 0.0, lse)[..., None]), 0.0)
    dp = np.einsum("bhie,bhje->bhij", dout, v)
    d = (dout * o).sum(-1)[..., None]
    ds = np.abs(p * (dp - d) * (1.0 - t * t))
    tq = w.scale * np.einsum("bhij,bhje->bhie", ds, np.abs(k))
    tk = w.scale * np.einsum("bhij,bhie->bhje", ds, np.abs(q))
    tv = np.einsum("bhij,bhie->bhje", p, np.abs(dout))
    return tq, _reduce_kv(w, torch.from_numpy(tk)).numpy(), _reduce_kv(w, torch.from_numpy(tv)).numpy()


TWO_KEYS = [
    # every row keeps keys 613 and 614 only (key range on a single document)
    (_odd("two_keys_range_bidir_softcap_gqa_bf16", "bf16", 6, 228, 615, wl.MASK_DOCUMENT_BIDIRECTIONAL, 0, (),
          5.0, H_kv=3), ([613], [615])),
    # a window of two: each row its own key and the one before
    (_odd("two_keys_window2_bf16", "bf16", 4, 700, 700, wl.MASK_SLIDING_WINDOW, 2), None),
]


@pytest.mark.parametrize("w,ranges", TWO_KEYS, ids=[c[0].name for c in TWO_KEYS])
def test_backward_two_key_rows(dev, w, ranges):
    """Rows with two live keys: each gradient element is a sum of two terms
    that may cancel, so the mean error is bounded by 2u times the mean of
    the terms' magnitude (rather than of the result, as elsewhere); the
    max-abs bound stays 8u of the reference's largest value."""
    (q, k, v, dout), doc, (dq, dk, dv) = _run(w, dev, None, ranges, seed=18)
    kwargs = dict(key_start=None if ranges is None else ranges[0], key_end=None if ranges is None else ranges[1])
    want = oracle.attention_backward(q.double().numpy(), _expand_kv(w, k).double().numpy(),
                                     _expand_kv(w, v).double().numpy(), dout.double().numpy(), w.kind,
                                     w.scale, w.window, doc, w.softcap, **kwargs)
    o, lse = oracle.attention(q.double().numpy(), _expand_kv(w, k).double().numpy(),
                              _expand_kv(w, v).double().numpy(), w.kind, w.scale, w.window, doc, w.softcap,
                              **kwargs)
    i = np.arange(w.L)[:, None]
    j = np.arange(w.S)[None, :]
    if ranges is not None:
        live = (j >= ranges[0][0]) & (j < ranges[1][0]) & np.ones((w.L, 1), bool)
    else:
        live = (i >= j) & (i - j < w.window)
    assert live.sum(1).max() == 2
    scales = _term_scales(w, q, k, v, dout, o, lse, live[None, None])
    u = U[w.dtype]
    for name, g, ref, sc in zip(("dq", "dk", "dv"), (dq, dk, dv),
                                (want[0], _reduce_kv(w, want[1]), _reduce_kv(w, want[2])), scales):
        got = g.float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        print(f"{w.name} {name}: max-abs {err.max():.3g} (bound {8 * u * np.abs(ref).max():.3g}), "
              f"mean-abs {err.mean():.3g} (2u mean |ref| {2 * u * np.abs(ref).mean():.3g}, "
              f"2u mean terms {2 * u * sc.mean():.3g})", flush=True)
        assert np.isfinite(got).all()
        assert err.max() <= 8 * u * np.abs(ref).max(), name
        assert err.mean() <= 2 * u * sc.mean(), name


def test_backward_one_key(dev):
    """One key (S = 1): P = 1 and O = V exactly, so dP - D = dO . (V - O) and
    with it dq and dk vanish; the kernel forms dP (MFMA) and D (the prep
    kernel) as two fp32 sums of the 64 exact products dO_e v_e, so dS is
    their rounding difference, at most 2 * 64 * 2^-24 sum_e |dO_e v_e| <=
    2^-16 sum_e |dO_e v_e| (with the soft-cap factor <= 1), and dq, dk are
    bounded through it; dv = sum_i dO_i keeps the usual bounds."""
    w = _odd("one_key_S1_softcap_bf16", "bf16", 3, 645, 1, wl.MASK_NONE, 0, (), 5.0, B=2)
    (q, k, v, dout), doc, (dq, dk, dv) = _run(w, dev, None, None, seed=74)
    want = oracle.attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     dout.double().numpy(), w.kind, w.scale, w.window, doc, w.softcap)
    qn, kn, vn, dn = (x.double().numpy() for x in (q, k, v, dout))
    ds_bound = 2.0 ** -16 * np.abs(dn * vn).sum(-1)  # [B, H, L]: |fl(dP) - fl(D)| per row
    dq_bound = w.scale * ds_bound[..., None] * np.abs(kn)  # the single key's row
    dk_bound = w.scale * (ds_bound[..., None] * np.abs(qn)).sum(2, keepdims=True)
    got_dq = dq.float().cpu().numpy().astype(np.float64)
    got_dk = dk.float().cpu().numpy().astype(np.float64)
    print(f"one key: dq max {np.abs(got_dq).max():.3g} (bound {dq_bound.max():.3g}), "
          f"dk max {np.abs(got_dk).max():.3g} (bound {dk_bound.max():.3g})", flush=True)
    assert np.abs(want[0]).max() < 1e-12 and np.abs(want[1]).max() < 1e-12
    assert np.all(np.abs(got_dq) <= dq_bound * (1 + 2.0 ** -8) + 1e-30)
    assert np.all(np.abs(got_dk) <= dk_bound * (1 + 2.0 ** -8) + 1e-30)
    _compare(w, dv, want[2], "one key dv")
