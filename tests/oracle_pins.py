"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the pages, a closed form, an invariance the pages state,
or an independent library routine. ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutants.py`` runs them on deliberately broken copies
to show that each plausible mistake fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NONE, CAUSAL, SLIDING, DOCUMENT = 0, 1, 2, 3
CAUSAL_LR, SLIDING_LR, DOCUMENT_BIDIR = 4, 5, 6
DENSE = 7


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Block mask and predicate pins
# ---------------------------------------------------------------------------

def check_flex_table_densities(orc, max_S=32768):
    """Token and block densities of the FlexAttention-on-MPS results table
    (causal and sliding-window rows, 128x128 blocks), to the printed 2 decimals."""
    g = _golden("flex_mps_densities.json")
    for row in g["rows"]:
        S, W = row["S"], row["W"]
        if S > max_S:
            continue
        kind, win = (CAUSAL, 0) if row["pattern"] == "causal" else (SLIDING, W)
        live = orc.count_live(kind, S, S, win)
        assert round(100.0 * live / (S * S), 2) == row["token_pct"], (row, live)
        kv_num, _, full_num, _ = orc.block_mask(kind, S, S, win, block=g["block"])
        nb = -(-S // g["block"])
        blocks = int(kv_num.sum() + full_num.sum())
        assert round(100.0 * blocks / (nb * nb), 2) == row["block_pct"], (row, blocks)


def check_live_pair_closed_forms(orc):
    """Live pairs: causal S(S+1)/2; window W*S - W(W-1)/2 (W <= S);
    document-causal sum over documents of n(n+1)/2; none L*S."""
    for S in (1, 7, 128, 1000):
        assert orc.count_live(CAUSAL, S, S) == S * (S + 1) // 2
        assert orc.count_live(NONE, S, S + 3) == S * (S + 3)
        for W in sorted({w for w in (1, 2, 37, S) if w <= S}):
            assert orc.count_live(SLIDING, S, S, W) == W * S - W * (W - 1) // 2, (S, W)
    bounds = (100, 190, 191)
    doc = wl.document_ids(300, bounds)
    sizes = np.diff([0, *bounds, 300])
    assert orc.count_live(DOCUMENT, 300, 300, doc=doc) == int(sum(n * (n + 1) // 2 for n in sizes))


def check_block_mask_worked_examples(orc):
    """The 2x2 causal example and the 3-document totals (hand derivation)."""
    g = _golden("block_mask_small.json")
    kv_num, kv_idx, full_num, full_idx = orc.block_mask(CAUSAL, 256, 256)
    ex = g["causal_256"]
    assert kv_num.tolist() == ex["kv_num_blocks"]
    assert kv_idx.tolist() == ex["kv_indices"]
    assert full_num.tolist() == ex["full_kv_num_blocks"]
    assert full_idx.tolist() == ex["full_kv_indices"]
    d = g["document_8192"]
    doc = wl.document_ids(8192, tuple(d["bounds"]))
    kv_num, _, full_num, _ = orc.block_mask(DOCUMENT, 8192, 8192, doc=doc)
    assert int(full_num.sum()) == d["full_total"]
    assert int(kv_num.sum()) == d["partial_total"]


def check_block_mask_window_closed_form(orc):
    """For W = 128*w the pair offsets i-j of block offset d = qb-kb span
    [128d-127, 128d+127]; the block is full iff that range sits inside [0, W-1]
    (1 <= d <= w-1) and partial iff it only overlaps (d == 0 or d == w)."""
    S = 2048
    nb = S // 128
    for w in (1, 2, 3):
        kv_num, kv_idx, full_num, full_idx = orc.block_mask(SLIDING, S, S, 128 * w)
        for qb in range(nb):
            full = [kb for kb in range(nb) if 1 <= qb - kb <= w - 1]
            part = [kb for kb in range(nb) if qb - kb in (0, w)]
            assert full_idx[qb, : full_num[qb]].tolist() == full
            assert kv_idx[qb, : kv_num[qb]].tolist() == part
            assert not full_idx[qb, full_num[qb]:].any() and not kv_idx[qb, kv_num[qb]:].any()


def check_block_mask_ragged_tail(orc):
    """Lengths not multiple of 128: out-of-range pairs are absent, so a tail
    block can never be full; kind none gives full interior blocks only."""
    L, S = 300, 200
    kv_num, kv_idx, full_num, full_idx = orc.block_mask(NONE, L, S)
    # blocks are (qb in 0..2) x (kb in 0..1); only (0,0) and (1,0) are whole.
    assert full_num.tolist() == [1, 1, 0]
    assert kv_num.tolist() == [1, 1, 2]
    assert kv_idx[2].tolist() == [0, 1]


# ---------------------------------------------------------------------------
# Attention pins
# ---------------------------------------------------------------------------

def _weights(orc, scores, kind=NONE, window=0, doc=None, softcap=0.0):
    """Attention weights of one row per query by the V = identity trick:
    with E=1, q=1, k_j = s_j and scale=1 the scores are s_j, and with V = I
    the output row is exactly the weight vector."""
    L, S = scores.shape
    k = np.zeros((1, 1, S, 1))
    out = np.zeros((L, S))
    lses = np.zeros(L)
    # scores differ per row, so run one row (one query) at a time
    for i in range(L):
        k[0, 0, :, 0] = scores[i]
        qi = np.ones((1, 1, L, 1))
        o, lse = orc.attention(qi, k, np.eye(S)[None, None], kind, 1.0, window, doc, softcap,
                               rows=[i])
        out[i] = o[0]
        lses[i] = lse[0]
    return out, lses


def check_tiled_softmax_equivalence(orc):
    """FlashAttention page: softmax over 4096 values computed tile by tile with
    a running max and running sum equals the plain softmax to double rounding
    (max error <= ~2e-18 on that page). The tiled form here is written
    independently of the oracle and compared with the oracle's weights."""
    g = _golden("tiled_softmax_error.json")
    n = g["n_values"]
    s = _rand(n, 3)
    w_or, _ = _weights(orc, s[None, :])
    w_or = w_or[0]
    for tile in g["tiles"]:
        m, l = -math.inf, 0.0
        chunks = []
        for t0 in range(0, n, tile):
            x = s[t0:t0 + tile]
            m_new = max(m, float(x.max()))
            l = l * math.exp(m - m_new) + float(np.exp(x - m_new).sum())
            chunks = [(c, mm) for c, mm in chunks] + [(x, m_new)]
            m = m_new
        w_tiled = np.concatenate([np.exp(x - mm) * math.exp(mm - m) for x, mm in chunks]) / l
        err = np.abs(w_tiled - w_or)
        assert err.max() <= 10 * max(g["max_abs_err"]), (tile, err.max())
        assert err.mean() <= 10 * max(g["mean_abs_err"]), (tile, err.mean())


def check_weights_are_a_distribution(orc):
    """Each non-empty row's weights sum to 1 and dead pairs weigh exactly 0."""
    L = S = 40
    scores = _rand((L, S), 5, 3.0)
    doc = wl.document_ids(S, (13, 29))
    for kind, W in ((NONE, 0), (CAUSAL, 0), (SLIDING, 5), (DOCUMENT, 0)):
        w, _ = _weights(orc, scores, kind, W, doc if kind == DOCUMENT else None)
        for i in range(L):
            dead = [j for j in range(S) if not _live_py(kind, W, doc, i, j)]
            assert np.all(w[i, dead] == 0.0), (kind, i)
            assert abs(w[i].sum() - 1.0) <= 1e-15, (kind, i, w[i].sum())


def _live_py(kind, W, doc, i, j):
    # restated from the page's mask_mod functions for the dead-pair check
    if kind == NONE:
        return True
    if kind == CAUSAL:
        return i >= j
    if kind == SLIDING:
        return i >= j and i - j < W
    return i >= j and doc[i] == doc[j]


def check_uniform_v(orc):
    """V rows all equal to v gives O_i = v for every row with a live key."""
    B, H, L, S, E = 1, 2, 70, 70, 8
    q, k = _rand((B, H, L, E), 7), _rand((B, H, S, E), 8)
    vrow = _rand(E, 9)
    v = np.broadcast_to(vrow, (B, H, S, E)).copy()
    doc = wl.document_ids(S, (20, 50))
    for kind, W, cap in ((NONE, 0, 0.0), (CAUSAL, 0, 0.0), (SLIDING, 9, 0.0),
                         (DOCUMENT, 0, 30.0)):
        o, _ = orc.attention(q, k, v, kind, 0.35, W, doc if kind == DOCUMENT else None, cap)
        assert np.abs(o - vrow).max() <= 1e-14, kind


def check_window_one_is_identity(orc):
    """Window W=1 leaves each query only its own key: O_i = V_i exactly and
    lse_i equals that single score."""
    B, H, L, E = 1, 2, 50, 16
    q, k, v = _rand((B, H, L, E), 10), _rand((B, H, L, E), 11), _rand((B, H, L, E), 12)
    o, lse = orc.attention(q, k, v, SLIDING, 0.25, 1)
    assert np.array_equal(o, v)
    single = 0.25 * np.einsum("bhle,bhle->bhl", q, k)
    assert np.abs(lse - single).max() <= 1e-13


def check_causal_first_row(orc):
    """Row 0 of a causal mask sees key 0 only: O_0 = V_0 exactly."""
    q, k, v = _rand((1, 3, 20, 8), 13), _rand((1, 3, 20, 8), 14), _rand((1, 3, 20, 8), 15)
    o, lse = orc.attention(q, k, v, CAUSAL, 0.5)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.abs(lse[:, :, 0] - 0.5 * (q[:, :, 0] * k[:, :, 0]).sum(-1)).max() <= 1e-13


def check_two_key_closed_form(orc):
    """E=2, q=(a,0), k1=(1,0), k2=(0,1): scores s1 = f(scale*a), s2 = f(0) = 0
    with f the identity or the soft-cap c*tanh(x/c) on the scaled score.
    Then O = sigmoid(s1) v1 + sigmoid(-s1) v2 and lse = log(1 + e^{s1})."""
    v1, v2 = np.array([1.5, -2.0, 0.25]), np.array([-0.5, 3.0, 1.0])
    k = np.array([[1.0, 0.0], [0.0, 1.0]])[None, None]
    v = np.stack([v1, v2])[None, None]
    for a, scale, cap in ((0.7, 1.0, 0.0), (-3.0, 0.125, 0.0), (200.0, 0.5, 30.0),
                          (-90.0, 0.5, 30.0), (4.0, 0.5, 30.0)):
        q = np.array([[a, 0.0]])[None, None]
        s1 = scale * a
        if cap:
            s1 = cap * math.tanh(s1 / cap)
        w1 = 1.0 / (1.0 + math.exp(-s1))
        o, lse = orc.attention(q, k, v, NONE, scale, softcap=cap)
        want = w1 * v1 + (1.0 - w1) * v2
        assert np.abs(o[0, 0, 0] - want).max() <= 1e-13, (a, scale, cap)
        assert abs(lse[0, 0, 0] - np.logaddexp(0.0, s1)) <= 1e-13, (a, scale, cap)


def check_scipy_softmax(orc):
    """Small random cases against scipy.special.softmax of the masked, scaled
    (and soft-capped) score table times V, for every mask kind; L != S."""
    B, H, L, S, E, Ev = 2, 2, 9, 13, 5, 3
    q, k, v = _rand((B, H, L, E), 16), _rand((B, H, S, E), 17), _rand((B, H, S, Ev), 18)
    doc = wl.document_ids(S, (4, 10))
    for kind, W, cap in ((NONE, 0, 0.0), (CAUSAL, 0, 0.0), (SLIDING, 3, 0.0),
                         (DOCUMENT, 0, 0.0), (CAUSAL, 0, 1.5)):
        scale = 0.6
        sc = scale * np.einsum("bhle,bhse->bhls", q, k)
        if cap:
            sc = cap * np.tanh(sc / cap)
        bias = np.array([[0.0 if _live_py(kind, W, doc, i, j) else -np.inf for j in range(S)]
                         for i in range(L)])
        want = scipy.special.softmax(sc + bias, axis=-1) @ v
        want_lse = scipy.special.logsumexp(sc + bias, axis=-1)
        o, lse = orc.attention(q, k, v, kind, scale, W, doc if kind == DOCUMENT else None, cap)
        assert np.abs(o - want).max() <= 1e-14, kind
        assert np.abs(lse - want_lse).max() <= 1e-13, kind


def check_empty_rows(orc):
    """A query with no live key returns zeros and lse = -inf (SDPA page,
    fully-masked-row aside). L=8 > S=3 with W=2: rows 4..7 see nothing."""
    q, k, v = _rand((1, 1, 8, 4), 19), _rand((1, 1, 3, 4), 20), _rand((1, 1, 3, 4), 21)
    o, lse = orc.attention(q, k, v, SLIDING, 0.5, 2)
    assert np.all(o[0, 0, 4:] == 0.0) and np.all(np.isneginf(lse[0, 0, 4:]))
    assert np.all(np.isfinite(lse[0, 0, :4])) and np.abs(o[0, 0, :4]).sum() > 0


def check_causal_prefix_invariance(orc):
    """SDPA page, pitfall 3: causal row i equals unmasked attention of q_i over
    keys 0..i (the one-token decode against a cache)."""
    q, k, v = _rand((1, 2, 24, 8), 22), _rand((1, 2, 24, 8), 23), _rand((1, 2, 24, 8), 24)
    o, lse = orc.attention(q, k, v, CAUSAL, 0.3)
    for i in (0, 5, 23):
        oi, li = orc.attention(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], NONE, 0.3)
        assert np.abs(o[:, :, i] - oi[:, :, 0]).max() <= 1e-14
        assert np.abs(lse[:, :, i] - li[:, :, 0]).max() <= 1e-14


def check_sliding_equals_window_slice(orc):
    """Window W: row i equals unmasked attention over keys i-W+1..i."""
    W = 6
    q, k, v = _rand((1, 2, 30, 8), 25), _rand((1, 2, 30, 8), 26), _rand((1, 2, 30, 8), 27)
    o, _ = orc.attention(q, k, v, SLIDING, 0.3, W)
    for i in (0, 3, 5, 6, 29):
        lo = max(0, i - W + 1)
        oi, _ = orc.attention(q[:, :, i:i + 1], k[:, :, lo:i + 1], v[:, :, lo:i + 1], NONE, 0.3)
        assert np.abs(o[:, :, i] - oi[:, :, 0]).max() <= 1e-14


def check_document_isolation(orc):
    """Block-mask page, document packing: no attention across documents, so the
    packed result equals each document run alone with a causal mask."""
    bounds = (11, 40)
    S = 57
    doc = wl.document_ids(S, bounds)
    q, k, v = _rand((1, 2, S, 8), 28), _rand((1, 2, S, 8), 29), _rand((1, 2, S, 8), 30)
    o, lse = orc.attention(q, k, v, DOCUMENT, 0.3, doc=doc)
    edges = [0, *bounds, S]
    for a, b in zip(edges[:-1], edges[1:]):
        od, ld = orc.attention(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], CAUSAL, 0.3)
        assert np.abs(o[:, :, a:b] - od).max() <= 1e-14
        assert np.abs(lse[:, :, a:b] - ld).max() <= 1e-14


def check_library_equivalence(orc):
    """SDPA page, section 1: the hand-written matmul-softmax-matmul attention
    and SDPA agree to ~1e-15 in fp64 and ~5e-7 in fp32 at (2,8,512,64).
    The oracle is compared with that composition in torch fp64 (same bound,
    with a small margin) and with torch fp32 (the fp32 bound)."""
    g = _golden("sdpa_naive_equivalence.json")
    B, H, L, E = g["shape"]
    q, k, v = _rand((B, H, L, E), 31), _rand((B, H, L, E), 32), _rand((B, H, L, E), 33)
    scale = 1.0 / math.sqrt(E)
    for name, kind in (("none", NONE), ("causal", CAUSAL)):
        o, _ = orc.attention(q, k, v, kind, scale)
        for dt, bound in ((torch.float64, 4 * g["fp64_max_abs"][name]),
                          (torch.float32, 4 * g["fp32_max_abs"][name])):
            tq, tk, tv = (torch.from_numpy(x).to(dt) for x in (q, k, v))
            sc = (tq @ tk.transpose(-2, -1).contiguous()) * scale
            if kind == CAUSAL:
                tri = torch.ones(L, L, dtype=torch.bool).tril()
                sc = sc.masked_fill(~tri, float("-inf"))
            ref = (torch.softmax(sc, dim=-1) @ tv).double().numpy()
            assert np.abs(o - ref).max() <= bound, (name, dt, np.abs(o - ref).max())


def check_softcap_limits(orc):
    """The soft-cap bounds every score by c, and a huge c leaves scores as they are."""
    q, k, v = _rand((1, 1, 12, 4), 34, 40.0), _rand((1, 1, 12, 4), 35, 40.0), _rand((1, 1, 12, 4), 36)
    o1, l1 = orc.attention(q, k, v, NONE, 0.5, softcap=1e12)
    o0, l0 = orc.attention(q, k, v, NONE, 0.5)
    assert np.abs(o1 - o0).max() <= 1e-9 and np.abs(l1 - l0).max() <= 1e-9
    _, lw = orc.attention(q, k, v, SLIDING, 0.5, 1, softcap=2.0)   # single key: lse = s'
    assert np.all(np.abs(lw) <= 2.0) and np.abs(lw).max() > 1.9


# ---------------------------------------------------------------------------
# Variant masks: bottom-right alignment and bidirectional documents
# ---------------------------------------------------------------------------

def check_kv_cache_alignment_example(orc):
    """SDPA page, pitfall 3: for L=1, S=6 the upper-left causal row is the
    printed [T, F, F, F, F, F]; the bottom-right row sees every key, and the
    one-query result equals the last row of full causal attention (and the
    unmasked one-query result), while the upper-left one does not."""
    g = _golden("sdpa_kv_cache_alignment.json")
    L, S = g["L"], g["S"]
    assert [orc.live(CAUSAL, 0, j, L=L, S=S) for j in range(S)] == g["upper_left_row"]
    assert [orc.live(CAUSAL_LR, 0, j, L=L, S=S) for j in range(S)] == g["lower_right_row"]
    q, k, v = _rand((1, 1, S, 8), 40), _rand((1, 1, S, 8), 41), _rand((1, 1, S, 8), 42)
    ref, ref_lse = orc.attention(q, k, v, CAUSAL, 0.35)
    ok, ok_lse = orc.attention(q[:, :, -1:], k, v, CAUSAL_LR, 0.35)
    un, _ = orc.attention(q[:, :, -1:], k, v, NONE, 0.35)
    bad, _ = orc.attention(q[:, :, -1:], k, v, CAUSAL, 0.35)
    assert np.abs(ok[:, :, 0] - ref[:, :, -1]).max() <= 1e-14
    assert np.abs(ok_lse[:, :, 0] - ref_lse[:, :, -1]).max() <= 1e-14
    assert np.abs(un - ok).max() <= 1e-14
    assert np.abs(bad[:, :, 0] - ref[:, :, -1]).max() > 1e-3


def check_lower_right_is_last_rows(orc):
    """Chunked inference (same page and pitfall): L queries at the end of an
    S-token sequence, bottom-right aligned, equal the last L rows of the full
    causal (or sliding-window) attention over all S tokens. L > S leaves the
    first L - S rows with no key (zeros, lse = -inf)."""
    S, W = 40, 7
    q, k, v = _rand((1, 2, S, 8), 43), _rand((1, 2, S, 8), 44), _rand((1, 2, S, 8), 45)
    for kind, lr, win in ((CAUSAL, CAUSAL_LR, 0), (SLIDING, SLIDING_LR, W)):
        full, full_lse = orc.attention(q, k, v, kind, 0.3, win)
        for L in (1, 3, 17, S):
            o, lse = orc.attention(q[:, :, S - L:], k, v, lr, 0.3, win)
            assert np.abs(o - full[:, :, S - L:]).max() <= 1e-14, (kind, L)
            assert np.abs(lse - full_lse[:, :, S - L:]).max() <= 1e-14, (kind, L)
    qq = _rand((1, 1, 9, 8), 46)
    o, lse = orc.attention(qq, k[:, :1, :5], v[:, :1, :5], CAUSAL_LR, 0.3)
    assert np.all(o[0, 0, :4] == 0.0) and np.all(np.isneginf(lse[0, 0, :4]))
    assert np.all(np.isfinite(lse[0, 0, 4:]))


def check_variant_live_pair_closed_forms(orc):
    """Live pairs: bottom-right causal with L <= S is sum_i (S - L + 1 + i) =
    L(S - L + 1) + L(L - 1)/2; with L > S it is S(S + 1)/2; bidirectional
    documents give sum over documents of n^2."""
    for L, S in ((1, 6), (5, 12), (12, 12), (7, 100), (20, 9)):
        want = L * (S - L + 1) + L * (L - 1) // 2 if L <= S else S * (S + 1) // 2
        assert orc.count_live(CAUSAL_LR, L, S) == want, (L, S)
    for L, S, W in ((4, 30, 5), (30, 30, 5), (10, 25, 1)):
        # each query sees min(W, position + 1) keys, position = i + S - L
        want = sum(min(W, i + S - L + 1) for i in range(L) if i + S - L >= 0)
        assert orc.count_live(SLIDING_LR, L, S, W) == want, (L, S, W)
    bounds = (100, 190, 191)
    doc = wl.document_ids(300, bounds)
    sizes = np.diff([0, *bounds, 300])
    assert orc.count_live(DOCUMENT_BIDIR, 300, 300, doc=doc) == int(sum(n * n for n in sizes))


def check_bidirectional_document_isolation(orc):
    """Packed documents without the causal part: the result equals each
    document run alone with no mask (block-diagonal attention)."""
    bounds = (11, 40)
    S = 57
    doc = wl.document_ids(S, bounds)
    q, k, v = _rand((1, 2, S, 8), 47), _rand((1, 2, S, 8), 48), _rand((1, 2, S, 8), 49)
    o, lse = orc.attention(q, k, v, DOCUMENT_BIDIR, 0.3, doc=doc)
    edges = [0, *bounds, S]
    for a, b in zip(edges[:-1], edges[1:]):
        od, ld = orc.attention(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], NONE, 0.3)
        assert np.abs(o[:, :, a:b] - od).max() <= 1e-14
        assert np.abs(lse[:, :, a:b] - ld).max() <= 1e-14


def check_variant_block_masks(orc):
    """Block classification of the variants, by hand: bottom-right causal with
    L=256, S=640 shifts the diagonal by 384 = 3 blocks (query block 0: kv
    blocks 0-2 full, 3 partial; block 1: 0-3 full, 4 partial); bidirectional
    documents on aligned boundaries give only full diagonal blocks."""
    kv_num, kv_idx, full_num, full_idx = orc.block_mask(CAUSAL_LR, 256, 640)
    assert full_num.tolist() == [3, 4] and kv_num.tolist() == [1, 1]
    assert full_idx[0, :3].tolist() == [0, 1, 2] and full_idx[1, :4].tolist() == [0, 1, 2, 3]
    assert kv_idx[0, 0] == 3 and kv_idx[1, 0] == 4
    doc = wl.document_ids(512, (256,))
    kv_num, _, full_num, full_idx = orc.block_mask(DOCUMENT_BIDIR, 512, 512, doc=doc)
    assert kv_num.tolist() == [0, 0, 0, 0] and full_num.tolist() == [2, 2, 2, 2]
    assert full_idx[:, :2].tolist() == [[0, 1], [0, 1], [2, 3], [2, 3]]


# ---------------------------------------------------------------------------
# Key padding (a kept key range per batch entry, ANDed with the mask)
# ---------------------------------------------------------------------------

def check_key_padding_equals_truncation(orc):
    """SDPA page, pitfall 1 and section 5: keeping keys [0, kept) equals
    running on the truncated K/V (right padding); keeping only the padding is
    a different result; with causal AND left padding of p tokens, rows p..
    equal causal attention over the unpadded tokens."""
    g = _golden("sdpa_key_padding.json")
    L, kept = g["right_padding"]["L"], g["right_padding"]["kept"]
    q, k, v = _rand((1, 1, L, 8), 60), _rand((1, 1, L, 8), 61), _rand((1, 1, L, 8), 62)
    ref, ref_lse = orc.attention(q, k[:, :, :kept], v[:, :, :kept], NONE, 0.35)
    ok, ok_lse = orc.attention(q, k, v, NONE, 0.35, key_start=[0], key_end=[kept])
    bad, _ = orc.attention(q, k, v, NONE, 0.35, key_start=[kept], key_end=[L])
    assert np.abs(ok - ref).max() <= 1e-15 and np.abs(ok_lse - ref_lse).max() <= 1e-15
    assert np.abs(bad - ref).max() > 1e-2
    L, p = g["left_padding"]["L"], g["left_padding"]["padded"]
    q, k, v = _rand((2, 3, L, 8), 63), _rand((2, 3, L, 8), 64), _rand((2, 3, L, 8), 65)
    full, full_lse = orc.attention(q, k, v, CAUSAL, 0.35, key_start=[p, p], key_end=[L, L])
    trunc, trunc_lse = orc.attention(q[:, :, p:], k[:, :, p:], v[:, :, p:], CAUSAL, 0.35)
    assert np.abs(full[:, :, p:] - trunc).max() <= 1e-15
    assert np.abs(full_lse[:, :, p:] - trunc_lse).max() <= 1e-15
    # the padded query rows themselves see no kept key at or before them
    assert np.all(full[:, :, :p] == 0.0) and np.all(np.isneginf(full_lse[:, :, :p]))


def check_key_padding_per_batch(orc):
    """Each batch entry takes its own range: the batched result equals every
    entry run alone, and an empty range leaves rows with no key."""
    S = 23
    q, k, v = _rand((3, 2, 19, 8), 66), _rand((3, 2, S, 8), 67), _rand((3, 2, S, 8), 68)
    starts, ends = [0, 5, 9], [S, 17, 9]
    o, lse = orc.attention(q, k, v, SLIDING, 0.3, 6, key_start=starts, key_end=ends)
    for b in range(3):
        ob, lb = orc.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], SLIDING, 0.3, 6,
                               key_start=[starts[b]], key_end=[ends[b]])
        assert np.abs(o[b:b + 1] - ob).max() <= 1e-15
        assert np.array_equal(np.isneginf(lse[b:b + 1]), np.isneginf(lb))
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse[2]))
    on, _ = orc.attention(q, k, v, SLIDING, 0.3, 6)
    assert np.abs(o[0] - on[0]).max() <= 1e-15  # the whole range is no padding


# ---------------------------------------------------------------------------
# User-supplied dense masks
# ---------------------------------------------------------------------------

def _band(L, S, lo, hi):
    """Boolean [L, S] with True where lo <= i - j <= hi (an input mask)."""
    d = np.arange(L)[:, None] - np.arange(S)[None, :]
    return (d >= lo) & (d <= hi)


def check_dense_mask_table_densities(orc):
    """The FlexAttention-on-MPS densities again, now from the patterns given
    as dense boolean masks (the form SDPA takes them in): token and block
    densities of the S = 8192 rows, to the printed 2 decimals."""
    g = _golden("flex_mps_densities.json")
    for row in g["rows"]:
        S, W = row["S"], row["W"]
        if S != 8192 or (W or 0) > 1024:
            continue
        m = _band(S, S, 0, S) if row["pattern"] == "causal" else _band(S, S, 0, W - 1)
        live = orc.count_live(DENSE, S, S, mask=m)
        assert round(100.0 * live / (S * S), 2) == row["token_pct"], (row, live)
        kv_num, _, full_num, _ = orc.block_mask(DENSE, S, S, block=g["block"], mask=m)
        nb = -(-S // g["block"])
        assert round(100.0 * int(kv_num.sum() + full_num.sum()) / (nb * nb), 2) == row["block_pct"], row


def check_pack_mask_worked_example(orc):
    """The bit layout on a hand-worked example (tests/golden/dense_mask_bits.json)."""
    g = _golden("dense_mask_bits.json")
    m = np.zeros((g["L"], g["S"]), bool)
    for i, kept in enumerate(g["kept"]):
        if kept == "all":
            m[i, :] = True
        else:
            m[i, kept] = True
    want = np.array([[int(w, 16) for w in row] for row in g["words"]], np.uint32)
    assert np.array_equal(orc.pack_mask(m), want)


def check_pack_mask_numpy(orc):
    """Bit packing equals numpy.packbits (little bit order) of the mask padded
    with False to a multiple of 128 keys, read as little-endian 32-bit words."""
    rng = np.random.default_rng(70)
    for L, S in ((3, 1), (5, 127), (4, 128), (7, 300), (2, 1000)):
        m = rng.random((L, S)) < 0.4
        padded = np.zeros((L, 128 * (-(-S // 128))), bool)
        padded[:, :S] = m
        want = np.packbits(padded, axis=1, bitorder="little").view("<u4")
        assert np.array_equal(orc.pack_mask(m), want), (L, S)


def check_dense_mask_matches_sdpa(orc):
    """Attention under a random dense boolean mask equals torch's
    scaled_dot_product_attention with that mask as attn_mask (True = take
    part), fp64 on the CPU, with and without the soft-cap written as a float
    bias; every row keeps at least one key."""
    rng = np.random.default_rng(71)
    B, H, L, S, E = 2, 3, 37, 53, 8
    q, k, v = _rand((B, H, L, E), 72), _rand((B, H, S, E), 73), _rand((B, H, S, E), 74)
    m = rng.random((L, S)) < 0.3
    m[np.arange(L), rng.integers(0, S, L)] = True
    o, lse = orc.attention(q, k, v, DENSE, 0.3, mask=m)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(m),
                                                           scale=0.3).numpy()
    assert np.abs(o - ref).max() <= 1e-13
    sc = (tq @ tk.transpose(-2, -1).contiguous()) * 0.3
    sc = sc.masked_fill(~torch.from_numpy(m), float("-inf"))
    assert np.abs(lse - torch.logsumexp(sc, dim=-1).numpy()).max() <= 1e-13


def check_dense_mask_empty_rows(orc):
    """A row whose mask keeps nothing gives O = 0 and lse = -inf; the others
    are unchanged by it."""
    q, k, v = _rand((1, 2, 6, 4), 75), _rand((1, 2, 9, 4), 76), _rand((1, 2, 9, 4), 77)
    m = np.ones((6, 9), bool)
    m[2] = False
    o, lse = orc.attention(q, k, v, DENSE, 0.5, mask=m)
    on, ln = orc.attention(q, k, v, NONE, 0.5)
    assert np.all(o[:, :, 2] == 0.0) and np.all(np.isneginf(lse[:, :, 2]))
    keep = [0, 1, 3, 4, 5]
    assert np.array_equal(o[:, :, keep], on[:, :, keep]) and np.array_equal(lse[:, :, keep], ln[:, :, keep])


def check_dense_mask_equals_rules(orc):
    """A rule written out as a dense mask gives the rule's result exactly
    (bottom-right causal with L < S, a sliding window, documents)."""
    q, k, v = _rand((1, 2, 40, 8), 78), _rand((1, 2, 70, 8), 79), _rand((1, 2, 70, 8), 80)
    cases = [(CAUSAL_LR, 0, None, _band(40, 70, -30, 70)),
             (SLIDING, 9, None, _band(40, 70, 0, 8))]
    doc = np.repeat([0, 1, 2], [25, 30, 15]).astype(np.int32)
    same = doc[:40, None] == doc[None, :70]
    cases.append((DOCUMENT, 0, doc, same & _band(40, 70, 0, 70)))
    for kind, win, d, m in cases:
        o1, l1 = orc.attention(q, k, v, kind, 0.4, win, d, softcap=5.0)
        o2, l2 = orc.attention(q, k, v, DENSE, 0.4, softcap=5.0, mask=m)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), kind
        a = orc.block_mask(kind, 40, 70, win, d, block=16)
        b = orc.block_mask(DENSE, 40, 70, block=16, mask=m)
        assert all(np.array_equal(x, y) for x, y in zip(a, b)), kind


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def _torch_attention(q, k, v, keep, scale, softcap=0.0):
    """Masked softmax attention composed of torch ops (fp64, CPU), for
    autograd: keep [L, S] or [B, 1, L, S] boolean."""
    sc = (q @ k.transpose(-2, -1).contiguous()) * scale
    if softcap > 0.0:
        sc = softcap * torch.tanh(sc / softcap)
    sc = sc.masked_fill(~keep, float("-inf"))
    return torch.softmax(sc, dim=-1) @ v


def check_backward_matches_autograd(orc):
    """dq, dk, dv of sum(dO * O) equal torch autograd through the composed
    attention (fp64), for the rule kinds, a dense mask, the soft-cap, key
    padding and grouped K/V heads (the gradient of a shared head is the sum
    over the query heads that read it)."""
    B, H, Hk, L, S, E = 2, 4, 2, 23, 31, 8
    rng = np.random.default_rng(81)
    doc = np.repeat([0, 1, 2], [9, 12, 10]).astype(np.int32)
    dense = rng.random((L, S)) < 0.4
    dense[np.arange(L), rng.integers(0, S, L)] = True
    i, j = np.arange(L)[:, None], np.arange(S)[None, :]
    cases = [
        (NONE, 0, None, None, np.ones((L, S), bool), 0.0, None),
        (CAUSAL_LR, 0, None, None, j <= i + (S - L), 0.0, None),
        (SLIDING, 5, None, None, (j <= i) & (i - j < 5), 7.0, None),
        (DOCUMENT_BIDIR, 0, doc, None, doc[:L, None] == doc[None, :S], 0.0, None),
        (DENSE, 0, None, dense, dense, 3.0, None),
        (CAUSAL_LR, 0, None, None, j <= i + (S - L), 0.0, ([2, 0], [31, 20])),
    ]
    q, dout = _rand((B, H, L, E), 82), _rand((B, H, L, E), 85)
    kk, vv = _rand((B, Hk, S, E), 83), _rand((B, Hk, S, E), 84)
    for kind, win, d, m, keep, cap, pad in cases:
        ke, ve = (np.repeat(x, H // Hk, axis=1) for x in (kk, vv))
        keep_b = np.broadcast_to(keep, (B, 1, L, S)).copy()
        if pad is not None:
            for b in range(B):
                keep_b[b, :, :, :pad[0][b]] = False
                keep_b[b, :, :, pad[1][b]:] = False
        dq, dk, dv = orc.attention_backward(q, ke, ve, dout, kind, 0.3, win, d, cap,
                                            key_start=None if pad is None else pad[0],
                                            key_end=None if pad is None else pad[1], mask=m)
        dk = dk.reshape(B, Hk, H // Hk, S, E).sum(2)
        dv = dv.reshape(B, Hk, H // Hk, S, E).sum(2)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, kk, vv))
        o = _torch_attention(tq, tk.repeat_interleave(H // Hk, 1), tv.repeat_interleave(H // Hk, 1),
                             torch.from_numpy(keep_b), 0.3, cap)
        (o * torch.from_numpy(dout)).sum().backward()
        for got, t in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.abs(got - t.grad.numpy()).max() <= 1e-12, kind


def check_backward_finite_differences(orc):
    """Gradients against central differences of the oracle's own forward
    (f = sum(dO * O)) on sampled elements of q, k and v, with the soft-cap
    and a sliding window."""
    rng = np.random.default_rng(86)
    q, k, v, dout = _rand((1, 2, 9, 4), 87), _rand((1, 2, 13, 4), 88), _rand((1, 2, 13, 4), 89), \
        _rand((1, 2, 9, 4), 90)
    args = dict(kind=SLIDING_LR, scale=0.45, window=6, softcap=2.5)
    dq, dk, dv = orc.attention_backward(q, k, v, dout, args["kind"], args["scale"], args["window"],
                                        softcap=args["softcap"])

    def f(q_, k_, v_):
        o, _ = orc.attention(q_, k_, v_, args["kind"], args["scale"], args["window"],
                             softcap=args["softcap"])
        return float((o * dout).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = (q, k, v)
            pos = {"q": 0, "k": 1, "v": 2}[name]
            fp = f(*[xp if t == pos else a[t] for t in range(3)])
            fm = f(*[xm if t == pos else a[t] for t in range(3)])
            assert abs((fp - fm) / (2 * h) - g[idx]) <= 1e-7, (name, idx)


def check_backward_dq_rows(orc):
    """The rows form of dq equals those rows of the whole backward."""
    q, k, v, dout = _rand((2, 2, 11, 4), 95), _rand((2, 2, 17, 4), 96), _rand((2, 2, 17, 4), 97), \
        _rand((2, 2, 11, 4), 98)
    dq, _, _ = orc.attention_backward(q, k, v, dout, CAUSAL_LR, 0.4, softcap=3.0)
    rows = np.array([0, 5, 11, 30, 43])
    got = orc.attention_backward_dq_rows(q, k, v, dout, CAUSAL_LR, 0.4, rows, softcap=3.0)
    assert np.abs(got - dq.reshape(-1, 4)[rows]).max() <= 1e-15


def check_backward_empty_rows_and_unseen_keys(orc):
    """A query row with no live key gets dq = 0; a key no query sees gets
    dk = dv = 0."""
    q, k, v, dout = _rand((1, 1, 6, 4), 91), _rand((1, 1, 8, 4), 92), _rand((1, 1, 8, 4), 93), \
        _rand((1, 1, 6, 4), 94)
    m = np.ones((6, 8), bool)
    m[3] = False
    m[:, 5] = False
    dq, dk, dv = orc.attention_backward(q, k, v, dout, DENSE, 0.5, mask=m)
    assert np.all(dq[0, 0, 3] == 0.0) and np.any(dq[0, 0, 2] != 0.0)
    assert np.all(dk[0, 0, 5] == 0.0) and np.all(dv[0, 0, 5] == 0.0)
    assert np.any(dk[0, 0, 4] != 0.0) and np.any(dv[0, 0, 4] != 0.0)


ALL_CHECKS = [
    check_flex_table_densities,
    check_live_pair_closed_forms,
    check_block_mask_worked_examples,
    check_block_mask_window_closed_form,
    check_block_mask_ragged_tail,
    check_tiled_softmax_equivalence,
    check_weights_are_a_distribution,
    check_uniform_v,
    check_window_one_is_identity,
    check_causal_first_row,
    check_two_key_closed_form,
    check_scipy_softmax,
    check_empty_rows,
    check_causal_prefix_invariance,
    check_sliding_equals_window_slice,
    check_document_isolation,
    check_library_equivalence,
    check_softcap_limits,
    check_kv_cache_alignment_example,
    check_lower_right_is_last_rows,
    check_variant_live_pair_closed_forms,
    check_bidirectional_document_isolation,
    check_variant_block_masks,
    check_key_padding_equals_truncation,
    check_key_padding_per_batch,
    check_dense_mask_table_densities,
    check_pack_mask_worked_example,
    check_pack_mask_numpy,
    check_dense_mask_matches_sdpa,
    check_dense_mask_empty_rows,
    check_dense_mask_equals_rules,
    check_backward_matches_autograd,
    check_backward_finite_differences,
    check_backward_empty_rows_and_unseen_keys,
    check_backward_dq_rows,
]
