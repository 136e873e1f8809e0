"""attn_forward_noalloc (the allocation-free forward for callers that cannot
allocate) against attn_forward / attn_forward_padded through the C ABI: two
calls in a row on the same per-GPU scratch, the second with a smaller input,
each equal bit for bit to the workspace entry point (the same kernels), and
so within the forward's tolerance of it. Also: a shape needing more scratch
than the array holds is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import block_sparse_attention_35_amd as bsa
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def _both(w: wl.Workload, dev, seed=0):
    print(f"no-alloc: {w.name} B={w.B} H={w.H} H_kv={w.kv_heads} L={w.L} S={w.S}", flush=True)
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, seed))
    doc = wl.make_doc(w)
    bm = bsa.create_block_mask(w.kind, w.L, w.S, window=w.window or None,
                               document_id=None if doc is None else torch.from_numpy(doc).to(dev),
                               device=dev)
    sm = "softcap" if w.softcap else None
    o_ref, lse_ref = bsa.attention(q, k, v, bm, score_mod=sm, softcap=w.softcap or 30.0,
                                   scale=w.scale, return_lse=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.L), float("nan"), dtype=torch.float32, device=dev)
    bsa.attention_noalloc(q, k, v, bm, out=o, lse=lse, score_mod=sm, softcap=w.softcap or 30.0,
                          scale=w.scale)
    torch.cuda.synchronize()
    return o, lse, o_ref, lse_ref, bsa.workspace_size(q, bm)


def _same(o, lse, o_ref, lse_ref, name):
    # the same kernels on the same inputs: identical bits, which is within
    # any tolerance (max-abs 1e-2 / mean-abs 1e-3 for bf16 and fp16)
    assert torch.equal(o, o_ref), f"{name}: O differs from attn_forward's"
    assert torch.equal(lse, lse_ref), f"{name}: lse differs from attn_forward's"
    err = (o.float() - o_ref.float()).abs()
    assert float(err.max()) <= 1e-2 and float(err.mean()) <= 1e-3


def test_noalloc_two_calls_second_smaller(dev):
    big = wl.WORKLOADS["causal_8192_bf16"]                      # split items: scratch in use
    small = wl.Workload("noalloc_causal_2304_bf16", 1, 3, 2304, 2304, 64, "bf16", wl.MASK_CAUSAL)
    for w in (big, small):
        o, lse, o_ref, lse_ref, need = _both(w, dev)
        assert need > 0, f"{w.name} should use the scratch"
        _same(o, lse, o_ref, lse_ref, w.name)


def test_noalloc_other_paths(dev):
    # split-KV decode (the scratch holds chunk partials), fp16 documents with
    # the soft-cap (split items), a window with no scratch at all, fp32
    cases = [wl.WORKLOADS["decode_gqa_b8_h32_kv8_s8192_bf16"],
             wl.Workload("noalloc_doc_f16", 1, 4, 3000, 3000, 64, "f16", wl.MASK_DOCUMENT, 0,
                         (700, 1900), 30.0),
             wl.WORKLOADS["sliding_8192_w256_bf16"],
             wl.WORKLOADS["causal_256_f32"]]
    for w in cases:
        o, lse, o_ref, lse_ref, _ = _both(w, dev)
        _same(o, lse, o_ref, lse_ref, w.name)


def test_noalloc_padded_matches_padded(dev):
    w = wl.WORKLOADS["causal_8192_keypad_b2_bf16"].with_(L=2048, S=2048,
                                                         key_ranges=((0, 2048), (300, 1700)))
    q, k, v = (x.to(dev) for x in wl.make_qkv(w, 3))
    bm = bsa.create_block_mask(w.kind, w.L, w.S, device=dev)
    ks = torch.tensor([a for a, _ in w.key_ranges], dtype=torch.int32, device=dev)
    ke = torch.tensor([b for _, b in w.key_ranges], dtype=torch.int32, device=dev)
    o_ref, lse_ref = bsa.attention(q, k, v, bm, return_lse=True, key_start=ks, key_end=ke)
    o, lse = torch.empty_like(q), torch.empty_like(lse_ref)
    bsa.attention_noalloc(q, k, v, bm, out=o, lse=lse, key_start=ks, key_end=ke)
    torch.cuda.synchronize()
    _same(o, lse, o_ref, lse_ref, "padded")


def test_noalloc_refuses_a_shape_beyond_the_scratch(dev):
    # B*H*nq = 2048 split query blocks of a 33 KiB partial slot: 69 MB > 64 MiB
    H, L = 32, 8192
    q = torch.empty(1, H, L, 64, dtype=torch.bfloat16, device=dev)
    bm = bsa.create_block_mask("causal", L, L, device=dev)
    assert bsa.workspace_size(q, bm) > (64 << 20)
    with pytest.raises(bsa.BsattnError) as ei:
        bsa.attention_noalloc(q, q, q, bm, out=torch.empty_like(q))
    assert ei.value.status == -2 and "scratch" in str(ei.value)
