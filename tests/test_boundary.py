"""The C ABI library: it loads, exports every function include/bsattn.h
declares, and its host-side validation returns the documented status codes.

Validation cases pass placeholder device addresses that are never
dereferenced: each case is invalid, so the library returns before it enqueues
anything. They run only where no GPU is visible, so a validation bug can never
turn into a launch on fake addresses.
"""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_attention_35_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="placeholder-address validation runs only without a GPU")

OK, INVALID, UNSUPPORTED = 0, -1, -2
FAKE = 0x10000  # 16-byte aligned placeholder address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("attn_build_block_mask", "attn_forward", "attn_forward_gqa",
                     "attn_num_blocks", "attn_status_string", "attn_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bsa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in bsattn.h but not exported"


def test_num_blocks():
    assert [bsa.num_blocks(n) for n in (0, 1, 127, 128, 129, 256, 8192, 32768)] == \
        [0, 1, 1, 1, 2, 2, 64, 256]
    lib = bsa._load()
    assert lib.attn_num_blocks(-1, 128) == -1
    assert lib.attn_num_blocks(100, 64) == -1


def test_status_strings():
    lib = bsa._load()
    assert lib.attn_status_string(OK) == b"ok"
    assert lib.attn_status_string(INVALID) == b"invalid argument"
    assert lib.attn_status_string(UNSUPPORTED) == b"unsupported"
    assert lib.attn_status_string(-3) == b"HIP runtime error"


def _bm(**kw):
    s = bsa._BlockMaskStruct()
    for f in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices", "schedule"):
        setattr(s, f, FAKE)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _build(kind=1, window=0, doc=None, q_len=256, kv_len=256, block=128, bm=None):
    lib = bsa._load()
    bm = _bm() if bm is None else bm
    return lib.attn_build_block_mask(kind, window, doc, q_len, kv_len, block, ctypes.byref(bm), None)


BUILD_CASES = [
    ("custom_kind_needs_its_builder", dict(kind=7), INVALID, "attn_build_block_mask_custom"),
    ("unknown_kind", dict(kind=8), INVALID, "kind"),
    ("negative_kind", dict(kind=-1), INVALID, "kind"),
    ("lower_right_window_zero", dict(kind=5, window=0), INVALID, "window"),
    ("bidirectional_document_without_ids", dict(kind=6, doc=None), INVALID, "document"),
    ("negative_len", dict(q_len=-1), INVALID, "negative"),
    ("block_64", dict(block=64), UNSUPPORTED, "block_size"),
    ("window_zero", dict(kind=2, window=0), INVALID, "window"),
    ("document_without_ids", dict(kind=3, doc=None), INVALID, "document"),
    ("null_array", dict(bm=_bm(kv_indices=None)), INVALID, "null"),
    ("too_many_kv_blocks", dict(kv_len=16385 * 128), UNSUPPORTED, "kv blocks"),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code,words", BUILD_CASES, ids=[c[0] for c in BUILD_CASES])
def test_build_block_mask_validation(name, kw, code, words):
    assert _build(**kw) == code
    assert words in bsa._load().attn_last_error().decode()


@no_gpu
def test_build_null_struct():
    lib = bsa._load()
    assert lib.attn_build_block_mask(1, 0, None, 256, 256, 128, None, None) == INVALID


def _built_mask(L=256, S=256, kind=1, window=0, doc=None):
    return _bm(q_len=L, kv_len=S, block_size=128, num_q_blocks=-(-L // 128),
               num_kv_blocks=-(-S // 128), kind=kind, window=window, document_id=doc)


WS_FAKE = 0x100000  # 256-byte aligned placeholder workspace, never dereferenced


def _fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, dtype=1, B=1, H=2, L=256, S=256, E=64,
         qs=None, ks=None, vs=None, os_=None, bm=None, score_mod=0, softcap=0.0, scale=0.125,
         ws=WS_FAKE, ws_bytes=1 << 30):
    lib = bsa._load()
    bm = _built_mask(L, S) if bm is None else bm

    def st(x):
        return None if x is None else (ctypes.c_int64 * 4)(*x)

    return lib.attn_forward(q, k, v, o, lse, dtype, B, H, L, S, E, st(qs), st(ks), st(vs),
                            st(os_), ctypes.byref(bm), score_mod, softcap, scale, ws, ws_bytes,
                            None)


FWD_CASES = [
    ("null_q", dict(q=None), INVALID, "non-null"),
    ("unknown_dtype", dict(dtype=9), UNSUPPORTED, "dtype"),
    ("zero_heads", dict(H=0), INVALID, "sizes"),
    ("head_dim_128", dict(E=128), UNSUPPORTED, "head dim"),
    ("mask_for_other_lengths", dict(bm=_built_mask(512, 512)), INVALID, "built for"),
    ("mask_not_built", dict(bm=_built_mask(256, 256, kind=2, window=0)), INVALID, "inconsistent"),
    ("document_mask_without_ids", dict(bm=_built_mask(256, 256, kind=3)), INVALID, "inconsistent"),
    ("lower_right_window_mask_not_built", dict(bm=_built_mask(256, 256, kind=5, window=0)), INVALID,
     "inconsistent"),
    ("bidirectional_mask_without_ids", dict(bm=_built_mask(256, 256, kind=6)), INVALID,
     "inconsistent"),
    ("custom_mask_without_bits", dict(bm=_built_mask(256, 256, kind=7)), INVALID, "inconsistent"),
    ("unknown_mask_kind", dict(bm=_built_mask(256, 256, kind=8)), INVALID, "inconsistent"),
    ("unknown_score_mod", dict(score_mod=4), INVALID, "score_mod"),
    ("softcap_zero", dict(score_mod=1, softcap=0.0), INVALID, "soft-cap"),
    ("softcap_nan", dict(score_mod=1, softcap=float("nan")), INVALID, "soft-cap"),
    ("scale_zero", dict(scale=0.0), INVALID, "scale"),
    ("scale_negative", dict(scale=-0.125), INVALID, "scale"),
    ("scale_inf", dict(scale=float("inf")), INVALID, "scale"),
    ("misaligned_k", dict(k=FAKE + 2), INVALID, "aligned"),
    ("head_dim_stride", dict(qs=(2 * 256 * 128, 256 * 128, 128, 2)), INVALID, "head-dim stride"),
    ("row_stride_breaks_alignment", dict(ks=(2 * 256 * 65, 256 * 65, 65, 1)), INVALID, "alignment"),
    ("negative_stride", dict(vs=(2 * 256 * 64, -256 * 64, 64, 1)), INVALID, "negative"),
    ("k_seq_stride_too_large", dict(ks=(0, 0, (1 << 24) + 8, 1)), UNSUPPORTED, "sequence stride"),
    ("v_seq_stride_too_large", dict(vs=(0, 0, (1 << 24) + 8, 1)), UNSUPPORTED, "sequence stride"),
    ("workspace_missing", dict(ws=None, ws_bytes=0), INVALID, "workspace"),
    ("workspace_misaligned", dict(ws=WS_FAKE + 16), INVALID, "workspace"),
    ("workspace_too_small", dict(ws_bytes=1024), INVALID, "workspace"),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code,words", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_validation(name, kw, code, words):
    assert _fwd(**kw) == code
    msg = bsa._load().attn_last_error().decode()
    assert words in msg, msg


def _fwd_gqa(H=4, H_kv=2, L=256, S=256, ks=None, ws_bytes=1 << 30):
    lib = bsa._load()
    bm = _built_mask(L, S)
    st = (lambda x: None if x is None else (ctypes.c_int64 * 4)(*x))
    return lib.attn_forward_gqa(FAKE, FAKE, FAKE, FAKE, None, 1, 1, H, H_kv, L, S, 64, None,
                                st(ks), None, None, ctypes.byref(bm), 0, 0.0, 0.125, WS_FAKE,
                                ws_bytes, None)


GQA_CASES = [
    ("kv_heads_zero", dict(H_kv=0), INVALID, "share"),
    ("kv_heads_not_a_divisor", dict(H=6, H_kv=4), INVALID, "share"),
    ("kv_heads_above_heads", dict(H=2, H_kv=4), INVALID, "share"),
    ("kv_head_stride_checked", dict(ks=(2 * 256 * 64, 65, 64, 1)), INVALID, "alignment"),
]


@no_gpu
def test_forward_gqa_single_kv_head_stride_unused():
    # with one K/V head its head stride is never used, so any value passes
    # validation; the call then fails only on the (too small) workspace
    assert _fwd_gqa(H=4, H_kv=1, ks=(256 * 64, 65, 64, 1), ws_bytes=16) == INVALID
    assert "workspace" in bsa._load().attn_last_error().decode()


@no_gpu
@pytest.mark.parametrize("name,kw,code,words", GQA_CASES, ids=[c[0] for c in GQA_CASES])
def test_forward_gqa_validation(name, kw, code, words):
    assert _fwd_gqa(**kw) == code
    msg = bsa._load().attn_last_error().decode()
    assert words in msg, msg


def test_binding_rejects_kv_heads_that_do_not_divide():
    q = torch.zeros(1, 6, 128, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsa.attention(q, k, k, block_mask=None)


@no_gpu
def test_forward_null_mask():
    lib = bsa._load()
    assert lib.attn_forward(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 1, 128, 128, 64, None, None,
                            None, None, None, 0, 0.0, 0.125, None, 0, None) == INVALID


def _ws_size(dtype, B, H, L, S=None):
    S = L if S is None else S
    n = ctypes.c_size_t(123)
    bm = _built_mask(L, S)
    assert bsa._load().attn_forward_workspace_size(dtype, B, H, ctypes.byref(bm),
                                                   ctypes.byref(n)) == OK
    return n.value


def test_workspace_size():
    # split items need ticket counters (a fixed region of 2048 int32, the
    # most a splitting call has) and one fp32 partial slot per query block
    # and head (the first of the two chunks to finish leaves its partial) of
    # 4 waves x 32 registers x 64 lanes plus a max and a sum per row
    slot = (4 * 32 * 64 + 2 * 128) * 4
    nq, bh = 64, 8
    counters = 2048 * 4
    assert _ws_size(1, 1, 8, 8192) == counters + nq * bh * slot
    assert _ws_size(2, 2, 4, 8192) == counters + nq * bh * slot
    assert _ws_size(1, 1, 1, 300) == counters + 3 * 1 * slot
    assert _ws_size(0, 1, 8, 8192) == 0            # fp32 never splits
    assert _ws_size(1, 1, 32, 8192) == counters + 64 * 32 * slot  # 2048 items
    assert _ws_size(1, 1, 33, 8192) == 0           # many items: no split
    assert _ws_size(1, 1, 8, 0) == 0               # no query blocks
    # decode (one query block, many kv blocks): split-KV, k = min(64,
    # ceil(512 / (B*H*nq)), nk / 2) chunks of one slot each
    assert _ws_size(1, 1, 8, 1, 8192) == counters + 1 * 32 * 8 * slot      # k = 32
    assert _ws_size(2, 4, 32, 16, 8192) == counters + 1 * 4 * 128 * slot   # k = 4
    assert _ws_size(1, 1, 8, 1, 640) == counters + 1 * 8 * slot            # nk = 5: two-way split


@no_gpu
def test_workspace_size_validation():
    lib = bsa._load()
    n = ctypes.c_size_t(0)
    assert lib.attn_forward_workspace_size(1, 1, 1, None, ctypes.byref(n)) == INVALID
    bm = _built_mask()
    assert lib.attn_forward_workspace_size(1, 0, 1, ctypes.byref(bm), ctypes.byref(n)) == INVALID
    assert lib.attn_forward_workspace_size(1, 1, 1, ctypes.byref(bm), None) == INVALID


def test_binding_rejects_cpu_tensors():
    q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsa.attention(q, q, q, block_mask=None)


def test_binding_rejects_float64():
    q = torch.zeros(1, 1, 128, 64, dtype=torch.float64)
    with pytest.raises(ValueError):
        bsa.attention(q, q, q, block_mask=None)


def test_mask_words():
    lib = bsa._load()
    assert [lib.attn_mask_words(n) for n in (0, 1, 128, 129, 8192)] == [0, 4, 4, 8, 256]
    assert lib.attn_mask_words(-1) == -1
    assert bsa.mask_words(1000) == 32


def _build_custom(bits=FAKE, q_len=256, kv_len=256, block=128, bm=None):
    lib = bsa._load()
    bm = _bm() if bm is None else bm
    return lib.attn_build_block_mask_custom(bits, q_len, kv_len, block, ctypes.byref(bm), None)


CUSTOM_BUILD_CASES = [
    ("null_bits", dict(bits=None), INVALID, "bits"),
    ("misaligned_bits", dict(bits=FAKE + 4), INVALID, "aligned"),
    ("negative_len", dict(kv_len=-3), INVALID, "negative"),
    ("block_64", dict(block=64), UNSUPPORTED, "block_size"),
    ("null_array", dict(bm=_bm(schedule=None)), INVALID, "null"),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code,words", CUSTOM_BUILD_CASES, ids=[c[0] for c in CUSTOM_BUILD_CASES])
def test_build_block_mask_custom_validation(name, kw, code, words):
    assert _build_custom(**kw) == code
    assert words in bsa._load().attn_last_error().decode()


PACK_CASES = [
    ("negative_len", dict(q_len=-1), INVALID, "negative"),
    ("short_row_stride", dict(row_stride=99), INVALID, "row_stride"),
    ("null_dense", dict(dense=None), INVALID, "non-null"),
    ("null_bits", dict(bits=None), INVALID, "non-null"),
    ("misaligned_bits", dict(bits=FAKE + 8), INVALID, "aligned"),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code,words", PACK_CASES, ids=[c[0] for c in PACK_CASES])
def test_pack_mask_validation(name, kw, code, words):
    a = dict(dense=FAKE, row_stride=100, q_len=10, kv_len=100, bits=FAKE)
    a.update(kw)
    lib = bsa._load()
    assert lib.attn_pack_mask(a["dense"], a["row_stride"], a["q_len"], a["kv_len"], a["bits"], None) == code
    assert words in lib.attn_last_error().decode()


def test_binding_custom_kind_needs_its_own_constructor():
    with pytest.raises(ValueError, match="create_block_mask_from_dense"):
        bsa.create_block_mask("custom", 128, 128)


def _bwd(dtype=1, B=1, H=2, H_kv=2, L=256, S=256, E=64, bm=None, score_mod=0, softcap=0.0, scale=0.125,
         ws=FAKE, ws_bytes=1 << 30, ptrs=None):
    lib = bsa._load()
    bm = _built_mask(L, S) if bm is None else bm
    p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE)
    p.update(ptrs or {})
    return lib.attn_backward(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"], p["dv"],
                             dtype, B, H, H_kv, L, S, E, ctypes.byref(bm), score_mod, softcap, scale,
                             None, None, ws, ws_bytes, None)


BWD_CASES = [
    ("fp32_misaligned_dk", dict(dtype=0, ptrs=dict(dk=FAKE + 4)), INVALID, "aligned"),
    ("unknown_dtype", dict(dtype=9), UNSUPPORTED, "dtype"),
    ("head_dim_128", dict(E=128), UNSUPPORTED, "head dim"),
    ("kv_heads_not_dividing", dict(H=3, H_kv=2), INVALID, "share"),
    ("null_dout", dict(ptrs=dict(dout=None)), INVALID, "non-null"),
    ("null_lse", dict(ptrs=dict(lse=None)), INVALID, "non-null"),
    ("misaligned_dq", dict(ptrs=dict(dq=FAKE + 2)), INVALID, "aligned"),
    ("mask_for_other_lengths", dict(bm=_built_mask(128, 256)), INVALID, "q_len"),
    ("bad_score_mod", dict(score_mod=5), INVALID, "score_mod"),
    ("softcap_zero", dict(score_mod=1, softcap=0.0), INVALID, "soft-cap"),
    ("bad_scale", dict(scale=float("nan")), INVALID, "scale"),
    ("workspace_too_small", dict(ws_bytes=16), INVALID, "workspace"),
    ("workspace_misaligned", dict(ws=FAKE + 16), INVALID, "workspace"),
    ("custom_mask_without_bits", dict(bm=_built_mask(256, 256, kind=7)), INVALID, "inconsistent"),
]


@no_gpu
@pytest.mark.parametrize("name,kw,code,words", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_validation(name, kw, code, words):
    assert _bwd(**kw) == code
    assert words in bsa._load().attn_last_error().decode()


def test_backward_workspace_size():
    lib = bsa._load()
    n = ctypes.c_size_t(0)
    bm = _built_mask(300, 700)  # nq = 3, nk = 6
    assert lib.attn_backward_workspace_size(2, 4, 2, ctypes.byref(bm), ctypes.byref(n)) == OK
    al = lambda x: (x + 255) // 256 * 256
    fixed = 2 * 8192 + 2 * al(2 * 4 * 300 * 4) + 2 * al(6 * 4) + 2 * al(6 * 3 * 4) + al((4 + 8 * 6) * 4)
    # few items: partial slots for split dK/dV (6 kv blocks x 2 x B*H_kv) and dQ (3 x 2 x B*H)
    assert n.value == fixed + al(6 * 2 * 4 * 16384 * 4) + al(3 * 2 * 8 * 8192 * 4)
    assert lib.attn_backward_workspace_size(0, 4, 2, ctypes.byref(bm), ctypes.byref(n)) == INVALID
    assert lib.attn_backward_workspace_size(2, 4, 3, ctypes.byref(bm), ctypes.byref(n)) == INVALID


# The binding's own argument checks (host logic, no GPU): every tensor the
# library writes through must have exactly the shape, dtype and device it
# assumes, or the call is refused before any pointer crosses the boundary.

def _fwd_tensors(dt=torch.bfloat16, B=2, H=4, Hk=2, L=256, S=384, E=64):
    q = torch.zeros(B, H, L, E, dtype=dt)
    k = torch.zeros(B, Hk, S, E, dtype=dt)
    v = torch.zeros(B, Hk, S, E, dtype=dt)
    return q, k, v


def test_forward_arg_checks_accept_a_valid_call():
    q, k, v = _fwd_tensors()
    out = torch.empty_like(q)
    lse = torch.empty(2, 4, 256)
    ws = torch.zeros(64, dtype=torch.uint8)
    ks = torch.zeros(2, dtype=torch.int32)
    assert bsa._check_forward_args(q, k, v, out, lse, ws, ks, ks) == (2, 4, 2, 256, 384, 64)
    assert bsa._check_forward_args(q, k, v, None, None, None, None, None) == (2, 4, 2, 256, 384, 64)


@pytest.mark.parametrize("case", [
    "out_small", "out_dtype", "out_stride", "out_device", "lse_shape", "lse_dtype",
    "lse_noncontig", "lse_device", "ws_dtype", "ws_device", "key_dtype", "key_shape",
    "key_noncontig", "key_device", "k_dim", "k_head_dim", "heads_not_dividing"])
def test_forward_arg_checks_reject(case):
    q, k, v = _fwd_tensors()
    out, lse, ws, ks = torch.empty_like(q), torch.empty(2, 4, 256), None, None
    meta = torch.device("meta")
    if case == "out_small":
        out = torch.empty(2, 4, 128, 64, dtype=q.dtype)
    elif case == "out_dtype":
        out = torch.empty(2, 4, 256, 64, dtype=torch.float16)
    elif case == "out_stride":
        out = torch.empty(2, 4, 64, 256, dtype=q.dtype).transpose(2, 3)
    elif case == "out_device":
        out = torch.empty(2, 4, 256, 64, dtype=q.dtype, device=meta)
    elif case == "lse_shape":
        lse = torch.empty(2, 4, 255)
    elif case == "lse_dtype":
        lse = torch.empty(2, 4, 256, dtype=torch.float64)
    elif case == "lse_noncontig":
        lse = torch.empty(2, 256, 4).transpose(1, 2)
    elif case == "lse_device":
        lse = torch.empty(2, 4, 256, device=meta)
    elif case == "ws_dtype":
        ws = torch.zeros(16, dtype=torch.int32)
    elif case == "ws_device":
        ws = torch.zeros(64, dtype=torch.uint8, device=meta)
    elif case == "key_dtype":
        ks = torch.zeros(2, dtype=torch.int64)
    elif case == "key_shape":
        ks = torch.zeros(3, dtype=torch.int32)
    elif case == "key_noncontig":
        ks = torch.zeros(4, dtype=torch.int32)[::2]
    elif case == "key_device":
        ks = torch.zeros(2, dtype=torch.int32, device=meta)
    elif case == "k_dim":
        k = k[0]
    elif case == "k_head_dim":
        k = torch.zeros(2, 2, 384, 32, dtype=q.dtype)
        v = k.clone()
    elif case == "heads_not_dividing":
        k = torch.zeros(2, 3, 384, 64, dtype=q.dtype)
        v = k.clone()
    with pytest.raises(ValueError):
        bsa._check_forward_args(q, k, v, out, lse, ws, ks, None)


@pytest.mark.parametrize("case", [
    "k_dim", "k_head_dim", "k_batch", "v_shape", "heads_not_dividing", "lse_device", "lse_shape",
    "out_shape", "dout_dtype", "key_noncontig", "key_device"])
def test_backward_arg_checks_reject(case):
    q, k, v = _fwd_tensors()
    out, dout, lse, ks = torch.empty_like(q), torch.empty_like(q), torch.empty(2, 4, 256), None
    meta = torch.device("meta")
    if case == "k_dim":
        k = k[0]
    elif case == "k_head_dim":
        k = torch.zeros(2, 2, 384, 32, dtype=q.dtype)
        v = k.clone()
    elif case == "k_batch":
        k = torch.zeros(1, 2, 384, 64, dtype=q.dtype)
        v = k.clone()
    elif case == "v_shape":
        v = torch.zeros(2, 2, 383, 64, dtype=q.dtype)
    elif case == "heads_not_dividing":
        k = torch.zeros(2, 3, 384, 64, dtype=q.dtype)
        v = k.clone()
    elif case == "lse_device":
        lse = torch.empty(2, 4, 256, device=meta)
    elif case == "lse_shape":
        lse = torch.empty(2, 4, 128)
    elif case == "out_shape":
        out = torch.empty(2, 4, 128, 64, dtype=q.dtype)
    elif case == "dout_dtype":
        dout = torch.empty_like(q, dtype=torch.float16)
    elif case == "key_noncontig":
        ks = torch.zeros(4, dtype=torch.int32)[::2]
    elif case == "key_device":
        ks = torch.zeros(2, dtype=torch.int32, device=meta)
    with pytest.raises(ValueError):
        bsa._check_backward_args(q, k, v, out, lse, dout, ks, None)


def test_backward_arg_checks_accept_a_valid_call():
    q, k, v = _fwd_tensors()
    got = bsa._check_backward_args(q, k, v, torch.empty_like(q), torch.empty(2, 4, 256),
                                   torch.empty_like(q), torch.zeros(2, dtype=torch.int32), None)
    assert got == (2, 4, 2, 256, 384, 64)


def test_schedule_len():
    lib = bsa._load()
    # a 4-entry header and two 4-entry descriptors per query block
    for L, S in ((0, 0), (1, 8192), (256, 256), (300, 200), (8192, 8192), (32768, 32768)):
        assert lib.attn_block_mask_schedule_len(L, S, 128) == 4 + 8 * ((L + 127) // 128)
        assert bsa.schedule_len(L, S) == 4 + 8 * ((L + 127) // 128)
    assert lib.attn_block_mask_schedule_len(-1, 128, 128) == -1
    assert lib.attn_block_mask_schedule_len(128, -1, 128) == -1
    assert lib.attn_block_mask_schedule_len(128, 128, 64) == -1
    with pytest.raises(bsa.BsattnError):
        bsa.schedule_len(-5, 10)


@no_gpu
def test_forward_noalloc_refuses_shapes_beyond_its_scratch():
    # 2048 split items (B*H*nq) with a 33 KiB partial slot each: above 64 MiB.
    # Refused on the host before the scratch is looked up or anything enqueued.
    lib = bsa._load()
    bm = _built_mask(8192, 8192)
    assert lib.attn_forward_noalloc(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 32, 32, 8192, 8192, 64,
                                    None, None, None, None, ctypes.byref(bm), 0, 0.0, 0.125,
                                    None, None, None) == UNSUPPORTED
    assert "scratch" in lib.attn_last_error().decode()
    assert lib.attn_forward_noalloc(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 2, 2, 256, 256, 64,
                                    None, None, None, None, None, 0, 0.0, 0.125,
                                    None, None, None) == INVALID
