"""Host-side checks of the C ABI: the library loads without a GPU, exports
every function include/vit.h declares, and rejects invalid arguments with
the documented status before anything is enqueued (these calls never reach
a kernel launch: every case fails validation)."""

import ctypes
import os

import pytest

import vision_transformer_encoder_amd as vit

OK, NULL, ALIGN, SHAPE, UNSUP, SEQ, WS, ALIAS, HIP = range(9)

A = 0x7f0000000000  # fake, 256-aligned device addresses: never dereferenced
B = A + (1 << 30)
C = A + (2 << 30)
D = A + (3 << 30)
E = A + (4 << 30)
F = A + (5 << 30)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vit.library_path):
        pytest.fail("libvit.so is not built (run __graft_entry__.build())")
    return vit.require_library()


def test_exports_every_declared_function(lib):
    names = vit.declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(vit._SIGS), "binding and header disagree"


def test_version_and_status_strings(lib):
    import re
    hdr = open(vit.header_path).read()
    declared = int(re.search(r"#define VIT_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.vit_abi_version() == declared == vit.ABI_VERSION
    for s in range(9):
        assert lib.vit_status_string(s)
    assert lib.vit_status_string(0) == b"ok"


def _cu(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr


def test_quant_validation(lib):
    f = lib.vit_quant_fp8_block128
    assert f(None, 128, 4, 128, 1, B, C, None) == NULL
    assert f(A + 8, 128, 4, 128, 1, B, C, None) == ALIGN
    assert f(A, 132, 4, 128, 1, B, C, None) == ALIGN            # ld % 8
    assert f(A, 128, -1, 128, 1, B, C, None) == SHAPE
    assert f(A, 64, 4, 128, 1, B, C, None) == SHAPE             # ld < cols
    assert f(A, 128, 4, 128, 2, B, C, None) == UNSUP
    assert f(A, 128, 4, 128, 1, A, C, None) == ALIAS
    assert f(A, 128, 4, 128, 1, B, B + 16, None) == ALIAS       # codes overlap scales
    assert f(A, 128, 0, 128, 1, None, None, None) == OK          # empty: no-op


def test_e4m3_and_layernorm_validation(lib):
    assert lib.vit_e4m3_encode(A, B, -1, None) == SHAPE
    assert lib.vit_e4m3_encode(A, B, 0, None) == OK
    assert lib.vit_e4m3_encode(None, B, 10, None) == NULL
    assert lib.vit_e4m3_encode(A, A + 16, 100, None) == ALIAS
    f = lib.vit_layernorm_quant_fp8
    assert f(A, 1152, B, C, 1e-6, 10, 1000, D, E, None, None) == SHAPE    # D % 128
    assert f(A, 1152, B, C, -1.0, 10, 1152, D, E, None, None) == SHAPE    # eps < 0
    assert f(A, 1152, None, C, 1e-6, 10, 1152, D, E, None, None) == NULL
    assert f(A, 1152, B, C, 1e-6, 10, 1152, D, E, A, None) == ALIAS       # prequant over x
    assert f(A, 1152, B, C, 1e-6, 0, 1152, D, E, None, None) == OK


def test_gemm_validation(lib):
    f = lib.vit_fp8_block128_gemm
    assert f(A, B, C, D, 16, 256, 256, None, None, 3, E, None, None, None, None) == UNSUP
    assert f(A, B, C, D, 16, 0, 256, None, None, 0, E, None, None, None, None) == SHAPE
    assert f(A, B, C, D, 16, 256, 256, None, None, 1, E, None, None, None, None) == NULL  # residual
    assert f(A, B, C, D, 16, 256, 256, None, None, 2, None, None, E, None, None) == NULL  # codes
    assert f(A, B, C, D, 16, 256, 256, None, None, 0, A + 64, None, None, None, None) == ALIAS
    assert f(A, B, C + 8, D, 16, 256, 256, None, None, 0, E, None, None, None, None) == ALIGN
    # in-place residual (same pointer) passes validation up to the overlap check of other inputs
    assert f(A, B, C, D, 16, 256, 256, None, E + 2, 1, E, None, None, None, None) == ALIGN
    assert f(A, B, C, D, 0, 256, 256, None, None, 0, E, None, None, None, None) == OK
    g = lib.vit_bf16_gemm
    assert g(A, 0, B, 16, 64, 12, None, None, 0, C, 64, None) == SHAPE   # K % 8
    assert g(A, 0, B, 16, 64, 64, None, None, 5, C, 64, None) == UNSUP
    assert g(A, 0, B, 16, 64, 64, None, None, 0, C, 32, None) == SHAPE   # ld_out < N
    assert g(A, 0, B, 16, 64, 64, None, None, 0, B, 64, None) == ALIAS
    assert g(A, 1, None, 16, 64, 64, None, None, 0, C, 64, None) == NULL


def test_rope_validation(lib):
    f = lib.vit_rope2d
    pos = E
    assert f(A, A + 2304, 3456, pos, 10, 16, 70, 10000.0, None) == UNSUP
    assert f(A, A + 2304, 1000, pos, 10, 16, 72, 10000.0, None) == SHAPE     # ld < H*hd
    assert f(A, A + 2304, 3456, pos, 10, 16, 72, -1.0, None) == SHAPE        # theta
    assert f(A, A + 16, 3456, pos, 10, 16, 72, 10000.0, None) == ALIAS       # q, k overlap in a row
    assert f(A, None, 3456, pos, 10, 16, 72, 10000.0, None) == NULL
    assert f(A, A + 2304, 3456, A + 2304 * 2, 10, 16, 72, 10000.0, None) == ALIAS  # pos inside qkv
    assert f(A, A + 2304, 3456, pos, 0, 16, 72, 10000.0, None) == OK


def test_attention_validation(lib):
    f = lib.vit_attention
    lib.vit_attention_workspace_size.restype = ctypes.c_size_t
    wsb = lib.vit_attention_workspace_size()
    assert wsb > 0 and wsb % 256 == 0
    cu = _cu([0, 5, 9])
    bad = _cu([1, 5, 9])
    dec = _cu([0, 6, 5])

    def call(q=A, ld=3456, o=D, cuh=cu, ns=2, T=9, hd=72, scale=0.1, ws=F, nb=None):
        return f(q, q + 2304, q + 4608, ld, o, 1152, E, cuh, ns, T, 16, hd, ctypes.c_float(scale), ws,
                 ctypes.c_size_t(wsb if nb is None else nb), None)

    assert call(hd=64) == UNSUP
    assert call(ld=(1 << 24) + 8) == SHAPE       # row stride above 2^24
    assert call(cuh=bad) == SEQ
    assert call(cuh=dec, T=5) == SEQ
    assert call(T=10) == SEQ                      # last offset != total
    assert call(o=A + 64) == ALIAS                # output inside qkv
    assert call(cuh=None) == NULL
    assert call(scale=0.0) == SHAPE
    assert call(ld=3452) == ALIGN
    assert call(ws=None) == WS                    # workspace missing
    assert call(nb=wsb - 1) == WS                 # workspace too small
    assert call(ws=F + 8) == ALIGN                # workspace misaligned
    assert call(ws=A) == ALIAS                    # workspace over qkv
    assert call(ws=D - 16) == ALIAS               # workspace running into the output
    empty = _cu([0])
    assert call(cuh=empty, ns=0, T=0, ws=None) == OK


def test_attention_noalloc_validation(lib):
    """The workspace-free entry point validates like vit_attention (every
    case here fails before the library looks at a device)."""
    f = lib.vit_attention_noalloc
    lib.vit_attention_noalloc_scratch_size.restype = ctypes.c_size_t
    assert lib.vit_attention_noalloc_scratch_size() >= lib.vit_attention_workspace_size()
    cu = _cu([0, 5, 9])

    def call(q=A, ld=3456, o=D, cuh=cu, ns=2, T=9, hd=72, scale=0.1, cud=E):
        return f(q, q + 2304, q + 4608, ld, o, 1152, cud, cuh, ns, T, 16, hd, ctypes.c_float(scale), None)

    assert call(hd=64) == UNSUP
    assert call(cuh=_cu([1, 5, 9])) == SEQ
    assert call(T=10) == SEQ
    assert call(o=A + 64) == ALIAS
    assert call(cuh=None) == NULL
    assert call(cud=None) == NULL
    assert call(q=A + 8) == ALIGN
    assert call(ld=3452) == ALIGN
    assert call(ld=(1 << 24) + 8) == SHAPE
    assert call(scale=float("inf")) == SHAPE
    assert call(cuh=_cu([0]), ns=0, T=0) == OK


def test_merge_validation_statuses(lib):
    f = lib.vit_merge2x2_layernorm
    grids = _cu([4, 6, 2, 2])
    odd = _cu([3, 6, 2, 2])
    G = F + 4096  # device token offsets
    assert f(A, 1152, B, G, odd, 2, 22, C, D, 1e-6, E, None) == SEQ
    assert f(A, 1152, B, G, grids, 2, 27, C, D, 1e-6, E, None) == SEQ    # sum h*w != T
    assert f(A, 4000, B, G, grids, 2, 28, C, D, 1e-6, E, None) == SHAPE  # 4D > 8192
    assert f(A, 1152, B, G, grids, 2, 28, C, D, 1e-6, A + 64, None) == ALIAS
    assert f(A, 1152, B, G, grids, 2, 28, C, D, 1e-6, G - 64, None) == ALIAS  # out over cu_seqlens
    assert f(A, 1152, None, G, grids, 2, 28, C, D, 1e-6, E, None) == NULL
    assert f(A, 1152, B, None, grids, 2, 28, C, D, 1e-6, E, None) == NULL     # device offsets
    assert f(A, 1152, B, G + 4, grids, 2, 28, C, D, 1e-6, E, None) == ALIGN


def test_pos_embed_interp_validation(lib):
    f = lib.vit_pos_embed_interp
    grids = _cu([46, 136, 3, 5])
    T = 46 * 136 + 15
    G = F + 4096  # device token offsets
    assert f(A, 48, 1152, B, G, grids, 2, T + 1, C, 1152, None) == SEQ      # sum h*w != T
    assert f(A, 48, 1152, B, G, _cu([0, 5]), 1, 0, C, 1152, None) == SEQ    # empty side
    assert f(A, 0, 1152, B, G, grids, 2, T, C, 1152, None) == SHAPE         # G < 1
    assert f(A, 1025, 1152, B, G, grids, 2, T, C, 1152, None) == SHAPE
    assert f(A, 48, 1150, B, G, grids, 2, T, C, 1152, None) == SHAPE        # dim % 8
    assert f(A, 48, 1152, B, G, grids, 2, T, C, 1148, None) == SHAPE        # ld_out < dim
    assert f(A, 48, 1152, B, G, grids, 2, T, C, 1156, None) == SHAPE        # ld_out % 8
    assert f(A, 48, 1152, B, G, None, 2, T, C, 1152, None) == NULL          # host grids
    assert f(None, 48, 1152, B, G, grids, 2, T, C, 1152, None) == NULL
    assert f(A, 48, 1152, None, G, grids, 2, T, C, 1152, None) == NULL
    assert f(A, 48, 1152, B, None, grids, 2, T, C, 1152, None) == NULL      # device offsets
    assert f(A, 48, 1152, B, G, grids, 2, T, None, 1152, None) == NULL
    assert f(A + 8, 48, 1152, B, G, grids, 2, T, C, 1152, None) == ALIGN
    assert f(A, 48, 1152, B, G, grids, 2, T, C + 8, 1152, None) == ALIGN
    assert f(A, 48, 1152, B, G + 4, grids, 2, T, C, 1152, None) == ALIGN
    assert f(A, 48, 1152, B, G, grids, 2, T, A + 4096, 1152, None) == ALIAS  # out over the table
    assert f(A, 48, 1152, B, G, grids, 2, T, B - 64, 1152, None) == ALIAS    # out over the grids
    assert f(A, 48, 1152, B, G, grids, 2, T, G - 64, 1152, None) == ALIAS    # out over cu_seqlens
    assert f(A, 48, 1152, B, G, _cu([]), 0, 0, C, 1152, None) == OK          # nothing to do


def test_smart_resize_host_logic_reproduces_the_page_table():
    # a host-only computation: the library is called directly, no GPU work
    import json
    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
    f = facts["smart_resize_rows"]
    for max_pixels, patches in f["rows"]:
        h, w = vit.vit_smart_resize(f["image_height"], f["image_width"], max_pixels=max_pixels)
        assert (h // 16) * (w // 16) == patches and h % 32 == 0 and w % 32 == 0


@pytest.mark.parametrize("hw", [(100, 100), (17, 900), (4000, 3000), (31, 33), (48, 48), (80, 80), (724, 2172)])
@pytest.mark.parametrize("limits", [(0, None), (0, 250000), (200000, None), (3136, 1000000)])
def test_smart_resize_host_logic_matches_the_oracle(hw, limits):
    from oracle import preprocess as P
    assert vit.vit_smart_resize(*hw, min_pixels=limits[0], max_pixels=limits[1]) == \
        P.smart_resize(*hw, min_pixels=limits[0], max_pixels=limits[1])


def test_smart_resize_and_preprocess_validation(lib):
    h, w = ctypes.c_int(0), ctypes.c_int(0)
    f = lib.vit_smart_resize
    assert f(0, 10, 32, 0, 0, ctypes.byref(h), ctypes.byref(w)) == SHAPE
    assert f(10, 10, 0, 0, 0, ctypes.byref(h), ctypes.byref(w)) == SHAPE
    assert f(10, 10, 32, 0, 0, None, ctypes.byref(w)) == NULL
    g = lib.vit_preprocess_frames
    mean = (ctypes.c_float * 3)(0.5, 0.5, 0.5)
    std = (ctypes.c_float * 3)(0.5, 0.5, 0.5)
    bad = (ctypes.c_float * 3)(0.5, 0.0, 0.5)
    m, s_, b_ = (ctypes.cast(x, ctypes.c_void_p) for x in (mean, std, bad))
    assert g(A, 1, 724, 2172, 736, 2170, m, s_, B, None) == SHAPE    # out width % 16
    assert g(A, 0, 724, 2172, 736, 2176, m, s_, B, None) == SHAPE    # no frames
    assert g(A, 1, 724, 2172, 736, 2176, m, b_, B, None) == SHAPE    # std = 0
    assert g(A, 1, 724, 2172, 736, 2176, None, s_, B, None) == NULL
    assert g(None, 1, 724, 2172, 736, 2176, m, s_, B, None) == NULL
    assert g(A, 1, 724, 2172, 736, 2176, m, s_, None, None) == NULL
    assert g(A, 1, 724, 2172, 736, 2176, m, s_, B + 4, None) == ALIGN
    assert g(A, 1, 724, 2172, 736, 2176, m, s_, A + 4096, None) == ALIAS


BF16_BLOCK_FIELDS = ("qkv_w", "proj_w", "fc1_w", "fc2_w")
FP8_MERGER_FIELDS = ("fc1_codes", "fc1_scales", "fc2_codes", "fc2_scales")


def _block_struct(null_field=None, misalign=None, bf16=False):
    """An FP8 block (bf16 weight pointers NULL), or with bf16=True a block
    whose bf16 weights are set as well."""
    s = vit._BlockW()
    for i, (name, _) in enumerate(vit._BlockW._fields_):
        if name in BF16_BLOCK_FIELDS and not bf16:
            continue
        setattr(s, name, A + i * (1 << 24))
    if null_field:
        setattr(s, null_field, None)
    if misalign:
        setattr(s, misalign, getattr(s, misalign) + 4)
    return s


def test_block_validation(lib):
    f = lib.vit_block_forward
    cu = _cu([0, 256])
    need = lib.vit_block_workspace_size(256)
    assert need >= 256 * (3456 * 2 + 1152 * 2 + 1152 + 4352)
    s = _block_struct()
    X, POS, CU, WSP = B, C, C + 4096, D
    assert f(ctypes.byref(s), X, 256, POS, CU, cu, 1, WSP, need - 1, None) == WS
    assert f(ctypes.byref(_block_struct("fc1_codes")), X, 256, POS, CU, cu, 1, WSP, need, None) == NULL
    assert f(ctypes.byref(_block_struct(misalign="qkv_scales")), X, 256, POS, CU, cu, 1, WSP, need, None) == ALIGN
    assert f(ctypes.byref(s), X, 256, POS, CU, _cu([0, 255]), 1, WSP, need, None) == SEQ
    assert f(ctypes.byref(s), X, 256, POS, CU, cu, 1, WSP + 64, need, None) == ALIGN   # 256-B workspace
    assert f(ctypes.byref(s), X, 256, POS, CU, cu, 1, X, need, None) == ALIAS          # x inside workspace
    assert f(None, X, 256, POS, CU, cu, 1, WSP, need, None) == NULL
    # precision switch: a partial bf16 set is rejected, a complete one needs no FP8 codes
    part = _block_struct()
    part.qkv_w = A
    assert f(ctypes.byref(part), X, 256, POS, CU, cu, 1, WSP, need, None) == NULL
    assert f(ctypes.byref(_block_struct(bf16=True, misalign="fc2_w")), X, 256, POS, CU, cu, 1, WSP, need,
             None) == ALIGN
    assert f(ctypes.byref(_block_struct(bf16=True, null_field="qkv_codes")), X, 256, POS, CU, cu, 1, WSP,
             need - 1, None) == WS


def test_layernorm_validation(lib):
    f = lib.vit_layernorm
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    X, G, Bt, O = A, B, B + 8192, C
    assert f(X, 1152, G, Bt, 1e-6, 16, 1000, O, 1152, None) == SHAPE  # D % 128
    assert f(X, 1000, G, Bt, 1e-6, 16, 1152, O, 1152, None) == SHAPE  # ld_x < D
    assert f(X, 1152, G, Bt, 1e-6, 16, 1152, O, 1000, None) == SHAPE  # ld_out < D
    assert f(X, 1152, G, Bt, -1.0, 16, 1152, O, 1152, None) == SHAPE  # eps
    assert f(X, 1152, G, Bt, 1e-6, 0, 1152, O, 1152, None) == OK
    assert f(None, 1152, G, Bt, 1e-6, 16, 1152, O, 1152, None) == NULL
    assert f(X, 1156, G, Bt, 1e-6, 16, 1152, O, 1152, None) == ALIGN  # ld_x % 8
    assert f(X + 8, 1152, G, Bt, 1e-6, 16, 1152, O, 1152, None) == ALIGN
    assert f(X, 1152, G, Bt, 1e-6, 16, 1152, X + 1024, 1152, None) == ALIAS


def test_encoder_validation(lib):
    f = lib.vit_encoder_forward
    w = vit._EncoderW()
    w.patch_w, w.patch_b = A, A + 4096
    for b in range(27):
        w.blocks[b] = _block_struct()
    for m in range(4):
        ms = vit._MergerW()
        for i, (name, _) in enumerate(vit._MergerW._fields_):
            if name not in FP8_MERGER_FIELDS:
                setattr(ms, name, B + i * (1 << 24))
        w.mergers[m] = ms
    grids = _cu([46, 136])
    T = 6256
    need = lib.vit_encoder_workspace_size(T, 1)
    PIX, GD, OUT, WSP = C, C - 4096, D, E
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, OUT, None, WSP, need - 256, None) == WS
    assert f(ctypes.byref(w), PIX, None, GD, _cu([46, 135]), 1, 46 * 135, OUT, None, WSP, need, None) == SEQ
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T + 2, OUT, None, WSP, need, None) == SEQ
    w.mergers[2].fc2_w = None
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, OUT, None, WSP, need, None) == NULL
    w.mergers[2].fc2_w = B
    w.mergers[1].fc1_codes = B  # partial FP8 merger set
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, OUT, None, WSP, need, None) == NULL
    w.mergers[1].fc1_codes = None
    w.blocks[13].proj_bias = None
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, OUT, None, WSP, need, None) == NULL
    w.blocks[13].proj_bias = A
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, WSP + 1024, None, WSP, need, None) == ALIAS
    # learned position table: one position source, a valid side, aligned
    w.pos_table, w.pos_grid_side = F, 48
    assert f(ctypes.byref(w), PIX, F + (1 << 24), GD, grids, 1, T, OUT, None, WSP, need, None) == SHAPE
    w.pos_grid_side = 0
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, OUT, None, WSP, need, None) == SHAPE
    w.pos_table, w.pos_grid_side = F + 8, 48
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, OUT, None, WSP, need, None) == ALIGN
    w.pos_table = F
    assert f(ctypes.byref(w), PIX, None, GD, grids, 1, T, OUT, None, WSP, need - 256, None) == WS


def test_workspace_sizes_monotone(lib):
    sizes = [lib.vit_block_workspace_size(t) for t in (1, 256, 6256, 6684)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    assert lib.vit_block_workspace_size(-1) == 0
    assert lib.vit_encoder_workspace_size(6256, 1) > lib.vit_block_workspace_size(6256)


def test_binding_rejects_mismatched_output_buffers():
    # caller-provided outputs are checked for shape, dtype and contiguity
    # before anything reaches the library
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    g = torch.ones(256, dtype=torch.bfloat16)
    good_s = torch.empty((4, 2), dtype=torch.float32)
    with pytest.raises(ValueError):
        vit.vit_layernorm_quant_fp8(x, g, g, out=(torch.empty((4, 128), dtype=torch.uint8), good_s))
    with pytest.raises(ValueError):
        vit.vit_layernorm_quant_fp8(x, g, g, out=(torch.empty((4, 256), dtype=torch.int8), good_s))
    with pytest.raises(ValueError):
        vit.vit_quant_fp8_block128(x, out=(torch.empty((4, 256), dtype=torch.uint8),
                                           torch.empty((2, 4), dtype=torch.float32).t()))
    with pytest.raises(ValueError):
        vit.vit_merge2x2_layernorm(x, [(2, 2)], g.repeat(4), g.repeat(4), out=torch.empty((1, 512), dtype=torch.bfloat16))
