"""C-ABI checks that need no GPU: the library loads, exports every entry point include/mxmoe.h
declares, and rejects bad arguments on the host (before any HIP call) with the documented codes."""
import ctypes
import os
import re

import pytest

from mx_quantized_grouped_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from mx_quantized_grouped_amd import build
        build.build()
    return B.lib()


def _declared():
    txt = open(os.path.join(ROOT, "include", "mxmoe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mxmoe_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert sorted(B.EXPORTS) == names


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(B.status_string(s), str) and B.status_string(s)


def test_route_validation(L):
    r = L.mxmoe_route
    assert r(None, 4, 8, 9, 0, None, None, None) == B.MXMOE_EINVAL        # k > E
    assert r(None, 4, 8, 0, 0, None, None, None) == B.MXMOE_EINVAL        # k < 1
    assert r(None, -1, 8, 2, 0, None, None, None) == B.MXMOE_EINVAL       # T < 0
    assert r(None, 4, 2000, 2, 0, None, None, None) == B.MXMOE_EINVAL     # E too large
    assert r(None, 4, 128, 64, 0, None, None, None) == B.MXMOE_EUNSUPPORTED
    assert r(None, 4, 8, 2, 5, None, None, None) == B.MXMOE_EINVAL        # bad dtype
    assert r(None, 4, 8, 2, 0, None, None, None) == B.MXMOE_EINVAL        # null pointers
    assert r(None, 0, 8, 2, 0, None, None, None) == B.MXMOE_OK            # T = 0 no-op
    assert r(ctypes.c_void_p(3), 4, 8, 2, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
             None) == B.MXMOE_EINVAL                                     # misaligned fp32


def test_gate_validation(L):
    gt = L.mxmoe_gate
    p = ctypes.c_void_p(4096)
    assert gt(p, p, 4, 100, 8, 1, p, None) == B.MXMOE_EINVAL                # H % 32 != 0
    assert gt(p, p, 4, 0, 8, 1, p, None) == B.MXMOE_EINVAL                  # H = 0
    assert gt(p, p, 4, 128, 0, 1, p, None) == B.MXMOE_EINVAL                # E < 1
    assert gt(p, p, 4, 128, 5000, 1, p, None) == B.MXMOE_EINVAL             # E too large
    assert gt(p, p, -1, 128, 8, 1, p, None) == B.MXMOE_EINVAL               # T < 0
    assert gt(p, p, 4, 128, 8, 7, p, None) == B.MXMOE_EINVAL                # bad dtype
    assert gt(None, p, 4, 128, 8, 1, p, None) == B.MXMOE_EINVAL             # null x
    assert gt(p, p, 4, 128, 8, 1, None, None) == B.MXMOE_EINVAL             # null logits
    assert gt(ctypes.c_void_p(4104), p, 4, 128, 8, 1, p, None) == B.MXMOE_EINVAL  # x misaligned
    assert gt(p, p, 4, 128, 8, 1, ctypes.c_void_p(4098), None) == B.MXMOE_EINVAL  # fp32 misaligned
    assert gt(None, None, 0, 128, 8, 1, None, None) == B.MXMOE_OK           # T = 0 no-op


def test_align_validation_and_capacity(L):
    assert L.mxmoe_align_capacity(3, 2, 1, 2) == 0                       # block_m not allowed
    # S = 6 slots, at most min(E+1, S) = 3 touched experts: 6 + 3*15 = 51, rounded up to 16 -> 64
    assert L.mxmoe_align_capacity(3, 2, 1, 16) == 64
    assert L.mxmoe_align_ex(None, 3, 2, 1, 20, None, None, None, None, None, 0, None) == B.MXMOE_EINVAL
    assert L.mxmoe_align_ex(None, 0, 2, 1, 16, None, None, None, None, None, 0, None) == B.MXMOE_OK
    assert L.mxmoe_align_ex(None, 3, 2, 1, 16, None, None, None, None, None, 0, None) == B.MXMOE_EINVAL
    # large variant needs scratch
    assert L.mxmoe_align_workspace_bytes(8192, 128, 8, 64) > 0
    p = ctypes.c_void_p(256)
    assert L.mxmoe_align_ex(p, 8192, 128, 8, 64, p, p, p, None, None, 0, None) == B.MXMOE_EWORKSPACE


def test_align_contract_form(L):
    # the form without offsets or workspace: same validation; sorts that need scratch are refused
    assert L.mxmoe_align(None, 3, 2, 1, 20, None, None, None, None) == B.MXMOE_EINVAL
    assert L.mxmoe_align(None, 0, 2, 1, 16, None, None, None, None) == B.MXMOE_OK
    assert L.mxmoe_align(None, 3, 2, 1, 16, None, None, None, None) == B.MXMOE_EINVAL
    p = ctypes.c_void_p(256)
    assert L.mxmoe_align_workspace_bytes(8192, 128, 8, 64) > 0
    assert L.mxmoe_align(p, 8192, 128, 8, 64, p, p, p, None) == B.MXMOE_EWORKSPACE
    assert L.mxmoe_align_workspace_bytes(455, 128, 8, 16) == 0   # 4095 slots: one workgroup


def test_capacity_formula(L):
    for T, E, k, bm in [(32, 128, 8, 16), (8192, 128, 8, 64), (1, 512, 8, 128), (6, 512, 8, 256)]:
        S = T * (k + 1)
        cap = S + min(E + 1, S) * (bm - 1)
        assert L.mxmoe_align_capacity(T, E, k, bm) == -(-cap // bm) * bm


def test_quantize_validation(L):
    q = L.mxmoe_quantize
    p = ctypes.c_void_p(256)
    assert q(p, 4, 33, 0, 2, p, p, None) == B.MXMOE_EINVAL                # K % 32
    assert q(p, 4, 64, 7, 2, p, p, None) == B.MXMOE_EINVAL                # src dtype
    assert q(p, 4, 64, 0, 0, p, p, None) == B.MXMOE_EINVAL                # fmt
    assert q(None, 4, 64, 0, 2, p, p, None) == B.MXMOE_EINVAL
    assert q(ctypes.c_void_p(8), 4, 64, 0, 2, p, p, None) == B.MXMOE_EINVAL  # misaligned
    assert q(None, 0, 64, 0, 2, None, None, None) == B.MXMOE_OK


def test_shape_validation_and_sizes(L):
    ok = B.Shape.of(32, 3072, 128, 8, 384, "mxfp8")
    assert B.mxmoe_workspace_bytes(ok) > 0
    bad = [B.Shape.of(32, 3000, 128, 8, 384), B.Shape.of(32, 3072, 128, 8, 380),
           B.Shape.of(32, 3072, 128, 0, 384), B.Shape.of(32, 3072, 128, 129, 384),
           B.Shape(32, 3072, 128, 8, 384, 2, 0, 0), B.Shape(32, 3072, 128, 8, 384, 0, 2, 0),
           B.Shape(32, 3072, 128, 8, 384, 9, 2, 0), B.Shape(32, 3072, 128, 8, 384, 2, 2, 4)]
    for s in bad:
        assert B.mxmoe_workspace_bytes(s) == 0
        assert L.mxmoe_forward(ctypes.byref(s), None, None, None, None, None, None, None, None, 0,
                               None) < 0
    # H % 128 != 0 (but % 32 == 0) is a valid shape the kernels do not cover
    assert L.mxmoe_forward(ctypes.byref(B.Shape.of(4, 160, 8, 2, 64)), None, None, None, None,
                           None, None, None, None, 0, None) == B.MXMOE_EUNSUPPORTED
    # prepacked sizes: fragment-major layout holds exactly the canonical bytes when K % 128 == 0
    E1, H, I = 129, 3072, 384
    assert B.mxmoe_prepacked_bytes(ok, 0) == E1 * 2 * I * H
    assert B.mxmoe_prepacked_bytes(ok, 1) == E1 * 2 * I * H // 32
    assert B.mxmoe_prepacked_bytes(ok, 2) == E1 * H * I
    # one scale dword per lane, 128-K step and group of four 16-row tiles: I = 384 is 3 steps
    assert B.mxmoe_prepacked_bytes(ok, 3) == E1 * (H // 64) * 3 * 256
    f4 = B.Shape.of(128, 3072, 128, 8, 768, "mxfp4")
    assert B.mxmoe_prepacked_bytes(f4, 0) == E1 * 2 * 768 * 3072 // 2
    bf = B.Shape.of(16, 256, 8, 2, 128, "bf16")
    assert B.mxmoe_prepacked_bytes(bf, 1) == 0 and B.mxmoe_prepacked_bytes(bf, 0) == 9 * 256 * 256 * 2
    pad = B.Shape.of(4, 256, 4, 2, 96, "mxfp8")       # K of down padded 96 -> 128
    assert B.mxmoe_prepacked_bytes(pad, 2) == 5 * 256 * 128


def test_forward_workspace_checks(L):
    s = B.Shape.of(32, 3072, 128, 8, 384, "mxfp8")
    need = B.mxmoe_workspace_bytes(s)
    p = ctypes.c_void_p(4096)
    args = [p] * 7
    assert L.mxmoe_forward(ctypes.byref(s), *args, p, need - 1, None) == B.MXMOE_EWORKSPACE
    assert L.mxmoe_forward(ctypes.byref(s), *args, ctypes.c_void_p(4096 + 64), need,
                           None) == B.MXMOE_EWORKSPACE                   # misaligned
    assert L.mxmoe_forward(ctypes.byref(s), *args[:6], None, p, need, None) == B.MXMOE_EINVAL
    o = B.Options(3, 0, 0, 0)
    assert B.mxmoe_workspace_bytes(s, o) == 0
    o = B.Options(0, 0, 48, 0)
    assert B.mxmoe_workspace_bytes(s, o) == 0


def test_workspace_view(L):
    s = B.Shape.of(32, 3072, 128, 8, 384, "mxfp8")
    off0, nb0, bm = B.mxmoe_workspace_view(s, None, B.VIEW_TOPK_IDS)
    # the control words of the one-launch path come first, at the same place in every plan
    assert off0 == B.WORKSPACE_CONTROL_BYTES and nb0 == 32 * 9 * 4 and bm == 16
    assert B.mxmoe_workspace_view(s, None, B.VIEW_STATUS)[:2] == (16, 4)
    big = B.Shape.of(8192, 3072, 128, 8, 384, "mxfp8")
    assert B.mxmoe_workspace_view(big, None, B.VIEW_STATUS)[:2] == (16, 4)
    off, nb, bm = B.mxmoe_workspace_view(s, B.Options(2, 2, 128, 0), B.VIEW_SORTED_IDS)
    assert bm == 128 and nb == 4 * L.mxmoe_align_capacity(32, 128, 8, 128)
    assert off % 256 == 0
    off, nb, _ = B.mxmoe_workspace_view(s, None, B.VIEW_XQ)
    assert nb == 32 * 3072 and off % 256 == 0
    off, nb, _ = B.mxmoe_workspace_view(s, None, B.VIEW_XS)
    assert nb == 32 * 96                                 # 3072 / 32 scale bytes, already 16-aligned
    sb = B.Shape.of(16, 256, 8, 2, 128, "bf16")
    assert B.mxmoe_workspace_view(sb, None, B.VIEW_XQ)[1] == 0   # bf16 weights: no activation codes
    srt = B.Options(0, 0, 0, 0, None, 0, 0, 0, B.MXMOE_LAYOUT_SORTED)
    off, nb, _ = B.mxmoe_workspace_view(s, srt, B.VIEW_H)
    cap = L.mxmoe_align_capacity(32, 128, 8, 16)
    assert nb == cap * 384 and off % 256 == 0            # I = 384 is three whole 128-K steps
    off, nb, _ = B.mxmoe_workspace_view(s, srt, B.VIEW_HS)
    assert nb == cap * 16                                # 12 scale bytes padded to 16
    assert B.mxmoe_workspace_view(sb, None, B.VIEW_H)[1] == L.mxmoe_align_capacity(16, 8, 2, 16) * 128 * 2
    assert B.mxmoe_workspace_view(sb, None, B.VIEW_HS)[1] == 0
    with pytest.raises(B.MxMoeError):
        B.mxmoe_workspace_view(s, None, 11)
    with pytest.raises(B.MxMoeError):
        B.mxmoe_workspace_view(s, None, -1)


def test_w4a4_plan(L):
    # MXFP4 activations with MXFP4 weights: E2M1 activation codes and intermediate take half the
    # bytes of E4M3 ones, with the same scale rows
    s = B.Shape.of(128, 3072, 128, 8, 768, "mxfp4", act_fmt="mxfp4")
    a8 = B.Shape.of(128, 3072, 128, 8, 768, "mxfp4")
    assert B.mxmoe_workspace_bytes(s) > 0
    assert B.mxmoe_workspace_view(s, None, B.VIEW_XQ)[1] == 128 * 3072 // 2
    for v in (B.VIEW_XS, B.VIEW_HS, B.VIEW_SORTED_IDS):
        assert B.mxmoe_workspace_view(s, None, v)[1] == B.mxmoe_workspace_view(a8, None, v)[1]
    assert 2 * B.mxmoe_workspace_view(s, None, B.VIEW_H)[1] == B.mxmoe_workspace_view(a8, None, B.VIEW_H)[1]
    pad = B.Shape.of(4, 256, 4, 2, 96, "mxfp4", act_fmt="mxfp4")     # K of down padded to 128
    assert B.mxmoe_workspace_view(pad, None, B.VIEW_H)[1] == L.mxmoe_align_capacity(4, 4, 2, 16) * 64
    # MXFP4 activations need MXFP4 weights; the one-launch path takes E4M3 activations only
    for wf in (B.MXMOE_BF16, B.MXMOE_MXFP8_E4M3):
        assert B.mxmoe_workspace_bytes(B.Shape(128, 3072, 128, 8, 768, wf, B.MXMOE_MXFP4_E2M1, 0)) == 0
    assert B.mxmoe_workspace_bytes(s, B.Options(0, 0, 0, 0, None, 1)) == 0
    assert B.mxmoe_workspace_bytes(s, B.Options(0, 0, 0, 0, None, -1)) > 0


def test_options_one_launch(L):
    dec = B.Shape.of(32, 3072, 128, 8, 384, "mxfp8")
    fused = B.Options(0, 0, 0, 0, None, 1)
    assert B.mxmoe_workspace_bytes(dec, fused) > 0
    # required but not allowed: large batches, bf16 weights, other combines or tile heights
    assert B.mxmoe_workspace_bytes(B.Shape.of(8192, 3072, 128, 8, 384, "mxfp8"), fused) == 0
    assert B.mxmoe_workspace_bytes(B.Shape.of(16, 256, 8, 2, 128, "bf16"), fused) == 0
    assert B.mxmoe_workspace_bytes(dec, B.Options(0, 3, 0, 0, None, 1)) == 0
    assert B.mxmoe_workspace_bytes(dec, B.Options(0, 0, 64, 0, None, 1)) == 0
    assert B.mxmoe_workspace_bytes(dec, B.Options(2, 0, 0, 0, None, 1)) == 0
    # invalid values
    for o in [B.Options(0, 0, 0, 0, None, 2), B.Options(0, 0, 0, 0, None, 0, -1),
              B.Options(0, 0, 0, 0, None, 0, 0, 2), B.Options(0, 0, 0, 0, None, 0, 0, 0, 3)]:
        assert B.mxmoe_workspace_bytes(dec, o) == 0


def _layout(shape, o=None):
    """'slots' for the slot-order plan (no tile map: views 3-5 are empty), else 'sorted'."""
    return "sorted" if B.mxmoe_workspace_view(shape, o, B.VIEW_BLOCK_EXPERT)[1] else "slots"


def test_options_layout(L):
    dec = B.Shape.of(32, 3072, 128, 8, 384, "mxfp8")
    slots = lambda *a: B.Options(*a, 0, None, 0, 0, 0, B.MXMOE_LAYOUT_SLOTS)
    sorted_ = B.Options(0, 0, 0, 0, None, 0, 0, 0, B.MXMOE_LAYOUT_SORTED)
    # automatic: slot order at decode over 128 experts (288 slots, 129 experts; 12 x 129 gate_up
    # units); the sorted layout for one or six tokens over 512 experts (fewer slots than experts),
    # small expert counts (few units: K is split), large batches and the atomic combine
    assert _layout(dec) == "slots"
    assert _layout(B.Shape.of(128, 3072, 128, 8, 768, "mxfp4", act_fmt="mxfp4")) == "slots"
    assert _layout(B.Shape.of(1, 2048, 512, 8, 512, "mxfp4")) == "sorted"
    assert _layout(B.Shape.of(6, 2048, 512, 8, 512, "mxfp4")) == "sorted"
    assert _layout(B.Shape.of(16, 256, 8, 2, 128, "bf16")) == "sorted"
    assert _layout(B.Shape.of(8192, 3072, 128, 8, 384, "mxfp8")) == "sorted"
    assert _layout(dec, B.Options(0, 2, 0, 0)) == "sorted"
    assert _layout(dec, sorted_) == "sorted"
    # the one-launch path has its own layout
    assert _layout(dec, B.Options(0, 0, 0, 0, None, 1)) == "sorted"
    # required: any small-M plan with 16-row tiles, a slot-row combine and at most 256 tokens
    assert _layout(dec, slots(0, 0, 0)) == "slots"
    assert _layout(B.Shape.of(1, 2048, 512, 8, 512, "mxfp4"), slots(1, 3, 16)) == "slots"
    assert B.mxmoe_workspace_view(dec, slots(0, 0, 0), B.VIEW_SORTED_IDS)[2] == 16
    for bad in [slots(2, 0, 0), slots(0, 2, 0), slots(1, 0, 32)]:
        assert B.mxmoe_workspace_bytes(dec, bad) == 0
    assert B.mxmoe_workspace_bytes(dec.with_T(257), slots(1, 0, 0)) == 0
    assert B.mxmoe_workspace_bytes(dec.with_T(256), slots(1, 0, 0)) > 0
    assert B.mxmoe_workspace_bytes(dec, B.Options(0, 0, 0, 0, None, 1, 0, 0, 2)) == 0
    # slot order: T intermediate rows and T list entries per expert (shared one included)
    assert B.mxmoe_workspace_view(dec, slots(0, 0, 0), B.VIEW_H)[1] == 129 * 32 * 384
    assert B.mxmoe_workspace_view(dec, slots(0, 0, 0), B.VIEW_HS)[1] == 129 * 32 * 16
    assert B.mxmoe_workspace_view(dec, slots(0, 0, 0), B.VIEW_SORTED_IDS)[1] == 129 * 32 * 4
    for v in (B.VIEW_BLOCK_EXPERT, B.VIEW_NUM_POST_PAD, B.VIEW_EXPERT_OFF):
        assert B.mxmoe_workspace_view(dec, slots(0, 0, 0), v)[1] == 0
    # at least the sorted layout's capacity: one token over 512 experts (144 rows) takes 513
    one = B.Shape.of(1, 2048, 512, 8, 512, "mxfp4")
    assert L.mxmoe_align_capacity(1, 512, 8, 16) < 513
    assert B.mxmoe_workspace_view(one, slots(1, 3, 16), B.VIEW_H)[1] == 513 * 512
    # the automatic choice keeps T rows per expert within 64 MiB: 256 tokens over 256 experts at
    # I = 2048 (257 * 256 * 2048 bytes) stays sorted, unless asked for
    big = B.Shape.of(256, 2048, 256, 8, 2048, "mxfp8")
    assert _layout(big) == "sorted" and _layout(big, slots(1, 1, 0)) == "slots"


def test_auto_launcher_thresholds(L):
    # the automatic plan's tile height: 128-row tiles (large-M) from 16 slots per expert, or from
    # 6 with more than 256 experts; 16-row tiles below
    def bm(T, E, k=8):
        return B.mxmoe_workspace_view(B.Shape.of(T, 2048, E, k, 512, "mxfp4"), None,
                                      B.VIEW_SORTED_IDS)[2]
    assert bm(229, 128) == 16 and bm(230, 128) == 128      # 9 * 230 = 2070 >= 16 * 129 = 2064
    assert bm(341, 512) == 16 and bm(342, 512) == 128      # 9 * 342 = 3078 >= 6 * 513 = 3078
    assert bm(128, 128) == 16 and bm(4096, 512) == 128
    assert B.mxmoe_workspace_view(B.Shape.of(4096, 2048, 512, 8, 512, "mxfp4"),
                                  B.Options(1, 0, 0, 0), B.VIEW_SORTED_IDS)[2] == 16


def test_options_unit_run(L):
    s = B.Shape.of(8192, 3072, 128, 8, 384, "mxfp8")
    assert B.mxmoe_workspace_bytes(s, B.Options(0, 0, 0, -1)) > 0     # one range per XCD
    assert B.mxmoe_workspace_bytes(s, B.Options(0, 0, 0, 5)) > 0      # runs of 5
    assert B.mxmoe_workspace_bytes(s, B.Options(0, 0, 0, -2)) == 0    # invalid


def test_gate_ex_tiles(L):
    p = ctypes.c_void_p(4096)
    assert L.mxmoe_gate_ex(p, p, 4, 128, 8, 1, 13, p, None) == B.MXMOE_EINVAL   # no such tile
    assert L.mxmoe_gate_ex(p, p, 4, 128, 8, 1, 99, p, None) == B.MXMOE_EINVAL
    assert L.mxmoe_gate_ex(None, None, 0, 128, 8, 1, 144, None, None) == B.MXMOE_OK  # T = 0


def test_32bit_offset_limits(L):
    # Activation codes, the intermediate and one expert's weights are addressed with 32-bit
    # offsets: shapes that would reach 2 GiB are refused on the host, before any HIP call.
    big = B.Shape.of(700000, 3072, 128, 8, 384, "mxfp8")       # T*H = 2.15 GB of codes
    assert B.mxmoe_workspace_bytes(big) == 0
    assert L.mxmoe_forward(ctypes.byref(big), *[ctypes.c_void_p(4096)] * 7,
                           ctypes.c_void_p(4096), 1 << 40, None) == B.MXMOE_EUNSUPPORTED
    # bf16 weights, I = 4096: the intermediate (cap * I * 2 bytes) crosses 2 GiB near 29K tokens
    assert B.mxmoe_workspace_bytes(B.Shape.of(20000, 1024, 8, 2, 4096, "bf16")) > 0
    assert B.mxmoe_workspace_bytes(B.Shape.of(90000, 1024, 8, 2, 4096, "bf16")) == 0
    # one expert's W13 past 2 GiB (2 * I * H bytes of E4M3 codes)
    huge_w = B.Shape.of(4, 32768, 4, 2, 32768, "mxfp8")
    assert B.mxmoe_prepacked_bytes(huge_w, 0) == 0 and B.mxmoe_workspace_bytes(huge_w) == 0
    assert B.mxmoe_prepacked_bytes(B.Shape.of(4, 16384, 4, 2, 32768, "mxfp4"), 0) > 0
