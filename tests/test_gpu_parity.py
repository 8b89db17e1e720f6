"""GPU parity: every step of the HIP path against the fp64 CPU oracle on the same seeded inputs.

Bit-exact: MX codes and scales of the quantiser, routing ids, the sorted layout. Within the stated
tolerance: routing weights (1e-6 relative) and the block output (max |err| <= 2e-2 * max |ref| and
sum |err| / sum |ref| <= 5e-3). Workloads of up to 128 tokens are compared on every output element;
the prefill-size workloads on a token sample that places a compared slot in every 128-row tile of
the layout (the oracle computes them token by token); routing and layout on every token. The
GEMM layouts are pinned bit for bit in test_gpu_exact.py."""
import numpy as np
import pytest
import torch

import workloads
from mx_quantized_grouped_amd import binding as B
from oracle import moe, mx

from gpu_support import (DEV, bf16_tensor, f64, inputs, oracle_result, oracle_weights,
                         packed_weights, shape_of, tolerance_ok)

pytestmark = pytest.mark.gpu

SMALL = ["tiny_bf16", "decode_mxfp8", "decode_mxfp4", "wide512_mxfp4_T1", "wide512_mxfp4_T6"]
LARGE = ["prefill_mxfp8", "wide512_mxfp4_T4096"]
ALL = SMALL + LARGE
# MXFP4 weights with MXFP4 activations (both MFMA operands E2M1); routing and layout are those of
# the MXFP8-activation workloads of the same shapes, so only the forward is parametrised over them
W4A4 = ["decode_w4a4", "wide512_w4a4_T4096"]


def _say(*a):
    print("[gpu-parity]", *a, flush=True)


def _pack_fp4(codes: np.ndarray) -> np.ndarray:
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


# ------------------------------------------------------------------------------- quantiser
def _quant_inputs(rng, rows, K):
    x = rng.standard_normal((rows, K)) * np.exp(rng.uniform(-12, 12, size=(rows, 1)))
    x[0] = 0.0                                        # all-zero blocks
    x[1, :32] = 2.0 ** -130                           # clamped scale
    x[2, :32] = [1.0625, 1.1875, -1.0] + [0.0] * 29   # ties
    x[3, :32] = -0.0
    x[4] = rng.integers(-6, 7, size=K) * 0.5          # many exact grid points and ties
    return x


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_bit_exact(fmt, src):
    _say("quantize", fmt, src)
    rng = np.random.default_rng(11)
    rows, K = 256, 512
    x = _quant_inputs(rng, rows, K)
    if src == "bf16":
        bits = workloads.bf16_bits_from_f32(x.astype(np.float32))
        xs = f64(bits)
        t = bf16_tensor(bits)
    else:
        xs = x.astype(np.float32).astype(np.float64)
        t = torch.from_numpy(xs.astype(np.float32)).to(DEV)
    codes, scales = B.mxmoe_quantize(t, fmt)
    torch.cuda.synchronize()
    el = "e4m3" if fmt == "mxfp8" else "e2m1"
    rc, rs = mx.quantize(xs, el)
    if fmt == "mxfp4":
        rc = _pack_fp4(rc)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("name", ["decode_mxfp4", "wide512_mxfp4_T6"])
def test_quantize_w4a4_activations(name):
    # The MXFP4-activation reading (W4A4): the GPU quantiser on a workload's bf16 activations,
    # decoded, equals the oracle's activation quantisation with E2M1 elements, value for value.
    _say("quantize w4a4 activations", name)
    w = workloads.get(name)
    xb = workloads.draw_x(w)
    codes, scales = B.mxmoe_quantize(bf16_tensor(xb), "mxfp4")
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    unpacked = np.stack([c & 0xF, c >> 4], axis=-1).reshape(w.T, w.H)
    got = mx.dequantize(unpacked, scales.cpu().numpy(), "e2m1")
    ref = moe.quantize_activation_rows(f64(xb), "mxfp4")
    assert np.array_equal(got, ref)


def test_quantize_exhaustive_bf16():
    # Every finite bf16 value, in blocks of 32 shuffled together (so each block's scale varies).
    _say("quantize exhaustive bf16")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = workloads.f32_from_bf16_bits(bits)
    bits = bits[np.isfinite(v)]
    bits = np.random.default_rng(0).permutation(bits)
    n = bits.size // 32 * 32
    bits = bits[:n].reshape(-1, 32)
    codes, scales = B.mxmoe_quantize(bf16_tensor(bits), "mxfp8")
    rc, rs = mx.quantize(f64(bits), "e4m3")
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("name", ["decode_mxfp8", "decode_mxfp4", "wide512_mxfp4_T1"])
def test_weight_quantisation_matches_oracle(name):
    _say("weights", name)
    w = workloads.get(name)
    loader, _ = packed_weights(name)
    el = "e4m3" if w.w_fmt == "mxfp8" else "e2m1"
    for e in [0, 1, w.E // 2, w.E]:
        a, b = workloads.draw_expert(w, e)
        for dev_c, dev_s, src in [(loader.w13[e], loader.s13[e], a), (loader.w2[e], loader.s2[e], b)]:
            rc, rs = mx.quantize(src.astype(np.float64), el)
            if el == "e2m1":
                rc = _pack_fp4(rc)
            assert np.array_equal(dev_s.cpu().numpy(), rs), (name, e)
            assert np.array_equal(dev_c.cpu().numpy(), rc), (name, e)


# ------------------------------------------------------------------------------- gate
def _gate_bound(xb, gb):
    """fp32 accumulation bound for the gate: |err| <= H * 2^-24 * sum_h |x_h w_h| per logit
    (recursive summation of H exact bf16 products, each partial sum rounded once; the products of
    two bf16 values are exact in fp32)."""
    H = xb.shape[1]
    return H * 2.0 ** -24 * (np.abs(f64(xb)) @ np.abs(f64(gb)).T)


@pytest.mark.parametrize("T,H,E", [(32, 3072, 128), (8192, 3072, 128), (6, 2048, 512),
                                   (700, 160, 515), (1500, 3072, 128),
                                   (1, 2048, 512), (37, 96, 70), (100, 64, 1), (65, 128, 130),
                                   (4096, 2048, 512), (300, 256, 130), (2100, 96, 520),
                                   (3000, 64, 200)])
def test_gate_parity(T, H, E):
    _say("gate", T, H, E)
    wl = workloads.Workload(f"gate_{T}_{H}_{E}", T, H, E, 1, 128, "mxfp8", "mxfp8", False, 9)
    xb, gb = workloads.draw_x(wl), workloads.draw_gate(wl)
    ref = moe.gate_logits(f64(xb), f64(gb))
    bound = _gate_bound(xb, gb)
    x, g = bf16_tensor(xb), bf16_tensor(gb)
    l32 = B.mxmoe_gate(x, g)
    l16 = B.mxmoe_gate(x, g, out_dtype=torch.bfloat16)
    again = B.mxmoe_gate(x, g)
    torch.cuda.synchronize()
    a = l32.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(a - ref) <= bound), np.max(np.abs(a - ref) - bound)
    assert torch.equal(l32, again)                      # fixed-order sums: reproducible
    b = l16.float().cpu().numpy().astype(np.float64)   # one more rounding, to bf16
    assert np.all(np.abs(b - ref) <= bound + 2.0 ** -8 * np.abs(ref))


def test_gate_tiles_agree():
    # Every tile shape of the gate, register or LDS-staged, splits K over the 4 waves the same way
    # and adds their partial sums in wave order, so the logits are bit-identical whatever tile the
    # launcher picks for a batch size.
    _say("gate tiles agree")
    wl = workloads.Workload("gate_tiles", 1100, 224, 140, 1, 128, "mxfp8", "mxfp8", False, 13)
    x, g = bf16_tensor(workloads.draw_x(wl)), bf16_tensor(workloads.draw_gate(wl))
    outs = {}
    for cfg in [11, 12, 14, 21, 22, 24, 28, 41, 42, 44, 48, 84, 124, 142, 144, 148]:
        outs[cfg] = B.mxmoe_gate(x, g, tile=cfg)
    torch.cuda.synchronize()
    for cfg, o in outs.items():
        assert torch.equal(o, outs[11]), cfg


def test_gate_then_route_and_forward():
    # gate -> route inside forward: the routing of the GPU's logits is the oracle's routing of
    # those same logits (bit-exact), and the block output is within tolerance of the oracle's
    _say("gate -> forward")
    name = "decode_mxfp8"
    w, xb, _ = inputs(name)
    _, packed = packed_weights(name)
    gb = workloads.draw_gate(w)
    x = bf16_tensor(xb)
    logits = B.mxmoe_gate(x, bf16_tensor(gb))
    shape = shape_of(w, "f32")
    ws = B.new_workspace(B.mxmoe_workspace_bytes(shape, None), DEV)
    y = B.mxmoe_forward(shape, x, logits, packed, workspace=ws)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lg - moe.gate_logits(f64(xb), f64(gb))) <= _gate_bound(xb, gb))
    ids, _ = _view(ws, shape, None, B.VIEW_TOPK_IDS)
    rid, _ = moe.route(lg, w.top_k)
    assert np.array_equal(ids.reshape(w.T, w.top_k + 1), rid)
    toks = np.arange(0, w.T, 4)
    ref = moe.moe_block(f64(xb), lg, oracle_weights(w), w.top_k, w.act_fmt, tokens=toks)
    st = moe.parity_stats(y.float().cpu().numpy().astype(np.float64)[toks], ref.y[toks])
    assert tolerance_ok(st), st


# ------------------------------------------------------------------------------- route
def _check_route(lg64, dev_logits, k):
    ids, wts = B.mxmoe_route(dev_logits, k)
    torch.cuda.synchronize()
    rid, rw = moe.route(lg64, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(wts.cpu().numpy(), rw, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("name", ALL)
def test_route_bit_exact(name):
    _say("route", name)
    w, _, lb = inputs(name)
    _check_route(f64(lb), bf16_tensor(lb), w.top_k)


def test_route_adversarial():
    _say("route adversarial")
    rng = np.random.default_rng(3)
    for E, k in [(8, 2), (128, 8), (512, 8), (1024, 63), (64, 64 - 1), (3, 3)]:
        T = 37
        lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32) * 0.5
        lg[rng.random(lg.shape) < 0.2] = -0.0
        lg[0] = 0.25                                  # all equal
        bits = workloads.bf16_bits_from_f32(lg)
        _check_route(f64(bits), bf16_tensor(bits), k)
        _check_route(lg.astype(np.float64), torch.from_numpy(lg).to(DEV), k)   # fp32 logits


# ------------------------------------------------------------------------------- align
@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("bm", [16, 64, 128])
def test_align_bit_exact(name, bm):
    _say("align", name, bm)
    w, _, lb = inputs(name)
    rid, _ = moe.route(f64(lb), w.top_k)
    L = moe.align(rid, w.E, bm)
    ids = torch.from_numpy(rid.astype(np.int32)).to(DEV)
    sorted_ids, bexp, npp, eoff = B.mxmoe_align(ids, w.E, bm)
    torch.cuda.synchronize()
    assert int(npp.item()) == L.num_post_pad
    assert np.array_equal(sorted_ids.cpu().numpy(), L.sorted_ids)
    assert np.array_equal(bexp.cpu().numpy(), L.block_expert)
    assert np.array_equal(eoff.cpu().numpy(), L.expert_off)


@pytest.mark.parametrize("name", ["decode_mxfp8", "wide512_mxfp4_T6"])
def test_align_contract_form(name):
    # mxmoe_align without offsets or workspace (sorts of at most 4096 slots), through the C ABI
    import ctypes
    _say("align contract form", name)
    w, _, lb = inputs(name)
    rid, _ = moe.route(f64(lb), w.top_k)
    L = moe.align(rid, w.E, 16)
    ids = torch.from_numpy(rid.astype(np.int32)).to(DEV)
    cap = B.mxmoe_align_capacity(w.T, w.E, w.top_k, 16)
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=DEV)
    bexp = torch.empty(cap // 16, dtype=torch.int32, device=DEV)
    npp = torch.empty(1, dtype=torch.int32, device=DEV)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = B.lib().mxmoe_align(vp(ids), w.T, w.E, w.top_k, 16, vp(sorted_ids), vp(bexp), vp(npp),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == B.MXMOE_OK
    assert int(npp.item()) == L.num_post_pad
    assert np.array_equal(sorted_ids.cpu().numpy(), L.sorted_ids)
    assert np.array_equal(bexp.cpu().numpy(), L.block_expert)


def test_align_random_shapes():
    _say("align random shapes")
    rng = np.random.default_rng(9)
    # up to 16 slots every wave derives the layout in registers (the first five shapes), up to
    # 4096 slots a workgroup sorts, beyond that the three-pass sort
    for T, E, k, bm in [(1, 1, 1, 16), (3, 2, 1, 32), (1, 1024, 15, 16), (2, 512, 7, 256),
                        (5, 2, 2, 64), (7, 1024, 8, 16), (32, 1, 1, 16), (500, 7, 3, 16),
                        (455, 9, 8, 256), (5000, 3, 2, 128), (129, 1024, 8, 16),
                        (2000, 1024, 8, 64)]:
        lg = rng.standard_normal((T, E))
        rid, _ = moe.route(lg, k)
        L = moe.align(rid, E, bm)
        s, b, n, o = B.mxmoe_align(torch.from_numpy(rid.astype(np.int32)).to(DEV), E, bm)
        assert int(n.item()) == L.num_post_pad
        assert np.array_equal(s.cpu().numpy(), L.sorted_ids)
        assert np.array_equal(b.cpu().numpy(), L.block_expert)
        assert np.array_equal(o.cpu().numpy(), L.expert_off)


def test_align_large_histograms():
    """Chunk histograms too large for the scan pass's LDS copy (73 chunks x 1025 experts): the
    scan walks them in global memory. Routing rows are drawn directly (k distinct experts per
    token, shared slot last) since only the layout is under test."""
    _say("align large histograms")
    rng = np.random.default_rng(11)
    T, E, k, bm = 8300, 1024, 8, 64
    rid = np.empty((T, k + 1), dtype=np.int64)
    for t in range(T):
        rid[t, :k] = rng.choice(E, size=k, replace=False)
    rid[:, k] = E
    L = moe.align(rid, E, bm)
    s, b, n, o = B.mxmoe_align(torch.from_numpy(rid.astype(np.int32)).to(DEV), E, bm)
    assert int(n.item()) == L.num_post_pad
    assert np.array_equal(s.cpu().numpy(), L.sorted_ids)
    assert np.array_equal(b.cpu().numpy(), L.block_expert)
    assert np.array_equal(o.cpu().numpy(), L.expert_off)


# ------------------------------------------------------------------------------- forward
def _run_forward(name, options=None, logits_dtype="bf16"):
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w, logits_dtype)
    x = bf16_tensor(xb)
    lg = bf16_tensor(lb) if logits_dtype == "bf16" else bf16_tensor(lb).float()
    ws = B.new_workspace(B.mxmoe_workspace_bytes(shape, options), DEV)
    y = B.mxmoe_forward(shape, x, lg, packed, workspace=ws, options=options)
    torch.cuda.synchronize()
    return w, shape, y, ws


def _view(ws, shape, options, which, dtype=torch.int32):
    off, nb, bm = B.mxmoe_workspace_view(shape, options, which)
    return ws[off:off + nb].view(dtype).cpu().numpy(), bm


def _check_slot_lists(lists, ids, E):
    T, k1 = ids.shape
    S = T * k1
    lists = lists.reshape(E + 1, T)
    flat = ids.reshape(-1)
    for e in range(E + 1):
        slots = np.flatnonzero(flat == e)
        want = np.concatenate([slots, np.full(T - len(slots), S)]).astype(np.int64)
        assert np.array_equal(lists[e].astype(np.int64), want), e


def _check_forward(name, options):
    w, shape, y, ws = _run_forward(name, options)
    r = oracle_result(name)
    toks = r.tokens
    if w.T <= 128:
        assert len(toks) == w.T
    # routing and layout inside forward: bit-exact on every token
    ids, _ = _view(ws, shape, options, B.VIEW_TOPK_IDS)
    assert np.array_equal(ids.reshape(w.T, w.top_k + 1), r.ids)
    sids, bm = _view(ws, shape, options, B.VIEW_SORTED_IDS)
    if B.mxmoe_workspace_view(shape, options, B.VIEW_BLOCK_EXPERT)[1]:
        L = moe.align(r.ids, w.E, bm)
        assert np.array_equal(sids, L.sorted_ids)
    else:  # slot order: expert e's slots in slot order at e*T, then the padding id S
        _check_slot_lists(sids, r.ids, w.E)
    yt = y.float().cpu().numpy().astype(np.float64)[toks]
    st = moe.parity_stats(yt, r.y[toks])
    _say(name, options and (options.launcher, options.combine), st)
    assert np.all(np.isfinite(yt))
    assert tolerance_ok(st), st
    return st


@pytest.mark.parametrize("name", ALL + W4A4)
def test_forward_parity_default(name):
    _say("forward", name)
    _check_forward(name, None)


@pytest.mark.parametrize("name", ["tiny_bf16", "decode_mxfp8", "decode_mxfp4", "wide512_mxfp4_T6",
                                  "prefill_mxfp8", "wide512_mxfp4_T4096"] + W4A4)
@pytest.mark.parametrize("launcher,combine", [(1, 2), (2, 1), (2, 2), (1, 1)])
def test_forward_parity_launchers(name, launcher, combine):
    _say("forward", name, launcher, combine)
    _check_forward(name, B.Options(launcher, combine, 0, 0))


# Both small-M row layouts on the decode workloads, each against the oracle. Where the sorted plan
# runs one wave per unit the two outputs are bit-identical (every output row is the same sums in
# the same order); with few units (tiny_bf16, the 512-expert workloads) the sorted plan splits K
# over four waves, which reorders the sums. Slot order on the 512-expert workloads (fewer slots
# than experts: most units find no rows) runs only when asked for.
@pytest.mark.parametrize("name", ["tiny_bf16", "decode_mxfp8", "decode_mxfp4", "wide512_mxfp4_T1",
                                  "wide512_mxfp4_T6"] + W4A4[:1])
@pytest.mark.parametrize("combine", [1, 3])
def test_forward_layouts(name, combine):
    _say("layouts", name, combine)
    outs = []
    for layout in (B.MXMOE_LAYOUT_SORTED, B.MXMOE_LAYOUT_SLOTS):
        o = B.Options(1, combine, 0, 0, None, 0, 0, 0, layout)
        _, shape, y, _ = _run_forward(name, o)
        has_layout = B.mxmoe_workspace_view(shape, o, B.VIEW_BLOCK_EXPERT)[1] > 0
        assert has_layout == (layout == B.MXMOE_LAYOUT_SORTED)
        _check_forward(name, o)
        outs.append(y.view(torch.int16).clone())
    if name.startswith("decode"):
        assert torch.equal(outs[0], outs[1])


def _check_act_codes(shape, ws, options, xbits):
    """The activation codes and scales forward left in its workspace against the oracle's MX rule
    (E2M1 codes two per byte, element 2i in the low nibble)."""
    T, H = xbits.shape
    xq, _ = _view(ws, shape, options, B.VIEW_XQ, torch.uint8)
    xs, _ = _view(ws, shape, options, B.VIEW_XS, torch.uint8)
    a4 = shape.act_fmt == B.MXMOE_MXFP4_E2M1
    rc, rs = mx.quantize(f64(xbits), "e2m1" if a4 else "e4m3")
    if a4:
        rc = _pack_fp4(rc)
    assert np.array_equal(xq.reshape(T, -1), rc)
    assert np.array_equal(xs.reshape(T, -1)[:, :H // 32], rs)


@pytest.mark.parametrize("name", ["decode_mxfp8", "wide512_mxfp4_T6", "prefill_mxfp8"] + W4A4)
def test_forward_activation_codes_bit_exact(name):
    # the in-forward quantiser (one-launch and split prologues) against the oracle, every code
    _say("activation codes", name)
    w, xb, _ = inputs(name)
    _, shape, _, ws = _run_forward(name, None)
    _check_act_codes(shape, ws, None, xb)


def test_forward_activation_codes_exhaustive_bf16():
    # every finite bf16 value once, shuffled into a 32 x 2048 activation matrix
    _say("activation codes exhaustive")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(workloads.f32_from_bf16_bits(bits))]
    bits = np.random.default_rng(3).permutation(bits)
    T, H = 32, 2048
    xb = np.zeros(T * H, dtype=np.uint16)
    xb[:bits.size] = bits
    xb = xb.reshape(T, H)
    wl = workloads.Workload("act_exhaustive", T, H, 4, 2, 128, "mxfp8", "mxfp8", False, 7)
    from mx_quantized_grouped_amd.weights import ExpertLoader
    shape = shape_of(wl)
    loader = ExpertLoader(shape, DEV)
    for e in range(wl.E + 1):
        loader.add_expert(e, *workloads.draw_expert(wl, e))
    packed = loader.finish()
    lb = workloads.draw_logits(wl)
    ws = B.new_workspace(B.mxmoe_workspace_bytes(shape, None), DEV)
    B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, workspace=ws)
    torch.cuda.synchronize()
    _check_act_codes(shape, ws, None, xb)


@pytest.mark.parametrize("bm", [16, 32, 128, 256])
def test_forward_block_m(bm):
    _say("forward block_m", bm)
    _check_forward("wide512_mxfp4_T4096", B.Options(2, 2, bm, 0))


def test_forward_logits_f32():
    _say("forward f32 logits")
    w, _, y, _ = _run_forward("decode_mxfp8", None, "f32")
    r = oracle_result("decode_mxfp8")
    yt = y.float().cpu().numpy().astype(np.float64)[r.tokens]
    assert tolerance_ok(moe.parity_stats(yt, r.y[r.tokens]))


def test_forward_slots_deterministic_and_permutation_invariant():
    _say("forward determinism / permutation")
    name = "decode_mxfp4"
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w)
    opt = B.Options(1, 1, 0, 0)
    y1 = B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, options=opt)
    y2 = B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, options=opt)
    perm = np.random.default_rng(1).permutation(w.T)
    yp = B.mxmoe_forward(shape, bf16_tensor(xb[perm]), bf16_tensor(lb[perm]), packed, options=opt)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(yp.view(torch.int16), y1[torch.from_numpy(perm).to(DEV)].view(torch.int16))


@pytest.mark.parametrize("name", ["tiny_bf16", "decode_mxfp8", "wide512_mxfp4_T1",
                                  "wide512_mxfp4_T6"])
def test_forward_graph_replay(name):
    # One forward captured in a HIP graph (the library only enqueues kernels on the caller's
    # stream) and replayed on new inputs written into the captured buffers, with eager forwards
    # and host synchronisations between the replays: every replay equals the eager result bit for
    # bit (same kernels, fixed-order combine).
    _say("graph replay", name)
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w)
    rng = np.random.default_rng(7)
    draws = [(xb, lb)] + [(xb[rng.permutation(w.T)], lb[rng.permutation(w.T)]) for _ in range(2)]
    xs, ls = bf16_tensor(xb), bf16_tensor(lb)
    ys = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    wss = B.new_workspace(B.mxmoe_workspace_bytes(shape), DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.mxmoe_forward(shape, xs, ls, packed, y=ys, workspace=wss)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.mxmoe_forward(shape, xs, ls, packed, y=ys, workspace=wss)
    torch.cuda.synchronize()
    for xr, lr in draws:
        ref = B.mxmoe_forward(shape, bf16_tensor(xr), bf16_tensor(lr), packed)
        torch.cuda.synchronize()
        xs.copy_(bf16_tensor(xr))
        ls.copy_(bf16_tensor(lr))
        ys.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["prefill_mxfp8", "wide512_mxfp4_T4096", "wide512_w4a4_T4096"])
def test_forward_unit_order_invariant(name):
    # The large-M launcher's unit order (runs of units per XCD turn; -1 = one contiguous range per
    # XCD, 1 = linear, 5 = runs that do not divide the unit count) only changes which workgroup
    # computes which output tile: every order must give the library's output bit for bit, so the
    # mapping covers every unit exactly once.
    _say("unit order", name)
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w)
    x, lg = bf16_tensor(xb), bf16_tensor(lb)
    ref = B.mxmoe_forward(shape, x, lg, packed)
    for run in (-1, 1, 5):
        y = B.mxmoe_forward(shape, x, lg, packed, options=B.Options(0, 0, 0, run))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), run


# ------------------------------------------------------------------------------- edge shapes
@pytest.mark.parametrize("T,H,E,k,I,fmt", [
    (1, 128, 1, 1, 32, "mxfp8"),      # one token, one routed expert
    (5, 256, 4, 4, 96, "mxfp8"),      # k == E; I not a multiple of 128 (padded K of down)
    (7, 384, 6, 2, 160, "mxfp4"),
    (17, 256, 8, 2, 64, "mxfp8"),     # one-launch prologue with one wave routing two tokens
    (33, 128, 16, 3, 64, "bf16"),     # just past the one-launch prologue
    (300, 256, 8, 2, 64, "mxfp8"),    # large-M launcher on a small problem
    (300, 256, 8, 2, 128, "bf16"),    # bf16 weights past the launcher threshold: AUTO runs the
                                      # one-wave large-M kernel with bf16 slot rows
    (5, 256, 4, 4, 96, "w4a4"),       # E2M1 intermediate with a padded K of down
    (300, 256, 8, 2, 64, "w4a4"),     # W4A4 on the one-wave large-M kernel (I / 32 = 2 chunks)
])
def test_forward_edge_shapes(T, H, E, k, I, fmt):
    _say("edge", T, H, E, k, I, fmt)
    w_fmt, act = {"bf16": ("bf16", "bf16"), "w4a4": ("mxfp4", "mxfp4")}.get(fmt, (fmt, "mxfp8"))
    wl = workloads.Workload(f"edge_{T}_{H}_{E}_{k}_{I}_{fmt}", T, H, E, k, I, w_fmt, act, False, 3)
    from mx_quantized_grouped_amd.weights import ExpertLoader
    shape = shape_of(wl)
    loader = ExpertLoader(shape, DEV)
    for e in range(E + 1):
        loader.add_expert(e, *workloads.draw_expert(wl, e))
    packed = loader.finish()
    xb, lb = workloads.draw_x(wl), workloads.draw_logits(wl)
    ref = moe.moe_block(f64(xb), f64(lb), oracle_weights(wl), k, wl.act_fmt)
    # AUTO, both launchers with every combine (bf16 slot rows on the one-wave large-M kernel when
    # I % 128 != 0 or the tile height is not 128 / 256, and on the streaming kernel), a short tile
    for opt in [None, B.Options(1, 1, 0, 0), B.Options(1, 3, 0, 0), B.Options(2, 2, 0, 0),
                B.Options(2, 3, 0, 0), B.Options(2, 1, 32, 0), B.Options(2, 3, 64, 0)]:
        y = B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, options=opt)
        torch.cuda.synchronize()
        st = moe.parity_stats(y.float().cpu().numpy(), ref.y)
        assert tolerance_ok(st), (opt and (opt.launcher, opt.combine, opt.block_m), st)


# 256-row layout blocks on the large-M launcher (each block runs as two 128-row tiles): odd and
# single K-step counts, fp8 and fp4 weights, experts with fewer rows than one block
@pytest.mark.parametrize("T,H,E,k,I,fmt", [
    (520, 384, 4, 2, 128, "mxfp8"),   # 3 K-steps: the step pairs end on a zero step
    (300, 128, 4, 3, 256, "mxfp4"),   # 1 K-step
    (700, 1024, 6, 2, 256, "mxfp8"),
    (600, 1024, 4, 2, 512, "mxfp8"),  # row-resident down pass at 4 K-steps (70 KB of LDS stages)
])
def test_forward_wide_tiles(T, H, E, k, I, fmt):
    _say("wide tiles", T, H, E, k, I, fmt)
    wl = workloads.Workload(f"wide_{T}_{H}_{E}_{k}_{I}_{fmt}", T, H, E, k, I, fmt, "mxfp8", False, 5)
    from mx_quantized_grouped_amd.weights import ExpertLoader
    shape = shape_of(wl)
    loader = ExpertLoader(shape, DEV)
    for e in range(E + 1):
        loader.add_expert(e, *workloads.draw_expert(wl, e))
    packed = loader.finish()
    xb, lb = workloads.draw_x(wl), workloads.draw_logits(wl)
    ref = moe.moe_block(f64(xb), f64(lb), oracle_weights(wl), k, wl.act_fmt)
    for opt in [B.Options(2, 3, 256, 0), B.Options(2, 1, 256, 0)]:
        y = B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, options=opt)
        torch.cuda.synchronize()
        st = moe.parity_stats(y.float().cpu().numpy(), ref.y)
        assert tolerance_ok(st), (opt.combine, st)


# Small-M launcher forced on ~380 16-row tiles (past the split-K unit count, so one wave per unit
# on gate_up and the shared-tile down pass): K-step counts 4, 12 and 8 (at 4 the fp8 ring drops
# from 3 stages to 2), 4 and 8 column chunks, fp8 / fp4 weights and E2M1 activations
@pytest.mark.parametrize("T,H,E,k,I,fmt", [
    (1100, 512, 40, 4, 128, "mxfp8"),
    (1100, 1536, 40, 4, 128, "mxfp4"),
    (1100, 1024, 40, 4, 256, "w4a4"),
])
def test_forward_small_m_many_tiles(T, H, E, k, I, fmt):
    _say("small-M many tiles", T, H, E, k, I, fmt)
    w_fmt, act = {"w4a4": ("mxfp4", "mxfp4")}.get(fmt, (fmt, "mxfp8"))
    wl = workloads.Workload(f"sa_{T}_{H}_{E}_{k}_{I}_{fmt}", T, H, E, k, I, w_fmt, act, False, 17)
    from mx_quantized_grouped_amd.weights import ExpertLoader
    shape = shape_of(wl)
    loader = ExpertLoader(shape, DEV)
    for e in range(E + 1):
        loader.add_expert(e, *workloads.draw_expert(wl, e))
    packed = loader.finish()
    xb, lb = workloads.draw_x(wl), workloads.draw_logits(wl)
    ref = moe.moe_block(f64(xb), f64(lb), oracle_weights(wl), k, wl.act_fmt)
    for opt in [B.Options(1, 1, 0, 0), B.Options(1, 3, 0, 0)]:
        y = B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, options=opt)
        torch.cuda.synchronize()
        st = moe.parity_stats(y.float().cpu().numpy(), ref.y)
        assert tolerance_ok(st), (opt.combine, st)


# Degenerate routing: equal logits send every token to experts 0 .. k-1 (ties go to the lower
# index), so two experts and the shared one hold every slot and the rest are untouched: the
# largest per-expert row counts the layout can have, on both launchers and every combine.
@pytest.mark.parametrize("T", [64, 1024])
def test_forward_all_tokens_one_expert_set(T):
    _say("degenerate routing", T)
    wl = workloads.Workload(f"ties_{T}", T, 512, 16, 2, 256, "mxfp8", "mxfp8", False, 11)
    from mx_quantized_grouped_amd.weights import ExpertLoader
    shape = shape_of(wl)
    loader = ExpertLoader(shape, DEV)
    for e in range(wl.E + 1):
        loader.add_expert(e, *workloads.draw_expert(wl, e))
    packed = loader.finish()
    xb = workloads.draw_x(wl)
    lb = np.zeros((T, wl.E), dtype=np.uint16)  # bf16 +0.0 everywhere
    ref = moe.moe_block(f64(xb), f64(lb), oracle_weights(wl), wl.top_k, wl.act_fmt)
    assert np.array_equal(ref.ids[:, :2], np.tile([0, 1], (T, 1)))
    for opt in [None, B.Options(1, 1, 0, 0), B.Options(1, 2, 0, 0), B.Options(2, 1, 0, 0),
                B.Options(2, 3, 0, 0)]:
        y = B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, options=opt)
        torch.cuda.synchronize()
        st = moe.parity_stats(y.float().cpu().numpy(), ref.y)
        assert tolerance_ok(st), (opt and (opt.launcher, opt.combine), st)


def test_forward_zero_tokens_is_noop():
    shape = B.Shape.of(0, 256, 8, 2, 128, "mxfp8")
    assert B.lib().mxmoe_forward(shape, None, None, None, None, None, None, None, None, 0,
                                 None) == 0
