"""Pins for the oracle's routing, sort and whole block (CPU only).

Routing and the sort are checked against brute force written differently and against hand
examples; the block against hand-worked closed forms (tests/golden/moe_worked_examples.txt), a dense
all-expert evaluation written with explicit loops, the shared expert as a plain dense MLP,
token-permutation invariance and textbook special cases."""
import math
import os

import numpy as np
import pytest

import workloads
from oracle import moe, mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------ gate
def test_gate_hand_example():
    # 2 tokens, 3 experts, H = 2: every logit worked by hand
    x = np.array([[1.0, 2.0], [-0.5, 4.0]])
    w = np.array([[1.0, 0.0], [0.25, -1.0], [3.0, 0.5]])
    assert moe.gate_logits(x, w).tolist() == [[1.0, -1.75, 4.0], [-0.5, -4.125, 0.5]]


def test_gate_matches_loops_and_one_hot_rows():
    rng = np.random.default_rng(5)
    x = workloads.f32_from_bf16_bits(workloads.bf16_bits_from_f32(
        rng.standard_normal((5, 64)).astype(np.float32))).astype(np.float64)
    w = workloads.f32_from_bf16_bits(workloads.bf16_bits_from_f32(
        (0.02 * rng.standard_normal((7, 64))).astype(np.float32))).astype(np.float64)
    ref = moe.gate_logits(x, w)
    for t in range(5):                       # brute force: one exact sum per logit
        for e in range(7):
            assert ref[t, e] == pytest.approx(math.fsum(x[t, h] * w[e, h] for h in range(64)),
                                              rel=1e-13, abs=1e-15)
    onehot = np.zeros((3, 64))
    onehot[0, 5] = onehot[1, 0] = onehot[2, 63] = 1.0   # expert e reads one column of x
    assert np.array_equal(moe.gate_logits(x, onehot), x[:, [5, 0, 63]])
    with pytest.raises(ValueError):
        moe.gate_logits(x, w[:, :32])


# ------------------------------------------------------------------------------------ route
def test_route_hand_examples():
    ids, w = moe.route(np.array([[1.0, 3.0, 3.0, 2.0]]), 2)
    assert ids.tolist() == [[1, 2, 4]]                  # tie 3 == 3 -> lower index first
    assert w.tolist() == [[0.5, 0.5, 1.0]]
    ids, _ = moe.route(np.array([[-0.0, 0.0, -1.0]]), 1)
    assert ids.tolist() == [[0, 3]]                      # -0 == +0 -> index 0
    ids, _ = moe.route(np.array([[0.0, -0.0, 5.0]]), 2)
    assert ids.tolist() == [[2, 0, 3]]
    ids, w = moe.route(np.array([[0.0, 1.0]]), 2)        # closed form for two selected logits
    assert ids.tolist() == [[1, 0, 2]]
    assert w[0, 0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    assert w[0, 1] == pytest.approx(math.exp(-1) / (1 + math.exp(-1)), rel=1e-15)


def test_route_all_equal_and_k_equals_E():
    ids, w = moe.route(np.full((3, 8), 0.25), 3)
    assert ids[:, :3].tolist() == [[0, 1, 2]] * 3
    assert np.allclose(w[:, :3], 1 / 3, rtol=1e-15, atol=0)
    lg = np.array([[0.5, -2.0, 3.0, 0.5, 1.0]])
    ids, w = moe.route(lg, 5)
    assert ids.tolist() == [[2, 4, 0, 3, 1, 5]]
    p = np.exp(lg[0] - lg[0].max())
    assert np.allclose(w[0, :5], (p / p.sum())[[2, 4, 0, 3, 1]], rtol=1e-14)


def test_route_brute_force_with_ties():
    # Small-integer logits make ties common; compare with numpy's lexsort (a different sort).
    rng = np.random.default_rng(0)
    for E, k in [(8, 2), (16, 4), (128, 8), (512, 8)]:
        lg = rng.integers(-3, 4, size=(40, E)).astype(np.float64) * 0.5
        lg[rng.random(lg.shape) < 0.1] = -0.0
        ids, w = moe.route(lg, k)
        for t in range(40):
            order = np.lexsort((np.arange(E), -lg[t] + 0.0))
            assert ids[t, :k].tolist() == order[:k].tolist()
            assert ids[t, k] == E and w[t, k] == 1.0
            assert abs(math.fsum(w[t, :k]) - 1.0) < 1e-12           # renormalised
            sel = lg[t, order[:k]]
            p = np.exp(sel - sel.max())
            assert np.allclose(w[t, :k], p / p.sum(), rtol=1e-14)


def test_route_rejects_bad_input():
    with pytest.raises(ValueError):
        moe.route(np.zeros((2, 4)), 5)
    with pytest.raises(ValueError):
        moe.route(np.array([[0.0, np.nan]]), 1)


# ------------------------------------------------------------------------------------ align
def test_align_hand_example():
    # T=3, k=1 (+ shared id 2), E=2, block 2. Flat slots: f=0:(t0,1) f=1:(t0,2) f=2:(t1,0)
    # f=3:(t1,2) f=4:(t2,1) f=5:(t2,2). Sentinel 6.
    ids = np.array([[1, 2], [0, 2], [1, 2]])
    L = moe.align(ids, 2, 2)
    assert L.sorted_ids.tolist() == [2, 6, 0, 4, 1, 3, 5, 6, 6, 6]
    assert L.block_expert.tolist() == [0, 1, 2, 2, -1]
    assert L.num_post_pad == 8
    assert L.expert_off.tolist() == [0, 2, 4, 8]
    assert L.counts.tolist() == [1, 2, 3]
    assert moe.align_capacity(3, 2, 1, 2) == 10              # 6 + 3*1 = 9 -> 10


def _align_brute(ids, E, bm):
    T, k1 = ids.shape
    S = T * k1
    pairs = sorted((int(ids[f // k1, f % k1]), f) for f in range(S))
    out, blocks = [], []
    for e in range(E + 1):
        fs = [f for (ee, f) in pairs if ee == e]
        if fs:
            n = -(-len(fs) // bm) * bm
            out += fs + [S] * (n - len(fs))
            blocks += [e] * (n // bm)
    return out, blocks


@pytest.mark.parametrize("bm", [1, 16, 32, 64, 128, 256])
def test_align_matches_brute_force(bm):
    rng = np.random.default_rng(bm)
    for T, E, k in [(1, 8, 2), (7, 16, 4), (64, 128, 8), (200, 512, 8)]:
        lg = rng.standard_normal((T, E))
        ids, _ = moe.route(lg, k)
        L = moe.align(ids, E, bm)
        want, blocks = _align_brute(ids, E, bm)
        assert L.num_post_pad == len(want)
        assert L.sorted_ids[:len(want)].tolist() == want
        assert L.block_expert[:len(blocks)].tolist() == blocks
        S = T * (k + 1)
        cap = moe.align_capacity(T, E, k, bm)
        assert len(L.sorted_ids) == cap and cap % bm == 0 and cap >= len(want)
        assert np.all(L.sorted_ids[len(want):] == S) and np.all(L.block_expert[len(blocks):] == -1)
        valid = L.sorted_ids[L.sorted_ids < S]
        assert sorted(valid.tolist()) == list(range(S))            # each slot exactly once
        for b, e in enumerate(blocks):                              # one expert per tile
            fs = L.sorted_ids[b * bm:(b + 1) * bm]
            fs = fs[fs < S]
            assert np.all(ids.reshape(-1)[fs] == e)


# ------------------------------------------------------------------------------------ block
def _const_weights(E, H, I, bytes_per_expert, fmt):
    """Every element of gate / up / down of expert e is 2^(b - 127) for its listed byte."""
    el = {"mxfp8": "e4m3", "mxfp4": "e2m1"}.get(fmt)
    one = {"e4m3": 0x38, "e2m1": 0x2}.get(el)
    w13c = np.full((E + 1, 2 * I, H), one, np.uint8) if el else None
    w13s = np.zeros((E + 1, 2 * I, H // 32), np.uint8)
    w2c = np.full((E + 1, H, I), one, np.uint8) if el else None
    w2s = np.zeros((E + 1, H, I // 32), np.uint8)
    for e, (bg, bu, bd) in enumerate(bytes_per_expert):
        w13s[e, :I], w13s[e, I:], w2s[e] = bg, bu, bd
    if el:
        return moe.ExpertWeights.from_mx(w13c, w13s, w2c, w2s, fmt)
    dense13 = np.repeat(2.0 ** (w13s.astype(np.float64) - 127), 32, axis=2)
    dense2 = np.repeat(2.0 ** (w2s.astype(np.float64) - 127), 32, axis=2)
    return moe.ExpertWeights.from_dense(dense13, dense2)


def test_block_hand_worked_examples():
    n = 0
    with open(os.path.join(GOLDEN, "moe_worked_examples.txt")) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if not ln:
                continue
            name, fmt, E, k, lg, per, expect = [p.strip() for p in ln.split("|")]
            E, k = int(E), int(k)
            per = [tuple(int(v) for v in grp.split(",")) for grp in per.split()]
            assert len(per) == E + 1
            W = _const_weights(E, 32, 32, per, fmt)
            logits = np.array([[float(v) for v in lg.split()]])
            r = moe.moe_block(np.ones((1, 32)), logits, W, k, "bf16" if fmt == "bf16" else "mxfp8")
            want = eval(expect, {"math": math})
            assert np.allclose(r.y, want, rtol=1e-14, atol=0), (name, r.y[0, :2], want)
            n += 1
    assert n == 3


def _tiny(T=5, H=64, E=4, k=2, I=64, fmt="mxfp8", seed=0):
    w = workloads.Workload("t", T, H, E, k, I, fmt, "bf16" if fmt == "bf16" else "mxfp8",
                           False, seed)
    x = workloads.f32_from_bf16_bits(workloads.draw_x(w)).astype(np.float64)
    lg = workloads.f32_from_bf16_bits(workloads.draw_logits(w)).astype(np.float64)
    W = moe.ExpertWeights.from_draws(lambda e: workloads.draw_expert(w, e), E, H, I, fmt)
    return w, x, lg, W


def _dense_loops(x, logits, W, k, act_fmt):
    """Every expert for every token with explicit loops, combined with a length-(E+1) weight vector
    that is zero off the selection (brute force; no grouping, no matmul)."""
    T, H = x.shape
    E = logits.shape[1]
    I = W.I
    xq = moe.quantize_activation_rows(x, act_fmt)
    y = np.zeros((T, H))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        p = [math.exp(logits[t, e] - logits[t, order[0]]) for e in order]
        wv = np.zeros(E + 1)
        for e, pe in zip(order, p):
            wv[e] = pe / math.fsum(p)
        wv[E] = 1.0
        for e in range(E + 1):
            w13, w2 = W(e)
            gate = [math.fsum(xq[t, h] * w13[i, h] for h in range(H)) for i in range(I)]
            up = [math.fsum(xq[t, h] * w13[I + i, h] for h in range(H)) for i in range(I)]
            a = np.array([g / (1 + math.exp(-g)) * u for g, u in zip(gate, up)])
            ah = moe.quantize_intermediate(a[None], act_fmt)[0]
            for n in range(H):
                y[t, n] += wv[e] * math.fsum(ah[i] * w2[n, i] for i in range(I))
    return y


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "bf16"])
def test_block_matches_dense_brute_force(fmt):
    w, x, lg, W = _tiny(fmt=fmt, T=4, H=64, E=4, k=2, I=32)
    r = moe.moe_block(x, lg, W, w.top_k, w.act_fmt)
    ref = _dense_loops(x, lg, W, w.top_k, w.act_fmt)
    assert np.allclose(r.y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())


def _shared_only_ones(H, I, E=2):
    """Routed experts all zero; every shared-expert weight 1."""
    def getter(e):
        if e == E:
            return np.ones((2 * I, H)), np.ones((H, I))
        return np.zeros((2 * I, H)), np.zeros((H, I))
    return moe.ExpertWeights(E, H, I, "mxfp8", getter)


@pytest.mark.parametrize("act_fmt,expect", [("mxfp4", 6144.0), ("mxfp8", 7168.0)])
def test_block_activation_format_closed_form(act_fmt, expect):
    # H = I = 32, every x = 0.5, only the shared expert (all weights 1) contributes.
    # Q1: amax 0.5 gives scale 2^(-1 - emax) and 0.5 lands on a grid point in both formats.
    # gate = up = 32 * 0.5 = 16; a = SiLU(16) * 16 = 256 / (1 + e^-16), 255.99997 in fp32.
    # Q2, E2M1 (emax 2): scale 2^(7 - 2) = 32, a / 32 = 7.99999 saturates to 6: a^ = 192.
    # Q2, E4M3 (emax 8): scale 2^(7 - 8) = 1/2, a * 2 = 511.9999 saturates to 448: a^ = 224.
    # down: y = 32 * a^ in every column (6144 and 7168).
    H = I = 32
    x = np.full((3, H), 0.5)
    lg = np.zeros((3, 2))
    r = moe.moe_block(x, lg, _shared_only_ones(H, I), 1, act_fmt)
    assert np.all(r.y == expect)


def test_mxfp4_activations_on_the_e2m1_grid():
    # Q1 for "mxfp4": every dequantised value of a 32-block is an E2M1 value (0, 0.5, 1, 1.5, 2, 3,
    # 4, 6 and negatives) times 2^(floor(log2 amax) - 2), with the block maximum mapped to [4, 8)
    # before rounding (so to 4 or 6).
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 128)) * np.exp2(rng.integers(-6, 6, (6, 1)))
    q = moe.quantize_activation_rows(x, "mxfp4")
    grid = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    for t in range(6):
        for b in range(4):
            blk, qb = x[t, 32 * b:32 * b + 32], q[t, 32 * b:32 * b + 32]
            s = math.floor(math.log2(np.abs(blk).max())) - 2
            assert all(abs(v) / 2.0 ** s in grid for v in qb)
            assert np.abs(qb).max() / 2.0 ** s in (4.0, 6.0)
    # and it is not the MXFP8 rule
    assert not np.array_equal(q, moe.quantize_activation_rows(x, "mxfp8"))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_block_w4a4_matches_dense_brute_force(fmt):
    w, x, lg, W = _tiny(fmt=fmt, T=3, H=64, E=4, k=2, I=32, seed=4)
    r = moe.moe_block(x, lg, W, w.top_k, "mxfp4")
    ref = _dense_loops(x, lg, W, w.top_k, "mxfp4")
    assert np.allclose(r.y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())


def test_shared_expert_equals_dense_mlp():
    # Routed experts with all-zero weights contribute nothing; the block must then equal the shared
    # expert run as a plain dense MLP on all tokens at once (matrix form, weight 1).
    w, x, lg, W = _tiny(T=6, H=64, E=4, k=2, I=64)
    w13s, w2s = W(w.E)

    def getter(e):
        if e == w.E:
            return w13s, w2s
        return np.zeros_like(w13s), np.zeros_like(w2s)
    Wz = moe.ExpertWeights(w.E, w.H, w.I, "mxfp8", getter)
    r = moe.moe_block(x, lg, Wz, w.top_k, "mxfp8")
    xq = mx.quantize_dequantize(x, "e4m3")
    G = xq @ w13s[:w.I].T
    U = xq @ w13s[w.I:].T
    A = (G / (1 + np.exp(-G))) * U
    Ah = mx.quantize_dequantize(A, "e4m3")
    Y = Ah @ w2s.T
    assert np.allclose(r.y, Y, rtol=1e-13, atol=1e-16)


def test_single_expert_is_dense_swiglu_mlp():
    # E = 1, k = 1: the routed weight renormalises to exactly 1, so y = MLP_0(x) + MLP_shared(x).
    w, x, lg, W = _tiny(T=3, H=64, E=1, k=1, I=32)
    r = moe.moe_block(x, lg, W, 1, "mxfp8")
    assert np.all(r.weights == 1.0) and np.all(r.ids == [[0, 1]] * 3)
    xq = mx.quantize_dequantize(x, "e4m3")
    y = np.zeros_like(x)
    for e in (0, 1):
        w13, w2 = W(e)
        G, U = xq @ w13[:32].T, xq @ w13[32:].T
        y += mx.quantize_dequantize((G / (1 + np.exp(-G))) * U, "e4m3") @ w2.T
    assert np.allclose(r.y, y, rtol=1e-13, atol=1e-16)


def test_q2_quantises_the_exact_swiglu_output():
    # Hand-worked block: amax 300 gives the shared exponent floor(log2 300) - 8 = 0, so the second
    # element is rounded on the E4M3 grid of [1, 2) (step 1/8). 1.0625 + 2^-40 lies just above the
    # midpoint of 1 and 1.125 and must round up to 1.125 (code 0x39); held in fp32 first it would
    # be exactly 1.0625, a tie, and go to the even code 0x38 (1.0).
    a = np.zeros((1, 32))
    a[0, 0], a[0, 1] = 300.0, 1.0625 + 2.0 ** -40
    q = moe.quantize_intermediate(a, "mxfp8")
    assert q[0, 1] == 1.125 and q[0, 0] == 288.0          # 300 -> grid step 32 in [256, 512)
    # the bf16 workload: one rounding of the exact value (1 + 2^-8 + 2^-30 -> 1 + 2^-7)
    b = np.array([[1.0 + 2.0 ** -8 + 2.0 ** -30]])
    assert moe.quantize_intermediate(b, "bf16")[0, 0] == 1.0 + 2.0 ** -7


def test_keep_intermediate_reports_q2_codes():
    w, x, lg, W = _tiny(T=3, H=64, E=4, k=2, I=64)
    r = moe.moe_block(x, lg, W, w.top_k, w.act_fmt, keep_intermediate=True)
    inter = r.extras["intermediate"]
    assert sorted(inter) == [(t, j) for t in range(3) for j in range(3)]
    xq = moe.quantize_activation_rows(x, "mxfp8")
    for (t, j), (codes, scales) in inter.items():
        w13, _ = W(int(r.ids[t, j]))
        g, u = xq[t] @ w13[:w.I].T, xq[t] @ w13[w.I:].T
        a = g / (1 + np.exp(-g)) * u
        assert np.array_equal(mx.dequantize(codes, scales, "e4m3"), moe.quantize_intermediate(a[None], "mxfp8")[0])


# ---------------------------------------------------------------- expert weights from draws
def _from_draws_explicit(a, b, el):
    """Quantisation of one expert's fp32 draws written out row by row: every row of W13 [2I, H]
    is cut into 32-element blocks along H, every row of W2 [H, I] along I, and each block is
    decoded as code value * 2^(byte - 127)."""
    def rows(m):
        out = np.empty(m.shape)
        for r in range(m.shape[0]):
            for c0 in range(0, m.shape[1], 32):
                codes, sb = mx.quantize(m[r, c0:c0 + 32][None], el)
                out[r, c0:c0 + 32] = mx.decode(codes[0], el) * 2.0 ** (int(sb[0, 0]) - 127)
        return out
    return rows(np.asarray(a, np.float64)), rows(np.asarray(b, np.float64))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_from_draws_quantises_along_k(fmt):
    # H != I, so blocks along the wrong axis would not even line up with the matrix shape.
    w = workloads.Workload("fd", 2, 96, 3, 2, 64, fmt, "mxfp8", False, 6)
    W = moe.ExpertWeights.from_draws(lambda e: workloads.draw_expert(w, e), w.E, w.H, w.I, fmt)
    el = {"mxfp8": "e4m3", "mxfp4": "e2m1"}[fmt]
    for e in range(w.E + 1):
        a, b = workloads.draw_expert(w, e)
        w13, w2 = W(e)
        assert w13.shape == (2 * w.I, w.H) and w2.shape == (w.H, w.I)
        ra, rb = _from_draws_explicit(a, b, el)
        assert np.array_equal(w13, ra) and np.array_equal(w2, rb)
        # and through from_mx on codes quantised along H (W13) and along I (W2)
        c13, s13 = mx.quantize(a.astype(np.float64), el)
        c2, s2 = mx.quantize(b.astype(np.float64), el)
        assert s13.shape == (2 * w.I, w.H // 32) and s2.shape == (w.H, w.I // 32)
        Wm = moe.ExpertWeights.from_mx(c13[None], s13[None], c2[None], s2[None], fmt)
        m13, m2 = Wm(0)
        assert np.array_equal(m13, w13) and np.array_equal(m2, w2)


def test_from_draws_axis_hand_worked():
    # W13 [2I = 64, H = 64], W2 [H = 64, I = 32]. Element (0, 0) of W13 is 0.011 and (0, 1) is 400:
    # along H its block has amax 400, shared exponent 0 (byte 127), and 0.011 falls in the
    # subnormal E4M3 range: 0.011 / 2^-9 = 5.63 -> 6 * 2^-9 = 0.01171875. Along the other axis its
    # block (column 0, rows 0..31) would have amax 0.011, shared exponent -7 - 8 = -15 (byte 112):
    # 0.011 * 2^15 = 360.4 -> 352 (grid step 32) -> 0.0107421875. W2 gets the same pair at (0, 0),
    # (0, 1), so its blocks run along I.
    w13 = np.zeros((64, 64), np.float32)
    w13[0, 0], w13[0, 1] = 0.011, 400.0
    w2 = np.zeros((64, 32), np.float32)
    w2[0, 0], w2[0, 1] = 0.011, 400.0
    W = moe.ExpertWeights.from_draws(lambda e: (w13, w2), 0, 64, 32, "mxfp8")
    a, b = W(0)
    assert a[0, 0] == 0.01171875 and b[0, 0] == 0.01171875
    # 400 is the midpoint of 384 and 416 (grid step 32 in [256, 512)): ties go to the even code
    assert a[0, 1] == 384.0 and b[0, 1] == 384.0
    # the scale bytes of those blocks
    _, s = mx.quantize(w13.astype(np.float64), "e4m3")
    assert s[0, 0] == 127
    _, sw = mx.quantize(w13.T.astype(np.float64), "e4m3")
    assert sw[0, 0] == 112                                   # the wrong axis: another byte


def test_token_permutation_invariance():
    w, x, lg, W = _tiny(T=9, H=64, E=6, k=3, I=32)
    r = moe.moe_block(x, lg, W, 3, "mxfp8")
    perm = np.random.default_rng(5).permutation(9)
    rp = moe.moe_block(x[perm], lg[perm], W, 3, "mxfp8")
    assert np.allclose(rp.y, r.y[perm], rtol=1e-13, atol=1e-16)
    assert np.array_equal(rp.ids, r.ids[perm])


def test_token_subset_matches_full():
    w, x, lg, W = _tiny(T=8, H=64, E=6, k=3, I=32)
    full = moe.moe_block(x, lg, W, 3, "mxfp8")
    sub = moe.moe_block(x, lg, W, 3, "mxfp8", tokens=[6, 1, 3])
    assert np.allclose(sub.y[[6, 1, 3]], full.y[[6, 1, 3]], rtol=1e-13, atol=1e-16)


def test_unit_scales_reduce_to_plain_fp8_gemm():
    # All scale bytes 127: the dequantised weights are the E4M3 code values themselves, so G1 is a
    # plain fp8 GEMM; checked against integer arithmetic on codes chosen to be small integers.
    rng = np.random.default_rng(7)
    ints = {0x00: 0, 0x38: 1, 0x40: 2, 0x44: 3, 0xB8: -1, 0xC0: -2}
    keys = np.array(list(ints))
    c13 = rng.choice(keys, size=(1, 64, 64)).astype(np.uint8)
    W = moe.ExpertWeights.from_mx(c13, np.full((1, 64, 2), 127, np.uint8),
                                  np.zeros((1, 64, 32), np.uint8),
                                  np.full((1, 64, 1), 127, np.uint8), "mxfp8")
    w13, _ = W(0)
    iv = np.vectorize(ints.get)(c13[0])
    assert np.array_equal(w13, iv.astype(np.float64))


def test_parity_stats_definition():
    s = moe.parity_stats(np.array([1.0, 2.0, 3.5]), np.array([1.0, 2.0, 4.0]))
    assert s["max_abs_err"] == 0.5 and s["max_rel"] == 0.125
    assert s["mean_rel"] == pytest.approx(0.5 / 7.0)


def test_workload_draws_are_seeded_and_shaped():
    w = workloads.get("tiny_bf16")
    a, b = workloads.draw_x(w), workloads.draw_x(w)
    assert a.shape == (16, 256) and a.dtype == np.uint16 and np.array_equal(a, b)
    w13, w2 = workloads.draw_expert(w, w.E)
    assert w13.shape == (256, 256) and w2.shape == (256, 128)
    xs = workloads.f32_from_bf16_bits(a)
    assert abs(xs.mean()) < 0.05 and abs(xs.std() - 1) < 0.05
    big = workloads.draw_expert(workloads.get("decode_mxfp8"), 3)[0]
    assert abs(big.std() - 0.02) < 1e-4
    z = workloads.get("prefill_mxfp8")
    lg = workloads.f32_from_bf16_bits(workloads.draw_logits(z.with_T(4096)))
    # Zipf bias: the column means fall by 1.1 * ln((e+1)/e) between neighbours
    m = lg.mean(axis=0)
    assert m[0] > m[1] > m[9] > m[99]
    assert abs((m[0] - m[9]) - 1.1 * math.log(10)) < 0.1
