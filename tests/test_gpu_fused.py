"""The one-launch decode path (routing, layout, gate_up, down and the final sum as roles of one grid)
against the oracle and against the separate-launch path.

- Every output element within the block's tolerance of the oracle, on every small-batch workload
  and on edge shapes; routing, the sorted layout and the activation codes it leaves in the workspace
  bit for bit.
- Bit-identical to the separate-launch path where both split K the same way (the same sums in
  the same order), and to itself call after call (fixed-order final sum).
- The bounded waits: with the layout held back from the host side every wait gives up after its
  spin limit, the kernel ends, the status word reads 1, and the next call on the same workspace is
  correct again (the control words were reset).
- HIP graph replay of the one launch equals the eager result on new inputs."""
import numpy as np
import pytest
import torch

import workloads
from mx_quantized_grouped_amd import binding as B
from mx_quantized_grouped_amd.weights import ExpertLoader
from oracle import moe, mx

from gpu_support import (DEV, bf16_tensor, f64, inputs, oracle_result, oracle_weights,
                         packed_weights, shape_of, tolerance_ok)

pytestmark = pytest.mark.gpu

FUSED = B.Options(0, 0, 0, 0, None, 1)
SEPARATE = B.Options(1, 1, 0, 0, None, -1)
SMALL_MX = ["decode_mxfp8", "decode_mxfp4", "wide512_mxfp4_T1", "wide512_mxfp4_T6"]


def _say(*a):
    print("[gpu-fused]", *a, flush=True)


def _run(shape, xb, lb, packed, options, ws=None):
    if ws is None:
        ws = B.new_workspace(B.mxmoe_workspace_bytes(shape, options), DEV)
    y = B.mxmoe_forward(shape, bf16_tensor(xb), bf16_tensor(lb), packed, workspace=ws,
                        options=options)
    torch.cuda.synchronize()
    return y, ws


def _view(ws, shape, options, which, dtype=torch.int32):
    off, nb, bm = B.mxmoe_workspace_view(shape, options, which)
    return ws[off:off + nb].view(dtype).cpu().numpy(), bm


@pytest.mark.parametrize("name", SMALL_MX)
def test_fused_parity(name):
    _say("parity", name)
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w)
    y, ws = _run(shape, xb, lb, packed, FUSED)
    assert B.workspace_status(shape, ws, FUSED) == 0
    r = oracle_result(name)
    assert len(r.tokens) == w.T
    ids, _ = _view(ws, shape, FUSED, B.VIEW_TOPK_IDS)
    assert np.array_equal(ids.reshape(w.T, w.top_k + 1), r.ids)
    sids, bm = _view(ws, shape, FUSED, B.VIEW_SORTED_IDS)
    L = moe.align(r.ids, w.E, bm)
    assert bm == 16 and np.array_equal(sids, L.sorted_ids)
    bexp, _ = _view(ws, shape, FUSED, B.VIEW_BLOCK_EXPERT)
    assert np.array_equal(bexp, L.block_expert)
    eoff, _ = _view(ws, shape, FUSED, B.VIEW_EXPERT_OFF)
    assert np.array_equal(eoff, L.expert_off)
    xq, _ = _view(ws, shape, FUSED, B.VIEW_XQ, torch.uint8)
    xs, _ = _view(ws, shape, FUSED, B.VIEW_XS, torch.uint8)
    rc, rs = mx.quantize(f64(xb), "e4m3")
    assert np.array_equal(xq.reshape(w.T, w.H), rc)
    assert np.array_equal(xs.reshape(w.T, -1)[:, :w.H // 32], rs)
    st = moe.parity_stats(y.float().cpu().numpy().astype(np.float64), r.y)
    _say(name, st)
    assert tolerance_ok(st), st


@pytest.mark.parametrize("name", ["decode_mxfp8", "decode_mxfp4", "wide512_mxfp4_T1"])
def test_fused_equals_separate_launches(name):
    # Same split of K (one wave per unit, or four waves taking every fourth K-step) on both paths:
    # the same fp32 sums in the same order, so the outputs are equal bit for bit; and one-launch
    # calls repeat bit for bit.
    _say("fused == separate", name)
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w)
    y1, ws = _run(shape, xb, lb, packed, FUSED)
    y2, _ = _run(shape, xb, lb, packed, FUSED, ws)
    ys, _ = _run(shape, xb, lb, packed, SEPARATE)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), ys.view(torch.int16))


@pytest.mark.parametrize("T,H,E,k,I,fmt", [
    (1, 128, 1, 1, 32, "mxfp8"),      # one token, one routed expert
    (5, 256, 4, 4, 96, "mxfp8"),      # k == E; I not a multiple of 128 (padded K of down)
    (7, 384, 6, 2, 160, "mxfp4"),
    (17, 256, 8, 2, 64, "mxfp8"),     # two shared-expert groups
    (40, 512, 3, 2, 128, "mxfp8"),    # experts with more than 16 rows (several gate_up passes)
    (70, 256, 200, 3, 64, "mxfp4"),   # tokens past 64 (the second membership word), E > 128
    (128, 256, 16, 8, 128, "mxfp8"),  # the largest batch of the path
])
def test_fused_edge_shapes(T, H, E, k, I, fmt):
    _say("edge", T, H, E, k, I, fmt)
    wl = workloads.Workload(f"fedge_{T}_{H}_{E}_{k}_{I}_{fmt}", T, H, E, k, I, fmt, "mxfp8",
                            False, 3)
    shape = shape_of(wl)
    loader = ExpertLoader(shape, DEV)
    for e in range(E + 1):
        loader.add_expert(e, *workloads.draw_expert(wl, e))
    packed = loader.finish()
    xb, lb = workloads.draw_x(wl), workloads.draw_logits(wl)
    ref = moe.moe_block(f64(xb), f64(lb), oracle_weights(wl), k, wl.act_fmt)
    y, ws = _run(shape, xb, lb, packed, FUSED)
    assert B.workspace_status(shape, ws, FUSED) == 0
    ids, _ = _view(ws, shape, FUSED, B.VIEW_TOPK_IDS)
    assert np.array_equal(ids.reshape(T, k + 1), ref.ids)
    st = moe.parity_stats(y.float().cpu().numpy().astype(np.float64), ref.y)
    assert tolerance_ok(st), st
    # fp32 logits take the other key path of the routers and of the membership test
    shape32 = shape_of(wl, "f32")
    ws32 = B.new_workspace(B.mxmoe_workspace_bytes(shape32, FUSED), DEV)
    y32 = B.mxmoe_forward(shape32, bf16_tensor(xb), bf16_tensor(lb).float(), packed,
                          workspace=ws32, options=FUSED)
    torch.cuda.synchronize()
    assert torch.equal(y32.view(torch.int16), y.view(torch.int16))


def test_fused_wait_gives_up_and_recovers():
    # The layout is never published (hold): the gate_up epilogues and the down units wait for it,
    # give up after 64 polls each, and the kernel ends; the status word says so. The next call on
    # the same workspace finds the control words reset and gives the right output.
    _say("bounded wait")
    name = "wide512_mxfp4_T6"
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w)
    held = B.Options(0, 0, 0, 0, None, 1, 64, 1)
    ws = B.new_workspace(B.mxmoe_workspace_bytes(shape, held), DEV)
    _run(shape, xb, lb, packed, held, ws)
    assert B.workspace_status(shape, ws, held) == 1
    y, _ = _run(shape, xb, lb, packed, FUSED, ws)
    assert B.workspace_status(shape, ws, FUSED) == 0
    ref, _ = _run(shape, xb, lb, packed, FUSED)
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["decode_mxfp8", "wide512_mxfp4_T1"])
def test_fused_graph_replay(name):
    # One launch captured in a HIP graph, replayed on new inputs written into the captured buffers
    # with eager calls and host synchronisations in between: every replay equals the eager result.
    _say("graph replay", name)
    w, xb, lb = inputs(name)
    _, packed = packed_weights(name)
    shape = shape_of(w)
    rng = np.random.default_rng(5)
    draws = [(xb, lb)] + [(xb[rng.permutation(w.T)], lb[rng.permutation(w.T)]) for _ in range(2)]
    xs, ls = bf16_tensor(xb), bf16_tensor(lb)
    ys = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    wss = B.new_workspace(B.mxmoe_workspace_bytes(shape, FUSED), DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.mxmoe_forward(shape, xs, ls, packed, y=ys, workspace=wss, options=FUSED)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.mxmoe_forward(shape, xs, ls, packed, y=ys, workspace=wss, options=FUSED)
    torch.cuda.synchronize()
    for xr, lr in draws:
        ref, _ = _run(shape, xr, lr, packed, FUSED)
        xs.copy_(bf16_tensor(xr))
        ls.copy_(bf16_tensor(lr))
        ys.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys.view(torch.int16), ref.view(torch.int16))
        assert B.workspace_status(shape, wss, FUSED) == 0
