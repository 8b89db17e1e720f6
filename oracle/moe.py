"""The MX-quantised MoE expert block, step by step in plain fp64 — the CPU oracle.

Test infrastructure only (tests/, the package smoke check and the bench's CPU baseline use it);
it shares no code with the GPU path. Each function states the passage it follows. The pages are:

  [M3]  "Lần theo điểm nghẽn: Tối ưu MiniMax M3 trên AMD Instinct MI355X" (gpuhub.net)
  [M3j] "AMD Instinct MI355X 上での MiniMax M3 の最適化" (agentlenshq.com), the same campaign
  [K3]  "Tối ưu hiệu năng Kimi K3 trong vLLM: Hành trình đạt thông lượng gấp 2,8 lần"
  [L3]  "Ling-3.0-flash: Tối ưu hóa độ trễ giải mã lên 54% trên 4 GPU Blackwell"

The block, per token t with bf16 activations x[t] and bf16 router logits l[t] (or logits from the
gate in front of it, step 0: l = x . W_g^T, [L3] "Sửa thước đo trước khi sửa máy"):
  1. route  : top-k routed experts by logit (ties to the lower index), softmax weights over the k
              selected, and the shared expert appended as slot k with weight 1   ([M3] shared-expert
              passage, Fig. 4: the shared expert is a table entry every token selects).
  2. align  : slots grouped expert by expert into tile-padded blocks (the layout the grouped GEMMs
              consume; [M3] local-shapes passage on grouped MoE programs).
  3. Q1     : x[t] -> MXFP8 (E4M3), one scale per 32 along H (MXFP4, E2M1, for the W4A4 reading).
  4. G1     : gate/up projection of the quantised row by the (dequantised) fused W13 of the expert.
  5. S      : SwiGLU, a = SiLU(gate) * up ([M3] shared-expert passage lists "gate/up projection,
              activation, down projection" as the dense expert MLP).
  6. Q2     : a -> MXFP8 per 32 along I (bf16 rounding in the unquantised workload).
  7. G2     : down projection by the (dequantised) W2 of the expert.
  8. combine: y[t] = sum over slots of weight * down output ([K3] deferred-finalize passage: the
              top-k finalize is the weighted sum back to token order).
Readings of points the pages leave open are listed with each function.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import mx


# ---------------------------------------------------------------- 0. gate (in front of route)
def gate_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """Router logits l[t, e] = sum_h x[t, h] * w_gate[e, h] in fp64.

    x: [T, H] and w_gate: [E, H] (bf16 values held in fp64). [L3] "Sửa thước đo trước khi sửa
    máy" names a bf16 gate in front of the router (a 2.6 MB gate-weight kernel): reading, the
    gate's operands are bf16 and its products are summed in at least fp32, so the exact sum of
    the bf16 products is the reference and a device result differs from it only by accumulation
    rounding. The definition is the matrix product itself."""
    x = np.asarray(x, dtype=np.float64)
    w_gate = np.asarray(w_gate, dtype=np.float64)
    if x.ndim != 2 or w_gate.ndim != 2 or x.shape[1] != w_gate.shape[1]:
        raise ValueError("need x [T, H] and w_gate [E, H]")
    return x @ w_gate.T


# ---------------------------------------------------------------- 1. route
def route(logits: np.ndarray, top_k: int):
    """Top-k routing with renormalised softmax weights and the shared slot.

    logits: [T, E] finite values (bf16 values held in fp64). For each token the experts are ordered
    by (logit descending, expert index ascending) — the fixed lowest-index tie-break, with -0 == +0
    — and the first top_k are taken, in that order. Selection is on logits: softmax is strictly
    increasing, and a monotone map cannot change a top-k order ([M3] speculative-indexer passage:
    only the top-k order matters and a positive rescale cannot change it). Weights are softmax
    restricted to the selected experts (equal to softmax over all E renormalised over the top k).
    The shared expert (id E) fills slot top_k with weight exactly 1 ([M3] Fig. 4).

    Returns ids int64 [T, top_k + 1] and weights fp64 [T, top_k + 1]."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("need 1 <= top_k <= E")
    if not np.all(np.isfinite(logits)):
        raise ValueError("router logits must be finite")
    ids = np.empty((T, top_k + 1), dtype=np.int64)
    w = np.empty((T, top_k + 1), dtype=np.float64)
    for t in range(T):
        row = logits[t]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        sel = order[:top_k]
        top = row[sel[0]]
        p = [math.exp(row[e] - top) for e in sel]
        s = math.fsum(p)
        ids[t, :top_k] = sel
        w[t, :top_k] = [v / s for v in p]
        ids[t, top_k] = E
        w[t, top_k] = 1.0
    return ids, w


# ---------------------------------------------------------------- 2. align
def align_capacity(T: int, E: int, top_k: int, block_m: int) -> int:
    """Upper bound on the padded slot count: every touched expert (at most min(E+1, S) of them)
    wastes at most block_m - 1 rows; rounded up to a whole block."""
    S = T * (top_k + 1)
    cap = S + min(E + 1, S) * (block_m - 1)
    return -(-cap // block_m) * block_m


@dataclass
class Layout:
    sorted_ids: np.ndarray      # [cap] flat slot ids; sentinel S = T*(k+1) in padding
    block_expert: np.ndarray    # [cap / block_m] expert of each block; -1 past the end
    num_post_pad: int           # padded slot count actually used
    expert_off: np.ndarray      # [E + 2] start of each expert's rows in sorted_ids (+ total)
    counts: np.ndarray          # [E + 1] slots per expert
    block_m: int


def align(ids: np.ndarray, E: int, block_m: int) -> Layout:
    """Counting sort of the flat slots f = t*(k+1) + j into expert-contiguous, tile-padded blocks.

    Experts 0..E (the shared expert E last) are laid out in ascending id order. Within an expert
    the slots keep ascending f (stable). Each expert's run is padded with the sentinel
    S = T*(k+1) to a multiple of block_m; experts with no slots get no blocks. Reading: the pages
    describe grouped MoE programs over expert-contiguous work ([M3] local-shapes passage) and
    GPU-resident counts turned into indices by fixed shapes plus padding ([L3] "Hình dạng của một
    bước batch-1"), not the layout itself; this is the plainest layout with those properties."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k1 = ids.shape
    S = T * k1
    flat = ids.reshape(-1)
    if np.any((flat < 0) | (flat > E)):
        raise ValueError("expert id out of range")
    cap = align_capacity(T, E, k1 - 1, block_m)
    sorted_ids = []
    block_expert = []
    counts = np.zeros(E + 1, dtype=np.int64)
    expert_off = np.zeros(E + 2, dtype=np.int64)
    for e in range(E + 1):
        expert_off[e] = len(sorted_ids)
        fs = [int(f) for f in np.nonzero(flat == e)[0]]      # ascending f
        counts[e] = len(fs)
        if not fs:
            continue
        padded = -(-len(fs) // block_m) * block_m
        sorted_ids += fs + [S] * (padded - len(fs))
        block_expert += [e] * (padded // block_m)
    expert_off[E + 1] = len(sorted_ids)
    num_post_pad = len(sorted_ids)
    sorted_ids += [S] * (cap - num_post_pad)
    block_expert += [-1] * (cap // block_m - len(block_expert))
    return Layout(np.array(sorted_ids, dtype=np.int64), np.array(block_expert, dtype=np.int64),
                  num_post_pad, expert_off, counts, block_m)


# ---------------------------------------------------------------- expert weights
class ExpertWeights:
    """Dequantised fp64 expert weights, one expert at a time (W13 [2I, H], W2 [H, I]).

    Built either from MX codes + scales already in hand (`from_mx`), from bf16-valued arrays
    (`from_dense`), or lazily from fp32 draws that this class quantises with the oracle's own MX
    quantiser (`from_draws`). Only experts that are asked for are decoded; a small cache keeps the
    most recent ones."""

    def __init__(self, E: int, H: int, I: int, fmt: str, getter, cache: int = 24):
        self.E, self.H, self.I, self.fmt = E, H, I, fmt
        self._get = getter
        self._cache: dict[int, tuple[np.ndarray, np.ndarray]] = {}
        self._order: list[int] = []
        self._cap = cache

    def __call__(self, e: int):
        if e in self._cache:
            return self._cache[e]
        val = self._get(e)
        self._cache[e] = val
        self._order.append(e)
        if len(self._order) > self._cap:
            self._cache.pop(self._order.pop(0), None)
        return val

    @staticmethod
    def from_mx(w13_codes, w13_scales, w2_codes, w2_scales, fmt: str) -> "ExpertWeights":
        """Codes [E+1, rows, K] (one code per byte), scale bytes [E+1, rows, K/32]."""
        E1, twoI, H = w13_codes.shape
        el = {"mxfp8": "e4m3", "mxfp4": "e2m1"}[fmt]

        def get(e):
            return (mx.dequantize(w13_codes[e], w13_scales[e], el),
                    mx.dequantize(w2_codes[e], w2_scales[e], el))
        return ExpertWeights(E1 - 1, H, twoI // 2, fmt, get)

    @staticmethod
    def from_dense(w13, w2) -> "ExpertWeights":
        """Unquantised weights (bf16 values) [E+1, 2I, H] and [E+1, H, I]."""
        E1, twoI, H = w13.shape

        def get(e):
            return np.asarray(w13[e], np.float64), np.asarray(w2[e], np.float64)
        return ExpertWeights(E1 - 1, H, twoI // 2, "bf16", get)

    @staticmethod
    def from_draws(draw, E: int, H: int, I: int, fmt: str) -> "ExpertWeights":
        """`draw(e)` returns the fp32 draws (W13, W2) of expert e; MX formats are quantised here
        along K (H for W13, I for W2) with the oracle's quantiser."""
        def get(e):
            a, b = draw(e)
            if fmt == "bf16":
                return np.asarray(a, np.float64), np.asarray(b, np.float64)
            el = {"mxfp8": "e4m3", "mxfp4": "e2m1"}[fmt]
            return mx.quantize_dequantize(a, el), mx.quantize_dequantize(b, el)
        return ExpertWeights(E, H, I, fmt, get)


# ---------------------------------------------------------------- 3..8 the block
def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


# Element format of the quantised activations. MXFP8 activations are the served configuration
# ([M3] opening results). For MXFP4 weights the pages give throughput but no activation format
# ([M3] opening results, the MXFP4 bullet); the "mxfp4" activation format reads W4A4 as the same MX
# rule with E2M1 elements (largest exponent 2) in both Q1 and Q2.
ACT_ELEMENT = {"mxfp8": "e4m3", "mxfp4": "e2m1"}


def quantize_activation_rows(x: np.ndarray, act_fmt: str) -> np.ndarray:
    """Q1: MX along the row, one scale per 32 values (E4M3 elements for "mxfp8", E2M1 for
    "mxfp4"); identity for bf16."""
    if act_fmt == "bf16":
        return np.asarray(x, np.float64)
    return mx.quantize_dequantize(x, ACT_ELEMENT[act_fmt])


def quantize_intermediate(a: np.ndarray, act_fmt: str) -> np.ndarray:
    """Q2 on the SwiGLU output, per slot row along I: the MX rule of Q1 (same element format)
    applied to the exact a; in the unquantised workload a is rounded to bf16 before the down
    projection. The dense expert MLP sequence of [M3]'s shared-expert passage stores the activation
    output between the two projections; the MX format of that store is the served format ([M3]
    opening results), so the rule applies to a as the activation defines it, with no intermediate
    precision in between."""
    a = np.asarray(a, np.float64)
    if act_fmt == "bf16":
        return mx.round_to_bf16(a)
    return mx.quantize_dequantize(a, ACT_ELEMENT[act_fmt])


@dataclass
class BlockResult:
    y: np.ndarray                 # [T, H] fp64 (rows not requested are zero)
    ids: np.ndarray               # [T, k+1]
    weights: np.ndarray           # [T, k+1]
    tokens: np.ndarray            # the tokens y was computed for
    extras: dict = field(default_factory=dict)


def moe_block(x: np.ndarray, logits: np.ndarray, weights: ExpertWeights, top_k: int,
              act_fmt: str, tokens=None, keep_intermediate: bool = False) -> BlockResult:
    """The whole block for the requested tokens (default: all), grouped by expert.

    x: [T, H] bf16 values (fp64), logits: [T, E]. For each expert e in ascending order the slots
    routed to it form one group ([M3] Fig. 4: routed and shared experts share one grouped-GEMM
    pass); their quantised rows are multiplied by the dequantised W13 of e (one fp64 matmul), SiLU(
    gate) * up is quantised per row (Q2), multiplied by W2 of e, and added into y[t] with the
    routing weight of the slot (weight applied after the down projection, in the combine).

    keep_intermediate: also return, in extras["intermediate"], each computed slot's Q2 result as
    {(t, j): (codes, scale bytes)} for MX activations (the MX quantiser's own output for the row)
    or {(t, j): bf16 values} for the unquantised workload."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    ids, w = route(logits, top_k)
    E = logits.shape[1]
    I = weights.I
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    xq = quantize_activation_rows(x[tokens], act_fmt)          # Q1 on the requested rows only
    y = np.zeros((T, H), dtype=np.float64)
    inter = {}
    sub_ids = ids[tokens]
    for e in range(E + 1):
        rr, jj = np.nonzero(sub_ids == e)                        # slots (token row, j) on expert e
        if rr.size == 0:
            continue
        order = np.argsort(tokens[rr] * (top_k + 1) + jj, kind="stable")
        rr, jj = rr[order], jj[order]
        w13, w2 = weights(e)
        gu = xq[rr] @ w13.T                                      # G1: [n_e, 2I]
        a = silu(gu[:, :I]) * gu[:, I:]                          # S
        ah = quantize_intermediate(a, act_fmt)                   # Q2
        d = ah @ w2.T                                            # G2: [n_e, H]
        wt = w[tokens[rr], jj]
        np.add.at(y, tokens[rr], wt[:, None] * d)                # combine
        if keep_intermediate:
            coded = (None if act_fmt == "bf16" else mx.quantize(a, ACT_ELEMENT[act_fmt]))
            for i, (r_, j_) in enumerate(zip(rr, jj)):
                key = (int(tokens[r_]), int(j_))
                inter[key] = ah[i] if coded is None else (coded[0][i], coded[1][i])
    return BlockResult(y=y, ids=ids, weights=w, tokens=tokens,
                       extras={"intermediate": inter} if keep_intermediate else {})


# ---------------------------------------------------------------- pass/fail measure
def parity_stats(y: np.ndarray, ref: np.ndarray) -> dict:
    """max |y - ref| / max |ref|  and  sum |y - ref| / sum |ref|  (the block's output tolerance is
    stated on these two), plus the cosine similarity the [M3] correctness-contracts passage uses
    to expose a broken expert mask."""
    y = np.asarray(y, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    err = np.abs(y - r)
    mx_ref = float(np.max(np.abs(r))) if r.size else 0.0
    sum_ref = float(np.sum(np.abs(r)))
    denom = float(np.linalg.norm(y) * np.linalg.norm(r))
    return {
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_ref": mx_ref,
        "max_rel": float(err.max() / mx_ref) if mx_ref > 0 else float(err.max() if err.size else 0),
        "mean_rel": float(err.sum() / sum_ref) if sum_ref > 0 else float(err.sum()),
        "cosine": float(np.dot(y, r) / denom) if denom > 0 else 1.0,
    }
