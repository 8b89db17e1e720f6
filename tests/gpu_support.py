"""Shared set-up for the GPU parity tests: seeded inputs on the device, weights prepared by the
library's own kernels, and the oracle's view of the same draws (quantised by the oracle itself)."""
from __future__ import annotations

import functools

import numpy as np
import torch

import workloads
from mx_quantized_grouped_amd import binding as B
from mx_quantized_grouped_amd.weights import ExpertLoader
from oracle import moe

DEV = "cuda"


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def f64(bits: np.ndarray) -> np.ndarray:
    return workloads.f32_from_bf16_bits(bits).astype(np.float64)


def shape_of(w: workloads.Workload, logits_dtype="bf16") -> B.Shape:
    return B.Shape.of(w.T, w.H, w.E, w.top_k, w.I, w.w_fmt, logits_dtype, w.act_fmt)


def packed_weights(name: str):
    """Prepacked device weights of a workload (independent of T), built with mxmoe_quantize and
    mxmoe_prepack from the seeded fp32 draws. Cached: workloads that differ only in T share one
    weight set."""
    w = workloads.get(name)
    key = (w.H, w.E, w.I, w.w_fmt, w.seed)
    if key not in _PACKED:
        if len(_PACKED) >= 3:
            _PACKED.pop(next(iter(_PACKED)))
        loader = ExpertLoader(shape_of(w), DEV)
        workloads.draw_all_experts(w, threads=8, callback=loader.add_expert)
        packed = loader.finish(keep_canonical=True)
        torch.cuda.synchronize()
        _PACKED[key] = (loader, packed)
    return _PACKED[key]


_PACKED: dict = {}


def oracle_weights(w: workloads.Workload) -> moe.ExpertWeights:
    return moe.ExpertWeights.from_draws(lambda e: workloads.draw_expert(w, e), w.E, w.H, w.I,
                                        w.w_fmt)


def oracle_weights_prefetched(w: workloads.Workload, experts, threads: int = 8,
                              ahead: int = 24) -> moe.ExpertWeights:
    """The oracle's expert weights for the experts a block computation will ask for, in the order
    it asks (ascending id), decoded ahead of use on a thread pool: the same per-expert decode, only
    overlapped (each expert takes ~0.5 s of numpy work at these sizes). At most `ahead` decoded
    experts are held at once."""
    from concurrent.futures import ThreadPoolExecutor
    decode = oracle_weights(w)._get
    order = [int(e) for e in sorted(set(int(e) for e in experts))]
    pool = ThreadPoolExecutor(threads)
    futs, nxt = {}, [0]

    def get(e):
        i = order.index(e) if e in order else -1
        while nxt[0] < len(order) and nxt[0] <= i + ahead:
            futs[order[nxt[0]]] = pool.submit(decode, order[nxt[0]])
            nxt[0] += 1
        f = futs.pop(e, None)
        out = f.result() if f is not None else decode(e)
        if nxt[0] >= len(order) and not futs:
            pool.shutdown(wait=False)
        return out
    return moe.ExpertWeights(w.E, w.H, w.I, w.w_fmt, get, cache=0)


@functools.lru_cache(maxsize=16)
def inputs(name: str):
    w = workloads.get(name)
    xb, lb = workloads.draw_x(w), workloads.draw_logits(w)
    return w, xb, lb


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], mid]))


# Workloads up to this many tokens are compared on every token; larger ones on a sample that
# puts at least one compared slot in every tile of the layout the large-M launcher uses.
FULL_COMPARE_MAX_T = 128


def covering_tokens(name: str, block_m: int = 128, seed: int = 0) -> np.ndarray:
    """Tokens of a workload such that every block_m-row tile of its sorted layout (the oracle's
    route and align) holds at least one slot of a chosen token, plus the first and last token.
    Within a tile the slot is drawn at random, so different rows of the tiles are covered."""
    w, _, lb = inputs(name)
    if w.T <= FULL_COMPARE_MAX_T:
        return np.arange(w.T)
    ids, _ = moe.route(f64(lb), w.top_k)
    L = moe.align(ids, w.E, block_m)
    S = w.slots
    rng = np.random.default_rng(seed)
    toks = {0, w.T - 1}
    for b in range(L.num_post_pad // block_m):
        rows = L.sorted_ids[b * block_m:(b + 1) * block_m]
        valid = rows[rows < S]
        if not any(int(f) // (w.top_k + 1) in toks for f in valid):
            toks.add(int(rng.choice(valid)) // (w.top_k + 1))
    return np.array(sorted(toks))


@functools.lru_cache(maxsize=16)
def oracle_result(name: str):
    """The oracle on every token (T <= 128) or on the tile-covering sample."""
    w, xb, lb = inputs(name)
    toks = covering_tokens(name)
    ids, _ = moe.route(f64(lb)[toks], w.top_k)
    W = oracle_weights_prefetched(w, np.unique(ids))
    return moe.moe_block(f64(xb), f64(lb), W, w.top_k, w.act_fmt, tokens=toks)


def tolerance_ok(stats: dict) -> bool:
    # The block's output tolerance: max |err| <= 2e-2 * max |ref| and sum|err| / sum|ref| <= 5e-3.
    return stats["max_rel"] <= 2e-2 and stats["mean_rel"] <= 5e-3
