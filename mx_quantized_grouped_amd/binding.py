"""Thin ctypes binding of libmxmoe.so (include/mxmoe.h), with the same entry-point names.

Argument marshalling only: torch supplies device memory (data_ptr) and the current HIP stream;
every step of the block runs in the library's HIP kernels. Importing works without a GPU; calling
raises if the library is not built."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxmoe.so")

# ----------------------------------------------------------------------------- constants
MXMOE_OK, MXMOE_EINVAL, MXMOE_EUNSUPPORTED, MXMOE_EWORKSPACE, MXMOE_EHIP = 0, -1, -2, -3, -4
MXMOE_BF16, MXMOE_F32, MXMOE_MXFP8_E4M3, MXMOE_MXFP4_E2M1 = 0, 1, 2, 3
MXMOE_LAUNCH_AUTO, MXMOE_LAUNCH_SMALL_M, MXMOE_LAUNCH_LARGE_M = 0, 1, 2
MXMOE_COMBINE_AUTO, MXMOE_COMBINE_SLOTS, MXMOE_COMBINE_ATOMIC, MXMOE_COMBINE_SLOTS_BF16 = 0, 1, 2, 3
MXMOE_LAYOUT_AUTO, MXMOE_LAYOUT_SORTED, MXMOE_LAYOUT_SLOTS = 0, 1, 2
(VIEW_TOPK_IDS, VIEW_TOPK_W, VIEW_SORTED_IDS, VIEW_BLOCK_EXPERT, VIEW_NUM_POST_PAD, VIEW_EXPERT_OFF,
 VIEW_XQ, VIEW_XS, VIEW_H, VIEW_HS, VIEW_STATUS) = range(11)
WORKSPACE_CONTROL_BYTES = 72 * 1024

FMT_BY_NAME = {"bf16": MXMOE_BF16, "f32": MXMOE_F32, "mxfp8": MXMOE_MXFP8_E4M3,
               "mxfp4": MXMOE_MXFP4_E2M1}

EXPORTS = [
    "mxmoe_status_string", "mxmoe_gate", "mxmoe_gate_ex", "mxmoe_route", "mxmoe_align_capacity", "mxmoe_align_workspace_bytes",
    "mxmoe_align", "mxmoe_align_ex", "mxmoe_quantize", "mxmoe_prepacked_bytes", "mxmoe_prepack",
    "mxmoe_workspace_bytes", "mxmoe_workspace_bytes_ex", "mxmoe_forward", "mxmoe_forward_ex",
    "mxmoe_workspace_view", "mxmoe_forward_noalloc",
]


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("I", ctypes.c_int32), ("w_fmt", ctypes.c_int32),
                ("act_fmt", ctypes.c_int32), ("logits_dtype", ctypes.c_int32)]

    @staticmethod
    def of(T, H, E, top_k, I, w_fmt="mxfp8", logits_dtype="bf16", act_fmt=None) -> "Shape":
        """act_fmt None: bf16 activations for bf16 weights, MXFP8 for MX weights."""
        wf = FMT_BY_NAME[w_fmt] if isinstance(w_fmt, str) else int(w_fmt)
        if act_fmt is None:
            af = MXMOE_BF16 if wf == MXMOE_BF16 else MXMOE_MXFP8_E4M3
        else:
            af = FMT_BY_NAME[act_fmt] if isinstance(act_fmt, str) else int(act_fmt)
        ld = FMT_BY_NAME[logits_dtype] if isinstance(logits_dtype, str) else int(logits_dtype)
        return Shape(T, H, E, top_k, I, wf, af, ld)

    def with_T(self, T: int) -> "Shape":
        return Shape(T, self.H, self.E, self.top_k, self.I, self.w_fmt, self.act_fmt,
                     self.logits_dtype)


MXMOE_STAGE_EVENTS = 5
STAGES = ("prologue", "gate_up", "down", "finalize")


class Options(ctypes.Structure):
    _fields_ = [("launcher", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("unit_run", ctypes.c_int32),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                ("fused", ctypes.c_int32), ("spin_limit", ctypes.c_int32),
                ("hold", ctypes.c_int32), ("layout", ctypes.c_int32)]


class MxMoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m mx_quantized_grouped_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sp, op = ctypes.POINTER(Shape), ctypes.POINTER(Options)
    sig = {
        "mxmoe_status_string": (ctypes.c_char_p, [i32]),
        "mxmoe_gate": (i32, [vp, vp, i32, i32, i32, i32, vp, vp]),
        "mxmoe_gate_ex": (i32, [vp, vp, i32, i32, i32, i32, i32, vp, vp]),
        "mxmoe_route": (i32, [vp, i32, i32, i32, i32, vp, vp, vp]),
        "mxmoe_align_capacity": (sz, [i32, i32, i32, i32]),
        "mxmoe_align_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "mxmoe_align": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp]),
        "mxmoe_align_ex": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "mxmoe_quantize": (i32, [vp, i32, i32, i32, i32, vp, vp, vp]),
        "mxmoe_prepacked_bytes": (sz, [sp, i32]),
        "mxmoe_prepack": (i32, [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "mxmoe_workspace_bytes": (sz, [sp]),
        "mxmoe_workspace_bytes_ex": (sz, [sp, op]),
        "mxmoe_forward": (i32, [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "mxmoe_forward_ex": (i32, [sp, op, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "mxmoe_workspace_view": (sz, [sp, op, i32, ctypes.POINTER(sz), ctypes.POINTER(i32)]),
        "mxmoe_forward_noalloc": (i32, [sp, vp, vp, vp, vp, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def status_string(status: int) -> str:
    try:
        return lib().mxmoe_status_string(int(status)).decode()
    except RuntimeError:
        return "library not built"


def _check(status: int, where: str):
    if status != MXMOE_OK:
        raise MxMoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t):
    return t.device


# ----------------------------------------------------------------------------- entry points
def mxmoe_status_string(status: int) -> str:
    return status_string(status)


def mxmoe_gate(x: torch.Tensor, w_gate: torch.Tensor, out_dtype=torch.float32, logits=None,
               stream=None, tile: int = 0):
    """Router logits x . w_gate^T (bf16 operands, fp32 sums) as a [T, E] fp32 or bf16 tensor.
    tile != 0 picks the kernel tile (mxmoe_gate_ex)."""
    T, H = x.shape
    E = w_gate.shape[0]
    if logits is None:
        logits = torch.empty((T, E), dtype=out_dtype, device=_dev(x))
    ld = MXMOE_F32 if logits.dtype == torch.float32 else MXMOE_BF16
    if tile:
        st = lib().mxmoe_gate_ex(_ptr(x), _ptr(w_gate), T, H, E, ld, tile, _ptr(logits),
                                 _stream(stream))
    else:
        st = lib().mxmoe_gate(_ptr(x), _ptr(w_gate), T, H, E, ld, _ptr(logits), _stream(stream))
    _check(st, "mxmoe_gate")
    return logits


def mxmoe_route(logits: torch.Tensor, top_k: int, topk_ids=None, topk_w=None, stream=None):
    T, E = logits.shape
    ld = MXMOE_F32 if logits.dtype == torch.float32 else MXMOE_BF16
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k + 1), dtype=torch.int32, device=_dev(logits))
    if topk_w is None:
        topk_w = torch.empty((T, top_k + 1), dtype=torch.float32, device=_dev(logits))
    _check(lib().mxmoe_route(_ptr(logits), T, E, top_k, ld, _ptr(topk_ids), _ptr(topk_w),
                             _stream(stream)), "mxmoe_route")
    return topk_ids, topk_w


def mxmoe_align_capacity(T: int, E: int, top_k: int, block_m: int) -> int:
    return int(lib().mxmoe_align_capacity(T, E, top_k, block_m))


def mxmoe_align_workspace_bytes(T: int, E: int, top_k: int, block_m: int) -> int:
    return int(lib().mxmoe_align_workspace_bytes(T, E, top_k, block_m))


def mxmoe_align(topk_ids: torch.Tensor, E: int, block_m: int, with_expert_off=True, stream=None):
    """The sort through mxmoe_align_ex (expert offsets, and the scratch a large sort needs, in
    tensors allocated here)."""
    T, k1 = topk_ids.shape
    top_k = k1 - 1
    cap = mxmoe_align_capacity(T, E, top_k, block_m)
    dev = _dev(topk_ids)
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    block_expert = torch.empty(cap // block_m if block_m else 0, dtype=torch.int32, device=dev)
    npp = torch.empty(1, dtype=torch.int32, device=dev)
    eoff = torch.empty(E + 2, dtype=torch.int32, device=dev) if with_expert_off else None
    wsb = mxmoe_align_workspace_bytes(T, E, top_k, block_m)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check(lib().mxmoe_align_ex(_ptr(topk_ids), T, E, top_k, block_m, _ptr(sorted_ids),
                                _ptr(block_expert), _ptr(npp), _ptr(eoff), _ptr(ws), wsb,
                                _stream(stream)), "mxmoe_align_ex")
    return sorted_ids, block_expert, npp, eoff


mxmoe_align_ex = mxmoe_align


def mxmoe_quantize(src: torch.Tensor, fmt="mxfp8", codes=None, scales=None, stream=None):
    rows, K = src.shape
    f = FMT_BY_NAME[fmt] if isinstance(fmt, str) else int(fmt)
    sd = MXMOE_F32 if src.dtype == torch.float32 else MXMOE_BF16
    cw = K if f == MXMOE_MXFP8_E4M3 else K // 2
    if codes is None:
        codes = torch.empty((rows, cw), dtype=torch.uint8, device=_dev(src))
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=_dev(src))
    _check(lib().mxmoe_quantize(_ptr(src), rows, K, sd, f, _ptr(codes), _ptr(scales),
                                _stream(stream)), "mxmoe_quantize")
    return codes, scales


def mxmoe_prepacked_bytes(shape: Shape, which: int) -> int:
    return int(lib().mxmoe_prepacked_bytes(ctypes.byref(shape), which))


def mxmoe_prepack(shape: Shape, w13, s13, w2, s2, out=None, stream=None):
    dev = _dev(w13)
    if out is None:
        out = [torch.empty(max(mxmoe_prepacked_bytes(shape, i), 1), dtype=torch.uint8, device=dev)
               for i in range(4)]
    _check(lib().mxmoe_prepack(ctypes.byref(shape), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                               *[_ptr(o) for o in out], _stream(stream)), "mxmoe_prepack")
    return out


def mxmoe_workspace_bytes(shape: Shape, options: Options | None = None) -> int:
    if options is None:
        return int(lib().mxmoe_workspace_bytes(ctypes.byref(shape)))
    return int(lib().mxmoe_workspace_bytes_ex(ctypes.byref(shape), ctypes.byref(options)))


def mxmoe_workspace_view(shape: Shape, options: Options | None, which: int):
    """(byte offset, byte size, block_m) of an intermediate inside forward's workspace."""
    nb, bm = ctypes.c_size_t(0), ctypes.c_int(0)
    off = lib().mxmoe_workspace_view(ctypes.byref(shape),
                                     ctypes.byref(options) if options is not None else None,
                                     which, ctypes.byref(nb), ctypes.byref(bm))
    if off == ctypes.c_size_t(-1).value:
        raise MxMoeError(MXMOE_EINVAL, "mxmoe_workspace_view")
    return int(off), int(nb.value), int(bm.value)


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A forward workspace of nbytes, zero-filled (its control words must start at zero; every
    forward call leaves them zero, so it can be reused for any later call)."""
    return torch.zeros(max(int(nbytes), WORKSPACE_CONTROL_BYTES), dtype=torch.uint8, device=device)


def workspace_status(shape: Shape, workspace: torch.Tensor, options: Options | None = None) -> int:
    """Status word of the last one-launch forward on this workspace (0 ok, 1 a wait gave up)."""
    off, nb, _ = mxmoe_workspace_view(shape, options, VIEW_STATUS)
    return int(workspace[off:off + nb].view(torch.int32).item())


def mxmoe_forward(shape: Shape, x, logits, packed, y=None, workspace=None,
                  options: Options | None = None, stream=None):
    """packed = (w13_p, s13_p, w2_p, s2_p) from mxmoe_prepack (scales may be None for bf16)."""
    if y is None:
        y = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=_dev(x))
    need = mxmoe_workspace_bytes(shape, options)
    if workspace is None:  # zeroed: the control words must start at zero
        workspace = new_workspace(need, _dev(x))
    w13p, s13p, w2p, s2p = packed
    args = [_ptr(x), _ptr(logits), _ptr(w13p), _ptr(s13p), _ptr(w2p), _ptr(s2p), _ptr(y),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)]
    if options is None:
        st = lib().mxmoe_forward(ctypes.byref(shape), *args)
    else:
        st = lib().mxmoe_forward_ex(ctypes.byref(shape), ctypes.byref(options), *args)
    _check(st, "mxmoe_forward")
    return y


NOALLOC_SCRATCH_BYTES = 32 << 20


def mxmoe_forward_noalloc(shape: Shape, x, logits, packed, y=None, stream=None):
    """mxmoe_forward with the library's device-resident workspace (no workspace argument)."""
    if y is None:
        y = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=_dev(x))
    w13p, s13p, w2p, s2p = packed
    _check(lib().mxmoe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w13p),
                                       _ptr(s13p), _ptr(w2p), _ptr(s2p), _ptr(y), _stream(stream)),
           "mxmoe_forward_noalloc")
    return y
