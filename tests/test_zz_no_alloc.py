"""mxmoe_forward_noalloc (workspace in the library's device-resident array) against mxmoe_forward
(caller's workspace): the same kernels on the same inputs, so the outputs must be equal bit for
bit. Two calls in a row on one GPU, the second with fewer tokens, so the second call runs on the
array the first one left behind; and a shape whose workspace exceeds the array is refused."""
import numpy as np
import pytest
import torch

import workloads
from mx_quantized_grouped_amd import binding as B

from gpu_support import DEV, bf16_tensor, packed_weights, shape_of

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[no-alloc]", *a, flush=True)


@pytest.mark.parametrize("name,Ts", [("decode_mxfp8", (32, 8)), ("wide512_mxfp4_T6", (6, 1)),
                                     ("decode_mxfp4", (128, 17))])
def test_noalloc_matches_forward(name, Ts):
    w = workloads.get(name)
    _, packed = packed_weights(name)
    big = w.with_T(max(Ts))
    xb, lb = workloads.draw_x(big), workloads.draw_logits(big)
    for T in Ts:
        _say(name, "T", T)
        shape = shape_of(w.with_T(T))
        assert B.mxmoe_workspace_bytes(shape) <= B.NOALLOC_SCRATCH_BYTES
        x, lg = bf16_tensor(xb[:T]), bf16_tensor(lb[:T])
        y_na = B.mxmoe_forward_noalloc(shape, x, lg, packed)
        y_ref = B.mxmoe_forward(shape, x, lg, packed)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), (name, T)
        assert torch.isfinite(y_na.float()).all()


def test_noalloc_refuses_large_workspace():
    w = workloads.get("prefill_mxfp8")
    _, packed = packed_weights("decode_mxfp8")            # same H, E, I and format
    shape = shape_of(w)
    assert B.mxmoe_workspace_bytes(shape) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros((w.T, w.E), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.MxMoeError) as ei:
        B.mxmoe_forward_noalloc(shape, x, lg, packed)
    assert ei.value.status == B.MXMOE_EWORKSPACE
