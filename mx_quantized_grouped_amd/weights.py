"""Load-time preparation of expert weights with the library's own kernels.

Expert matrices arrive one expert at a time as fp32 (or bf16) host arrays; they are uploaded,
quantised on the GPU to MX (mxmoe_quantize, along K) into canonical buffers, and finally converted
into the kernel-native layout (mxmoe_prepack). All arithmetic runs in the HIP library."""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


class ExpertLoader:
    def __init__(self, shape: B.Shape, device="cuda"):
        self.shape = shape
        self.device = torch.device(device)
        E1, H, I = shape.E + 1, shape.H, shape.I
        self.fmt = shape.w_fmt
        if self.fmt == B.MXMOE_BF16:
            self.w13 = torch.empty((E1, 2 * I, H), dtype=torch.bfloat16, device=self.device)
            self.w2 = torch.empty((E1, H, I), dtype=torch.bfloat16, device=self.device)
            self.s13 = self.s2 = None
        else:
            div = 1 if self.fmt == B.MXMOE_MXFP8_E4M3 else 2
            self.w13 = torch.empty((E1, 2 * I, H // div), dtype=torch.uint8, device=self.device)
            self.w2 = torch.empty((E1, H, I // div), dtype=torch.uint8, device=self.device)
            self.s13 = torch.empty((E1, 2 * I, H // 32), dtype=torch.uint8, device=self.device)
            self.s2 = torch.empty((E1, H, I // 32), dtype=torch.uint8, device=self.device)
        self._seen = np.zeros(E1, dtype=bool)

    def add_expert(self, e: int, w13, w2):
        """w13 [2I, H] (gate rows then up rows) and w2 [H, I] of expert e (E = shared)."""
        t13 = torch.as_tensor(np.ascontiguousarray(w13)).to(self.device, non_blocking=False)
        t2 = torch.as_tensor(np.ascontiguousarray(w2)).to(self.device, non_blocking=False)
        if self.fmt == B.MXMOE_BF16:
            self.w13[e].copy_(t13.to(torch.bfloat16))
            self.w2[e].copy_(t2.to(torch.bfloat16))
        else:
            f = "mxfp8" if self.fmt == B.MXMOE_MXFP8_E4M3 else "mxfp4"
            B.mxmoe_quantize(t13.float().contiguous(), f, codes=self.w13[e], scales=self.s13[e])
            B.mxmoe_quantize(t2.float().contiguous(), f, codes=self.w2[e], scales=self.s2[e])
        self._seen[e] = True

    def add_expert_mx(self, e: int, c13, s13, c2, s2):
        """Canonical MX codes and scale bytes of expert e as they are: c13 [2I, H] and c2 [H, I]
        one code per byte (E2M1 codes are packed here, element 2i in the low nibble), s13
        [2I, H/32] and s2 [H, I/32] scale bytes."""
        if self.fmt == B.MXMOE_BF16:
            raise ValueError("bf16 weights carry no MX codes")

        def codes(c):
            c = np.asarray(c, dtype=np.uint8)
            if self.fmt == B.MXMOE_MXFP4_E2M1:
                c = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
            return torch.from_numpy(np.ascontiguousarray(c)).to(self.device)
        self.w13[e].copy_(codes(c13))
        self.w2[e].copy_(codes(c2))
        self.s13[e].copy_(torch.from_numpy(np.ascontiguousarray(s13, dtype=np.uint8)).to(self.device))
        self.s2[e].copy_(torch.from_numpy(np.ascontiguousarray(s2, dtype=np.uint8)).to(self.device))
        self._seen[e] = True

    def finish(self, keep_canonical: bool = False):
        """Prepack; returns the packed tuple (w13_p, s13_p, w2_p, s2_p)."""
        if not self._seen.all():
            missing = np.nonzero(~self._seen)[0][:8].tolist()
            raise ValueError(f"experts not loaded: {missing} ...")
        packed = B.mxmoe_prepack(self.shape, self.w13, self.s13, self.w2, self.s2)
        if not keep_canonical:
            torch.cuda.current_stream().synchronize()
            self.w13 = self.w2 = self.s13 = self.s2 = None
        return packed
