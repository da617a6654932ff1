"""The step on either side of the attention: a synthetic DiT self-attention block.

A video DiT block computes Q, K, V with one projection of the token
activations, runs attention, and projects the attention output back to the
model width; RotateAttention replaces the attention in the middle (RotateAttention
page, Abstract, which also quotes an end-to-end speed-up).  No trained weights
exist here, so the weights are seeded random and only the timing means
anything.

Layout is where the block loses time around an attention kernel: the
projection writes Q, K, V token-major ([B][N][3][H][D]) and the output
projection wants O token-major ([B][N][H][D]).  With ``fused=True`` the
prologue reads Q, K, V in place through strides and the attention kernels
write O in the output projection's layout, so there are no transposition
passes; ``fused=False`` makes the contiguous [B][H][N][D] copies a plain
boundary needs, for comparison.  The projections are plain library GEMMs
(torch matmul on hipBLASLt), except with ``gemm_prologue=True``: then the QKV
projection is the library's own kernel with the prologue as its epilogue
(rotattn_qkv_proj_prepare), so Q, K and V never reach memory in fp16.
"""
from __future__ import annotations

import numpy as np

from . import rotattn as R


class DiTAttentionBlock:
    def __init__(self, shape: R.Shape, width: int, rr: R.RopeRotDevice, seed: int = 0,
                 device: str = "cuda"):
        import torch
        self.torch = torch
        self.shape = shape
        self.width = width
        self.rr = rr
        B, H, N, D = shape.B, shape.H, shape.N, shape.D
        g = torch.Generator(device="cpu").manual_seed(seed)
        hd = H * D
        # seeded random weights of unit gain: x ~ N(0, 1) gives Q, K, V ~ N(0, 1)
        self.w_qkv = (torch.randn(width, 3 * hd, generator=g) / np.sqrt(width)).half().to(device)
        self.w_qkv_rows = self.w_qkv.t().contiguous()    # [3 H D][width]: output channels as rows
        self.w_o = (torch.randn(hd, width, generator=g) / np.sqrt(hd)).half().to(device)
        self.ws = torch.empty(R.workspace_bytes(shape), dtype=torch.uint8, device=device)
        self.prep = R.PreparedDevice(shape, with_rope=True, device=device)
        self.qkv = torch.empty((B, N, 3 * hd), dtype=torch.float16, device=device)
        self.o_tok = torch.empty((B, N, H, D), dtype=torch.float16, device=device)

    def forward(self, x, fp16: bool = False, fused: bool = True, gemm_prologue: bool = False):
        """x: [B][N][width] fp16 -> [B][N][width] fp16.  fp16=True runs every
        head through the FP16 attention (the full-precision baseline)."""
        torch = self.torch
        s = self.shape
        B, H, N, D = s.B, s.H, s.N, s.D
        mask = np.ones(B * H, np.uint8) if fp16 else None
        if gemm_prologue:
            R.qkv_proj_prepare(s, x, self.w_qkv_rows, None, self.rr, self.prep, mask)
            o = self.o_tok.permute(0, 2, 1, 3)
            if fp16:
                R.fp16_fwd_prepared(s, self.prep, o, head_select=mask)
            else:
                R.int4_fwd(s, self.prep, o)
            return torch.matmul(self.o_tok.view(B, N, H * D), self.w_o)
        torch.matmul(x, self.w_qkv, out=self.qkv)
        q, k, v = self.qkv.view(B, N, 3, H, D).permute(2, 0, 3, 1, 4)   # [B][H][N][D] views
        o = self.o_tok.permute(0, 2, 1, 3)                               # [B][H][N][D] view
        if not fused:
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            o = torch.empty((B, H, N, D), dtype=torch.float16, device=x.device)
        R.mixed_fwd(s, q, k, v, self.rr, mask, self.ws, o)
        if not fused:
            self.o_tok.copy_(o.permute(0, 2, 1, 3))
        return torch.matmul(self.o_tok.view(B, N, H * D), self.w_o)
