"""One MoE layer's resident state and its hot-path call sequence, over the C
ABI.  Allocation through torch (device memory only); all arithmetic in the
library's kernels.

    layer = Layer(E=512, H=2560, I=640, k=10)
    layer.set_router(W_r, bias)                        # fp32 device tensors
    layer.load_experts_fp32(e0, gate, up, down)        # quantized + packed on device
    bufs = layer.alloc(T)                              # every per-step buffer
    y = layer.forward(x_bf16, bufs, residual=True)     # router -> quant -> FFN -> combine
    fb = layer.alloc_fused(T)                          # decode: the fused layer (3 kernels at 1 token)
    y = layer.forward_fused(x_bf16, fb, residual=True)
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (MOE_FMT_CB3G128, MOE_FMT_NVFP4, dims, moe_combine,
               moe_expert_ffn_decode, moe_expert_ffn_prefill, moe_ffn_workspace_bytes,
               moe_layer_decode, moe_layer_decode_rescaled, moe_layer_decode_workspace_bytes,
               moe_pack_codebook,
               moe_pack_nvfp4, moe_packed_bytes, moe_quantize_act, moe_quantize_weights,
               moe_router_topk)



# Up to this many tokens the decode GEMVs are the faster expert FFN; above,
# the grouped GEMM (32-row expert tiles) is (measured layer steps at H 2560,
# I 640, E 512, k 10, NVFP4 gate/up: 100 vs 105 us at 12 tokens, 127 vs 117 us
# at 16, 218 vs 178 us at 32; codebook gate/up: 124 vs 128 us at 12 tokens,
# 162 vs 153 us at 16).  Both give the same result up to fp32 order.
DECODE_FFN_MAX_T = 12

class Layer:
    def __init__(self, E: int, H: int, I: int, k: int, fmt_gate_up: int = MOE_FMT_NVFP4,
                 device="cuda"):
        self.E, self.H, self.I, self.k = E, H, I, k
        self.fmt = fmt_gate_up
        self.device = torch.device(device)
        self.d = dims(E, H, I, k, fmt_gate_up)
        self.gate_up = torch.empty(moe_packed_bytes(self.d, 0), dtype=torch.uint8, device=self.device)
        self.down = torch.empty(moe_packed_bytes(self.d, 1), dtype=torch.uint8, device=self.device)
        self.ts_gate = torch.zeros(E, dtype=torch.float32, device=self.device)
        self.ts_up = torch.zeros(E, dtype=torch.float32, device=self.device)
        self.ts_down = torch.zeros(E, dtype=torch.float32, device=self.device)
        self.W_r: Optional[torch.Tensor] = None
        self.bias: Optional[torch.Tensor] = None
        # static (calibrated) NVFP4 tensor scale of h per expert, or None
        self.h_ts: Optional[torch.Tensor] = None

    # -------------------------------------------------------------- weights
    def experts(self) -> dict:
        return dict(gate_up=self.gate_up, down=self.down,
                    ts_gate=self.ts_gate if self.fmt == MOE_FMT_NVFP4 else None,
                    ts_up=self.ts_up if self.fmt == MOE_FMT_NVFP4 else None,
                    ts_down=self.ts_down, h_ts=self.h_ts)

    def set_static_h_scales(self, h_ts: Optional[torch.Tensor]):
        """Static NVFP4 tensor scales of h ([E] fp32, >= 0), or None for the
        per-row dynamic scale."""
        if h_ts is not None:
            assert h_ts.shape == (self.E,) and h_ts.dtype == torch.float32
            h_ts = h_ts.contiguous()
        self.h_ts = h_ts

    def set_router(self, W_r: torch.Tensor, bias: Optional[torch.Tensor] = None):
        assert W_r.shape == (self.E, self.H) and W_r.dtype == torch.float32
        self.W_r = W_r.contiguous()
        self.bias = None if bias is None else bias.contiguous()

    def quantize_plain(self, W: torch.Tensor):
        """W [n, rows, cols] fp32 -> (codes [n,rows,cols/2], scales [n,rows,cols/16], ts [n])."""
        n, rows, cols = W.shape
        codes = torch.empty((n, rows, cols // 2), dtype=torch.uint8, device=W.device)
        scales = torch.empty((n, rows, cols // 16), dtype=torch.uint8, device=W.device)
        ts = torch.empty(n, dtype=torch.float32, device=W.device)
        moe_quantize_weights(W.contiguous(), n, rows, cols, codes, scales, ts)
        return codes, scales, ts

    def load_experts_fp32(self, e0: int, gate: Optional[torch.Tensor], up: Optional[torch.Tensor],
                          down: torch.Tensor):
        """Quantize (NVFP4, one tensor scale per matrix) and pack experts
        e0 .. e0+n-1 from fp32 device weights gate/up [n, I, H], down [n, H, I].
        gate/up may be None for a codebook layer."""
        n = down.shape[0]
        dc, ds, dts = self.quantize_plain(down)
        if gate is not None:
            gc, gs, gts = self.quantize_plain(gate)
            uc, us, uts = self.quantize_plain(up)
            moe_pack_nvfp4(self.d, e0, n, gc, gs, uc, us, dc, ds, self.gate_up, self.down)
            self.ts_gate[e0:e0 + n] = gts
            self.ts_up[e0:e0 + n] = uts
        else:
            moe_pack_nvfp4(self.d, e0, n, None, None, None, None, dc, ds, self.gate_up, self.down)
        self.ts_down[e0:e0 + n] = dts

    def load_codebook(self, e0: int, gate_cb, gate_idx, up_cb, up_idx):
        """Codebook gate/up for experts e0 .. e0+n-1: cb [n, I, H/128, 8] fp16,
        idx [n, I, H] uint8."""
        n = gate_cb.shape[0]
        moe_pack_codebook(self.d, e0, n, gate_cb.contiguous().view(torch.int16),
                          gate_idx.contiguous(), up_cb.contiguous().view(torch.int16),
                          up_idx.contiguous(), self.gate_up)

    # -------------------------------------------------------------- step
    def alloc(self, T: int, prefill: Optional[bool] = None) -> dict:
        """Every buffer one step at T tokens needs (so a step allocates nothing)."""
        dev = self.device
        if prefill is None:
            prefill = T > DECODE_FFN_MAX_T
        ws_bytes = moe_ffn_workspace_bytes(self.d, T, prefill)
        return dict(
            T=T, prefill=prefill,
            logits=torch.empty((T, self.E), dtype=torch.float32, device=dev),
            ids=torch.empty((T, self.k), dtype=torch.int32, device=dev),
            w=torch.empty((T, self.k), dtype=torch.float32, device=dev),
            x_codes=torch.empty((T, self.H // 2), dtype=torch.uint8, device=dev),
            x_scales=torch.empty((T, self.H // 16), dtype=torch.uint8, device=dev),
            x_ts=torch.empty(T, dtype=torch.float32, device=dev),
            out=torch.empty((T, self.k, self.H), dtype=torch.float32, device=dev),
            y=torch.empty((T, self.H), dtype=torch.int16, device=dev),
            ws=torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev),
            ws_bytes=ws_bytes,
        )

    def forward(self, x: torch.Tensor, b: dict, residual: bool = False, dbg: Optional[dict] = None,
                stream=None) -> torch.Tensor:
        """x: [T, H] bf16 (or its int16 bits).  Returns y [T, H] as int16 bf16 bits
        (b['y'])."""
        T = b["T"]
        xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
        moe_router_topk(xb, self.W_r, self.bias, T, self.d, b["ids"], b["w"], b["logits"], stream)
        moe_quantize_act(xb, T, self.H, b["x_codes"], b["x_scales"], b["x_ts"], stream)
        xq = (b["x_codes"], b["x_scales"], b["x_ts"])
        ffn = moe_expert_ffn_prefill if b["prefill"] else moe_expert_ffn_decode
        ffn(self.d, self.experts(), xq, b["ids"], T, b["out"], b["ws"], b["ws_bytes"], dbg, stream)
        moe_combine(b["out"], b["w"], xb if residual else None, T, self.k, self.H, b["y"], stream)
        return b["y"]

    # -------------------------------------------------------------- fused decode
    def alloc_fused(self, T: int) -> dict:
        """Buffers of the fused decode layer (T <= 16)."""
        dev = self.device
        ws_bytes = moe_layer_decode_workspace_bytes(self.d, T)
        return dict(T=T, ws_bytes=ws_bytes,
                    ws=torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev),
                    ids=torch.empty((T, self.k), dtype=torch.int32, device=dev),
                    w=torch.empty((T, self.k), dtype=torch.float32, device=dev),
                    y=torch.empty((T, self.H), dtype=torch.int16, device=dev))

    def forward_fused(self, x: torch.Tensor, b: dict, residual: bool = False, stream=None):
        xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
        moe_layer_decode(self.d, self.experts(), xb, self.W_r, self.bias, b["T"], residual,
                         b["y"], b["ids"], b["w"], b["ws"], b["ws_bytes"], stream)
        return b["y"]

    def forward_stack(self, x_in: torch.Tensor, b: dict, target_rms: float, stream=None):
        """One layer of the stack: x_in (the previous layer's output) brought
        back to target_rms per token, then the fused layer with the residual
        add (moe_rms_norm + forward_fused in one call, bit for bit)."""
        xb = x_in.view(torch.int16) if x_in.dtype == torch.bfloat16 else x_in
        moe_layer_decode_rescaled(self.d, self.experts(), xb, target_rms, self.W_r, self.bias, b["T"],
                                  b["y"], b["ids"], b["w"], b["ws"], b["ws_bytes"], stream)
        return b["y"]
