"""One MoE expert layer on the GPU through the C ABI: route -> FC1+SwiGLU -> FC2 -> finalize
(or FC2 and finalize fused).

Buffers are allocated once per shape; run() enqueues the four calls on the
current stream and allocates nothing.  The FC weights are FP4Weights
(NVFP4/MXFP4) or FP8Weights (W8A16).
"""
from __future__ import annotations

import torch

from . import (GEMV_MAX_ROWS, QMOE_PATH_AUTO, QMOE_PATH_GEMV, QMOE_PATH_GROUPED, QMOE_SWIGLU_CONCAT, FP4Weights,
               FP8Weights, alloc_layer_workspace, alloc_workspace, fc_workspace_bytes, fp8_workspace_bytes,
               layer_decode_workspace_bytes, layer_persistent_workspace_bytes, qmoe_finalize,
               qmoe_fp4_gemv_fc1_swiglu, qmoe_fp4_gemv_fc2, qmoe_fp4_gemv_fc2_finalize, qmoe_fp4_moe_layer_decode,
               qmoe_fp4_moe_layer_persistent, qmoe_fp4_resolve_path, qmoe_fp4_route_fc1_swiglu,
               qmoe_fp8_gemv_fc1_swiglu, qmoe_fp8_gemv_fc2, qmoe_route_topk, qmoe_route_topk_router_weights)


class MoELayer:
    def __init__(self, T: int, E: int, k: int, H: int, I: int, w1: FP4Weights, w2: FP4Weights,
                 path: int = QMOE_PATH_AUTO, act=None, device="cuda"):
        self.T, self.E, self.k, self.H, self.I = T, E, k, H, I
        self.w1, self.w2, self.path, self.act = w1, w2, path, act
        R = T * k
        dev = torch.device(device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        self.p2e = torch.empty((R,), dtype=torch.int32, device=dev)
        self.e2p = torch.empty((R,), dtype=torch.int32, device=dev)
        self.h = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((R, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.fp8 = isinstance(w1, FP8Weights)
        if self.fp8:
            need = max(fp8_workspace_bytes(1, T, k, w1, act, path), fp8_workspace_bytes(2, T, k, w2, None, path))
        else:
            need = max(fc_workspace_bytes(1, T, k, w1, path, act), fc_workspace_bytes(2, T, k, w2, path),
                       fc_workspace_bytes(3, T, k, w2, path))
        # single-token decode: routing folded into the FC1 GEMV launch.  Every
        # FC1 workgroup runs the routing; with more tokens (a wave routes
        # several, or the grid takes more than one round of resident
        # workgroups) that costs more than the launch it saves (measured:
        # T=1 20.2 -> 19.2 us, T=4 32.3 -> 33.7 us, T=8 52.3 -> 62.9 us)
        self.route_in_fc1 = not self.fp8 and path != QMOE_PATH_GROUPED and T == 1 and R <= GEMV_MAX_ROWS
        # decode window with both FCs on the GEMV: the whole layer in one call
        # (FC1's SwiGLU folded into FC2's staging, h not written)
        fits = (not self.fp8 and R <= GEMV_MAX_ROWS and w2.w.shape[0] == w1.w.shape[0]
                and w2.w.shape[1] == w1.w.shape[2] and 2 * w2.w.shape[2] == w1.w.shape[1])
        # used where measured to pay: T <= 2 and FC1 in at most eight k chunks
        # (H <= 2048), so FC2's staging reads every plane ahead of its weights
        # (NVFP4 E=256, H=2048, I=768, one box, against the separate calls:
        # T=1 17.3 vs 18.8 us, T=2 23.8 vs 24.4, T=4 29.8 vs 29.2, T=8 43.2
        # vs 40.8; MXFP4 T=8, H=4096: 193 vs 169 us)
        self.layer_decode = (fits and path != QMOE_PATH_GROUPED and T <= 2 and H <= 2048
                             and qmoe_fp4_resolve_path(T, k, w1, path) == QMOE_PATH_GEMV
                             and qmoe_fp4_resolve_path(T, k, w2, path) == QMOE_PATH_GEMV)
        # the whole layer in one kernel launch (qmoe_fp4_moe_layer_persistent)
        concat = act is not None and len(tuple(act)) > 3 and tuple(act)[3] == QMOE_SWIGLU_CONCAT
        self.layer_persistent = (fits and path != QMOE_PATH_GROUPED and H % 32 == 0 and H <= 16384 and I <= 4096
                                 and (not concat or I % 256 == 0) and w1.fmt == w2.fmt
                                 and qmoe_fp4_resolve_path(T, k, w1, path) == QMOE_PATH_GEMV)
        self.ws_layer = (alloc_layer_workspace(layer_persistent_workspace_bytes(T, k, w1, w2, act), dev)
                         if self.layer_persistent else None)
        # run(fused=True) takes the one-launch layer up to four tokens of a
        # hidden size up to 2048, where it measured faster than the
        # multi-launch calls (NVFP4 E=256, H=2048, I=768, one box: T=1 16.4
        # vs 16.7 us, T=2 20.5 vs 23.4, T=4 25.6 vs 28.6); from five tokens
        # the multi-launch calls are faster (T=5 32.8 vs 35.0, T=6 34.3 vs
        # 35.0, T=7 36.9 vs 37.7, T=8 38.3 vs 39.8); at hidden size 4096
        # (MXFP4 T=8) the multi-launch calls 164 against 233 us
        self.one_launch = self.layer_persistent and T <= 4 and H <= 2048
        if not self.fp8 and R <= GEMV_MAX_ROWS:  # route_fc1() is callable
            need = max(need, fc_workspace_bytes(4, T, k, w1, path, act))
        self.decode_layer_callable = fits
        if fits:  # decode_layer() is callable
            need = max(need, layer_decode_workspace_bytes(T, k, w1, w2, act))
        self.ws = alloc_workspace(need, dev)

    def set_weights(self, w1: FP4Weights, w2: FP4Weights):
        self.w1, self.w2 = w1, w2

    def route(self, logits, router_weights=None):
        if router_weights is None:
            qmoe_route_topk(logits, self.k, self.topk_idx, self.topk_w, self.offsets, self.p2e, self.e2p)
        else:
            qmoe_route_topk_router_weights(logits, router_weights, self.k, self.topk_idx, self.topk_w, self.offsets,
                                           self.p2e, self.e2p)

    def fc1(self, x):
        if self.fp8:
            qmoe_fp8_gemv_fc1_swiglu(x, self.k, self.w1, self.offsets, self.p2e, self.h, self.ws, self.act,
                                     self.path)
        else:
            qmoe_fp4_gemv_fc1_swiglu(x, self.k, self.w1, self.offsets, self.p2e, self.h, self.ws, self.act,
                                     self.path)

    def route_fc1(self, logits, x, router_weights=None):
        qmoe_fp4_route_fc1_swiglu(logits, router_weights, x, self.k, self.w1, self.topk_idx, self.topk_w,
                                  self.offsets, self.p2e, self.e2p, self.h, self.ws, self.act)

    def decode_layer(self, logits, x, router_weights=None, route_in_fc1=None):
        """The whole layer by qmoe_fp4_moe_layer_decode (h and y are not written)."""
        rin = self.route_in_fc1 if route_in_fc1 is None else route_in_fc1
        qmoe_fp4_moe_layer_decode(logits, router_weights, x, self.k, self.w1, self.w2, self.topk_idx, self.topk_w,
                                  self.offsets, self.p2e, self.e2p, self.out, self.ws, self.act, rin)

    def persistent_layer(self, logits, x, router_weights=None):
        """The whole layer by qmoe_fp4_moe_layer_persistent (one kernel launch; h and y are not written)."""
        qmoe_fp4_moe_layer_persistent(logits, router_weights, x, self.k, self.w1, self.w2, self.topk_idx,
                                      self.topk_w, self.offsets, self.p2e, self.e2p, self.out, self.ws_layer,
                                      self.act)

    def fc2(self):
        if self.fp8:
            qmoe_fp8_gemv_fc2(self.h, self.T, self.k, self.w2, self.offsets, self.y, self.ws, self.path)
        else:
            qmoe_fp4_gemv_fc2(self.h, self.T, self.k, self.w2, self.offsets, self.y, self.ws, self.path)

    def finalize(self):
        qmoe_finalize(self.y, self.topk_w, self.e2p, self.out)

    def fc2_finalize(self):
        qmoe_fp4_gemv_fc2_finalize(self.h, self.k, self.w2, self.offsets, self.topk_w, self.e2p, self.out, self.ws,
                                   self.path)

    def run(self, logits, x, fused: bool = False, router_weights=None):
        """route -> FC1+SwiGLU -> FC2 -> finalize; fused=True runs the decode
        window's layer in one kernel launch where it can (the persistent
        layer), else as one call of a few launches (routing inside FC1 at
        T = 1, SwiGLU inside FC2's staging, FC2 + finalize fused: h and y are
        not written), else FC2 and the finalize as one call (y not written);
        router_weights [T][E] selects DeepSeek-style mixing weights."""
        if fused and self.one_launch:
            self.persistent_layer(logits, x, router_weights)
            return self.out
        if fused and self.layer_decode:
            self.decode_layer(logits, x, router_weights)
            return self.out
        if fused and self.route_in_fc1:
            self.route_fc1(logits, x, router_weights)
        else:
            self.route(logits, router_weights)
            self.fc1(x)
        if fused and not self.fp8:  # FP8 has no fused FC2 + finalize call
            self.fc2_finalize()
        else:
            self.fc2()
            self.finalize()
        return self.out
