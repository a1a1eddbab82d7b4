"""A layer object over the C ABI: packs checkpoint-layout weights once and runs
``moe_forward`` on the current HIP stream.  Allocation (torch) and argument
marshalling only; all arithmetic happens in libmoe.so.
"""
import torch

from . import (combine_workspace_bytes, max_blocks, max_padded_rows, moe_align,
               moe_forward, moe_gemm1_act, moe_gemm2_combine, moe_pack_w2, moe_pack_w13,
               moe_quant_act, moe_route, moe_prepare, packed_bytes, problem, align_workspace_bytes,
               workspace_bytes, weights)


def _bytes(n, device):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


class MoELayer:
    """Packed weights of one MoE layer plus the per-call plumbing.

    w13, w2: checkpoint layout on the device (uint16 bf16 bits, uint8 e4m3
    codes, or uint8 packed int4 / fp4); scales as the header describes (uint8
    E8M0 for the MX modes); a1, a2: 0-d float32 device tensors for the
    per-tensor modes.
    """

    def __init__(self, H, I, E_routed, top_k, act, quant, w13, w2, w13_scale=None,
                 w2_scale=None, a1=None, a2=None, n_shared=0, shared_gate=1.0,
                 renormalize=True, src_I=None, swap_halves=False, block_m=0):
        self.kw = dict(H=H, I=I, E_routed=E_routed, top_k=top_k, act=act, quant=quant,
                       n_shared=n_shared, shared_gate=shared_gate, renormalize=renormalize,
                       block_m=block_m)
        dev = w13.device
        self.device = dev
        p = self.problem(0)
        b13, s13 = packed_bytes(p, 13)
        b2, s2 = packed_bytes(p, 2)
        self.w13 = _bytes(b13, dev)
        self.w2 = _bytes(b2, dev)
        self.s13 = _bytes(s13, dev)
        self.s2 = _bytes(s2, dev)
        src_I = I if src_I is None else src_I
        moe_pack_w13(p, w13, src_I, swap_halves, w13_scale, self.w13, self.s13)
        moe_pack_w2(p, w2, src_I, w2_scale, self.w2, self.s2)
        self.a1, self.a2 = a1, a2
        self.w = weights(self.w13, self.w2, self.s13 if s13 else None, self.s2 if s2 else None,
                         a1, a2)
        self._ws = None

    def problem(self, T):
        return problem(T=T, **self.kw)

    def workspace(self, T):
        need = workspace_bytes(self.problem(T))
        if self._ws is None or self._ws.numel() < need:
            self._ws = _bytes(need, self.device)
        return self._ws

    def forward(self, x, logits=None, topk_ids=None, topk_w=None, out=None):
        H, K = self.kw["H"], self.kw["top_k"] + self.kw["n_shared"]
        if x.dim() != 2 or x.shape[1] != H:
            raise ValueError(f"x must be [T, {H}], got {tuple(x.shape)}")
        T = x.shape[0]
        for t, name, cols in ((logits, "logits", self.kw["E_routed"]), (topk_ids, "topk_ids", K),
                              (topk_w, "topk_w", K), (out, "out", H)):
            if t is not None and tuple(t.shape) != (T, cols):
                raise ValueError(f"{name} must be [{T}, {cols}], got {tuple(t.shape)}")
        p = self.problem(T)
        if out is None:
            out = torch.empty((T, self.kw["H"]), dtype=torch.bfloat16, device=self.device)
        moe_forward(p, self.w, x, logits, topk_ids, topk_w, out, self.workspace(T))
        return out

    # ---- the same pass as separate entry points, for tests and timing
    def buffers(self, T):
        p = self.problem(T)
        K = self.kw["top_k"] + self.kw["n_shared"]
        dev, H, I = self.device, self.kw["H"], self.kw["I"]
        q = self.kw["quant"]
        rows, blocks = max_padded_rows(p), max_blocks(p)
        E = self.kw["E_routed"] + self.kw["n_shared"]
        b = dict(
            topk_ids=torch.empty((T, K), dtype=torch.int32, device=dev),
            topk_w=torch.empty((T, K), dtype=torch.float32, device=dev),
            sorted_ids=torch.empty(max(rows, 1), dtype=torch.int32, device=dev),
            block_expert=torch.empty(max(blocks, 1), dtype=torch.int32, device=dev),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            num_padded=torch.empty(1, dtype=torch.int32, device=dev),
            align_ws=_bytes(align_workspace_bytes(p), dev),
            xq=None if q == "bf16" else torch.empty((T, H), dtype=torch.uint8, device=dev),
            xs=torch.empty((T, H // 128), dtype=torch.float32, device=dev)
            if q == "fp8_block" else
            torch.empty((T, H // 32), dtype=torch.uint8, device=dev) if q.startswith("mx") else None,
            a2=torch.empty((max(rows, 1), I), dtype=torch.bfloat16 if q == "bf16" else torch.uint8,
                           device=dev),
            a2s=torch.empty((max(rows, 1), I // 128), dtype=torch.float32, device=dev)
            if q == "fp8_block" else
            torch.empty((max(rows, 1), I // 32), dtype=torch.uint8, device=dev)
            if q.startswith("mx") else None,
            y=_bytes(combine_workspace_bytes(p), dev),
            out=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
        )
        return b

    def route(self, T, logits, b):
        moe_route(self.problem(T), logits, b["topk_ids"], b["topk_w"])

    def prepare(self, T, logits, x, b):
        """Routing, fp8 quantisation of x and alignment (one launch at decode sizes)."""
        moe_prepare(self.problem(T), logits, b["topk_ids"], b["topk_w"],
                    None if self.kw["quant"] == "bf16" else x, self.a1, b["xq"], b["xs"],
                    b["sorted_ids"], b["block_expert"], b["offsets"], b["num_padded"],
                    b["align_ws"])

    def align(self, T, b):
        moe_align(self.problem(T), b["topk_ids"], b["sorted_ids"], b["block_expert"],
                  b["offsets"], b["num_padded"], b["align_ws"])

    def quant(self, T, x, b):
        if self.kw["quant"] != "bf16":
            moe_quant_act(self.problem(T), x, self.a1, b["xq"], b["xs"])

    def gemm1(self, T, x, b):
        xin = x if self.kw["quant"] == "bf16" else b["xq"]
        moe_gemm1_act(self.problem(T), xin, b["xs"], self.w, b["sorted_ids"],
                      b["block_expert"], b["num_padded"], b["a2"], b["a2s"])

    def gemm2(self, T, b):
        moe_gemm2_combine(self.problem(T), b["a2"], b["a2s"], self.w, b["sorted_ids"],
                          b["block_expert"], b["num_padded"], b["topk_ids"], b["topk_w"],
                          b["y"], b["out"])
