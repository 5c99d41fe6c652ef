"""torch.autograd wrapper around the forward and backward entry points.

Allocation of outputs and of the backward workspace is done with torch (the
caller's device memory); every arithmetic step runs in libneoxattn.
"""

from __future__ import annotations

import torch

from . import (NEOX_POS_ALIBI, NEOX_POS_ROPE, neox_attn_bwd_ex, neox_attn_fwd_ex,
               neox_rope_attn_bwd_workspace_size, neox_rope_attn_fwd_workspace_size,
               neox_rope_table_prepare)


class NeoxAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, rotary_dim, rope_base, causal, softmax_scale, alibi, alibi_slopes,
                doc_offsets, out_f32):
        B, H, S, D = q.shape
        pos = NEOX_POS_ALIBI if alibi else NEOX_POS_ROPE
        o = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=q.device)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
        kw = dict(pos=pos, rotary_dim=rotary_dim, rope_base=rope_base, alibi_slopes=alibi_slopes,
                  causal=causal, softmax_scale=softmax_scale, doc_offsets=doc_offsets)
        ws = None
        if rotary_dim > 0 and not alibi:
            with torch.cuda.device(q.device):
                neox_rope_table_prepare(S, rotary_dim, rope_base)
        if rotary_dim > 0 and not alibi and q.dtype in (torch.bfloat16, torch.float16):
            ws = torch.empty(neox_rope_attn_fwd_workspace_size(B, H, S, D), dtype=torch.uint8,
                             device=q.device)
        neox_attn_fwd_ex(q, k, v, o, lse, out_f32=out_f32, workspace=ws, **kw)
        ctx.kw = kw
        ctx.out_f32 = out_f32
        ctx.save_for_backward(q, k, v, o, lse)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        B, H, S, D = q.shape
        do = do.to(q.dtype)
        o_in = o.to(q.dtype) if o.dtype != q.dtype else o
        if do.stride(3) != 1:
            do = do.contiguous()
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        ws = torch.empty(neox_rope_attn_bwd_workspace_size(B, H, S, D), dtype=torch.uint8,
                         device=q.device)
        neox_attn_bwd_ex(q, k, v, o_in, do, lse, dq, dk, dv, workspace=ws, **ctx.kw)
        return dq, dk, dv, None, None, None, None, None, None, None, None
