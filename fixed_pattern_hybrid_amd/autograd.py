"""torch.autograd glue for the SAF hybrid attention layer.

``hybrid_attention(q, k, v, a, r, frozen)`` returns O of the layer and, on
``backward()``, the gradients of q, k, v (the library's two-pass backward:
``saf_hybrid_attn_bwd``) and, when a or r require them, of the frozen heads'
pattern parameters (``saf_pattern_grad``, the trainable-pattern variant of
"When Can Attention Heads Be Statically Defined?", Appendix C.3.2).  Every
value is computed by the HIP library; this module only saves the forward's
outputs for the backward and passes tensors to the binding.

Limits are the library's: bf16 or fp32 tensors [B, H, T, D] with unit stride
along D; a, r fp32 [H, Tp] contiguous.  Grouped-query K/V (Hkv < H) run
forward only: their backward raises NotImplementedError, as the C ABI
refuses it.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import binding as B

__all__ = ["HybridAttentionFn", "hybrid_attention"]


class HybridAttentionFn(torch.autograd.Function):
    """O = hybrid layer(q, k, v; a, r, frozen) with the library's backward."""

    @staticmethod
    def forward(ctx, q, k, v, a, r, frozen, softmax_scale):
        frz = tuple(int(x) for x in frozen)
        o, lse = B.saf_hybrid_attn_fwd(q, k, v, frz, a, r, softmax_scale=softmax_scale)
        ctx.save_for_backward(q, k, v, o, lse, a, r)
        ctx.frozen = frz
        ctx.softmax_scale = softmax_scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, a, r = ctx.saved_tensors
        if v.shape[1] != o.shape[1]:
            raise NotImplementedError("grouped-query K/V (Hkv < H): the library has no backward for it")
        if not do.is_contiguous():  # e.g. the expanded gradient of a sum
            do = do.contiguous()
        dq = dk = dv = da = dr = None
        if any(ctx.needs_input_grad[:3]):
            dq, dk, dv = B.saf_hybrid_attn_bwd(q, k, v, o, do, lse, ctx.frozen, a, r,
                                               softmax_scale=ctx.softmax_scale)
        if ctx.needs_input_grad[3] or ctx.needs_input_grad[4]:
            da, dr = B.saf_pattern_grad(v, o, do, lse, ctx.frozen, a, r)
        return (dq if ctx.needs_input_grad[0] else None, dk if ctx.needs_input_grad[1] else None,
                dv if ctx.needs_input_grad[2] else None, da if ctx.needs_input_grad[3] else None,
                dr if ctx.needs_input_grad[4] else None, None, None)


def hybrid_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor, r: torch.Tensor,
                     frozen: Sequence[int], softmax_scale: Optional[float] = None) -> torch.Tensor:
    """O of the hybrid layer, differentiable in q, k, v and (for the frozen
    heads) a and r.  frozen: length-H sequence of 0/1.

    Under bf16 autocast on the GPU, q, k and v are cast to bf16 (the bf16
    path; their gradients flow back through the cast) while a and r stay
    fp32; other autocast dtypes leave the inputs as given (the library has
    bf16 and fp32 paths only)."""
    if torch.is_autocast_enabled("cuda") and torch.get_autocast_dtype("cuda") == torch.bfloat16:
        q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    with torch.autocast("cuda", enabled=False):
        return HybridAttentionFn.apply(q, k, v, a, r, frozen, softmax_scale)
