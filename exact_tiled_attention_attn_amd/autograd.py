"""torch.autograd integration: attention whose backward keeps linear state.

``attention(q, k, v, ...)`` runs the library's forward and registers a
backward that calls the library's backward.  What autograd keeps between the
two is exactly Q, K, V, the output O and the row statistics L: the score and
probability tiles are rebuilt from them when the gradients are needed (the
"What Ordinary Autograd Saves" page, closing section on the custom backward;
the alphabetamath page, reverse procedure).  Retained state is therefore
linear in n, 2nd + nv elements of the input dtype plus 4n bytes per head,
where a tiled forward traced by ordinary autograd retains tile-sized tensors
for every tile (quadratic in total).

``self_attention(x, ...)`` is the shared-input form Q = K = V = X
(HarshvardhanJ README, self-attention; scale 1 there): autograd adds the
three gradient contributions, dX = dQ + dK + dV.

Like the rest of the binding this only marshals arguments; the arithmetic
runs in the HIP kernels behind ``include/attn.h``.
"""

from __future__ import annotations

import torch

from . import _binding

__all__ = ["attention", "self_attention"]


class _Attention(torch.autograd.Function):
    """O, L = attention(Q, K, V); backward from (Q, K, V, O, L) alone."""

    @staticmethod
    def forward(ctx, q, k, v, scale, mask_mode, mask, deterministic, causal_offset, dropout_p, dropout_seed):
        o, lse = _binding.fwd(q, k, v, scale, mask_mode, mask, causal_offset=causal_offset, dropout_p=dropout_p,
                              dropout_seed=dropout_seed)
        # The mask words are caller-owned input storage, like Q, K and V; they
        # are kept as a reference, not as saved state.
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.mask_mode, ctx.mask, ctx.deterministic = scale, mask_mode, mask, deterministic
        ctx.causal_offset, ctx.dropout = causal_offset, (dropout_p, dropout_seed)
        ctx.mark_non_differentiable(lse)
        ctx.set_materialize_grads(False)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        if torch.is_grad_enabled():
            # create_graph=True: the library's backward is not itself
            # differentiable, so a second-order term would silently be zero.
            raise RuntimeError("attention: double backward (create_graph=True) is not supported")
        q, k, v, o, lse = ctx.saved_tensors
        if do is None:
            return (None,) * 10
        dq, dk, dv = _binding.bwd(q, k, v, o, do, lse, ctx.scale, ctx.mask_mode, ctx.mask,
                                  deterministic=ctx.deterministic, causal_offset=ctx.causal_offset,
                                  dropout_p=ctx.dropout[0], dropout_seed=ctx.dropout[1])
        needs = ctx.needs_input_grad
        return (dq if needs[0] else None, dk if needs[1] else None, dv if needs[2] else None,
                None, None, None, None, None, None, None)


def attention(q, k, v, scale=None, mask_mode="none", mask=None, *, deterministic=True,
              return_lse=False, causal_offset=0, dropout_p=0.0, dropout_seed=0):
    """Exact softmax attention, differentiable in Q, K, V.

    q [B, H, n, d]; k [B, H, nk, d]; v [B, H, nk, v] (nk may differ from n).

    scale: the c of s_ij = c <Q_i, K_j> (default 1 / sqrt(d)).  mask_mode is
    "none", "causal" or "bitmask" (then ``mask`` holds the LSB-first uint32
    words, [H, n, ceil(nk / 32)] or [B, H, n, ceil(nk / 32)]); with "causal",
    key j is allowed for query i iff j <= i + causal_offset.  deterministic
    selects the bitwise-reproducible dQ pass.  dropout_p / dropout_seed:
    dropout on the weights, the backward replaying the same keep decisions
    (counter-based, nothing stored).  L (fp32 natural-log
    logsumexp per row) is returned with ``return_lse`` and carries no
    gradient.
    """
    if scale is None:
        scale = q.shape[-1] ** -0.5
    # The library takes rows with a unit element stride; other layouts are
    # copied (autograd routes the gradients back through the copies).
    q, k, v = (t if t.stride(-1) == 1 else t.contiguous() for t in (q, k, v))
    o, lse = _Attention.apply(q, k, v, float(scale), mask_mode, mask, bool(deterministic),
                              int(causal_offset), float(dropout_p), int(dropout_seed))
    return (o, lse) if return_lse else o


def self_attention(x, scale=1.0, mask_mode="none", mask=None, *, deterministic=True):
    """attention(X, X, X): one input, whose gradient is dQ + dK + dV (d = v = X's width)."""
    return attention(x, x, x, scale, mask_mode, mask, deterministic=deterministic)
