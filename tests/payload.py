"""What autograd retains for the backward pass, measured with saved-tensor hooks.

The measurement of the "What Ordinary Autograd Saves" page ("Looking at what
autograd keeps"): every tensor autograd stashes passes through the pack hook;
bytes are summed once per distinct (storage, offset, shape, strides, dtype),
so a buffer stashed by several operations counts once while distinct views
of one storage count separately.  Storage the caller owns (Q, K, V) counts
too: the figure is what the backward graph can reach.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


def buffer_key(t: torch.Tensor) -> tuple:
    """Identity of one retained buffer: the page's definition, kept so that
    the figures compare with its own."""
    return (t.untyped_storage().data_ptr(), t.storage_offset(), tuple(t.shape), tuple(t.stride()), t.dtype)


@dataclass
class Retained:
    """Buffers the pack hook saw: bytes per distinct buffer, and hook calls."""

    sizes: dict = field(default_factory=dict)
    events: int = 0

    @property
    def bytes(self) -> int:
        return sum(self.sizes.values())


def retained_by(run) -> Retained:
    """Call ``run()`` -- a forward pass and its backward -- with a pack hook
    that records every tensor autograd saves for the backward."""
    seen = Retained()

    def pack(t):
        seen.events += 1
        seen.sizes.setdefault(buffer_key(t), t.numel() * t.element_size())
        return (t.detach(),)  # a fresh alias: the hook keeps no reference to the graph's tensor

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda packed: packed[0]):
        run()
    return seen


def traced_tiled_forward(q, k, v, scale, block):
    """Online-softmax forward over key blocks in plain torch ops, traced by autograd.

    The tiled forward of the "What Ordinary Autograd Saves" page ("The
    implementation under test"), query and key blocks of ``block`` rows, for
    [n, d] inputs: running max, rescaled sum and rescaled output per query
    block.  Used only to show what ordinary autograd keeps for it.
    """
    n = q.shape[0]
    outs = []
    for i0 in range(0, n, block):
        qb = q[i0:i0 + block]
        m = torch.full((qb.shape[0], 1), float("-inf"), dtype=q.dtype)
        l = torch.zeros((qb.shape[0], 1), dtype=q.dtype)
        acc = torch.zeros((qb.shape[0], v.shape[1]), dtype=q.dtype)
        for j0 in range(0, n, block):
            s = (qb @ k[j0:j0 + block].T) * scale
            m_new = torch.maximum(m, s.amax(dim=1, keepdim=True))
            alpha = torch.exp(m - m_new)
            p = torch.exp(s - m_new)
            l = alpha * l + p.sum(dim=1, keepdim=True)
            acc = alpha * acc + p @ v[j0:j0 + block]
            m = m_new
        outs.append(acc / l)
    return torch.cat(outs)
