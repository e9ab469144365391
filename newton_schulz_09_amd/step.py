"""A whole Muon hot-path step over a set of 2-D parameter matrices: Nesterov
momentum on every gradient, then NS5 of every momentum output (the order of
the Muon section's summary paragraph, Synced report on Modded-NanoGPT).

Memory is laid out for one GPU's HBM: the gradients, momentum buffers,
momentum outputs and orthogonalised updates are four flat float32 buffers
with a view per matrix, so momentum is a single streaming launch over all
parameters, and NS5 is one batched call over all matrices (each product of
each NS5 step is a single launch over every matrix that shares a tile size).
"""

import torch

from . import muon


class MuonStep:
    def __init__(self, shapes, device="cuda", mu=0.95, steps=muon.NS5_STEPS, eps=muon.NS5_EPS):
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        if not self.shapes or any(len(s) != 2 or min(s) < 1 for s in self.shapes):
            raise ValueError("shapes must be a non-empty list of (rows, cols) with rows, cols >= 1")
        self.device = torch.device(device)
        self.mu, self.steps, self.eps = float(mu), int(steps), float(eps)
        # matrices start on 64-element (256-byte) boundaries
        self.offsets, total = [], 0
        for r, c in self.shapes:
            self.offsets.append(total)
            total += (r * c + 63) // 64 * 64
        self.total = total
        kw = dict(dtype=torch.float32, device=self.device)
        self.grad = torch.zeros(total, **kw)
        self.buf = torch.zeros(total, **kw)
        self.u = torch.zeros(total, **kw)
        self.out = torch.zeros(total, **kw)
        self.grads = self._views(self.grad)
        self.bufs = self._views(self.buf)
        self.us = self._views(self.u)
        self.outs = self._views(self.out)
        self.groups = {}
        for i, s in enumerate(self.shapes):
            self.groups.setdefault(s, []).append(i)
        need = muon.batched_workspace_size(self.shapes)
        if need == 0:
            raise muon.MuonError(muon.MUON_ERR_UNSUPPORTED, "a shape is beyond the supported limits")
        self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)

    def _views(self, flat):
        return [flat[o:o + r * c].view(r, c) for o, (r, c) in zip(self.offsets, self.shapes)]

    def momentum(self):
        muon.momentum_nesterov(self.grad, self.buf, self.u, self.mu)

    def orthogonalise(self, events=None):
        """NS5 of every momentum output in one batched call: each product of
        each NS5 step is one launch over all matrices (``events``: see
        ``muon.ns5_batched``)."""
        muon.ns5_batched(self.us, self.outs, steps=self.steps, eps=self.eps, workspace=self.workspace,
                         events=events)

    def last_recorded(self):
        """Event pairs recorded by the last ``orthogonalise(events=...)``."""
        return muon.ns5_batched.last_recorded

    def fused_step(self, events=None):
        """The whole step in one call: momentum fused with the first pass of
        the norm, then NS5; ``us`` is not written (u never exists in
        float32).  ``events``: see ``muon.ns5_batched``."""
        muon.ns5_batched(self.grads, self.outs, steps=self.steps, eps=self.eps, workspace=self.workspace,
                         events=events, bufs=self.bufs, mu=self.mu)
        return self.outs

    def apply_step(self, lr):
        """The whole step with its parameter update, in one call: the
        parameters ``params`` (allocated as zeros on first use, one flat
        float32 buffer laid out like the gradients) become ``p - lr * NS5(u)``;
        the update O is never stored."""
        if not hasattr(self, "param"):
            self.param = torch.zeros(self.total, dtype=torch.float32, device=self.device)
            self.params = self._views(self.param)
        muon.ns5_batched(self.grads, self.params, steps=self.steps, eps=self.eps, workspace=self.workspace,
                         bufs=self.bufs, mu=self.mu, lr=lr)
        return self.params

    def step(self):
        """Enqueue one step on the current stream; results land in ``outs``
        (and the new state in ``bufs``)."""
        self.momentum()
        self.orthogonalise()
        return self.outs

    def nominal_ns5_flops(self):
        return sum(muon.ns5_flops(r, c, self.steps) for r, c in self.shapes)

    def momentum_bytes(self):
        return 16 * sum(r * c for r, c in self.shapes)
