"""Modal distillation of long filters on the GPU, through the C ABI.

Each head's target filter h [H][L] is fitted by a d-mode modal filter
(poles lambda, residues R, skip D) under the filter-discrepancy objective
sum_t (hhat[t] - h[t])^2 (Laughing Hyena Distillery review, 提出的方法), by
Adam steps that keep every pole inside the unit disc.  Each step is two
library calls (objective and gradient, then the update); torch only holds the
buffers.  The fitted tables plug straight into :class:`ModalHyena`.

Starts:
  init="circle": poles on the circle |lambda| = r_init at angles pi (n + 1/2) / d,
                 residues zero, D = h[0];
  init="fit":    the library's host-side matrix-pencil fit of the target taps
                 (hyena_modal_fit_init: poles from the pencil of the first taps,
                 residues by least squares over all taps, D = h[0]) -- the
                 Prony-type modal reduction, which Adam then refines.
hankel_order() gives each head's order from its Hankel singular values, from
which d can be chosen.
"""

from __future__ import annotations

import math

from . import binding as hb


class ModalDistiller:
    def __init__(self, target, d: int, r_init: float = 0.9, device="cuda", init: str = "circle",
                 r_max: float = 0.9999):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.target = torch.as_tensor(target, dtype=torch.float32).to(self.device).contiguous()
        self.H, self.L = int(self.target.shape[0]), int(self.target.shape[1])
        self.d = int(d)
        H, d_ = self.H, self.d
        e = dict(dtype=torch.float32, device=self.device)
        if init == "fit":
            p, r, sk = hb.hyena_modal_fit_init(self.target.cpu().numpy(), d_, r_max)
            self.poles = torch.from_numpy(p).to(self.device).contiguous()
            self.residues = torch.from_numpy(r).to(self.device).contiguous()
            self.skip = torch.from_numpy(sk).to(self.device).contiguous()
        elif init == "circle":
            ang = torch.tensor([math.pi * (n + 0.5) / d_ for n in range(d_)], dtype=torch.float64)
            poles = torch.stack([r_init * torch.cos(ang), r_init * torch.sin(ang)], -1)
            self.poles = poles.to(torch.float32)[None].repeat(H, 1, 1).to(self.device).contiguous()
            self.residues = torch.zeros((H, d_, 2), **e)
            self.skip = self.target[:, 0].clone()
        else:
            raise ValueError(f"unknown start {init!r}")
        self.g_poles = torch.zeros((H, d_, 2), **e)
        self.g_res = torch.zeros((H, d_, 2), **e)
        self.g_skip = torch.zeros((H,), **e)
        self.m = torch.zeros((H * d_ * 4 + H,), **e)
        self.v = torch.zeros((H * d_ * 4 + H,), **e)
        self.loss = torch.zeros((H,), **e)
        self.desc = hb.make_desc(0, H, H, d_, hb.HM_F32, self.poles, self.residues, self.skip)
        n = hb.hyena_distill_workspace(self.desc, self.L)
        self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        self.t = 0

    def objective(self, loss=None, stream=None):
        """Loss [H] and gradients (in self.g_*) at the current parameters."""
        loss = self.loss if loss is None else loss
        hb.hyena_distill_grad(self.desc, self.L, self.target, loss, self.g_poles, self.g_res, self.g_skip,
                              self.ws, stream=stream)
        return loss

    def step(self, lr: float, loss=None, r_max: float = 0.9999, stream=None):
        """One Adam step; the loss before the step goes to ``loss`` (default self.loss)."""
        self.objective(loss, stream)
        self.t += 1
        hb.hyena_distill_adam_step(self.H, self.d, self.poles, self.residues, self.skip, self.g_poles, self.g_res,
                                   self.g_skip, self.m, self.v, self.t, lr, r_max=r_max, stream=stream)

    def fit(self, steps: int, lr: float = 1e-2, r_max: float = 0.9999, stream=None):
        """Run ``steps`` Adam steps; returns the loss history [steps][H] (device)."""
        hist = self.torch.empty((steps, self.H), dtype=self.torch.float32, device=self.device)
        for i in range(steps):
            self.step(lr, loss=hist[i], r_max=r_max, stream=stream)
        return hist


def hankel_order(target, n: int = 64, rel_tol: float = 1e-6):
    """Per head of target [H][L] (host or device): the number of Hankel singular
    values above rel_tol x the largest (the real order of the filter; d complex
    modes give at most 2d)."""
    import numpy as np
    t = target.detach().float().cpu().numpy() if hasattr(target, "detach") else np.asarray(target, np.float32)
    return hb.hyena_modal_order(t, n, rel_tol)
