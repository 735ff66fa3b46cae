"""A projected Hyena stack over the C ABI (argument marshalling only).

Each layer: in_proj (D -> 3D) of the layer input with each token's row scaled
by its inverse RMS (fused into the projection) -> the modal Hyena operator on
[q|k|v] (contiguous thirds of the in_proj output) -> out_proj (D -> D).  No
bias, no residual.
The stack's output at the last prompt position is the first generation input;
each later generation input is the previous step's output.  Every computation
is a library call; torch only provides device memory, views and streams.
"""

from __future__ import annotations

from . import binding as hb

RMS_EPS = 1e-6


class HyenaStack:
    """Per-layer tables and weights (device tensors) plus preallocated buffers.

    layers: list of (ModalParams-like with poles/residues/skip, W_in [3D][D],
    W_out [D][D]); weights are torch bfloat16 tensors on ``device`` (or numpy
    bfloat16 bit patterns, copied to the device).
    """

    def __init__(self, layers, batch: int, prompt_len: int, device="cuda", fused: bool = True):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.B, self.L = int(batch), int(prompt_len)
        self.w_in, self.w_out, self.ops = [], [], []
        for params, w_in, w_out in layers:
            self.w_in.append(self._bf16(w_in))
            self.w_out.append(self._bf16(w_out))
            D = self.w_out[-1].shape[0]
            self.ops.append(hb.ModalHyena(params.poles, params.residues, params.skip, self.B, D, "bf16",
                                          device=self.device))
        self.D = D
        self.nl = len(self.ops)
        B, L, D = self.B, self.L, self.D
        e = dict(device=self.device)
        bf = torch.bfloat16
        M = B * L
        # prompt buffers
        self.x = [torch.empty((M, D), dtype=bf, **e), torch.empty((M, D), dtype=bf, **e)]
        self.qkv = torch.empty((M, 3 * D), dtype=bf, **e)
        self.y = torch.empty((M, D), dtype=bf, **e)
        # generation buffers
        self.xd = torch.empty((B, D), dtype=bf, **e)      # step input (and, fed back, output)
        self.xd_mid = [torch.empty((B, D), dtype=bf, **e), torch.empty((B, D), dtype=bf, **e)]
        self.qkvd = torch.empty((B, 3 * D), dtype=bf, **e)
        self.yd = torch.empty((B, D), dtype=bf, **e)
        self.states = [op.new_state() for op in self.ops]
        # split-K scratch of the generation-step projections
        ws = max(hb.hyena_dense_workspace(B, 3 * D, D), hb.hyena_dense_workspace(B, D, D))
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, **e) if ws > 0 else None
        # generation step: in_proj and decode fused into one launch where the
        # library supports the shape (packed in_proj rows), else two calls
        self.w_in_packed = None
        if fused and D % 16 == 0:
            self.w_in_packed = []
            for w in self.w_in:
                wp = torch.empty_like(w)
                hb.hyena_pack_in_proj_bf16(D, D, w, D, wp)
                self.w_in_packed.append(wp)

    def _bf16(self, w):
        torch = self.torch
        if isinstance(w, torch.Tensor):
            return w.to(self.device, torch.bfloat16).contiguous()
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).to(self.device)

    # ------------------------------------------------------------ one layer

    def _layer(self, l, x, out, M, qkv, y, rows_time, prefill: bool):
        D = self.D
        ws = None if prefill else self.ws
        hb.hyena_dense_rms_bf16(M, 3 * D, D, x, D, self.w_in[l], D, RMS_EPS, qkv, 3 * D, workspace=ws)
        if prefill:
            B, L = rows_time
            q3 = qkv.view(B, L, 3 * D)
            self.ops[l].prefill(q3[:, :, :D], q3[:, :, D:2 * D], q3[:, :, 2 * D:], y=y.view(B, L, D),
                                state_out=self.states[l])
        else:
            self.ops[l].decode_step(qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:], self.states[l], y=y)
        hb.hyena_dense_bf16(M, D, D, y, D, self.w_out[l], D, None, out, D, workspace=ws)

    def _layer_step(self, l, x, out):
        """One generated token through layer l: fused in_proj + decode when supported."""
        D, B = self.D, self.B
        if self.w_in_packed is not None:
            st = hb.hyena_layer_step_bf16(self.ops[l].desc, x, D, self.w_in_packed[l], RMS_EPS, self.states[l],
                                          self.yd, D)
            if st == hb.HM_OK:
                hb.hyena_dense_bf16(B, D, D, self.yd, D, self.w_out[l], D, None, out, D, workspace=self.ws)
                return
        self._layer(l, x, out, B, self.qkvd, self.yd, None, False)

    def prefill(self, x_in, record=None):
        """x_in: [B][L][D] bf16 prompt input.  Returns the stack output [B*L][D].

        record(l, x): called with each layer's input (a device view) before the layer.
        """
        M = self.B * self.L
        src = x_in.reshape(M, self.D)
        for l in range(self.nl):
            if record is not None:
                record(l, src)
            dst = self.x[l % 2]
            self._layer(l, src, dst, M, self.qkv, self.y, (self.B, self.L), True)
            src = dst
        return src

    def start_generation(self, prompt_out):
        """Copy the output at the last prompt position into the step input buffer."""
        self.xd.copy_(prompt_out.view(self.B, self.L, self.D)[:, -1, :])

    def decode_step(self, record=None):
        """One generated token for every batch row: reads self.xd, writes the output back to self.xd."""
        src = self.xd
        for l in range(self.nl):
            if record is not None:
                record(l, src)
            dst = self.xd if l == self.nl - 1 else self.xd_mid[l % 2]
            self._layer_step(l, src, dst)
            src = dst
        return self.xd
