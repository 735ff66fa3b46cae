"""A projected Hyena stack over the C ABI (argument marshalling only).

Each layer: in_proj (D -> 3D) of the layer input with each token's row scaled
by its inverse RMS -> the modal Hyena operator on [q|k|v] (contiguous thirds
of the in_proj output) -> out_proj (D -> D).  No bias, no residual.  For the
prompt the inverse RMS is a row pass of its own (hyena_row_rms) whose result
is the in_proj's row scale: the prompt GEMM without a fused sum of squares is
the faster one at these shapes (measured on MI355X, B * L = 131072, D = 2048:
0.09 + 2.79 ms against 3.56 ms fused).  A generated token's in_proj computes
its RMS inside the projection.
The stack's output at the last prompt position is the first generation input;
each later generation input is the previous step's output.  Every computation
is a library call; torch only provides device memory, views and streams.

Generation paths, fastest first (chosen once, from the shape):
  "deferred": per layer two launches with the state kept one input behind:
      the gate (RMS-fused in_proj, u = k v, y = q (D u + rho)), whose launch
      also prepares the next layer's readout from its state, then out_proj;
      each layer holds s = x - u_prev, u_prev and rho;
  "fused":    in_proj and decode step in one launch (hyena_layer_step_bf16),
      then out_proj;
  "separate": in_proj, decode step and out_proj as three calls.
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

    def __init__(self, layers, batch: int, prompt_len: int, device="cuda", fused: bool = True,
                 deferred: bool = True):
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
        self.inv_rms = torch.empty(M, dtype=torch.float32, **e)  # the prompt rows' inverse RMS
        # generation buffers
        self.xd = torch.empty((B, D), dtype=bf, **e)      # step input (and, fed back, output)
        self.xd_mid = [torch.empty((B, D), dtype=bf, **e), torch.empty((B, D), dtype=bf, **e)]
        self.qkvd = torch.empty((B, 3 * D), dtype=bf, **e)
        self.yd = torch.empty((B, D), dtype=bf, **e)
        self.states = [op.new_state() for op in self.ops]
        # split-K scratch of the generation-step projections
        ws = max(hb.hyena_dense_workspace(B, 3 * D, D), hb.hyena_dense_workspace(B, D, D))
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, **e) if ws > 0 else None
        # generation step: the deferred state where hyena_layer_gate_bf16 covers
        # the shape (B <= 64, D = 2048, D/H a multiple of 16, d in {8, 16, 32});
        # else in_proj and decode fused into one launch (packed in_proj rows);
        # else three calls
        self.deferred = bool(fused and deferred and B <= 64 and D == 2048 and D // self.ops[0].H % 16 == 0
                             and all(op.d in (8, 16, 32) for op in self.ops))
        if self.deferred:
            self.u_prev = [torch.zeros((B, D), dtype=torch.float32, **e) for _ in range(self.nl)]
            self.rho = [torch.zeros((B, D), dtype=torch.float32, **e) for _ in range(self.nl)]
        self.w_in_packed = None
        if fused and D % 16 == 0:
            self.w_in_packed = []
            for w in self.w_in:
                wp = torch.empty((3 * D, D), dtype=w.dtype, device=w.device)
                hb.hyena_pack_in_proj_bf16(D, D, w, w.stride(0), wp)
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
        if prefill:
            hb.hyena_row_rms(x, M, D, x.stride(0), RMS_EPS, self.inv_rms)
            hb.hyena_dense_bf16(M, 3 * D, D, x, x.stride(0), self.w_in[l], self.w_in[l].stride(0), self.inv_rms, qkv,
                                3 * D)
        else:
            hb.hyena_dense_rms_bf16(M, 3 * D, D, x, x.stride(0), self.w_in[l], self.w_in[l].stride(0), RMS_EPS, qkv,
                                    3 * D, workspace=ws)
        if prefill:
            B, L = rows_time
            q3 = qkv.view(B, L, 3 * D)
            self.ops[l].prefill(q3[:, :, :D], q3[:, :, D:2 * D], q3[:, :, 2 * D:], y=y.view(B, L, D),
                                state_out=self.states[l])
        else:
            self.ops[l].decode_step(qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:], self.states[l], y=y)
        hb.hyena_dense_bf16(M, D, D, y, y.stride(0), self.w_out[l], self.w_out[l].stride(0), None, out,
                            out.stride(0), workspace=ws)

    def _layer_step(self, l, x, out):
        """One generated token through layer l: fused in_proj + decode when supported."""
        D, B = self.D, self.B
        if self.deferred:
            # the next layer's prepare rides in this gate's launch
            nxt = (l + 1) % self.nl
            st = hb.hyena_layer_gate_bf16(self.ops[l].desc, x, x.stride(0), self.w_in_packed[l], RMS_EPS,
                                          self.rho[l], self.u_prev[l], self.yd, self.yd.stride(0),
                                          self.ops[nxt].desc, self.states[nxt], self.u_prev[nxt], self.rho[nxt])
            if st != hb.HM_OK:
                raise hb.HMError(st, "hyena_layer_gate_bf16")
            hb.hyena_dense_bf16(B, D, D, self.yd, self.yd.stride(0), self.w_out[l], self.w_out[l].stride(0),
                                None, out, out.stride(0), workspace=self.ws)
            return
        if self.w_in_packed is not None:
            st = hb.hyena_layer_step_bf16(self.ops[l].desc, x, x.stride(0), self.w_in_packed[l], RMS_EPS,
                                          self.states[l], self.yd, self.yd.stride(0))
            if st == hb.HM_OK:
                hb.hyena_dense_bf16(B, D, D, self.yd, self.yd.stride(0), self.w_out[l], self.w_out[l].stride(0),
                                    None, out, out.stride(0), workspace=self.ws)
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
        """Copy the output at the last prompt position into the step input buffer
        (deferred path: every layer's state s = the prefill's state, u_prev = 0,
        and layer 0's readout prepared for the first generated token; every other
        layer's prepare rides in the gate launch of the layer before it)."""
        self.xd.copy_(prompt_out.view(self.B, self.L, self.D)[:, -1, :])
        if self.deferred:
            for u in self.u_prev:
                u.zero_()
            hb.hyena_decode_prepare(self.ops[0].desc, self.states[0], self.u_prev[0], self.rho[0])

    def state_of(self, l):
        """Layer l's modal state x [B][H][d][P][2] between tokens (for inspection):
        on the deferred path s + u_prev (u_prev added to the real part of every
        mode) for layers 1.. (and layer 0 before the first token); layer 0 has
        been prepared for the coming token (its stored s is lambda x): None."""
        st = self.states[l]
        if not self.deferred:
            return st.clone()
        if l == 0:
            return None
        B, H, d, P = st.shape[0], st.shape[1], st.shape[2], st.shape[3]
        x = st.clone()
        x[..., 0] += self.u_prev[l].view(B, H, 1, P)
        return x

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
