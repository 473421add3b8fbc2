"""BeamDecoder: owns a torch-allocated workspace and one context of the C ABI.

PyTorch provides device memory and the stream here; every step of the decode
runs in the HIP library.  Methods map one-to-one onto gdn_beam_* calls.
"""
from __future__ import annotations

import torch

from . import binding as B

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class BeamDecoder:
    def __init__(self, R, H, d_k, d_v, T_max, W_max, V_max, io="bf16", wout="bf16",
                 device="cuda", H_K=0):
        self.cfg = B.make_config(R, H, d_k, d_v, T_max, W_max, V_max, io, wout, H_K)
        self.io, self.wout = io, wout
        self.shape = dict(R=R, H=H, H_K=H_K or H, d_k=d_k, d_v=d_v, T_max=T_max, W_max=W_max,
                          V_max=V_max)
        self.ws_bytes = B.gdn_beam_workspace_bytes(self.cfg)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        off = (-self.ws.data_ptr()) % 256            # the ABI wants a 256-byte aligned base
        self.ws_ptr = self.ws.data_ptr() + off
        self.device = torch.device(device)
        self.ctx = None

    @staticmethod
    def _stream(stream):
        return torch.cuda.current_stream() if stream is None else stream

    def init(self, S_ctx, W0, stream=None):
        self.close()
        self.ctx = B.gdn_beam_init(self.cfg, S_ctx, W0, self.ws_ptr, self.ws_bytes,
                                   self._stream(stream))
        return self

    def step(self, t, q, k, v, alpha, beta, o, stream=None):
        B.gdn_beam_step(self.ctx, t, q, k, v, alpha, beta, o, self._stream(stream))

    def fullstate_step(self, t, S_ctx, q, k, v, alpha, beta, o, states, stream=None):
        """The FullState baseline in place of step(t); `states` is a device buffer of
        fullstate_bytes() bytes (see alloc_states)."""
        B.gdn_fullstate_step(self.ctx, t, S_ctx, q, k, v, alpha, beta, o, states,
                             states.numel() * states.element_size(), self._stream(stream))

    def fullstate_bytes(self):
        return B.gdn_fullstate_bytes(self.cfg)

    def alloc_states(self):
        return torch.empty(self.fullstate_bytes() // 4, dtype=torch.float32, device=self.device)

    def select(self, t, o, Wout, V, W_next, parent, token, score, forced_parent=None,
               forced_token=None, stream=None):
        B.gdn_beam_select(self.ctx, t, o, Wout, V, W_next, forced_parent, forced_token,
                          parent, token, score, self._stream(stream))

    def query(self):
        return B.gdn_beam_query(self.ctx)

    def export(self, what, stream=None):
        n = B.gdn_beam_export_bytes(self.ctx, what)
        s = self.shape
        R, H, T, W = s["R"], s["H"], s["T_max"], s["W_max"]
        shapes = {
            B.GDN_EXPORT_ANCESTRY: ((R, W, T), torch.int32),
            B.GDN_EXPORT_TOKENS: ((R, W, T), torch.int32),
            B.GDN_EXPORT_CUM: ((R, W), torch.float32),
            B.GDN_EXPORT_GTR_ALPHA: ((R, H, T, W), torch.float32),
            B.GDN_EXPORT_GTR_DELTA: ((R, H, T, W, s["d_v"]), torch.float32),
            B.GDN_EXPORT_GTR_KEY: ((R, s["H_K"], T, W, s["d_k"]), _DT[self.io]),
            B.GDN_EXPORT_STATUS: ((1,), torch.int32),
        }
        shape, dt = shapes[what]
        out = torch.empty(shape, dtype=dt, device=self.device)
        assert out.numel() * out.element_size() == n
        B.gdn_beam_export(self.ctx, what, out, n, self._stream(stream))
        return out

    @staticmethod
    def time_steps(capacity):
        """Make the next `capacity` step launches (of any decoder: a process-wide count)
        record their own kernel time."""
        B.gdn_beam_time_steps(capacity)

    @staticmethod
    def step_times(cap):
        """(durations in ms of the timed step launches, in launch order; number recorded)."""
        return B.gdn_beam_step_times(cap)

    def close(self):
        if self.ctx is not None:
            B.gdn_beam_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prefill(S_out, k, v, alpha, beta, offsets, stream=None):
    """S_out [R,H,d_v,d_k] <- eq. (3) over stacked prompt tokens (see gdn_beam_prefill);
    k [N,H_K,d_k] may hold fewer (key) heads than v [N,H,d_v] (grouped value heads)."""
    R, H, d_v, d_k = S_out.shape
    N = k.shape[0]
    B.gdn_beam_prefill(R, H, k.shape[1], d_k, d_v, N, k, v, alpha, beta, offsets, S_out,
                       torch.cuda.current_stream() if stream is None else stream)
