"""BeamDecoder: owns a torch-allocated workspace and one context of the C ABI.

PyTorch provides device memory and the stream here; every step of the decode
runs in the HIP library.  Methods map one-to-one onto gdn_beam_* calls.
"""
from __future__ import annotations

import torch

from . import binding as B

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _need(name, x, shape, dtype, device):
    """Refuse, on the host and before any launch, a tensor the kernels would read or
    write out of its bounds or misread: wrong shape, dtype or device, or not dense."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(x).__name__}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {tuple(shape)}")
    if x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if x.device.type != "cuda" or (device.index is not None and x.device.index != device.index):
        raise ValueError(f"{name}: on {x.device}, expected {device}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: not contiguous")


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
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.ctx = None

    @staticmethod
    def _stream(stream):
        return torch.cuda.current_stream() if stream is None else stream

    def _step_inputs(self, q, k, v, alpha, beta, o):
        s = self.shape
        _, W = B.gdn_beam_query(self.ctx)
        R, H, HK = s["R"], s["H"], s["H_K"]
        io = _DT[self.io]
        _need("q", q, (R, HK, W, s["d_k"]), io, self.device)
        _need("k", k, (R, HK, W, s["d_k"]), io, self.device)
        _need("v", v, (R, H, W, s["d_v"]), io, self.device)
        _need("alpha", alpha, (R, H, W), torch.float32, self.device)
        _need("beta", beta, (R, H, W), torch.float32, self.device)
        _need("o", o, (R, H, W, s["d_v"]), torch.float32, self.device)

    def _ctx(self):
        if self.ctx is None:
            raise RuntimeError("BeamDecoder: init() first")
        return self.ctx

    def init(self, S_ctx, W0, stream=None):
        s = self.shape
        _need("S_ctx", S_ctx, (s["R"], s["H"], s["d_v"], s["d_k"]), torch.float32, self.device)
        self.close()
        self.ctx = B.gdn_beam_init(self.cfg, S_ctx, W0, self.ws_ptr, self.ws_bytes,
                                   self._stream(stream))
        return self

    def step(self, t, q, k, v, alpha, beta, o, stream=None):
        self._ctx()
        self._step_inputs(q, k, v, alpha, beta, o)
        B.gdn_beam_step(self.ctx, t, q, k, v, alpha, beta, o, self._stream(stream))

    def fullstate_step(self, t, S_ctx, q, k, v, alpha, beta, o, states, stream=None):
        """The FullState baseline in place of step(t); `states` is a device buffer of
        fullstate_bytes() bytes (see alloc_states)."""
        self._ctx()
        s = self.shape
        if S_ctx is not None:                          # read at t = 0 only
            _need("S_ctx", S_ctx, (s["R"], s["H"], s["d_v"], s["d_k"]), torch.float32, self.device)
        self._step_inputs(q, k, v, alpha, beta, o)
        if not isinstance(states, torch.Tensor) or not states.is_cuda or not states.is_contiguous():
            raise ValueError("states: expected a dense device tensor (see alloc_states)")
        if states.numel() * states.element_size() < self.fullstate_bytes():
            raise ValueError(f"states: {states.numel() * states.element_size()} bytes, "
                             f"expected at least {self.fullstate_bytes()}")
        B.gdn_fullstate_step(self.ctx, t, S_ctx, q, k, v, alpha, beta, o, states,
                             states.numel() * states.element_size(), self._stream(stream))

    def fullstate_bytes(self):
        return B.gdn_fullstate_bytes(self.cfg)

    def alloc_states(self):
        return torch.empty(self.fullstate_bytes() // 4, dtype=torch.float32, device=self.device)

    def select(self, t, o, Wout, V, W_next, parent, token, score, forced_parent=None,
               forced_token=None, stream=None):
        self._ctx()
        s = self.shape
        _, W = B.gdn_beam_query(self.ctx)
        R = s["R"]
        _need("o", o, (R, s["H"], W, s["d_v"]), torch.float32, self.device)
        _need("Wout", Wout, (s["d_v"], V), _DT[self.wout], self.device)
        _need("parent", parent, (R, W_next), torch.int32, self.device)
        _need("token", token, (R, W_next), torch.int32, self.device)
        _need("score", score, (R, W_next), torch.float32, self.device)
        if (forced_parent is None) != (forced_token is None):
            raise ValueError("forced_parent and forced_token go together")
        if forced_parent is not None:
            _need("forced_parent", forced_parent, (R, W_next), torch.int32, self.device)
            _need("forced_token", forced_token, (R, W_next), torch.int32, self.device)
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


def prefill(S_out, k, v, alpha, beta, offsets, stream=None, chunked=True, workspace=None):
    """S_out [R,H,d_v,d_k] <- eq. (3) over stacked prompt tokens (see gdn_beam_prefill);
    k [N,H_K,d_k] may hold fewer (key) heads than v [N,H,d_v] (grouped value heads).
    chunked: the chunked form, with `workspace` (a uint8 device tensor of at least
    gdn_beam_prefill_workspace_bytes) or a fresh one; otherwise token by token."""
    R, H, d_v, d_k = S_out.shape
    N = k.shape[0]
    dev = S_out.device
    _need("S_out", S_out, (R, H, d_v, d_k), torch.float32, dev)
    HK = k.shape[1] if k.dim() == 3 else -1
    _need("k", k, (N, HK, d_k), torch.float32, dev)
    _need("v", v, (N, H, d_v), torch.float32, dev)
    _need("alpha", alpha, (N, H), torch.float32, dev)
    _need("beta", beta, (N, H), torch.float32, dev)
    _need("offsets", offsets, (R + 1,), torch.int32, dev)
    nbytes = 0
    if chunked:
        nbytes = B.gdn_beam_prefill_workspace_bytes(H, d_k, d_v, N)
        if workspace is None and nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        if workspace is not None:
            _need("workspace", workspace, (workspace.numel(),), torch.uint8, dev)
            nbytes = workspace.numel()
    else:
        workspace = None
    B.gdn_beam_prefill(R, H, k.shape[1], d_k, d_v, N, k, v, alpha, beta, offsets, S_out,
                       workspace, nbytes,
                       torch.cuda.current_stream() if stream is None else stream)
