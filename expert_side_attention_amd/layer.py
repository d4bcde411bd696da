"""torch-facing wrapper of the C ABI: device tensors in, device tensors out.

PyTorch is used for device memory and streams only; the layer itself runs in
libafd_ffn.so.  The wrapper checks dtypes, shapes and devices, keeps the
weight tensors alive (the library borrows them) and passes raw pointers.
"""
from __future__ import annotations

import torch

from . import _ffi as F

_MODES = {"f32": F.AFD_MODE_F32, "bf16": F.AFD_MODE_BF16,
          "w8a8": F.AFD_MODE_W8A8_E4M3}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_fp8_1x128(x: torch.Tensor, stream=None):
    """E4M3 codes (uint8) and fp32 scales [rows, cols/128] of a bf16 or fp32
    matrix."""
    if x.dtype not in (torch.bfloat16, torch.float32) or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bf16 or fp32 tensor")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    fn = F.afd_quant_fp8_1x128 if x.dtype == torch.bfloat16 else F.afd_quant_fp8_1x128_f32
    fn(x.data_ptr(), rows, cols, q.data_ptr(), s.data_ptr(), _stream(stream))
    return q, s


def quantize_fp8_128x128(w: torch.Tensor, stream=None):
    """E4M3 codes and fp32 128x128 block scales of a bf16 [..., N, K] stack."""
    if w.dtype != torch.bfloat16 or w.dim() < 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous bf16 tensor with >= 2 dims")
    *lead, n, k = w.shape
    rows = w.numel() // k
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    s = torch.empty((*lead, n // 128, k // 128), dtype=torch.float32, device=w.device)
    F.afd_quant_fp8_128x128(w.data_ptr(), rows, k, q.data_ptr(), s.data_ptr(),
                            _stream(stream))
    return q, s


class FfnLayer:
    """One MoE FFN-service layer on the current HIP device.

    Weights: router_w [E, h]; gate_w, up_w [E, I, h]; down_w [E, h, I];
    shared sh_* with I_s; dtypes fp32 (mode "f32"), bf16 ("bf16"), or uint8
    E4M3 codes with fp32 block scales and a bf16 router ("w8a8")."""

    def __init__(self, *, mode, hidden, num_experts, top_k, inter, max_tokens,
                 router_w, gate_w, up_w, down_w, router_b=None,
                 gate_s=None, up_s=None, down_s=None, num_shared=0,
                 shared_inter=0, sh_gate_w=None, sh_up_w=None, sh_down_w=None,
                 sh_gate_s=None, sh_up_s=None, sh_down_s=None, single_launch=False,
                 split_gemms=False):
        if mode not in _MODES:
            raise ValueError(f"mode must be one of {sorted(_MODES)}")
        self.mode = mode
        dev = router_w.device
        h, E, I, S, Is = hidden, num_experts, inter, num_shared, shared_inter
        act = torch.float32 if mode == "f32" else torch.bfloat16
        wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "w8a8": torch.uint8}[mode]
        _need(router_w, "router_w", act, (E, h), dev)
        if router_b is not None:
            _need(router_b, "router_b", torch.float32, (E,), dev)
        _need(gate_w, "gate_w", wdt, (E, I, h), dev)
        _need(up_w, "up_w", wdt, (E, I, h), dev)
        _need(down_w, "down_w", wdt, (E, h, I), dev)
        if mode == "w8a8":
            _need(gate_s, "gate_s", torch.float32, (E, I // 128, h // 128), dev)
            _need(up_s, "up_s", torch.float32, (E, I // 128, h // 128), dev)
            _need(down_s, "down_s", torch.float32, (E, h // 128, I // 128), dev)
        if S:
            _need(sh_gate_w, "sh_gate_w", wdt, (S, Is, h), dev)
            _need(sh_up_w, "sh_up_w", wdt, (S, Is, h), dev)
            _need(sh_down_w, "sh_down_w", wdt, (S, h, Is), dev)
            if mode == "w8a8":
                _need(sh_gate_s, "sh_gate_s", torch.float32, (S, Is // 128, h // 128), dev)
                _need(sh_up_s, "sh_up_s", torch.float32, (S, Is // 128, h // 128), dev)
                _need(sh_down_s, "sh_down_s", torch.float32, (S, h // 128, Is // 128), dev)
        self._keep = [router_w, router_b, gate_w, up_w, down_w, gate_s, up_s, down_s,
                      sh_gate_w, sh_up_w, sh_down_w, sh_gate_s, sh_up_s, sh_down_s]
        self.device = dev
        self.hidden, self.num_experts, self.top_k = h, E, top_k
        self.inter, self.shared_inter = I, Is
        self.num_shared, self.max_tokens = S, max_tokens
        self.act_dtype = act
        cfg = F.afd_ffn_config(
            abi_version=F.AFD_FFN_ABI_VERSION, mode=_MODES[mode], hidden=h,
            num_experts=E, top_k=top_k, inter=I, num_shared=S, shared_inter=Is,
            max_tokens=max_tokens, has_router_bias=int(router_b is not None),
            single_launch=int(bool(single_launch)), split_gemms=int(bool(split_gemms)))
        self.single_launch = bool(single_launch)
        self.split_gemms = bool(split_gemms)
        w = F.afd_ffn_weights(*[_ptr(t) for t in self._keep])
        self._cfg, self._w = cfg, w
        with torch.cuda.device(dev):
            self._h = F.afd_ffn_create(cfg, w)

    def sibling(self) -> "FfnLayer":
        """Another handle (own workspace) over the same weights, for a second
        micro-batch on another stream."""
        k = self._keep
        return FfnLayer(mode=self.mode, hidden=self.hidden, num_experts=self.num_experts,
                        top_k=self.top_k, inter=self.inter, max_tokens=self.max_tokens,
                        router_w=k[0], router_b=k[1], gate_w=k[2], up_w=k[3], down_w=k[4],
                        gate_s=k[5], up_s=k[6], down_s=k[7], num_shared=self.num_shared,
                        shared_inter=self.shared_inter, sh_gate_w=k[8], sh_up_w=k[9],
                        sh_down_w=k[10], sh_gate_s=k[11], sh_up_s=k[12], sh_down_s=k[13],
                        single_launch=self.single_launch, split_gemms=self.split_gemms)

    def forward(self, hidden: torch.Tensor, out: torch.Tensor = None, stream=None,
                trace: bool = False):
        """out [T, h] = layer(hidden [T, h]).  With trace=True also returns a
        dict of the routing/dispatch intermediates of this call (router
        logits, ids, weights, dispatch, tile counts; W8A8: quantised input
        and z)."""
        T = hidden.shape[0]
        _need(hidden, "hidden", self.act_dtype, (T, self.hidden), self.device)
        if out is None:
            out = torch.empty_like(hidden)
        _need(out, "out", self.act_dtype, (T, self.hidden), self.device)
        s = _stream(stream)
        if not trace:
            F.afd_ffn_forward(self._h, hidden.data_ptr(), out.data_ptr(), T, s)
            return out
        d, k, E = self.device, self.top_k, self.num_experts
        tr = {"topk_ids": torch.empty((T, k), dtype=torch.int32, device=d),
              "topk_w": torch.empty((T, k), dtype=torch.float32, device=d),
              "counts": torch.empty((E,), dtype=torch.int32, device=d),
              "offsets": torch.empty((E + 1,), dtype=torch.int32, device=d),
              "perm": torch.empty((T * k,), dtype=torch.int32, device=d),
              "slot_row": torch.empty((T, k), dtype=torch.int32, device=d),
              "logits": torch.empty((T, E), dtype=torch.float32, device=d),
              "num_tiles": torch.empty((2,), dtype=torch.int32, device=d),
              "sync_timeouts": torch.empty((1,), dtype=torch.int32, device=d)}
        if self.mode == "w8a8":
            R = T * k + self.num_shared * T
            Z = max(self.inter, self.shared_inter if self.num_shared else 0)
            tr["x_q"] = torch.empty((T, self.hidden), dtype=torch.uint8, device=d)
            tr["x_s"] = torch.empty((T, self.hidden // 128), dtype=torch.float32, device=d)
            tr["z_q"] = torch.empty((R, Z), dtype=torch.uint8, device=d)
            tr["z_s"] = torch.empty((R, Z // 128), dtype=torch.float32, device=d)
        ct = F.afd_ffn_trace(**{n: tr[n].data_ptr() for n in tr})
        F.afd_ffn_forward_traced(self._h, hidden.data_ptr(), out.data_ptr(), T, s, ct)
        return out, tr

    def forward_static(self, hidden: torch.Tensor, out: torch.Tensor = None, stream=None):
        """The same layer through afd_ffn_forward_static: no handle, the
        library's fixed per-device scratch as workspace, nothing allocated by
        the library (out is allocated here when not given)."""
        T = hidden.shape[0]
        _need(hidden, "hidden", self.act_dtype, (T, self.hidden), self.device)
        if out is None:
            out = torch.empty_like(hidden)
        _need(out, "out", self.act_dtype, (T, self.hidden), self.device)
        F.afd_ffn_forward_static(self._cfg, self._w, hidden.data_ptr(), out.data_ptr(), T,
                                 _stream(stream))
        return out

    def profile_enable(self, stages=()):
        mask = 0
        for n in stages:
            mask |= 1 << F.STAGE_INDEX[n]
        F.afd_ffn_profile_enable(self._h, mask)

    def profile_read(self):
        return F.afd_ffn_profile_read(self._h)

    def close(self):
        if getattr(self, "_h", None) is not None:
            F.afd_ffn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
