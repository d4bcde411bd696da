"""Put a seeded synthetic layer (afd_inputs) on the GPU and wrap it.

Weights are drawn on the host expert by expert (threads) and copied straight
into preallocated device stacks, so no full host copy of a 20+ GB weight set
is ever held.  For W8A8 the bf16 stacks are quantised on the device by the
library's own 128x128 block quantiser and then freed.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from afd_inputs import SyntheticLayer

from .layer import FfnLayer, quantize_fp8_128x128


def to_device(a: np.ndarray, device, bf16: bool):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf16 else a)
    t = t.to(device)
    return t.view(torch.bfloat16) if bf16 else t


def hidden_tensor(syn: SyntheticLayer, device):
    return to_device(syn.hidden(), device, syn.shape.mode != "f32")


def build_layer(syn: SyntheticLayer, device, max_tokens=None, threads=16, single_launch=False,
                split_gemms=False):
    """FfnLayer holding the synthetic layer's weights on `device`
    (single_launch: forwards of at most 16 tokens as one launch; split_gemms:
    one launch per weight-streaming GEMM)."""
    s = syn.shape
    bf16 = s.mode != "f32"
    dt = torch.bfloat16 if bf16 else torch.float32
    E, I, h = s.E, s.I, s.h
    gate = torch.empty((E, I, h), dtype=dt, device=device)
    up = torch.empty((E, I, h), dtype=dt, device=device)
    down = torch.empty((E, h, I), dtype=dt, device=device)

    def put(dst, arr):
        src = torch.from_numpy(arr.view(np.int16) if bf16 else arr)
        dst.copy_(src.view(torch.bfloat16) if bf16 else src)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for e, mats in enumerate(ex.map(syn.expert, range(E))):
            put(gate[e], mats[0])
            put(up[e], mats[1])
            put(down[e], mats[2])
    sh = [None] * 3
    if s.S:
        sh = [torch.stack([to_device(syn.shared(j)[m], device, bf16) for j in range(s.S)])
              for m in range(3)]
    router_w = to_device(syn.router_weight(), device, bf16)
    b = syn.router_bias()
    router_b = None if b is None else torch.from_numpy(b).to(device)
    kw = dict(mode=s.mode, hidden=h, num_experts=E, top_k=s.k, inter=I,
              max_tokens=max_tokens or s.T, router_w=router_w, router_b=router_b,
              num_shared=s.S, shared_inter=s.Is, single_launch=single_launch,
              split_gemms=split_gemms)
    if s.mode == "w8a8":
        (gq, gs), (uq, us), (dq, ds) = (quantize_fp8_128x128(t) for t in (gate, up, down))
        kw.update(gate_w=gq, up_w=uq, down_w=dq, gate_s=gs, up_s=us, down_s=ds)
        if s.S:
            (a, as_), (b_, bs), (c, cs) = (quantize_fp8_128x128(t) for t in sh)
            kw.update(sh_gate_w=a, sh_up_w=b_, sh_down_w=c, sh_gate_s=as_,
                      sh_up_s=bs, sh_down_s=cs)
        torch.cuda.synchronize(device)
        del gate, up, down, sh
    else:
        kw.update(gate_w=gate, up_w=up, down_w=down)
        if s.S:
            kw.update(sh_gate_w=sh[0], sh_up_w=sh[1], sh_down_w=sh[2])
    return FfnLayer(**kw)
