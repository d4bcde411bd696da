"""Attention/FFN micro-pipeline on one MI355X (host-side harness, not on the
kernel path).

AFD runs attention and the experts on separate GPU pools and passes
micro-batches back and forth between them, so that in steady state a layer
costs the longer of the two stages plus the hand-over rather than their sum
(A/F 分离 page, 深入推导 / 微流水; the vLLM AFD plugin page lists MoE
ubatching and dual-batch overlap for the same reason).  This module runs that
schedule on one GPU:

* the FFN service is this library's layer, one handle per micro-batch;
* the attention service is a stand-in written with plain torch operations:
  decode attention of each token over its own KV cache (H query heads that
  share one K/V head of width d over L cached positions), the output
  projection and the residual.  It is the load the FFN service is paired
  with, not part of the library.

Three placements of one schedule:

* ``serial``: both services on one stream (co-located, nothing overlaps);
* ``overlap``: one stream per service over the whole chip;
* ``split``: one stream per service, each confined to its own compute units
  (HIP CU masks, whole blocks of 8 CUs), the blocks shared out by the
  rate-matching rule of ``afd_plan.split_gpus`` - a one-chip stand-in for
  separate attention and FFN pools.

The schedule is plain data (``ping_pong_schedule``), so its ordering is
checked without a GPU.
"""
from __future__ import annotations

import ctypes
import time
from dataclasses import dataclass
from typing import List, Optional, Sequence

from . import afd_plan

CU_BLOCK = 8  # the runtime accepts CU masks made of whole, aligned 8-CU blocks


@dataclass(frozen=True)
class Op:
    kind: str            # "attn" or "ffn"
    layer: int
    mb: int
    stream: int          # 0 = attention stream, 1 = FFN stream
    waits: tuple         # indices of earlier ops this one waits for


def ping_pong_schedule(layers: int, micro_batches: int) -> List[Op]:
    """Ops of `layers` layers for `micro_batches` micro-batches, in issue order.

    Micro-batch m of layer l: attention reads the hidden state the FFN wrote
    for (l - 1, m) and writes the FFN input; the FFN then reads that and writes
    the next hidden state.  So attn(l, m) waits for ffn(l - 1, m), and
    ffn(l, m) waits for attn(l, m); those two edges also order every reuse of
    the per-micro-batch buffers.  Micro-batches are otherwise independent,
    which is what lets one service work on m + 1 while the other works on m.
    """
    if layers < 1 or micro_batches < 1:
        raise ValueError("need at least one layer and one micro-batch")
    ops: List[Op] = []
    last_ffn = [None] * micro_batches
    for l in range(layers):
        for m in range(micro_batches):
            w = () if last_ffn[m] is None else (last_ffn[m],)
            ops.append(Op("attn", l, m, 0, w))
            a = len(ops) - 1
            ops.append(Op("ffn", l, m, 1, (a,)))
            last_ffn[m] = len(ops) - 1
    return ops


def cu_mask_words(blocks: Sequence[int], num_cus: int) -> List[int]:
    """32-bit CU-mask words enabling the given 8-CU blocks of a chip."""
    if num_cus % CU_BLOCK:
        raise ValueError(f"{num_cus} CUs is not a whole number of {CU_BLOCK}-CU blocks")
    nblk = num_cus // CU_BLOCK
    if not blocks:
        raise ValueError("a CU mask needs at least one block")
    words = [0] * ((num_cus + 31) // 32)
    for b in blocks:
        if not 0 <= b < nblk:
            raise ValueError(f"block {b} outside 0..{nblk - 1}")
        for c in range(b * CU_BLOCK, (b + 1) * CU_BLOCK):
            words[c // 32] |= 1 << (c % 32)
    return words


def split_blocks(t_attn: float, t_ffn: float, num_cus: int):
    """(attention blocks, FFN blocks): 8-CU blocks shared out by cost, as the
    pages share GPUs between the pools."""
    n_a, n_f = afd_plan.split_gpus(t_attn, t_ffn, num_cus // CU_BLOCK)
    return list(range(n_a)), list(range(n_a, n_a + n_f))


class MaskedStream:
    """A HIP stream whose kernels run only on the given 8-CU blocks."""

    def __init__(self, blocks: Sequence[int], num_cus: int, device=0):
        import torch
        self._hip = ctypes.CDLL("libamdhip64.so")
        words = cu_mask_words(blocks, num_cus)
        arr = (ctypes.c_uint32 * len(words))(*words)
        raw = ctypes.c_void_p()
        with torch.cuda.device(device):
            rc = self._hip.hipExtStreamCreateWithCUMask(ctypes.byref(raw),
                                                        ctypes.c_uint32(len(words)), arr)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with status {rc}")
        self._raw = raw
        self.stream = torch.cuda.ExternalStream(raw.value, device=device)
        self.blocks = list(blocks)

    def close(self):
        import torch
        if self._raw is not None:
            torch.cuda.synchronize()
            rc = self._hip.hipStreamDestroy(self._raw)
            self._raw = None
            if rc != 0:
                raise RuntimeError(f"hipStreamDestroy failed with status {rc}")


class AttentionStub:
    """Decode attention stand-in for one micro-batch of T tokens (torch ops).

    out = x + softmax(q K^T / sqrt(d)) V Wo with q = x Wq split into H heads
    of width d that share one K/V head; K is stored transposed, [T, d, L], and
    V as [T, L, d], so both batched products take a contiguous right operand.
    """

    def __init__(self, T: int, h: int, L: int, heads: int = 16, d: int = 512,
                 device="cuda:0", seed: int = 0):
        import torch
        g = torch.Generator(device=device).manual_seed(seed)
        bf = torch.bfloat16

        def rnd(*shape, std):
            return (torch.randn(*shape, generator=g, device=device) * std).to(bf)

        self.T, self.h, self.L, self.H, self.d = T, h, L, heads, d
        self.wq = rnd(h, heads * d, std=h ** -0.5)
        self.wo = rnd(heads * d, h, std=(heads * d) ** -0.5 * 0.1)
        self.kt = rnd(T, d, L, std=1.0)
        self.v = rnd(T, L, d, std=1.0)
        self.scale = d ** -0.5

    def kv_bytes(self) -> int:
        return 2 * self.T * self.L * self.d * 2

    def forward(self, x, out):
        import torch
        q = (x @ self.wq).view(self.T, self.H, self.d)
        s = torch.bmm(q, self.kt)
        p = torch.softmax(s.float() * self.scale, dim=-1).to(torch.bfloat16)
        o = torch.bmm(p, self.v).view(self.T, self.H * self.d)
        torch.add(x, o @ self.wo, out=out)
        return out


def run_schedule(ops: Sequence[Op], attn: Sequence[AttentionStub], ffn, hbuf, abuf,
                 streams) -> None:
    """Enqueue `ops`: attention of micro-batch m maps hbuf[m] -> abuf[m], the
    FFN maps abuf[m] -> hbuf[m].  streams = (attention stream, FFN stream)
    (the same stream twice for the co-located placement)."""
    import torch
    done: List[Optional[torch.cuda.Event]] = []
    for op in ops:
        st = streams[op.stream]
        for w in op.waits:
            st.wait_event(done[w])
        with torch.cuda.stream(st):
            if op.kind == "attn":
                attn[op.mb].forward(hbuf[op.mb], abuf[op.mb])
            else:
                ffn[op.mb].forward(abuf[op.mb], out=hbuf[op.mb], stream=st)
        ev = torch.cuda.Event()
        ev.record(st)
        done.append(ev)


def time_schedule(layers: int, attn, ffn, hbuf, abuf, streams, reset) -> float:
    """Wall time (ms) of `layers` layers after one untimed layer; `reset()`
    restores the input hidden states first."""
    import torch
    M = len(ffn)
    reset()
    run_schedule(ping_pong_schedule(1, M), attn, ffn, hbuf, abuf, streams)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_schedule(ping_pong_schedule(layers, M), attn, ffn, hbuf, abuf, streams)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def stage_ms(fn, reps: int) -> float:
    import torch
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / reps


def measure(ffn_layers, xs, attn, layers: int = 20, reps: int = 20,
            placements=("serial", "overlap", "split")) -> dict:
    """Per-layer period (ms, all micro-batches) of each placement, the stage
    times it is compared with, and whether every placement produced the same
    hidden states.  ffn_layers[m] / attn[m] / xs[m] belong to micro-batch m."""
    import torch
    M = len(ffn_layers)
    if not (len(xs) == len(attn) == M):
        raise ValueError("one FFN handle, one attention stub and one input per micro-batch")
    dev = xs[0].device
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    hbuf = [x.clone() for x in xs]
    abuf = [torch.empty_like(x) for x in xs]

    def reset():
        for hb, x in zip(hbuf, xs):
            hb.copy_(x)

    def attn_all(st):
        with torch.cuda.stream(st):
            for m in range(M):
                attn[m].forward(hbuf[m], abuf[m])

    def ffn_all(st):
        for m in range(M):
            ffn_layers[m].forward(abuf[m], out=hbuf[m], stream=st)

    whole = torch.cuda.Stream(device=dev)
    reset()
    t_a = stage_ms(lambda: attn_all(whole), reps)
    t_f = stage_ms(lambda: ffn_all(whole), reps)
    res = {"micro_batches": M, "layers": layers, "num_cus": num_cus,
           "t_attn_ms": t_a, "t_ffn_ms": t_f,
           "model_ms": afd_plan.pipeline_period(t_a, t_f), "period_ms": {}}
    finals = {}
    for p in placements:
        opened = []
        try:
            if p == "serial":
                streams = (whole, whole)
            elif p == "overlap":
                streams = (whole, torch.cuda.Stream(device=dev))
            elif p == "split":
                ab, fb = split_blocks(t_a, t_f, num_cus)
                sa = MaskedStream(ab, num_cus, dev.index or 0)
                opened.append(sa)
                sf = MaskedStream(fb, num_cus, dev.index or 0)
                opened.append(sf)
                streams = (sa.stream, sf.stream)
                reset()
                res["split"] = {"attn_cus": len(ab) * CU_BLOCK, "ffn_cus": len(fb) * CU_BLOCK,
                                "t_attn_ms": stage_ms(lambda: attn_all(sa.stream), reps),
                                "t_ffn_ms": stage_ms(lambda: ffn_all(sf.stream), reps)}
            else:
                raise ValueError(f"unknown placement {p!r}")
            ms = time_schedule(layers, attn, ffn_layers, hbuf, abuf, streams, reset)
            res["period_ms"][p] = ms / layers
            finals[p] = [hb.clone() for hb in hbuf]
        finally:
            for s in opened:
                s.close()
    ref = finals.get(placements[0])
    res["outputs_identical"] = all(
        all(torch.equal(a, b) for a, b in zip(ref, f)) for f in finals.values())
    res["finals"] = finals
    return res
