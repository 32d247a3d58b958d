"""A greedy decode chain built only from the library's calls.

One step from token t (the chain has no other state):
  h = embed(head, t)                                   (tied embedding)
  per layer l:  u, us = rmsq(h, wn_l)
                a     = [gate_l; up_l] u               (one q4mv over both)
                m, ms = swq(a, inter)
                h     = h + down_l m                   (q4mv_add, in place)
  u, us = rmsq(h, wn_final);  logits = head u;  t' = argmax(logits)

Three ways to run it, with the same bits (and, in AttnDecodeChain below,
the same chain with an attention block in every layer):
  fused=False      the steps as listed: 1 + 4 per layer + 4 kernels
  fused=True       rmsq in the products' prologues, SwiGLU in the gate/up
                   product's epilogue (gate and up rows interleaved), the
                   down product forming its group sums, argmax's first half
                   in the head product's epilogue: 1 + 2 per layer + 2 kernels
  persistent=True  the embedding and every layer in one persistent kernel
                   (q4_decode_layers), then the fused head: 3 kernels
  one_launch=True  the whole step, the head and its argmax included, in one
                   persistent kernel (q4_decode_token)

The token lives on the device: argmax writes it where the next step's embed
reads it, so a step captured once as a graph can be replayed token after
token with a single host wait (for reading the token) per step.

This is the structure "Metal: queued rmsq, swq, gdn and atq kernels and a
4-row q4mv, so a decode token is one command buffer with one wait" (#1440)
describes for a whole decode token (Verification: one command buffer, one
wait), restricted to the products, norms and SwiGLU the chain uses.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (ATQ_D, BLOCK_MAX_LAYERS, BLOCK_MAX_POS, FIXED, AttnBlock, BlockStack, Graph,
               Mailbox, MlpLayer, Q4Matrix, q4_argmax, q4_argmax_ws_bytes, q4_atq,
               q4_atq_ws_bytes, q4_decode_block_ws_bytes, q4_decode_blocks, q4_decode_layers,
               q4_decode_token,
               q4_decode_layers_ws_bytes, q4_embed, q4_pos_advance, q4mv, q4mv_add,
               q4mv_argmax_ws_bytes, q4mv_norm, q4mv_norm_argmax, q4mv_norm_swiglu, rmsq, swq)


def _stack_rows(a: dict, b: dict) -> dict:
    """[a; b] as one matrix: rows of a, then rows of b (same cols)."""
    assert a["cols"] == b["cols"]
    return {"q": np.concatenate([a["q"], b["q"]]), "s": np.concatenate([a["s"], b["s"]]),
            "b": np.concatenate([a["b"], b["b"]]), "rows": a["rows"] + b["rows"],
            "cols": a["cols"]}


def _interleave_rows(a: dict, b: dict) -> dict:
    """Rows a0, b0, a1, b1, ... (same shape)."""
    assert a["cols"] == b["cols"] and a["rows"] == b["rows"]
    il = lambda x, y: np.stack([x, y], axis=1).reshape(2 * x.shape[0], *x.shape[1:])
    return {"q": il(a["q"], b["q"]), "s": il(a["s"], b["s"]), "b": il(a["b"], b["b"]),
            "rows": 2 * a["rows"], "cols": a["cols"]}


class DecodeChain:
    def __init__(self, weights: dict, mode: int = FIXED, layers: int | None = None,
                 device: str = "cuda", fused: bool = True, persistent: bool = False,
                 one_launch: bool = False):
        self.mode = mode
        self.persistent = persistent or one_launch
        self.one_launch = one_launch
        self.fused = fused or self.persistent
        self.hidden = int(weights["hidden"])
        self.inter = int(weights["inter"])
        self.vocab = int(weights["vocab"])
        self.eps = float(weights["eps"])
        L = len(weights["layers"]) if layers is None else layers
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        self.layers = []
        for lw in weights["layers"][:L]:
            gu = (_interleave_rows if self.fused else _stack_rows)(lw["gate"], lw["up"])
            self.layers.append({
                "wn": f32(lw["wn"]),
                "gu": Q4Matrix.from_host(gu, device),
                "down": Q4Matrix.from_host(lw["down"], device),
            })
        self.wn_final = f32(weights["wn_final"])
        self.head = Q4Matrix.from_host(weights["head"], device)
        z = lambda n, dt=torch.float32: torch.zeros(n, dtype=dt, device=device)
        self.tok = z(1, torch.int32)
        self.h = z(self.hidden)
        self.u = z(self.hidden)
        self.us = z(self.hidden // 64)
        self.a = z(2 * self.inter)
        self.m = z(self.inter)
        self.ms = z(self.inter // 64)
        self.logits = z(self.vocab)
        self.ws = z((q4_argmax_ws_bytes(self.vocab) + 7) // 8, torch.int64)
        self.amax_ws = z((q4mv_argmax_ws_bytes() + 7) // 8, torch.int64)
        self.mlp = [MlpLayer(lw["gu"], lw["down"], lw["wn"]) for lw in self.layers]
        self.stack_ws = z((q4_decode_layers_ws_bytes() + 7) // 8, torch.int64)
        self.graph = None
        self.mailbox = None
        # the copies and fills above ran on the current stream; the chain may
        # run on another one
        torch.cuda.synchronize()

    def kernels_per_token(self) -> int:
        if self.one_launch:
            return 1
        if self.persistent:
            return 3
        return 3 + 2 * len(self.layers) if self.fused else 5 + 4 * len(self.layers)

    def bytes_per_token(self) -> int:
        """Algorithmic bytes one step moves: weights and scales of every
        product (codes cols/2, s and b 8 per group per row), plus the small
        vectors each kernel reads and writes."""
        def prod(w):
            return w.rows * (w.cols // 2 + 8 * (w.cols // 64)) + 4 * (w.cols + w.cols // 64 + w.rows)
        total = prod(self.head) + self.hidden * 2 + 4 * self.vocab  # embed row, argmax read
        for lw in self.layers:
            total += prod(lw["gu"]) + prod(lw["down"]) + 4 * self.hidden  # residual read
            total += 4 * (3 * self.hidden + self.hidden // 64)             # rmsq
            total += 4 * (3 * self.inter + self.inter // 64)               # swq
        return total + 4 * (3 * self.hidden + self.hidden // 64)

    def enqueue_step(self, stream) -> None:
        """Every kernel of one step, in order, on `stream`."""
        if self.one_launch:
            q4_decode_token(self.head, self.tok, self.mlp, self.wn_final, self.eps, self.h,
                            self.logits, self.stack_ws, mode=self.mode, stream=stream)
            return
        if self.persistent:
            q4_decode_layers(self.head, self.tok, self.mlp, self.eps, self.h, self.stack_ws,
                             mode=self.mode, stream=stream)
            q4mv_norm_argmax(self.head, self.h, self.wn_final, self.eps, self.logits, self.tok,
                             self.amax_ws, mode=self.mode, stream=stream)
            return
        q4_embed(self.head, self.tok, self.h, stream=stream)
        if self.fused:
            for lw in self.layers:
                q4mv_norm_swiglu(lw["gu"], self.h, lw["wn"], self.eps, self.m, mode=self.mode,
                                 stream=stream)
                q4mv_add(lw["down"], self.m, None, self.h, self.h, mode=self.mode, stream=stream)
            q4mv_norm_argmax(self.head, self.h, self.wn_final, self.eps, self.logits, self.tok,
                             self.amax_ws, mode=self.mode, stream=stream)
            return
        for lw in self.layers:
            rmsq(self.h, lw["wn"], self.eps, self.u, self.us, stream=stream)
            q4mv(lw["gu"], self.u, self.us, self.a, mode=self.mode, stream=stream)
            swq(self.a, self.inter, self.m, self.ms, mode=self.mode, stream=stream)
            q4mv_add(lw["down"], self.m, self.ms, self.h, self.h, mode=self.mode, stream=stream)
        rmsq(self.h, self.wn_final, self.eps, self.u, self.us, stream=stream)
        q4mv(self.head, self.u, self.us, self.logits, mode=self.mode, stream=stream)
        q4_argmax(self.logits, self.tok, self.ws, stream=stream)

    def capture(self, stream: torch.cuda.Stream) -> Graph:
        """One step as a graph; it ends with a post of the new token to the
        chain's mailbox (the host can wait on that instead of the stream)."""
        if self.mailbox is None:
            self.mailbox = Mailbox(1)
        g = Graph(stream)
        g.begin()
        try:
            self.enqueue_step(stream)
            self.mailbox.post(self.tok, stream=stream)
        finally:
            g.end()
        self.graph = g
        return g

    def set_token(self, t: int) -> None:
        self.tok.fill_(int(t))

    def run(self, tok0: int, steps: int, stream: torch.cuda.Stream, use_graph: bool = True,
            on_step=None, wait: str = "stream") -> list:
        """Decodes `steps` tokens from `tok0`; returns them (host ints).
        One host wait per token, to read it: wait="stream" copies the token
        to pinned memory and synchronises the stream; wait="mailbox" (graph
        only) spins on the mailbox that the graph's last kernel fills.
        `on_step(i, chain)` runs after token i is known, e.g. to read the
        logits."""
        if use_graph and self.graph is None:
            self.capture(stream)
        if wait == "mailbox" and not use_graph:
            raise ValueError("the mailbox wait needs the captured graph")
        with torch.cuda.stream(stream):
            self.set_token(tok0)
        out = []
        pinned = torch.empty(1, dtype=torch.int32, pin_memory=True)
        if wait == "mailbox":
            stream.synchronize()  # earlier posts have all landed
        target = self.mailbox.seq if self.mailbox is not None else 0
        for i in range(steps):
            if use_graph:
                self.graph.launch(stream)
            else:
                self.enqueue_step(stream)
            if wait == "mailbox":
                target += 1
                out.append(self.mailbox.wait(target)[0])
            else:
                with torch.cuda.stream(stream):
                    pinned.copy_(self.tok, non_blocking=True)
                stream.synchronize()
                out.append(int(pinned[0]))
            if on_step is not None:
                stream.synchronize()
                on_step(i, self)
        if wait == "mailbox":
            stream.synchronize()
        return out


class AttnDecodeChain(DecodeChain):
    """The decode chain with an attention block in every layer, on the fused
    per-stage kernels.  One step from token t at position p:

      h = embed(head, t)
      per layer l:  [q; g; k; v] = qgkv_l rmsq(h, wa_l)     (q4mv_norm)
                    o, os = atq(q, g, k, v, ..., caches_l, p)  (q4_atq)
                    h = h + O_l o                            (q4mv_add)
                    m = swq([gate_l; up_l] rmsq(h, wn_l))    (q4mv_norm_swiglu)
                    h = h + down_l m                         (q4mv_add)
      t' = argmax(head rmsq(h, wn_final));  p = p + 1

    Token and position live on the device, so one captured step is
    replayed token after token; 4 + 5 per layer kernels.  The
    attention block is the product set's Q/K/V/O stages given their
    dataflow (the gate rows are an addition: the attention step gates its
    output).  persistent=True runs every layer in one persistent launch
    (q4_decode_blocks over stacks of at most 32 layers, caches of at most
    4096 positions): 5 kernels for up to 32 layers, the same bits."""

    def __init__(self, weights: dict, mode: int = FIXED, layers: int | None = None,
                 device: str = "cuda", persistent: bool = False):
        self.mode = mode
        self.persistent = persistent
        self.fused = True
        self.hidden = int(weights["hidden"])
        self.inter = int(weights["inter"])
        self.vocab = int(weights["vocab"])
        self.eps = float(weights["eps"])
        self.hq, self.hkv = int(weights["hq"]), int(weights["hkv"])
        self.max_pos = int(weights["max_pos"])
        L = len(weights["layers"]) if layers is None else layers
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        z = lambda *n, dt=torch.float32: torch.zeros(*n, dtype=dt, device=device)
        self.layers = []
        for lw in weights["layers"][:L]:
            self.layers.append({
                "wa": f32(lw["wa"]), "wq": f32(lw["wq"]), "wk": f32(lw["wk"]),
                "qgkv": Q4Matrix.from_host(lw["qgkv"], device),
                "o": Q4Matrix.from_host(lw["o"], device),
                "wn": f32(lw["wn"]),
                "gu": Q4Matrix.from_host(_interleave_rows(lw["gate"], lw["up"]), device),
                "down": Q4Matrix.from_host(lw["down"], device),
                "kc": z(self.hkv, self.max_pos, ATQ_D),
                "vc": z(self.hkv, self.max_pos, ATQ_D),
            })
        self.wn_final = f32(weights["wn_final"])
        self.head = Q4Matrix.from_host(weights["head"], device)
        self.cos_tab, self.sin_tab = f32(weights["cos_tab"]), f32(weights["sin_tab"])
        self.tok = z(1, dt=torch.int32)
        self.pos = z(1, dt=torch.int32)
        self.h = z(self.hidden)
        D = ATQ_D
        self.y = z((2 * self.hq + 2 * self.hkv) * D)
        hq, hkv = self.hq, self.hkv
        self.q, self.g = self.y[:hq * D], self.y[hq * D:2 * hq * D]
        self.k = self.y[2 * hq * D:2 * hq * D + hkv * D]
        self.v = self.y[2 * hq * D + hkv * D:]
        self.o = z(hq * D)
        self.os = z(hq * 2)
        self.m = z(self.inter)
        self.logits = z(self.vocab)
        self.amax_ws = z((q4mv_argmax_ws_bytes() + 7) // 8, dt=torch.int64)
        self.atq_ws = z((q4_atq_ws_bytes(hq, hkv) + 7) // 8, dt=torch.int64)
        if persistent:
            if self.max_pos > BLOCK_MAX_POS:
                raise ValueError("the persistent layers hold at most %d positions" % BLOCK_MAX_POS)
            for lw in self.layers:
                lw["blk"] = AttnBlock(lw["qgkv"], lw["o"], lw["wa"], lw["wq"], lw["wk"], lw["kc"],
                                      lw["vc"], MlpLayer(lw["gu"], lw["down"], lw["wn"]))
            blks = [lw["blk"] for lw in self.layers]
            self.stacks = [BlockStack(blks[i:i + BLOCK_MAX_LAYERS])
                           for i in range(0, len(blks), BLOCK_MAX_LAYERS)]
            self.block_ws = z((q4_decode_block_ws_bytes() + 7) // 8, dt=torch.int64)
        self.graph = None
        self.mailbox = None
        torch.cuda.synchronize()

    def kernels_per_token(self) -> int:
        # embed, the layers, the head and argmax's final kernel, the
        # position advance
        if self.persistent:
            return 4 + len(self.stacks)
        return 4 + 5 * len(self.layers)

    def bytes_per_token(self) -> int:
        """Algorithmic bytes at position 0: every product's weights and
        scales plus the small vectors (the caches grow by 2 rows per layer
        per token and are read once per step: 1 KiB per position and layer
        per key/value head, not counted here)."""
        def prod(w):
            return w.rows * (w.cols // 2 + 8 * (w.cols // 64)) + 4 * (w.cols + w.cols // 64 + w.rows)
        total = prod(self.head) + self.hidden * 2 + 4 * self.vocab
        for lw in self.layers:
            total += prod(lw["qgkv"]) + prod(lw["o"]) + prod(lw["gu"]) + prod(lw["down"])
            total += 8 * self.hidden + 4 * (3 * self.hidden)  # residual reads, norms
        return total

    def set_position(self, p: int, clear_caches: bool = True) -> None:
        """Position of the next step (caches cleared by default: a new
        sequence)."""
        self.pos.fill_(int(p))
        if clear_caches:
            for lw in self.layers:
                lw["kc"].zero_()
                lw["vc"].zero_()

    def enqueue_step(self, stream) -> None:
        q4_embed(self.head, self.tok, self.h, stream=stream)
        if self.persistent:
            for st in self.stacks:
                q4_decode_blocks(st, self.eps, self.h, self.pos, self.cos_tab, self.sin_tab,
                                 self.block_ws, mode=self.mode, stream=stream)
            q4mv_norm_argmax(self.head, self.h, self.wn_final, self.eps, self.logits, self.tok,
                             self.amax_ws, mode=self.mode, stream=stream)
            q4_pos_advance(self.pos, stream=stream)
            return
        for lw in self.layers:
            q4mv_norm(lw["qgkv"], self.h, lw["wa"], self.eps, self.y, mode=self.mode, stream=stream)
            q4_atq(self.q, self.g, self.k, self.v, lw["wq"], lw["wk"], self.eps, self.cos_tab,
                   self.sin_tab, lw["kc"], lw["vc"], self.pos, self.o, self.os, self.atq_ws,
                   stream=stream)
            q4mv_add(lw["o"], self.o, self.os, self.h, self.h, mode=self.mode, stream=stream)
            q4mv_norm_swiglu(lw["gu"], self.h, lw["wn"], self.eps, self.m, mode=self.mode,
                             stream=stream)
            q4mv_add(lw["down"], self.m, None, self.h, self.h, mode=self.mode, stream=stream)
        q4mv_norm_argmax(self.head, self.h, self.wn_final, self.eps, self.logits, self.tok,
                         self.amax_ws, mode=self.mode, stream=stream)
        q4_pos_advance(self.pos, stream=stream)

    def run(self, tok0: int, steps: int, stream: torch.cuda.Stream, use_graph: bool = True,
            on_step=None, wait: str = "stream", pos0: int = 0) -> list:
        """As DecodeChain.run, from position `pos0` with empty caches."""
        if pos0 + steps > self.max_pos:
            raise ValueError("the caches hold %d positions" % self.max_pos)
        with torch.cuda.stream(stream):
            self.set_position(pos0)
        return super().run(tok0, steps, stream, use_graph=use_graph, on_step=on_step, wait=wait)
