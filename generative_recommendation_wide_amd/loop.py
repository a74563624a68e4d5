"""Device-resident multi-step decode loop (xLLM generative-recommendation design doc,
section 3.2: fixed-step execution prepares every step's buffers up front and keeps the
rounds on the device with no per-step device-to-host round trip; section 6: each round
runs the forward, the beam search and the next round's input preparation on the device).

Per step d: beam_select picks the new beams (their parents become row d of parent_idx),
then beam_attn_decode runs once per layer at depth d.  Beam state ping-pongs between two
preallocated buffers; nothing in run() synchronises with the host.  grw_backtrack turns
(token, parent) rows into the final semantic-ID tuples.
"""
from __future__ import annotations

import torch


class DecodeLoop:
    def __init__(self, ws, S: int, C: int, trie=None, device="cuda", overlap: bool = False, fanout: bool = False):
        """ws: a bound Workspace; trie: (row_ptr, code, n_internal) device tensors, optionally
        followed by (dense_slot, dense_mask) for nodes with dense child masks, or None;
        overlap: run each layer's unshared stage on a side stream beside its shared stage
        (beam_attn_decode_overlap) instead of the fused unshared + merge kernel; fanout: the
        first step expands each request's prompt beam to its best W children (first-step
        fan-out) instead of top_k."""
        from . import _lib  # noqa: F401  (the library must be loaded)
        self.ws, self.S, self.C = ws, S, C
        sumW = ws.sumW
        self.W = max(ws.W)
        self.K = max(ws.K)
        self.trie = trie
        dev = torch.device(device)
        self.scores = torch.empty(2, sumW, dtype=torch.float32, device=dev)
        self.nodes = torch.empty(2, sumW, dtype=torch.int32, device=dev)
        self.tokens = torch.empty(S, sumW, dtype=torch.int32, device=dev)
        self.parents = torch.empty(S, sumW, dtype=torch.int32, device=dev)   # parent_idx
        self.sid = torch.empty(sumW, S, dtype=torch.int32, device=dev)
        self.side_stream = torch.cuda.Stream(device=dev) if overlap else None
        self.fanout = fanout

    def select_step(self, d: int, logprobs, stream=None, noise=None, temperature: float = 0.0,
                    raw_logits: bool = False):
        """Selection at depth d; with noise, the Gumbel top-k at the given temperature; with
        raw_logits, `logprobs` holds raw logits and the row log-softmax is fused in.  A trie
        with dense child masks (five-tuple) goes through beam_select_ex."""
        from . import beam_select, beam_select_ex, beam_select_gumbel, beam_select_logits
        cur, nxt = d % 2, (d + 1) % 2
        fan = self.fanout and d == 0
        if fan or (self.trie is not None and len(self.trie) > 3):
            beam_select_ex(self.ws, logprobs, self.scores[cur], self.nodes[cur], self.trie, self.W, self.K, self.C,
                           self.tokens[d], self.parents[d], self.scores[nxt], self.nodes[nxt], noise, temperature,
                           raw_logits, stream, fan)
            return
        row_ptr, code, n_int = self.trie if self.trie is not None else (None, None, 0)
        if raw_logits:
            beam_select_logits(self.ws, logprobs, noise, temperature, self.scores[cur], self.nodes[cur],
                               row_ptr, code, n_int, self.W, self.K, self.C, self.tokens[d], self.parents[d],
                               self.scores[nxt], self.nodes[nxt], stream)
        elif noise is None:
            beam_select(self.ws, logprobs, self.scores[cur], self.nodes[cur], row_ptr, code, n_int,
                        self.W, self.K, self.C, self.tokens[d], self.parents[d], self.scores[nxt],
                        self.nodes[nxt], stream)
        else:
            beam_select_gumbel(self.ws, logprobs, noise, temperature, self.scores[cur], self.nodes[cur],
                               row_ptr, code, n_int, self.W, self.K, self.C, self.tokens[d], self.parents[d],
                               self.scores[nxt], self.nodes[nxt], stream)

    def attn_step(self, d: int, layer, out, stream=None):
        from . import beam_attn_decode, beam_attn_decode_overlap
        args = (self.ws, layer["q"][d], layer["k_s"], layer["v_s"], layer.get("k_scale"), layer.get("v_scale"),
                layer["k_u"], layer["v_u"], self.parents, d, out)
        if self.side_stream is not None:
            beam_attn_decode_overlap(*args, self.side_stream, stream)
        else:
            beam_attn_decode(*args, stream)

    def run(self, logprobs, layers, out, stream=None, steps=None, noise=None, temperature: float = 0.0,
            raw_logits: bool = False):
        """logprobs: sequence of S device tensors [sumW][C]; layers: sequence of dicts with
        q [S][sumW][Hq][D], k_s, v_s, k_scale, v_scale, k_u, v_u (device tensors);
        out: [sumW][Hq][D] float32 device tensor, or a list with one per layer;
        noise: None, or a sequence of S device tensors [sumW][C] of Gumbel draws for the
        sampled selection at the given temperature; raw_logits: logprobs holds raw logits
        and the selection fuses their log-softmax."""
        from . import grw_backtrack
        steps = self.S if steps is None else steps
        self.ws.beams_init(self.scores[0], self.nodes[0], stream)
        for d in range(steps):
            self.select_step(d, logprobs[d], stream, None if noise is None else noise[d], temperature, raw_logits)
            for li, layer in enumerate(layers):
                self.attn_step(d, layer, out[li] if isinstance(out, (list, tuple)) else out, stream)
        if steps == self.S:
            grw_backtrack(self.ws, self.tokens, self.parents, self.S, self.sid, stream)

    def capture(self, logprobs, layers, out, steps=None):
        """Record run() as one HIP graph (xLLM design doc, section 3.2, and the FlashRec
        announcement: the decode steps as one captured graph, with no host work between
        kernels).  Every kernel of the loop reads and writes preallocated buffers and the
        library records no memset, so replaying the graph repeats run() exactly.  One eager
        run first performs the library's one-time set-up outside the capture.  Returns the
        torch.cuda.CUDAGraph; call .replay() on it."""
        self.run(logprobs, layers, out, steps=steps)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(logprobs, layers, out, steps=steps)
        return graph

    def final_scores(self):
        return self.scores[self.S % 2]

    def final_nodes(self):
        return self.nodes[self.S % 2]
