"""Decode-loop driver of the compression step: append one row per step, compress
when the buffer is full.

The pages describe R-KV as compressing periodically during decoding with a
fixed buffer on top of the budget ("R-KV: Redundancy-aware KV Cache
Compression for Reasoning Models", atlas.scime.ai summary, "Approach"), with
the knobs kv_budget, window_size, mix_lambda, divide_method and
divide_length, step_length / 128 in the example ("R-KV: decoding-time KV
cache compression for reasoning models", hysenlabs page, "What the redundancy
scoring actually does at decode time"), and compression switched off when
the budget or the buffer is zero (same page, "Three install paths with
different levels of commitment"). Reading used here: every unit's cache holds
at most kv_budget + divide_length rows; when an append makes it full, the
step compresses it back to kv_budget rows, so events fall every
divide_length steps once the first kv_budget + divide_length rows exist.

Dense layout: each unit's rows live in a [units, kv_budget + divide_length,
128] buffer; compression writes the kept rows into a second buffer of the
same shape (the kernels work out of place) and the two swap. The window
queries are a ring of the last window_size query rows of each query head,
put in time order for each event. All units advance together (one row per
unit per step), as in batched decoding of equal-length sequences.

Every step of the compression itself runs in the HIP library (rkv_compress);
this driver only moves rows into place and decides when to call it.

With ``use_graph`` the compression call is captured once per ping-pong
parity into a HIP graph (through torch.cuda.CUDAGraph) and replayed at every
later event, the analogue of the piecewise CUDA-graph capture the pages
mention for the serving port ("R-KV: decoding-time KV cache compression for
reasoning models", hysenlabs page, "Three install paths with different levels
of commitment"). The window queries are first copied, in time order, into a
fixed buffer outside the graph, since their ring position moves between
events; every other argument of the call is a fixed buffer already. The
library issues no memset or host copy on the dense path, so the captured
launches are the whole call.
"""
from __future__ import annotations

from . import HEAD_DIM, compress, workspace_size


class DecodeLoop:
    def __init__(self, units: int, gqa_group: int, kv_budget: int = 1024, window_size: int = 8,
                 divide_length: int = 128, mix_lambda: float = 0.1, dtype=None, device="cuda",
                 capacity: int = 0, use_graph: bool = False):
        import torch
        self.units, self.gqa, self.budget, self.window = units, gqa_group, kv_budget, window_size
        self.divide_length, self.lam = divide_length, mix_lambda
        self.active = kv_budget > 0 and divide_length > 0
        if self.active and kv_budget <= window_size:
            raise ValueError("kv_budget must exceed window_size")
        cap = kv_budget + divide_length if self.active else capacity
        if cap <= 0:
            raise ValueError("compression is off (kv_budget or divide_length is 0): give a capacity")
        self.capacity = cap
        dt = torch.bfloat16 if dtype is None else dtype
        shape = (units, cap, HEAD_DIM)
        self._K = [torch.zeros(shape, dtype=dt, device=device) for _ in range(2)]
        self._V = [torch.zeros(shape, dtype=dt, device=device) for _ in range(2)]
        self._cur = 0
        self._q = torch.zeros((units, gqa_group, window_size, HEAD_DIM), dtype=dt, device=device)
        self._qpos = 0                     # ring slot of the next query row
        self.length = 0                    # rows held per unit
        self.step_count = 0
        self.events = 0
        if self.active:
            self._kept = torch.empty((units, kv_budget), dtype=torch.int32, device=device)
            dname = "bf16" if dt == torch.bfloat16 else "f32"
            nbytes = workspace_size(units, cap, gqa_group, window_size, kv_budget, dname)
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.use_graph = bool(use_graph) and self.active
        self._qbuf = torch.zeros_like(self._q) if self.use_graph else None
        self._graphs = [None, None]        # captured compression per parity
        self.on_event = None               # callback(loop) before each compression

    @property
    def K(self):
        """Rows held per unit: [units, length, 128] (a view)."""
        return self._K[self._cur][:, :self.length]

    @property
    def V(self):
        return self._V[self._cur][:, :self.length]

    def window_queries(self):
        """The last window_size query rows of each query head in time order:
        [units, G, w, 128] (contiguous)."""
        import torch
        return torch.roll(self._q, shifts=-self._qpos, dims=2).contiguous()

    def append(self, k, v, q) -> bool:
        """Append step rows k, v [units, 128] and q [units, G, 128]. Returns
        True when this step compressed the cache."""
        if self.length >= self.capacity:
            raise RuntimeError("cache full and compression is off")
        self._K[self._cur][:, self.length] = k
        self._V[self._cur][:, self.length] = v
        self._q[:, :, self._qpos] = q
        self._qpos = (self._qpos + 1) % self.window
        self.length += 1
        self.step_count += 1
        if self.active and self.length == self.capacity:
            self.compress()
            return True
        return False

    def _compress_call(self, cur: int, q):
        nxt = 1 - cur
        compress(self._K[cur][:, :self.capacity], self._V[cur][:, :self.capacity], q,
                 self.budget, self.window, self.lam,
                 K_out=self._K[nxt][:, :self.budget], V_out=self._V[nxt][:, :self.budget],
                 kept_idx=self._kept, workspace=self._ws)

    def _compress_graphed(self, cur: int):
        import torch
        self._qbuf.copy_(self.window_queries())
        g = self._graphs[cur]
        if g is None:
            # one eager call on a side stream first, as capture requires
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self._compress_call(cur, self._qbuf)
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._compress_call(cur, self._qbuf)
            self._graphs[cur] = g
        g.replay()

    def compress(self):
        """Compress every unit from `length` rows to kv_budget rows."""
        if self.on_event is not None:
            self.on_event(self)
        if self.length != self.capacity:
            raise RuntimeError("compression runs on a full buffer")
        if self.use_graph:
            self._compress_graphed(self._cur)
        else:
            self._compress_call(self._cur, self.window_queries())
        self._cur = 1 - self._cur
        self.length = self.budget
        self.events += 1

    @property
    def last_kept(self):
        """Kept indices of the last event: int32 [units, kv_budget]."""
        return self._kept
