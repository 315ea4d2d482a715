"""Caller-side plumbing for one batched decode step: upload host arrays into a pool and device
buffers, then enqueue the library calls. Used by the tests, the smoke check and the bench.

Nothing here computes any part of attention: it copies arrays and calls the C ABI.
"""

from __future__ import annotations

import contextlib

import numpy as np
import torch

from . import binding as B


def on_stream(stream):
    """Context in which torch's allocations and fills are ordered on ``stream`` (None: the current
    stream), the stream the library calls of a runner are enqueued on."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def to_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Host storage array (np.float32, or np.uint16 bf16 bits) -> CPU tensor of the storage dtype."""
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False))
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)


def to_numpy(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device/CPU tensor of the storage dtype -> host storage array (bits preserved)."""
    t = t.detach().cpu().contiguous()
    if dtype == "f32":
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


class PagedStep:
    """One append-then-decode step over a paged pool.

    ``case`` provides (duck-typed): dtype, num_q_heads, num_kv_heads, head_dim, num_blocks,
    rope_theta, rope_max_pos, positions, dest, kv_lens, block_tables, k_pool, v_pool, k_new,
    v_new, q, scale. With a RoPE table the queries are rotated by the append into ``q_rot`` and the
    decode reads those; without one the decode reads ``q`` directly."""

    def __init__(self, case, device: str = "cuda", stream=None):
        self.case = case
        self.dtype = case.dtype
        self.device = device
        self.stream = stream
        desc = B.make_desc("paged", case.dtype, case.num_kv_heads, case.head_dim,
                           num_blocks=case.num_blocks, rope_max_pos=case.rope_max_pos,
                           rope_theta=case.rope_theta)
        self.kv = B.alloc_pool(desc, device=device, stream=stream)
        self.kv.k.copy_(to_torch(case.k_pool, case.dtype))
        self.kv.v.copy_(to_torch(case.v_pool, case.dtype))
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        self.block_tables = dev(case.block_tables.astype(np.int32))
        self.bt_stride = int(case.block_tables.shape[1])
        self.positions = dev(case.positions.astype(np.int32))
        self.dest = dev(case.dest.astype(np.int32))
        self.kv_lens = dev(case.kv_lens.astype(np.int32))
        self.k_new = to_torch(case.k_new, case.dtype).to(device)
        self.v_new = to_torch(case.v_new, case.dtype).to(device)
        self.q = to_torch(case.q, case.dtype).to(device)
        self.rope = case.rope_max_pos > 0
        self.q_rot = torch.empty_like(self.q) if self.rope else None
        self.batch = len(case.kv_lens)
        self.H_q = case.num_q_heads
        self.D = case.head_dim
        self.max_kv_len = int(case.kv_lens.max(initial=0))
        self.out = torch.empty((self.batch, self.H_q, self.D), dtype=torch.float32, device=device)
        self.lse = torch.empty((self.batch, self.H_q), dtype=torch.float32, device=device)
        need = B.pa_decode_attention(self.kv.pool, self.q, self.H_q * self.D, 1, self.H_q,
                                     self.block_tables, self.bt_stride, self.kv_lens, self.batch,
                                     self.max_kv_len, case.scale, out=self.out,
                                     query_workspace=True)
        # zero-filled once: its first bytes are the decode kernel's work counter; allocated and
        # filled on the calls' stream, so the fill is ordered before their first launch
        with on_stream(stream):
            self.workspace = (torch.zeros(need, dtype=torch.uint8, device=device) if need > 0
                              else None)

    @property
    def q_decode(self) -> torch.Tensor:
        return self.q_rot if self.rope else self.q

    def append(self):
        B.pa_append_kv(self.kv.pool, self.block_tables, self.bt_stride, self.positions, self.dest,
                       self.k_new, self.v_new, self.q if self.rope else None,
                       self.q_rot, self.H_q if self.rope else 0, self.batch, stream=self.stream)

    def decode(self, with_lse: bool = True):
        B.pa_decode_attention(self.kv.pool, self.q_decode, self.H_q * self.D, 1, self.H_q,
                              self.block_tables, self.bt_stride, self.kv_lens, self.batch,
                              self.max_kv_len, self.case.scale, workspace=self.workspace,
                              out=self.out, lse=self.lse if with_lse else None,
                              stream=self.stream)

    def step(self):
        self.append()
        self.decode()

    def fused_step(self, with_lse: bool = True):
        """append + decode in one call (pa_append_decode_attention): the same results as step()."""
        B.pa_append_decode_attention(self.kv.pool, self.block_tables, self.bt_stride,
                                     self.positions, self.dest, self.k_new, self.v_new, self.q,
                                     self.q_rot, self.H_q, self.kv_lens, self.batch,
                                     self.max_kv_len, self.case.scale, workspace=self.workspace,
                                     out=self.out, lse=self.lse if with_lse else None,
                                     stream=self.stream)


class MultiQueryStep:
    """Multi-query paged attention: n_q shared queries per row over ragged per-row keys.

    ``case`` provides: dtype, num_heads (query heads), head_dim, n_q, num_blocks, kv_lens,
    block_tables, k_pool and v_pool ([num_blocks][H_kv][16][dh]: the pool's head count is taken from
    them), q ([n_q][H][dh], shared by all rows), scale."""

    def __init__(self, case, device: str = "cuda", stream=None):
        self.case = case
        self.stream = stream
        desc = B.make_desc("paged", case.dtype, int(case.k_pool.shape[1]), case.head_dim,
                           num_blocks=case.num_blocks)
        self.kv = B.alloc_pool(desc, device=device, stream=stream)
        self.kv.k.copy_(to_torch(case.k_pool, case.dtype))
        self.kv.v.copy_(to_torch(case.v_pool, case.dtype))
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        self.block_tables = dev(case.block_tables.astype(np.int32))
        self.bt_stride = int(case.block_tables.shape[1])
        self.kv_lens = dev(case.kv_lens.astype(np.int32))
        self.q = to_torch(case.q, case.dtype).to(device)
        self.batch = len(case.kv_lens)
        self.max_kv_len = int(case.kv_lens.max(initial=0))
        shape = (self.batch, case.n_q, case.num_heads, case.head_dim)
        self.out = torch.empty(shape, dtype=torch.float32, device=device)
        self.lse = torch.empty(shape[:3], dtype=torch.float32, device=device)

    def decode(self, with_lse: bool = True):
        c = self.case
        B.pa_decode_attention(self.kv.pool, self.q, 0, c.n_q, c.num_heads, self.block_tables,
                              self.bt_stride, self.kv_lens, self.batch, self.max_kv_len, c.scale,
                              out=self.out, lse=self.lse if with_lse else None,
                              stream=self.stream)


class PaddedLockstep:
    """A right-padded lockstep batch: pool [batch_cap][H_kv][seq_cap][D] plus the calls on it.

    The caller fills ``kv.k``/``kv.v`` (torch views) and passes per-step device arrays."""

    def __init__(self, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 batch_cap: int, seq_cap: int, rope_theta: float = 0.0, rope_max_pos: int = 0,
                 device: str = "cuda", stream=None):
        self.dtype = dtype
        self.H_q, self.H_kv, self.D = num_q_heads, num_kv_heads, head_dim
        self.device = device
        self.stream = stream
        desc = B.make_desc("padded", dtype, num_kv_heads, head_dim, batch_cap=batch_cap,
                           seq_cap=seq_cap, rope_max_pos=rope_max_pos, rope_theta=rope_theta)
        self.kv = B.alloc_pool(desc, device=device, stream=stream)
        self.rope = rope_max_pos > 0
        self._ws = None
        self._ws_batch = None

    def append(self, positions, dest, k_new, v_new, q_in=None, q_out=None):
        B.pa_append_kv(self.kv.pool, None, 1, positions, dest, k_new, v_new, q_in, q_out,
                       self.H_q if q_in is not None else 0, positions.shape[0],
                       stream=self.stream)

    def _workspace_for(self, need: int, batch: int):
        # one workspace for every call: grown when too small, and zero-filled again when the
        # batch changes (its counters sit at offsets set by batch x heads). Allocation and fill
        # run on the calls' stream, so they are ordered after the previous call (whose last
        # workgroups re-arm the counters) and before the next one.
        with on_stream(self.stream):
            if need > 0 and (self._ws is None or self._ws.numel() < need):
                self._ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            elif need > 0 and self._ws_batch != batch:
                self._ws.zero_()
        if need > 0:
            self._ws_batch = batch

    def _outputs(self, batch: int):
        with on_stream(self.stream):
            out = torch.empty((batch, self.H_q, self.D), dtype=torch.float32, device=self.device)
            lse = torch.empty((batch, self.H_q), dtype=torch.float32, device=self.device)
        return out, lse

    def decode(self, q, gap_start, gap_end, kv_cols: int, scale: float):
        batch = q.shape[0]
        out, lse = self._outputs(batch)
        need = B.pa_decode_attention_padded(self.kv.pool, q, self.H_q, batch, gap_start, gap_end,
                                            kv_cols, scale, out=out, query_workspace=True)
        self._workspace_for(need, batch)
        B.pa_decode_attention_padded(self.kv.pool, q, self.H_q, batch, gap_start, gap_end, kv_cols,
                                     scale, workspace=self._ws if need > 0 else None, out=out,
                                     lse=lse, stream=self.stream)
        return out, lse

    def append_decode(self, positions, dest, k_new, v_new, q, q_out, gap_start, gap_end,
                      kv_cols: int, scale: float):
        """append + decode in one call (pa_append_decode_attention_padded): the same results as
        append() followed by decode() on the rotated queries."""
        batch = q.shape[0]
        out, lse = self._outputs(batch)
        need = B.pa_append_decode_attention_padded(self.kv.pool, positions, dest, k_new, v_new, q,
                                                   q_out, self.H_q, gap_start, gap_end, kv_cols,
                                                   batch, scale, out=out, query_workspace=True)
        self._workspace_for(need, batch)
        B.pa_append_decode_attention_padded(self.kv.pool, positions, dest, k_new, v_new, q, q_out,
                                            self.H_q, gap_start, gap_end, kv_cols, batch, scale,
                                            workspace=self._ws if need > 0 else None, out=out,
                                            lse=lse, stream=self.stream)
        return out, lse


class PagedLockstepGraph:
    """One paged lockstep decode step -- append at the rows' positions and decode over kv_lens in
    one pa_append_decode_attention call (+ the log-sum-exp merge), then pa_advance_lockstep
    (position += 1, kv_len = position + 1) --
    recorded once as a HIP graph and replayed per token ("NeuroGrid releases", v0.8.0: the decode
    step replayed as a graph, lengths and positions in device buffers).

    The caller writes each token's keys, values and queries into ``k_new``, ``v_new`` and ``q_in``
    (in place) and keeps ``block_tables`` filled for the positions ahead; ``max_kv_len`` is the
    host bound for every replay (it sizes the launch and the workspace). Run ``step()`` once
    before ``capture()`` so that every kernel has been loaded."""

    def __init__(self, pool, block_tables, positions, num_q_heads: int, max_kv_len: int,
                 scale: float, device: str = "cuda"):
        d = pool.pool.desc
        self.pool = pool
        self.H_q, self.H_kv, self.D = num_q_heads, d.num_kv_heads, d.head_dim
        self.dtype = "bf16" if d.dtype == B.PA_BF16 else "f32"
        tdt = torch.bfloat16 if d.dtype == B.PA_BF16 else torch.float32
        self.batch = int(positions.shape[0])
        self.block_tables = block_tables
        self.bt_stride = int(block_tables.shape[1])
        self.positions = positions
        self.kv_lens = (positions + 1).to(torch.int32)
        self.max_kv_len = int(max_kv_len)
        self.scale = float(scale)
        self.k_new = torch.zeros((self.batch, self.H_kv, self.D), dtype=tdt, device=device)
        self.v_new = torch.zeros_like(self.k_new)
        self.q_in = torch.zeros((self.batch, self.H_q, self.D), dtype=tdt, device=device)
        self.q_out = torch.zeros_like(self.q_in)
        self.out = torch.zeros((self.batch, self.H_q, self.D), dtype=torch.float32, device=device)
        self.lse = torch.zeros((self.batch, self.H_q), dtype=torch.float32, device=device)
        need = B.pa_decode_attention(pool.pool, self.q_out, self.H_q * self.D, 1, self.H_q,
                                     block_tables, self.bt_stride, self.kv_lens, self.batch,
                                     self.max_kv_len, self.scale, out=self.out,
                                     query_workspace=True)
        # zero-filled before first use (the work counter); every step leaves it at zero again
        self.workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=device)
        self._need = need
        self.graph = None

    def step(self):
        # append + decode in one call (the append folded into the decode launch), the merge, then
        # the add-one kernel
        rope = self.pool.pool.desc.rope_max_pos > 0
        B.pa_append_decode_attention(self.pool.pool, self.block_tables, self.bt_stride,
                                     self.positions, None, self.k_new, self.v_new, self.q_in,
                                     self.q_out if rope else None, self.H_q, self.kv_lens,
                                     self.batch, self.max_kv_len, self.scale,
                                     workspace=self.workspace if self._need else None,
                                     out=self.out, lse=self.lse)
        B.pa_advance_lockstep(self.positions, self.kv_lens, None, self.batch)

    def capture(self):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        self.graph = g

    def replay(self):
        self.graph.replay()
