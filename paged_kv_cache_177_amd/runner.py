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
    """Paged lockstep decode steps recorded as a HIP graph and replayed ("NeuroGrid releases",
    v0.8.0: the decode step replayed as a graph, lengths and positions in device buffers,
    kv_len = position + 1 on the GPU).

    A token is one pa_lockstep_decode_step call: the append at the rows' positions, the decode over
    position + 1 tokens (merging its own splits) and the next positions, in one launch. The
    positions alternate between two device buffers (token i reads ``pos[i % 2]`` and writes the
    other); with an odd count of tokens per graph a copy brings them back to ``pos[0]`` at the end.
    With ``one_launch=False`` a token is pa_append_decode_attention followed by the add-one kernel
    (pa_advance_lockstep) on one buffer, the two-kernel form.

    One graph holds ``tokens`` consecutive tokens: token i reads its keys, values and queries from
    ``k_new[i]``, ``v_new[i]`` and ``q_in[i]`` and writes ``out[i]``/``lse[i]`` (its rotated queries
    to ``q_out[i]``), so a replay advances every row by ``tokens`` tokens with one launch from the
    host. The caller writes the inputs in place before a replay and keeps ``block_tables`` filled
    for the positions ahead; ``max_kv_len`` is the host bound for every step (it sizes the launch
    and the workspace). Run ``step()`` once before ``capture()`` so that every kernel has been
    loaded."""

    def __init__(self, pool, block_tables, positions, num_q_heads: int, max_kv_len: int,
                 scale: float, device: str = "cuda", tokens: int = 1, one_launch: bool = True):
        d = pool.pool.desc
        self.pool = pool
        self.H_q, self.H_kv, self.D = num_q_heads, d.num_kv_heads, d.head_dim
        self.dtype = "bf16" if d.dtype == B.PA_BF16 else "f32"
        tdt = torch.bfloat16 if d.dtype == B.PA_BF16 else torch.float32
        self.tokens = int(tokens)
        self.one_launch = bool(one_launch)
        self.batch = int(positions.shape[0])
        self.block_tables = block_tables
        self.bt_stride = int(block_tables.shape[1])
        # pos[0] holds the positions between replays; pos[1] is the other buffer of the pair
        self.pos = torch.stack([positions.to(torch.int32), positions.to(torch.int32)]).to(device)
        self.kv_lens = (positions + 1).to(torch.int32).to(device)  # two-kernel form only
        self.max_kv_len = int(max_kv_len)
        self.scale = float(scale)
        T, Bt = self.tokens, self.batch
        self.k_new = torch.zeros((T, Bt, self.H_kv, self.D), dtype=tdt, device=device)
        self.v_new = torch.zeros_like(self.k_new)
        self.q_in = torch.zeros((T, Bt, self.H_q, self.D), dtype=tdt, device=device)
        self.q_out = torch.zeros_like(self.q_in)
        self.out = torch.zeros((T, Bt, self.H_q, self.D), dtype=torch.float32, device=device)
        self.lse = torch.zeros((T, Bt, self.H_q), dtype=torch.float32, device=device)
        need = B.pa_decode_attention(pool.pool, self.q_out[0], self.H_q * self.D, 1, self.H_q,
                                     block_tables, self.bt_stride, self.kv_lens, self.batch,
                                     self.max_kv_len, self.scale, out=self.out[0],
                                     query_workspace=True)
        # zero-filled before first use (the work counter); every step leaves it at zero again
        self.workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=device)
        self._need = need
        self.graph = None

    @property
    def positions(self) -> torch.Tensor:
        """The rows' positions between replays (the next token's)."""
        return self.pos[0]

    def set_positions(self, positions: torch.Tensor):
        self.pos[0].copy_(positions)
        self.kv_lens.copy_(positions + 1)

    def token(self, i: int):
        """Token i of a replay."""
        rope = self.pool.pool.desc.rope_max_pos > 0
        ws = self.workspace if self._need else None
        q_out = self.q_out[i] if rope else None
        if self.one_launch:
            B.pa_lockstep_decode_step(self.pool.pool, self.block_tables, self.bt_stride,
                                      self.pos[i % 2], self.pos[(i + 1) % 2], self.k_new[i],
                                      self.v_new[i], self.q_in[i], q_out, self.H_q, self.batch,
                                      self.max_kv_len, self.scale, workspace=ws, out=self.out[i],
                                      lse=self.lse[i])
        else:
            B.pa_append_decode_attention(self.pool.pool, self.block_tables, self.bt_stride,
                                         self.pos[0], None, self.k_new[i], self.v_new[i],
                                         self.q_in[i], q_out, self.H_q, self.kv_lens,
                                         self.batch, self.max_kv_len, self.scale, workspace=ws,
                                         out=self.out[i], lse=self.lse[i])
            B.pa_advance_lockstep(self.pos[0], self.kv_lens, None, self.batch)

    def step(self):
        """The graph's work issued eagerly: every token in turn."""
        for i in range(self.tokens):
            self.token(i)
        if self.one_launch and self.tokens % 2 == 1:
            self.pos[0].copy_(self.pos[1])

    def capture(self):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        self.graph = g

    def replay(self):
        self.graph.replay()
