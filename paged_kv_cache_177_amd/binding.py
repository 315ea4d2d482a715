"""ctypes binding of libpa.so: the four C calls under the same names, plus a small pool wrapper.

Argument marshalling only -- every step of the path runs in the library's kernels. Device memory
and streams come from PyTorch: tensors are passed as ``data_ptr()`` and the stream as
``torch.cuda.current_stream().cuda_stream`` (on ROCm, torch's ``cuda`` namespace is HIP).
The library must be built (``python -m paged_kv_cache_177_amd.build``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import LIB

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_CAPACITY, PA_ERR_HIP = range(6)
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
                4: "PA_ERR_CAPACITY", 5: "PA_ERR_HIP"}
PA_F32, PA_BF16 = 0, 1
PA_PAGED, PA_PADDED = 0, 1

EXPORTS = ("pa_alloc_pool", "pa_append_kv", "pa_decode_attention", "pa_decode_attention_padded",
           "pa_decode_attention_block_sparse", "pa_advance_lockstep", "pa_append_kv_qk_norm",
           "pa_tokenize_kv", "pa_pack_projection", "pa_append_decode_attention",
           "pa_append_decode_attention_padded", "pa_lse_merge", "pa_decode_attention_noalloc",
           "pa_lockstep_decode_step")
NOALLOC_SCRATCH_BYTES = 16 << 20
NOALLOC_MAX_ROW_HEADS = 16384


class PaError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} returned {STATUS_NAMES.get(status, status)}")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("batch_cap", ctypes.c_int32), ("seq_cap", ctypes.c_int32),
                ("rope_max_pos", ctypes.c_int32), ("rope_theta", ctypes.c_double)]


class Pool(ctypes.Structure):
    _fields_ = [("desc", PoolDesc), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p),
                ("bytes", ctypes.c_size_t)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIZE_P = ctypes.POINTER(ctypes.c_size_t)
_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libpa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python -m paged_kv_cache_177_amd.build`")
    lib = ctypes.CDLL(path)
    lib.pa_alloc_pool.argtypes = [ctypes.POINTER(PoolDesc), _P, ctypes.c_size_t, _SIZE_P,
                                  ctypes.POINTER(Pool), _P]
    lib.pa_append_kv.argtypes = [ctypes.POINTER(Pool), _P, _I32, _P, _P, _P, _P, _P, _P, _I32,
                                 _I32, _P]
    lib.pa_decode_attention.argtypes = [ctypes.POINTER(Pool), _P, ctypes.c_int64, _I32, _I32, _P,
                                        _I32, _P, _I32, _I32, ctypes.c_float, _P, ctypes.c_size_t,
                                        _SIZE_P, _P, _P, _P]
    lib.pa_decode_attention_padded.argtypes = [ctypes.POINTER(Pool), _P, _I32, _I32, _P, _P, _I32,
                                               ctypes.c_float, _P, ctypes.c_size_t, _SIZE_P, _P,
                                               _P, _P]
    lib.pa_decode_attention_block_sparse.argtypes = [ctypes.POINTER(Pool), _P, ctypes.c_int64,
                                                     _I32, _I32, _P, _I32, _P, _I32, _I32,
                                                     ctypes.c_float, _P, _I32, _P, _P, _P]
    lib.pa_advance_lockstep.argtypes = [_P, _P, _P, _I32, _P]
    lib.pa_tokenize_kv.argtypes = [ctypes.POINTER(Pool), _P, _I32, _P, _I32, _P, _I32, _I32, _P,
                                   _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _P]
    lib.pa_pack_projection.argtypes = [_P, _I32, _I32, _P, _P]
    lib.pa_append_kv_qk_norm.argtypes = [ctypes.POINTER(Pool), _P, _I32, _P, _P, _P, _P, _P, _P,
                                         _I32, _I32, _P, _P, ctypes.c_float, _P]
    lib.pa_append_decode_attention.argtypes = [ctypes.POINTER(Pool), _P, _I32, _P, _P, _P, _P,
                                               _P, _P, _I32, _P, _I32, _I32, ctypes.c_float, _P,
                                               ctypes.c_size_t, _SIZE_P, _P, _P, _P]
    lib.pa_append_decode_attention_padded.argtypes = [ctypes.POINTER(Pool), _P, _P, _P, _P, _P,
                                                      _P, _I32, _P, _P, _I32, _I32,
                                                      ctypes.c_float, _P, ctypes.c_size_t,
                                                      _SIZE_P, _P, _P, _P]
    lib.pa_lse_merge.argtypes = [_P, _P, _I32, ctypes.c_int64, _I32, _P, _P, _P]
    lib.pa_lockstep_decode_step.argtypes = [ctypes.POINTER(Pool), _P, _I32, _P, _P, _P, _P, _P,
                                            _P, _I32, _I32, _I32, ctypes.c_float, _P,
                                            ctypes.c_size_t, _SIZE_P, _P, _P, _P]
    lib.pa_decode_attention_noalloc.argtypes = [ctypes.POINTER(Pool), _P, ctypes.c_int64, _I32,
                                                _I32, _P, _I32, _P, _I32, _I32, ctypes.c_float,
                                                _P, _P, _P]
    for name in EXPORTS:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(call: str, status: int) -> None:
    if status != PA_OK:
        raise PaError(call, status)


# ------------------------------------------------------------------------------------------
# The four calls (raw: pointers as tensors or ints, status raised as PaError)
# ------------------------------------------------------------------------------------------
def pa_alloc_pool(desc: PoolDesc, dev_buf=None, stream=None) -> tuple[int, Pool | None]:
    """Size query (dev_buf None) -> (bytes, None); else carve ``dev_buf`` -> (bytes, Pool)."""
    lib = load_library()
    need = ctypes.c_size_t(0)
    if dev_buf is None:
        _check("pa_alloc_pool", lib.pa_alloc_pool(ctypes.byref(desc), None, 0,
                                                   ctypes.byref(need), None, None))
        return need.value, None
    pool = Pool()
    nbytes = dev_buf.numel() * dev_buf.element_size()
    _check("pa_alloc_pool", lib.pa_alloc_pool(ctypes.byref(desc), _ptr(dev_buf), nbytes,
                                               ctypes.byref(need), ctypes.byref(pool),
                                               _stream(stream)))
    return need.value, pool


def pa_append_kv(pool: Pool, block_tables, bt_stride: int, positions, dest, k_new, v_new,
                 q_in=None, q_out=None, num_q_heads: int = 0, batch: int | None = None,
                 stream=None) -> None:
    lib = load_library()
    if batch is None:
        batch = positions.shape[0]
    _check("pa_append_kv", lib.pa_append_kv(ctypes.byref(pool), _ptr(block_tables), bt_stride,
                                             _ptr(positions), _ptr(dest), _ptr(k_new),
                                             _ptr(v_new), _ptr(q_in), _ptr(q_out), num_q_heads,
                                             batch, _stream(stream)))


def pa_decode_attention(pool: Pool, q, q_row_stride: int, n_q: int, num_q_heads: int,
                        block_tables, bt_stride: int, kv_lens, batch: int, max_kv_len: int,
                        scale: float, workspace=None, out=None, lse=None, stream=None,
                        query_workspace: bool = False) -> int:
    """Enqueue the decode; with ``query_workspace`` only return the workspace bytes needed."""
    lib = load_library()
    need = ctypes.c_size_t(0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode_attention(ctypes.byref(pool), _ptr(q), q_row_stride, n_q, num_q_heads,
                                 _ptr(block_tables), bt_stride, _ptr(kv_lens), batch, max_kv_len,
                                 ctypes.c_float(scale), _ptr(workspace), ws_bytes,
                                 ctypes.byref(need) if query_workspace else None, _ptr(out),
                                 _ptr(lse), _stream(stream))
    _check("pa_decode_attention", st)
    return need.value


def pa_decode_attention_noalloc(pool: Pool, q, q_row_stride: int, n_q: int, num_q_heads: int,
                                block_tables, bt_stride: int, kv_lens, batch: int,
                                max_kv_len: int, scale: float, out=None, lse=None,
                                stream=None) -> None:
    """Enqueue the decode on the library's own per-device scratch (no workspace argument)."""
    lib = load_library()
    st = lib.pa_decode_attention_noalloc(ctypes.byref(pool), _ptr(q), q_row_stride, n_q,
                                         num_q_heads, _ptr(block_tables), bt_stride,
                                         _ptr(kv_lens), batch, max_kv_len, ctypes.c_float(scale),
                                         _ptr(out), _ptr(lse), _stream(stream))
    _check("pa_decode_attention_noalloc", st)


def pa_decode_attention_block_sparse(pool: Pool, q, q_row_stride: int, n_q: int,
                                     num_q_heads: int, block_tables, bt_stride: int, kv_lens,
                                     batch: int, max_kv_len: int, scale: float, block_mask,
                                     mask_kv_blocks: int, out=None, lse=None, stream=None) -> None:
    """Enqueue the block-sparse multi-query decode (block_mask: uint8 device
    [batch][ceil(n_q / 16)][mask_kv_blocks])."""
    lib = load_library()
    st = lib.pa_decode_attention_block_sparse(ctypes.byref(pool), _ptr(q), q_row_stride, n_q,
                                              num_q_heads, _ptr(block_tables), bt_stride,
                                              _ptr(kv_lens), batch, max_kv_len,
                                              ctypes.c_float(scale), _ptr(block_mask),
                                              mask_kv_blocks, _ptr(out), _ptr(lse),
                                              _stream(stream))
    _check("pa_decode_attention_block_sparse", st)


def pa_append_kv_qk_norm(pool: Pool, block_tables, bt_stride: int, positions, dest, k_new,
                         v_new, q_in, q_out, num_q_heads: int, batch: int, q_norm_weight,
                         k_norm_weight, eps: float, stream=None) -> None:
    lib = load_library()
    st = lib.pa_append_kv_qk_norm(ctypes.byref(pool), _ptr(block_tables), bt_stride,
                                  _ptr(positions), _ptr(dest), _ptr(k_new), _ptr(v_new),
                                  _ptr(q_in), _ptr(q_out), num_q_heads, batch,
                                  _ptr(q_norm_weight), _ptr(k_norm_weight), ctypes.c_float(eps),
                                  _stream(stream))
    _check("pa_append_kv_qk_norm", st)


def pa_pack_projection(w, packed=None, stream=None):
    """Pack a bf16 [out_features][in_features] weight into matrix-core fragment order (a new
    tensor of the same size unless ``packed`` is given); returns the packed tensor."""
    import torch

    lib = load_library()
    if packed is None:
        packed = torch.empty_like(w)
    st = lib.pa_pack_projection(_ptr(w), w.shape[0], w.shape[1], _ptr(packed), _stream(stream))
    _check("pa_pack_projection", st)
    return packed


def pa_tokenize_kv(pool: Pool, neuron_table, time_table, value_table, w_k_packed, w_v_packed,
                   offsets, neuron_ids, time_bins, value_ids, block_tables, bt_stride: int,
                   batch: int, max_events: int, stream=None) -> None:
    """Tables: fp32 [rows][model_dim] tensors; w_k_packed/w_v_packed: the bf16 [H * dh][model_dim]
    weights after pa_pack_projection."""
    lib = load_library()
    st = lib.pa_tokenize_kv(ctypes.byref(pool), _ptr(neuron_table), neuron_table.shape[0],
                            _ptr(time_table), time_table.shape[0], _ptr(value_table),
                            value_table.shape[0], neuron_table.shape[1], _ptr(w_k_packed),
                            _ptr(w_v_packed),
                            _ptr(offsets), _ptr(neuron_ids), _ptr(time_bins), _ptr(value_ids),
                            neuron_ids.shape[0], _ptr(block_tables), bt_stride, batch, max_events,
                            _stream(stream))
    _check("pa_tokenize_kv", st)


def pa_advance_lockstep(positions, kv_lens=None, dest=None, batch: int | None = None,
                        stream=None) -> None:
    """Enqueue positions += 1, kv_lens = positions + 1, dest += 1 (int32 device tensors)."""
    lib = load_library()
    n = positions.shape[0] if batch is None else batch
    st = lib.pa_advance_lockstep(_ptr(positions), _ptr(kv_lens), _ptr(dest), n, _stream(stream))
    _check("pa_advance_lockstep", st)


def pa_decode_attention_padded(pool: Pool, q, num_q_heads: int, batch: int, gap_start, gap_end,
                               kv_cols: int, scale: float, workspace=None, out=None, lse=None,
                               stream=None, query_workspace: bool = False) -> int:
    lib = load_library()
    need = ctypes.c_size_t(0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_decode_attention_padded(ctypes.byref(pool), _ptr(q), num_q_heads, batch,
                                        _ptr(gap_start), _ptr(gap_end), kv_cols,
                                        ctypes.c_float(scale), _ptr(workspace), ws_bytes,
                                        ctypes.byref(need) if query_workspace else None, _ptr(out),
                                        _ptr(lse), _stream(stream))
    _check("pa_decode_attention_padded", st)
    return need.value


def pa_append_decode_attention(pool: Pool, block_tables, bt_stride: int, positions, dest, k_new,
                               v_new, q, q_out, num_q_heads: int, kv_lens, batch: int,
                               max_kv_len: int, scale: float, workspace=None, out=None, lse=None,
                               stream=None, query_workspace: bool = False) -> int:
    """Append + decode in one call; with ``query_workspace`` only return the workspace bytes."""
    lib = load_library()
    need = ctypes.c_size_t(0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_append_decode_attention(ctypes.byref(pool), _ptr(block_tables), bt_stride,
                                        _ptr(positions), _ptr(dest), _ptr(k_new), _ptr(v_new),
                                        _ptr(q), _ptr(q_out), num_q_heads, _ptr(kv_lens), batch,
                                        max_kv_len, ctypes.c_float(scale), _ptr(workspace),
                                        ws_bytes, ctypes.byref(need) if query_workspace else None,
                                        _ptr(out), _ptr(lse), _stream(stream))
    _check("pa_append_decode_attention", st)
    return need.value


def pa_lockstep_decode_step(pool: Pool, block_tables, bt_stride: int, positions, positions_out,
                            k_new, v_new, q, q_out, num_q_heads: int, batch: int,
                            max_kv_len: int, scale: float, workspace=None, out=None, lse=None,
                            stream=None, query_workspace: bool = False) -> int:
    """Append + decode (kv_len = position + 1) + positions_out = positions + 1, in one launch;
    with ``query_workspace`` only return the workspace bytes."""
    lib = load_library()
    need = ctypes.c_size_t(0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_lockstep_decode_step(ctypes.byref(pool), _ptr(block_tables), bt_stride,
                                     _ptr(positions), _ptr(positions_out), _ptr(k_new),
                                     _ptr(v_new), _ptr(q), _ptr(q_out), num_q_heads, batch,
                                     max_kv_len, ctypes.c_float(scale), _ptr(workspace), ws_bytes,
                                     ctypes.byref(need) if query_workspace else None, _ptr(out),
                                     _ptr(lse), _stream(stream))
    _check("pa_lockstep_decode_step", st)
    return need.value


def pa_append_decode_attention_padded(pool: Pool, positions, dest, k_new, v_new, q, q_out,
                                      num_q_heads: int, gap_start, gap_end, kv_cols: int,
                                      batch: int, scale: float, workspace=None, out=None,
                                      lse=None, stream=None,
                                      query_workspace: bool = False) -> int:
    """Lockstep append + padded decode in one call."""
    lib = load_library()
    need = ctypes.c_size_t(0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pa_append_decode_attention_padded(ctypes.byref(pool), _ptr(positions), _ptr(dest),
                                               _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(q_out),
                                               num_q_heads, _ptr(gap_start), _ptr(gap_end),
                                               kv_cols, batch, ctypes.c_float(scale),
                                               _ptr(workspace), ws_bytes,
                                               ctypes.byref(need) if query_workspace else None,
                                               _ptr(out), _ptr(lse), _stream(stream))
    _check("pa_append_decode_attention_padded", st)
    return need.value


def pa_lse_merge(out_parts, lse_parts, num_parts: int, n: int, head_dim: int, out, lse=None,
                 stream=None) -> None:
    """Merge per-part (out, lse) results over disjoint key sets into one (out, lse)."""
    lib = load_library()
    _check("pa_lse_merge", lib.pa_lse_merge(_ptr(out_parts), _ptr(lse_parts), num_parts, n,
                                            head_dim, _ptr(out), _ptr(lse), _stream(stream)))


# ------------------------------------------------------------------------------------------
# Convenience: a pool backed by one torch uint8 device buffer
# ------------------------------------------------------------------------------------------
_TORCH_DTYPE = {PA_F32: torch.float32, PA_BF16: torch.bfloat16}
_NAME_TO_DTYPE = {"f32": PA_F32, "bf16": PA_BF16}


@dataclass
class KVPool:
    """A carved pool: ``pool`` is the C view, ``buffer`` keeps the device memory alive,
    ``k``/``v`` are typed torch views ([num_blocks][H_kv][16][D] or [B][H_kv][S][D])."""
    desc: PoolDesc
    pool: Pool
    buffer: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    rope_cos: torch.Tensor | None
    rope_sin: torch.Tensor | None

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.desc.dtype]


def make_desc(layout: str, dtype: str, num_kv_heads: int, head_dim: int, num_blocks: int = 0,
              batch_cap: int = 0, seq_cap: int = 0, rope_max_pos: int = 0,
              rope_theta: float = 0.0) -> PoolDesc:
    return PoolDesc(layout=PA_PAGED if layout == "paged" else PA_PADDED,
                    dtype=_NAME_TO_DTYPE[dtype], num_kv_heads=num_kv_heads, head_dim=head_dim,
                    block_size=16, num_blocks=num_blocks, batch_cap=batch_cap, seq_cap=seq_cap,
                    rope_max_pos=rope_max_pos, rope_theta=rope_theta)


def alloc_pool(desc: PoolDesc, device="cuda", stream=None) -> KVPool:
    nbytes, _ = pa_alloc_pool(desc)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _, pool = pa_alloc_pool(desc, buf, stream)
    td = _TORCH_DTYPE[desc.dtype]
    el = torch.tensor([], dtype=td).element_size()
    if desc.layout == PA_PAGED:
        shape = (desc.num_blocks, desc.num_kv_heads, 16, desc.head_dim)
    else:
        shape = (desc.batch_cap, desc.num_kv_heads, desc.seq_cap, desc.head_dim)
    n = 1
    for s in shape:
        n *= s
    base = buf.data_ptr()
    k = buf[pool.k - base: pool.k - base + n * el].view(td).view(shape)
    v = buf[pool.v - base: pool.v - base + n * el].view(td).view(shape)
    cos = sin = None
    if desc.rope_max_pos > 0:
        tn = desc.rope_max_pos * (desc.head_dim // 2) * 4
        tshape = (desc.rope_max_pos, desc.head_dim // 2)
        cos = buf[pool.rope_cos - base: pool.rope_cos - base + tn].view(torch.float32).view(tshape)
        sin = buf[pool.rope_sin - base: pool.rope_sin - base + tn].view(torch.float32).view(tshape)
    return KVPool(desc=desc, pool=pool, buffer=buf, k=k, v=v, rope_cos=cos, rope_sin=sin)
