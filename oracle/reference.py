"""Plain fp64 reference for paged decode attention, written straight from the pages.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``. It shares no code with the HIP library and imports none of it.

Sources (page title, then section):
  [NG-0.7]  NeuroGrid releases, v0.7.0 "Paged KV Cache": fixed 16-token K/V blocks, per-sequence
            block tables, a paged-attention kernel that reads K/V through the block table, GQA.
  [NG-0.6]  NeuroGrid releases, v0.6.0 "Flash Decode Attention Kernel": online softmax over KV
            tiles without materialising the score matrix.
  [NG-0.5]  NeuroGrid releases, v0.5.0 "LFM2 Hybrid Architecture Support", Architecture: a
            per-head RMSNorm of the queries and keys, applied before RoPE.
  [NG-0.8]  NeuroGrid releases, v0.8.0 "Key Changes": lengths read from device buffers,
            kv_len = position + 1.
  [HX-1]    helexa PR #121 "continuous batching -- batched decode + engine", commit "slice 1"
            (batched lockstep decode groundwork): per-row RoPE positions gathered as (B,1,half)
            cos/sin tables and applied rotate-half; keys stored post-RoPE so padding is
            position-inert; right-padded lockstep KV; one additive padding-gap mask per row
            covering [prefix_len, padded_len).
  [HX-3a]   same PR, commit "slice 3a" (batch-row extraction): a row keeps its prefix
            [0, prefix_len) plus its decode columns [padded_len, padded_len + steps).
  [CX-K]    cortex-engine write-up, kernels section, block-sparse cross-attention: FlashAttention-2
            style online softmax (running max, log-sum, output statistics); a fully masked row
            yields zeros, not NaN; many latent queries attend to ragged spike tokens.
  [CX-T]    cortex-engine write-up, model section and kernels section (fused spike tokenizer):
            each spike event (neuron_id, time_bin, value) becomes the sum of three embedding-table
            rows, one per field, giving a flat, ragged sequence of tokens per sample.

Storage conventions (the pages fix only "16-token blocks"; the rest is this library's contract):
  paged pool   K, V each [num_blocks][H_kv][16][D]; token t of row b lives at
               (block_tables[b][t // 16], t % 16).
  padded pool  K, V each [batch_cap][H_kv][seq_cap][D]; token column c of row b lives at [b, :, c].
  dtypes       "f32" arrays are np.float32; "bf16" arrays are np.uint16 bit patterns.

Open points of the pages and the reading taken here:
  * RoPE constants: inv_i = theta ** (-2 i / D) and the angle p * inv_i in fp64, cos/sin rounded
    once to fp32 (Python ``math`` on the host's libm). Rotate-half pairs element i with i + D/2.
  * The rotation itself runs in fp32 with every product and sum rounded separately (no fused
    multiply-add), so that the stored keys are reproducible bit for bit.
  * GQA: query head h reads KV head h // G with G = H_q / H_kv (consecutive grouping).
  * A row with no valid key gives out = 0 and lse = -inf.
  * Block-sparse cross-attention [CX-K]: the mask is given per (block of 16 consecutive queries,
    16-token key block); query i of a row attends exactly to the keys of the blocks j with
    keep[i // 16][j]. The pages state only a boolean tile mask computed outside the kernel; the
    16 x 16 tile granularity is this library's reading (one matrix-core tile of queries by one
    K/V block of keys).
"""

from __future__ import annotations

import math

import numpy as np

BLOCK = 16


# --------------------------------------------------------------------------------------------
# Storage dtype conversions
# --------------------------------------------------------------------------------------------
def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to fp64. bf16 -> fp64 is exact (the bf16 bits are the top half of fp32)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def f32_to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage dtype.

    bf16 keeps the top 16 bits of the fp32 pattern after round-to-nearest, ties-to-even: add
    0x7FFF plus the lowest kept bit, then truncate. NaN stays NaN (quiet bit forced on).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32.copy()
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = ((u >> np.uint64(16)) | np.uint64(0x40)) & np.uint64(0xFFFF)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


# --------------------------------------------------------------------------------------------
# RoPE [HX-1]
# --------------------------------------------------------------------------------------------
def rope_tables(theta: float, head_dim: int, max_pos: int) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin tables [max_pos][head_dim/2] in fp32.

    Frequency i (i < D/2) is theta ** (-2 i / D); the angle at position p is p times that, both in
    fp64; each cosine and sine is rounded once to fp32. Pure-Python loop over ``math.cos``/``sin``.
    """
    half = head_dim // 2
    cos = np.empty((max_pos, half), dtype=np.float32)
    sin = np.empty((max_pos, half), dtype=np.float32)
    for i in range(half):
        inv = float(theta) ** (-2 * i / head_dim)
        for p in range(max_pos):
            a = p * inv
            cos[p, i] = math.cos(a)
            sin[p, i] = math.sin(a)
    return cos, sin


def rope_rotate_f32(x32: np.ndarray, c32: np.ndarray, s32: np.ndarray) -> np.ndarray:
    """Rotate-half in fp32 [HX-1]: the first and second halves of the head form pairs (i, i + D/2).

        r[i]       = x[i] * c[i]       - x[i + D/2] * s[i]
        r[i + D/2] = x[i + D/2] * c[i] + x[i] * s[i]

    Each product, sum and difference is a separate fp32 operation (numpy float32 ufuncs round each
    result to nearest-even; nothing is fused). ``c32``/``s32`` broadcast against x[..., :D/2].
    """
    x32 = np.asarray(x32, dtype=np.float32)
    half = x32.shape[-1] // 2
    x1 = x32[..., :half]
    x2 = x32[..., half:]
    c = np.asarray(c32, dtype=np.float32)
    s = np.asarray(s32, dtype=np.float32)
    r1 = np.subtract(np.multiply(x1, c), np.multiply(x2, s))
    r2 = np.add(np.multiply(x2, c), np.multiply(x1, s))
    return np.concatenate([r1, r2], axis=-1).astype(np.float32)


# --------------------------------------------------------------------------------------------
# Per-head QK RMSNorm [NG-0.5]
# --------------------------------------------------------------------------------------------
def rms_norm_head_f32(x32: np.ndarray, w32: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm on a query or key head before RoPE [NG-0.5]: y = x * r * w with
    r = 1 / sqrt(mean(x^2) + eps), in fp32.

    The pages fix no arithmetic; the reading taken (the library's contract, chosen so that results
    reproduce bit for bit): every product, sum, quotient and square root is a separate correctly
    rounded fp32 operation, y_i = (x_i * r) * w_i, mean = ss / D, and the sum of squares ss runs
    over the rotate-half pairs first, s_i = x_i * x_i + x_{i+D/2} * x_{i+D/2} (i < D/2), then a
    pairwise tree over i that adds neighbours at every level: (s_0 + s_1), (s_2 + s_3), ..., then
    those sums in pairs, and so on. x32 (..., D); w32 (D,); eps a float (rounded to fp32).

    That summation order is not from the pages: it was chosen to be the order in which the GPU
    kernel's lanes can form the sum (one lane per rotate-half pair, then a butterfly across
    neighbouring lanes), so that a bit-exact comparison is possible at all. A bit match with the
    kernel therefore shows that the kernel follows this order, nothing more. What pins the
    function to the mathematics is its distance from RMSNorm computed in fp64 and by torch
    (test_rms_norm_close_to_fp64_and_torch: within a few fp32 ulps) and the closed forms in the
    same test file (constant heads, power-of-two scaling, weights, zero heads)."""
    x = np.asarray(x32, dtype=np.float32)
    w = np.asarray(w32, dtype=np.float32)
    D = x.shape[-1]
    half = D // 2
    # IEEE fp32 throughout, as on the GPU: squares may overflow to inf, and with eps = 0 an all-zero
    # head gives 1 / sqrt(0) = inf and then 0 * inf = NaN; numpy's warnings for those are muted
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        s = np.add(np.multiply(x[..., :half], x[..., :half]),
                   np.multiply(x[..., half:], x[..., half:]))
        while s.shape[-1] > 1:
            s = np.add(s[..., 0::2], s[..., 1::2])
        ss = s[..., 0]
        ms = np.divide(ss, np.float32(D))
        r = np.divide(np.float32(1.0), np.sqrt(np.add(ms, np.float32(eps))))
        return np.multiply(np.multiply(x, r[..., None]), w).astype(np.float32)


# --------------------------------------------------------------------------------------------
# append_kv [HX-1], [NG-0.7]
# --------------------------------------------------------------------------------------------
def append_kv(k_pool, v_pool, dtype, layout, block_tables, positions, dest, k_new, v_new,
              cos=None, sin=None, q_in=None, q_norm_w=None, k_norm_w=None, norm_eps=None):
    """One new token per row, written into copies of the pools.

    Row b's key is rotated at its logical position ``positions[b]`` (when tables are given), rounded
    to the storage dtype and stored with its value at token index ``dest[b]``: slot
    (block_tables[b][dest // 16], dest % 16) for the paged layout, column ``dest`` for the padded
    one. The value is stored unchanged. ``q_in`` (if given) is rotated at the same positions.
    With ``k_norm_w``/``q_norm_w`` (fp32 (D,)) and ``norm_eps``, every key head (and query head) is
    RMS-normalised first (``rms_norm_head_f32``), then rotated [NG-0.5: per-head RMSNorm on
    Q/K before RoPE]. Returns (k_pool', v_pool', q_out or None).
    """
    norm = k_norm_w is not None
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    B = len(positions)
    rope = cos is not None
    q_out = None
    if q_in is not None:
        q_out = np.array(q_in, copy=True)
    for b in range(B):
        p = int(positions[b])
        t = int(dest[b])
        kb = np.asarray(k_new[b])
        if rope or norm:
            x = storage_to_f64(kb, dtype).astype(np.float32)  # exact widening
            if norm:
                x = rms_norm_head_f32(x, k_norm_w, norm_eps)
            if rope:
                x = rope_rotate_f32(x, cos[p][None, :], sin[p][None, :])
            kb = f32_to_storage(x, dtype)
        if layout == "paged":
            blk = int(block_tables[b][t // BLOCK])
            k_out[blk, :, t % BLOCK, :] = kb
            v_out[blk, :, t % BLOCK, :] = v_new[b]
        elif layout == "padded":
            k_out[b, :, t, :] = kb
            v_out[b, :, t, :] = v_new[b]
        else:
            raise ValueError(layout)
        if q_in is not None and (rope or norm):
            xq = storage_to_f64(np.asarray(q_in[b]), dtype).astype(np.float32)
            if norm:
                xq = rms_norm_head_f32(xq, q_norm_w, norm_eps)
            if rope:
                xq = rope_rotate_f32(xq, cos[p][None, :], sin[p][None, :])
            q_out[b] = f32_to_storage(xq, dtype)
    return k_out, v_out, q_out


# --------------------------------------------------------------------------------------------
# Gathers [NG-0.7], [HX-1]
# --------------------------------------------------------------------------------------------
def gather_paged(k_pool, v_pool, dtype, bt_row, kv_len):
    """Row's first kv_len tokens through its block table, as contiguous fp64 (n, H_kv, D) arrays."""
    t = np.arange(int(kv_len))
    blk = np.asarray(bt_row)[t // BLOCK]
    slot = t % BLOCK
    K = storage_to_f64(k_pool[blk, :, slot, :], dtype)
    V = storage_to_f64(v_pool[blk, :, slot, :], dtype)
    return K, V


def gather_padded_columns(k_pad, v_pad, dtype, b, columns):
    """Columns of padded row b, as fp64 (n, H_kv, D) arrays."""
    cols = np.asarray(columns, dtype=np.int64)
    K = storage_to_f64(np.moveaxis(k_pad[b][:, cols, :], 1, 0), dtype)
    V = storage_to_f64(np.moveaxis(v_pad[b][:, cols, :], 1, 0), dtype)
    return K, V


# --------------------------------------------------------------------------------------------
# Attention over one row's gathered keys
# --------------------------------------------------------------------------------------------
def attend_two_pass(q, K, V, scale):
    """Exact softmax attention for one row, two passes (max, then exponentials).

    q (n_q, H_q, D), K/V (n, H_kv, D), all fp64. Query head h uses KV head h // G.
    s_j = scale * <q_h, K_j>; m = max_j s_j; w_j = exp(s_j - m); out = sum_j w_j V_j / sum_j w_j;
    lse = m + ln(sum_j w_j). No keys: out = 0, lse = -inf [CX-K].
    """
    n_q, H_q, D = q.shape
    n, H_kv, _ = K.shape
    G = H_q // H_kv
    out = np.zeros((n_q, H_q, D), dtype=np.float64)
    lse = np.full((n_q, H_q), -np.inf, dtype=np.float64)
    if n == 0:
        return out, lse
    for h in range(H_q):
        g = h // G
        s = scale * (q[:, h, :] @ K[:, g, :].T)  # (n_q, n)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        out[:, h, :] = (w @ V[:, g, :]) / l
        lse[:, h] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def attend_brute_force(q, K, V, scale):
    """The same definition as scalar loops with ``math.fsum``/``math.exp`` (tiny inputs only)."""
    n_q, H_q, D = q.shape
    n, H_kv, _ = K.shape
    G = H_q // H_kv
    out = np.zeros((n_q, H_q, D), dtype=np.float64)
    lse = np.full((n_q, H_q), -np.inf, dtype=np.float64)
    if n == 0:
        return out, lse
    for i in range(n_q):
        for h in range(H_q):
            g = h // G
            s = [scale * math.fsum(float(q[i, h, d]) * float(K[j, g, d]) for d in range(D))
                 for j in range(n)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = math.fsum(w)
            for d in range(D):
                out[i, h, d] = math.fsum(w[j] * float(V[j, g, d]) for j in range(n)) / l
            lse[i, h] = m + math.log(l)
    return out, lse


def attend_online_tiled(q, K, V, scale, tile=BLOCK):
    """Online softmax over key tiles [NG-0.6], [CX-K]: a running max, a running sum and a rescaled
    output accumulator, one tile of keys at a time. Self-check of the two-pass form."""
    n_q, H_q, D = q.shape
    n, H_kv, _ = K.shape
    G = H_q // H_kv
    out = np.zeros((n_q, H_q, D), dtype=np.float64)
    lse = np.full((n_q, H_q), -np.inf, dtype=np.float64)
    for h in range(H_q):
        g = h // G
        m = np.full((n_q,), -np.inf)
        l = np.zeros((n_q,))
        acc = np.zeros((n_q, D))
        for t0 in range(0, n, tile):
            s = scale * (q[:, h, :] @ K[t0:t0 + tile, g, :].T)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            p = np.exp(s - m_new[:, None])
            l = l * alpha + p.sum(axis=1)
            acc = acc * alpha[:, None] + p @ V[t0:t0 + tile, g, :]
            m = m_new
        ok = l > 0
        out[ok, h, :] = acc[ok] / l[ok, None]
        lse[ok, h] = m[ok] + np.log(l[ok])
    return out, lse


def merge_partials(outs, lses):
    """Combine per-chunk normalised outputs o_s with their log-sum-exps lse_s:
    M = max_s lse_s; w_s = exp(lse_s - M); out = sum_s w_s o_s / sum_s w_s; lse = M + ln sum_s w_s.
    Chunks with lse = -inf carry no weight; if every chunk is empty the result is (0, -inf)."""
    outs = np.asarray(outs, dtype=np.float64)  # (S, ..., D)
    lses = np.asarray(lses, dtype=np.float64)  # (S, ...)
    M = lses.max(axis=0)
    safe_M = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_M), 0.0)
    W = w.sum(axis=0)
    num = (w[..., None] * outs).sum(axis=0)
    out = np.where(W[..., None] > 0, num / np.where(W > 0, W, 1.0)[..., None], 0.0)
    lse = np.where(W > 0, safe_M + np.log(np.where(W > 0, W, 1.0)), -np.inf)
    return out, lse


def attend_split_merge(q, K, V, scale, bounds):
    """Split the keys at ``bounds`` (sorted cut points), attend to each chunk, merge the partials."""
    cuts = [0] + list(bounds) + [K.shape[0]]
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = attend_two_pass(q, K[a:b], V[a:b], scale)
        outs.append(o)
        lses.append(l)
    return merge_partials(outs, lses)


def attend_block_sparse(q, K, V, scale, keep):
    """Block-sparse cross-attention for one row [CX-K]: query i attends to the keys of the 16-token
    blocks j with keep[i // 16, j] and to no other; with no kept key it gives out = 0 and
    lse = -inf (the guard for a fully masked row).

    q (n_q, H_q, D), K/V (n, H_kv, D) fp64; keep bool (ceil(n_q / 16), >= ceil(n / 16)).
    Each query is exact softmax attention over its kept key set (the two-pass definition)."""
    n_q, H_q, D = q.shape
    n = K.shape[0]
    out = np.zeros((n_q, H_q, D), dtype=np.float64)
    lse = np.full((n_q, H_q), -np.inf, dtype=np.float64)
    for i in range(n_q):
        cols = [t for t in range(n) if keep[i // BLOCK, t // BLOCK]]
        if cols:
            o, l = attend_two_pass(q[i:i + 1], K[cols], V[cols], scale)
            out[i] = o[0]
            lse[i] = l[0]
    return out, lse


def attend_block_mask_additive(q, K, V, scale, keep):
    """The same block-sparse attention written as dense scores plus an additive mask: -inf on the
    scores of dropped (query, key) pairs, then one softmax per query; a query whose scores are all
    -inf gives out = 0 and lse = -inf. Self-check of ``attend_block_sparse``."""
    n_q, H_q, D = q.shape
    n, H_kv, _ = K.shape
    G = H_q // H_kv
    out = np.zeros((n_q, H_q, D), dtype=np.float64)
    lse = np.full((n_q, H_q), -np.inf, dtype=np.float64)
    if n == 0:
        return out, lse
    qi = np.arange(n_q)[:, None] // BLOCK
    kj = np.arange(n)[None, :] // BLOCK
    add = np.where(keep[qi, kj], 0.0, -np.inf)  # (n_q, n)
    for h in range(H_q):
        g = h // G
        s = scale * (q[:, h, :] @ K[:, g, :].T) + add
        m = s.max(axis=1)
        live = np.isfinite(m)
        w = np.exp(s[live] - m[live, None])
        l = w.sum(axis=1)
        out[live, h, :] = (w @ V[:, g, :]) / l[:, None]
        lse[live, h] = m[live] + np.log(l)
    return out, lse


# --------------------------------------------------------------------------------------------
# Batched decode entry points (the operations the library exports)
# --------------------------------------------------------------------------------------------
def decode_paged(k_pool, v_pool, dtype, block_tables, kv_lens, q, scale, shared_q=False):
    """Paged decode [NG-0.7]: every row attends over its own first kv_len tokens, gathered through
    its block table. q is (B, n_q, H_q, D) or (B, H_q, D); with ``shared_q`` it is (n_q, H_q, D)
    and every row uses the same queries. Returns fp64 (B, n_q, H_q, D) outputs and (B, n_q, H_q)
    log-sum-exps."""
    B = len(kv_lens)
    outs, lses = [], []
    for b in range(B):
        if shared_q:
            qb = storage_to_f64(np.asarray(q), dtype)
        else:
            qb = storage_to_f64(np.asarray(q[b]), dtype)
        if qb.ndim == 2:
            qb = qb[None]
        K, V = gather_paged(k_pool, v_pool, dtype, block_tables[b], kv_lens[b])
        o, l = attend_two_pass(qb, K, V, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def padded_valid_columns(gap_start, gap_end, kv_cols):
    """Valid columns of a right-padded lockstep row [HX-1]: [0, gap_start) and [gap_end, kv_cols)."""
    return np.concatenate([np.arange(int(gap_start)), np.arange(int(gap_end), int(kv_cols))])


def decode_padded(k_pad, v_pad, dtype, gap_start, gap_end, kv_cols, q, scale):
    """Lockstep decode over right-padded KV [HX-1]: row b attends over its valid columns only."""
    B = len(gap_start)
    outs, lses = [], []
    for b in range(B):
        qb = storage_to_f64(np.asarray(q[b]), dtype)
        if qb.ndim == 2:
            qb = qb[None]
        cols = padded_valid_columns(gap_start[b], gap_end[b], kv_cols)
        K, V = gather_padded_columns(k_pad, v_pad, dtype, b, cols)
        o, l = attend_two_pass(qb, K, V, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def decode_padded_additive_mask(k_pad, v_pad, dtype, gap_start, gap_end, kv_cols, q, scale):
    """The literal form of [HX-1]: attend over every column [0, kv_cols) with an additive mask that
    is -inf on [gap_start, gap_end) and 0 elsewhere. Only meaningful when the gap holds finite
    values (a NaN in a masked column would still reach the output through 0 * NaN)."""
    B = len(gap_start)
    H_kv = k_pad.shape[1]
    outs, lses = [], []
    for b in range(B):
        qb = storage_to_f64(np.asarray(q[b]), dtype)
        if qb.ndim == 2:
            qb = qb[None]
        n_q, H_q, D = qb.shape
        G = H_q // H_kv
        cols = np.arange(int(kv_cols))
        K, V = gather_padded_columns(k_pad, v_pad, dtype, b, cols)
        mask = np.zeros(len(cols))
        mask[int(gap_start[b]):int(gap_end[b])] = -np.inf
        out = np.zeros((n_q, H_q, D))
        lse = np.full((n_q, H_q), -np.inf)
        for h in range(H_q):
            g = h // G
            s = scale * (qb[:, h, :] @ K[:, g, :].T) + mask[None, :]
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            out[:, h, :] = (w @ V[:, g, :]) / l
            lse[:, h] = m[:, 0] + np.log(l[:, 0])
        outs.append(out)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


# --------------------------------------------------------------------------------------------
# Lockstep re-batching on the padded layout [HX-1], [HX-3a]
# --------------------------------------------------------------------------------------------
def extract_row_padded(k_pad, v_pad, b, prefix_len, padded_len, steps):
    """Row b of a padded batch as a contiguous (H_kv, prefix_len + steps, D) history: its prefix
    [0, prefix_len) followed by its decode columns [padded_len, padded_len + steps); the gap is
    dropped [HX-3a]."""
    cols = np.concatenate([np.arange(prefix_len), np.arange(padded_len, padded_len + steps)])
    return k_pad[b][:, cols, :].copy(), v_pad[b][:, cols, :].copy()


def assemble_padded(histories, seq_cap, fill):
    """Right-pad every row's contiguous (H_kv, n_b, D) history to the batch maximum and stack them
    on the batch axis [HX-1]. Columns past a row's history hold ``fill``. Returns
    (k_pad, v_pad, prefix_lens, padded_len) with k_pad/v_pad of shape [B][H_kv][seq_cap][D]."""
    B = len(histories)
    H_kv, _, D = histories[0][0].shape
    dt = histories[0][0].dtype
    k_pad = np.full((B, H_kv, seq_cap, D), fill, dtype=dt)
    v_pad = np.full((B, H_kv, seq_cap, D), fill, dtype=dt)
    prefix = np.array([h[0].shape[1] for h in histories], dtype=np.int32)
    for b, (kh, vh) in enumerate(histories):
        k_pad[b, :, :kh.shape[1], :] = kh
        v_pad[b, :, :vh.shape[1], :] = vh
    return k_pad, v_pad, prefix, int(prefix.max(initial=0))


def decode_paged_block_sparse(k_pool, v_pool, dtype, block_tables, kv_lens, q, scale, keep,
                              shared_q=False):
    """Block-sparse multi-query decode over the paged pool [CX-K], [NG-0.7]: row b's queries attend
    over its first kv_len tokens (gathered through its block table), restricted by keep[b]
    (bool (B, ceil(n_q / 16), >= ceil(max kv_len / 16))). q as for ``decode_paged``."""
    B = len(kv_lens)
    outs, lses = [], []
    for b in range(B):
        qb = storage_to_f64(np.asarray(q if shared_q else q[b]), dtype)
        if qb.ndim == 2:
            qb = qb[None]
        K, V = gather_paged(k_pool, v_pool, dtype, block_tables[b], kv_lens[b])
        o, l = attend_block_sparse(qb, K, V, scale, np.asarray(keep[b], dtype=bool))
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# --------------------------------------------------------------------------------------------
# Fused spike tokenizer + K/V projection into the paged pool [CX-T], [NG-0.7]
# --------------------------------------------------------------------------------------------
def spike_embed_f32(n_emb, t_emb, v_emb, neuron_ids, time_bins, value_ids):
    """Token embeddings [CX-T]: x = (n_emb[neuron] + t_emb[bin]) + v_emb[value], each sum one
    fp32 operation in this order (tables fp32 (rows, Dm))."""
    n = np.asarray(n_emb, dtype=np.float32)[np.asarray(neuron_ids)]
    t = np.asarray(t_emb, dtype=np.float32)[np.asarray(time_bins)]
    v = np.asarray(v_emb, dtype=np.float32)[np.asarray(value_ids)]
    return np.add(np.add(n, t), v).astype(np.float32)


def tokenize_kv(k_pool, v_pool, n_emb, t_emb, v_emb, w_k, w_v, offsets, neuron_ids, time_bins,
                value_ids, block_tables, max_events=None):
    """Write the keys and values of every spike token into copies of the bf16 paged pools.

    Row b's tokens are its events offsets[b] .. offsets[b+1] - 1, in order; token t goes to slot
    (block_tables[b][t // 16], t % 16) [NG-0.7]. Its embedding x ([CX-T], ``spike_embed_f32``) is
    rounded to bf16 (the matrix-core input); key = x . W_k^T and value = x . W_v^T with the bf16
    weights [H * dh][Dm], summed in fp64 (the exact real value up to fp64 rounding), then rounded
    to bf16 (through fp32) and split into heads of dh. Returns (k_pool', v_pool', kexact, vexact, sumabs):
    the fp64 products before rounding and, per output, sum_i |x_i w_i| (for error bounds).
    With ``max_events``, a row's tokens past that count are not written."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    H, dh = k_pool.shape[1], k_pool.shape[3]
    x = spike_embed_f32(n_emb, t_emb, v_emb, neuron_ids, time_bins, value_ids)
    xb = storage_to_f64(f32_to_storage(x, "bf16"), "bf16")  # bf16 input, exact in fp64
    wk = storage_to_f64(np.asarray(w_k), "bf16")
    wv = storage_to_f64(np.asarray(w_v), "bf16")
    kx = xb @ wk.T  # (E, H * dh) fp64
    vx = xb @ wv.T
    sabs = np.abs(xb) @ np.maximum(np.abs(wk), np.abs(wv)).T
    kb = f32_to_storage(kx.astype(np.float32), "bf16")
    vb = f32_to_storage(vx.astype(np.float32), "bf16")
    offsets = np.asarray(offsets)
    for b in range(len(offsets) - 1):
        for e in range(int(offsets[b]), int(offsets[b + 1])):
            t = e - int(offsets[b])
            if max_events is not None and t >= max_events:
                break
            blk = int(block_tables[b][t // BLOCK])
            k_out[blk, :, t % BLOCK, :] = kb[e].reshape(H, dh)
            v_out[blk, :, t % BLOCK, :] = vb[e].reshape(H, dh)
    return k_out, v_out, kx, vx, sabs
