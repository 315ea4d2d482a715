"""Block masks for the block-sparse multi-query call (host side, numpy).

The kernel is policy-agnostic: it takes a boolean mask over (block of 16 queries, 16-token key
block) and skips the dropped tiles ("cortex-engine write-up", kernels section: the mask is computed
outside the kernel from which (latent, event) block pairs overlap in time). This module holds one
such policy.
"""

from __future__ import annotations

import numpy as np

BLOCK = 16


def temporal_block_mask(token_bins, n_q: int, n_bins: int, halo: int = 1,
                        mask_kv_blocks: int | None = None) -> np.ndarray:
    """Keep flags, uint8 [batch][ceil(n_q / 16)][mask_kv_blocks], from temporal overlap.

    The n_q latent queries are spread evenly over the window's n_bins time bins: query block k
    covers bins [k * n_bins / QB, (k + 1) * n_bins / QB) with QB = ceil(n_q / 16), widened by
    ``halo`` bins on each side. Key block j of a row covers the bins of its tokens (tokens are in
    time order, so its first and last token bound it). A tile is kept when the two ranges overlap.
    ``token_bins[b]`` is row b's per-token time bin; blocks past a row's last token are dropped.
    """
    batch = len(token_bins)
    qb = (n_q + BLOCK - 1) // BLOCK
    nkb = max(1, max(((len(t) + BLOCK - 1) // BLOCK for t in token_bins), default=1))
    width = nkb if mask_kv_blocks is None else int(mask_kv_blocks)
    if width < nkb:
        raise ValueError("mask_kv_blocks is smaller than the longest row's key blocks")
    k = np.arange(qb)
    lo_q = k * n_bins / qb - halo           # query block k covers [lo_q, hi_q)
    hi_q = (k + 1) * n_bins / qb + halo
    mask = np.zeros((batch, qb, width), dtype=np.uint8)
    for b, bins in enumerate(token_bins):
        bins = np.asarray(bins)
        n = len(bins)
        if n == 0:
            continue
        starts = np.arange(0, n, BLOCK)
        first = bins[starts]
        last = bins[np.minimum(starts + BLOCK, n) - 1]
        # key block covers [first, last + 1); overlap with [lo_q, hi_q)
        keep = (first[None, :] < hi_q[:, None]) & (last[None, :] + 1 > lo_q[:, None])
        mask[b, :, : len(starts)] = keep
    return mask
