"""Blocks past 4 GiB into the pool: the decode kernels and the multi-query kernel form K and V
block addresses from 64-bit block bases (the multi-query kernel through per-block buffer
resources). An ~8.6 GiB pool holds the used blocks at its far end; results are checked against
the oracle over those blocks alone (the block table remapped to them)."""

import numpy as np
import pytest
import torch

import workloads as W
from paged_kv_cache_177_amd import binding as B
from paged_kv_cache_177_amd.runner import to_torch

from _parity import check_rows, log, mq_wave_tokens

pytestmark = pytest.mark.gpu

H_Q, H_KV, D = 8, 2, 32  # 2 KiB per block in each of K and V (bf16)


def test_blocks_past_4gib_into_the_pool():
    rng = np.random.default_rng(88)
    lens = np.array([700, 1500, 33], np.int32)  # 1500 tokens: two splits, merged in the grid
    nblk = [(int(n) + 15) // 16 for n in lens]
    used = sum(nblk)
    blk_bytes = H_KV * 16 * D * 2
    far = (1 << 32) // blk_bytes + 5  # the first used block starts past 4 GiB into K
    k_host = W.to_storage(rng.standard_normal((used, H_KV, 16, D), dtype=np.float32), "bf16")
    v_host = W.to_storage(rng.standard_normal((used, H_KV, 16, D), dtype=np.float32), "bf16")
    perm = rng.permutation(used).astype(np.int32)
    stride = max(nblk)
    local = np.zeros((len(lens), stride), np.int32)
    off = 0
    for b, nb in enumerate(nblk):
        local[b, :nb] = perm[off:off + nb]
        local[b, nb:] = perm[off + nb - 1]  # entries past the row's blocks: a valid block
        off += nb
    desc = B.make_desc("paged", "bf16", H_KV, D, num_blocks=far + used)
    pool = B.alloc_pool(desc)
    log(f"[far] pool {pool.k.numel() * 2 * 2 / 2**30:.2f} GiB, used blocks from {far} "
        f"({far * blk_bytes / 2**30:.3f} GiB into K)")
    pool.k[far:far + used].copy_(to_torch(k_host, "bf16").cuda())
    pool.v[far:far + used].copy_(to_torch(v_host, "bf16").cuda())
    bt = torch.from_numpy(local + np.int32(far)).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    scale = float(np.float32(1.0 / np.sqrt(D)))
    n = len(lens)
    mx = int(lens.max())

    # paged decode, one query per row
    q = W.to_storage(rng.standard_normal((n, H_Q, D), dtype=np.float32), "bf16")
    dq = to_torch(q, "bf16").cuda()
    out = torch.empty((n, H_Q, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((n, H_Q), dtype=torch.float32, device="cuda")
    need = B.pa_decode_attention(pool.pool, dq, H_Q * D, 1, H_Q, bt, stride, lens_d, n, mx, scale,
                                 out=out, query_workspace=True)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    B.pa_decode_attention(pool.pool, dq, H_Q * D, 1, H_Q, bt, stride, lens_d, n, mx, scale,
                          workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    check_rows(out.cpu().numpy(), lse.cpu().numpy(), k_host, v_host, "bf16", local, lens, q,
               scale, "far blocks decode")

    # multi-query, 40 queries shared by the rows
    n_q = 40
    qm = W.to_storage(rng.standard_normal((n_q, H_Q, D), dtype=np.float32), "bf16")
    dqm = to_torch(qm, "bf16").cuda()
    outm = torch.empty((n, n_q, H_Q, D), dtype=torch.float32, device="cuda")
    lsem = torch.empty((n, n_q, H_Q), dtype=torch.float32, device="cuda")
    B.pa_decode_attention(pool.pool, dqm, 0, n_q, H_Q, bt, stride, lens_d, n, mx, scale,
                          out=outm, lse=lsem)
    torch.cuda.synchronize()
    check_rows(outm.cpu().numpy(), lsem.cpu().numpy(), k_host, v_host, "bf16", local, lens, qm,
               scale, "far blocks multi-query", q_shared=True, wave_tokens=mq_wave_tokens(lens))
