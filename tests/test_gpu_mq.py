"""GPU parity of the multi-query (matrix-core) path against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from paged_kv_cache_177_amd import binding as B
from paged_kv_cache_177_amd.runner import MultiQueryStep, to_torch

from _parity import (assert_attention_close, check_rows, check_rows_block_sparse, log,
                     mq_wave_tokens)

pytestmark = pytest.mark.gpu


def check_mq(case, shared=True):
    log(f"[mq] case={case.name} B={case.batch} n_q={case.n_q} H={case.num_heads} "
        f"D={case.head_dim} max_kv={case.max_kv_len}")
    r = MultiQueryStep(case)
    r.decode()
    torch.cuda.synchronize()
    # every row against the oracle: the acceptance tolerance and the derived fp32 bound, element
    # by element
    rec = check_rows(r.out.cpu().numpy(), r.lse.cpu().numpy(), case.k_pool, case.v_pool,
                     case.dtype, case.block_tables, case.kv_lens, case.q, case.scale,
                     f"mq {case.name}", q_shared=True, wave_tokens=mq_wave_tokens(case.kv_lens))
    log(f"[mq] ok case={case.name} max_err={rec['max']:.2e} mean_err={rec['mean']:.2e} "
        f"ratio={rec['ratio']:.3f}")
    return r


def test_mq_workload():
    """16 samples x 256 latent queries over ~820 spike tokens each, 8 heads of 32, bf16."""
    check_mq(W.mq())


def test_mq_workload_sharpened():
    """The same geometry with queries and keys scaled up so the softmax is far from uniform."""
    check_mq(W.mq(seed=5, q_gain=40.0, kv_gain=40.0))


def _random_mq(seed, kv, n_q, H_q, H_kv, D):
    """N(0,1) queries/keys/values in a shuffled paged pool (generic multi-query stress case)."""
    c = W.make_paged_case(f"mq-rand-{seed}", seed, [max(x - 1, 0) for x in kv], H_q, H_kv, D,
                          "bf16")
    rng = np.random.default_rng(seed + 1000)
    q = W.to_storage(rng.standard_normal((n_q, H_q, D), dtype=np.float32), "bf16")
    # append the step's token so every row has exactly kv[b] keys
    kp, vp, _ = O.append_kv(c.k_pool, c.v_pool, "bf16", "paged", c.block_tables, c.positions,
                            c.dest, c.k_new, c.v_new)
    kv_lens = np.asarray(kv, np.int32)
    return W.MQCase(name=c.name, dtype="bf16", num_heads=H_q, head_dim=D, n_q=n_q,
                    num_blocks=c.num_blocks, poison_block=c.poison_block, kv_lens=kv_lens,
                    block_tables=c.block_tables, k_pool=kp, v_pool=vp, q=q, scale=c.scale,
                    seed=seed)


@pytest.mark.parametrize("D,H_q,H_kv,n_q", [
    (32, 4, 4, 37), (64, 4, 4, 37), (128, 4, 4, 37),
    (32, 8, 2, 13),  # GQA: a workgroup's two 16-row sub-tiles mix queries and heads; 26 of 32 rows
])
def test_mq_random_ragged(D, H_q, H_kv, n_q):
    kv = [1, 15, 16, 17, 300, 821, 1333]
    c = _random_mq(40 + D + H_kv, kv, n_q, H_q, H_kv, D)
    check_mq(c)


def test_mq_gqa_partial_tile_and_empty_rows():
    """G = 4 (query rows are (query, head) pairs), 5 queries -> a partial 16-row tile; a row with
    no keys gives zeros and -inf."""
    H_q, H_kv, D, n_q = 8, 2, 64, 5
    kv = [0, 1, 40, 700]
    c = W.make_paged_case("mq-gqa", 51, [max(x - 1, 0) for x in kv], H_q, H_kv, D, "bf16")
    kp, vp, _ = O.append_kv(c.k_pool, c.v_pool, "bf16", "paged", c.block_tables, c.positions,
                            c.dest, c.k_new, c.v_new)
    rng = np.random.default_rng(52)
    q = W.to_storage(rng.standard_normal((n_q, H_q, D), dtype=np.float32), "bf16")
    kv_lens = np.asarray(kv, np.int32)
    desc = B.make_desc("paged", "bf16", H_kv, D, num_blocks=c.num_blocks)
    pool = B.alloc_pool(desc)
    pool.k.copy_(to_torch(kp, "bf16"))
    pool.v.copy_(to_torch(vp, "bf16"))
    bt = torch.from_numpy(c.block_tables).cuda()
    lens = torch.from_numpy(kv_lens).cuda()
    dq = to_torch(q, "bf16").cuda()
    out = torch.empty((len(kv), n_q, H_q, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((len(kv), n_q, H_q), dtype=torch.float32, device="cuda")
    B.pa_decode_attention(pool.pool, dq, 0, n_q, H_q, bt, c.bt_stride, lens, len(kv),
                          int(kv_lens.max()), c.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    wt = mq_wave_tokens(kv_lens)
    check_rows(out.cpu().numpy(), lse.cpu().numpy(), kp, vp, "bf16", c.block_tables, kv_lens, q,
               c.scale, "mq gqa", q_shared=True, wave_tokens=wt)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    # per-row queries (q_row_stride != 0) give each row its own queries
    q2 = W.to_storage(rng.standard_normal((len(kv), n_q, H_q, D), dtype=np.float32), "bf16")
    dq2 = to_torch(q2, "bf16").cuda()
    B.pa_decode_attention(pool.pool, dq2, n_q * H_q * D, n_q, H_q, bt, c.bt_stride, lens,
                          len(kv), int(kv_lens.max()), c.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    check_rows(out.cpu().numpy(), lse.cpu().numpy(), kp, vp, "bf16", c.block_tables, kv_lens, q2,
               c.scale, "mq per-row queries", wave_tokens=wt)


# ---------------------------------------------------------------------------------------------
# Block-sparse multi-query decode (query blocks of 16 x 16-token key blocks)
# ---------------------------------------------------------------------------------------------
def _sparse_call(pool, dq, q_row_stride, n_q, H_q, bt, bt_stride, lens, batch, max_len, scale,
                 keep, out_shape):
    mask = torch.from_numpy(np.ascontiguousarray(keep.astype(np.uint8))).cuda()
    out = torch.full(out_shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(out_shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    B.pa_decode_attention_block_sparse(pool, dq, q_row_stride, n_q, H_q, bt, bt_stride, lens,
                                       batch, max_len, scale, mask, keep.shape[2], out=out,
                                       lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_mq_block_sparse_temporal_mask():
    """The latent workload under the temporal-overlap mask (about 10% of the tiles kept)."""
    from paged_kv_cache_177_amd.masks import temporal_block_mask

    c = W.mq()
    keep = temporal_block_mask(c.token_bins, c.n_q, c.n_bins, halo=1)
    log(f"[mq-sparse] temporal mask {keep.shape} kept {keep.mean():.3f}")
    r = MultiQueryStep(c)
    shape = (c.batch, c.n_q, c.num_heads, c.head_dim)
    out, lse = _sparse_call(r.kv.pool, r.q, 0, c.n_q, c.num_heads, r.block_tables, r.bt_stride,
                            r.kv_lens, c.batch, r.max_kv_len, c.scale, keep, shape)
    o_ref, l_ref = O.decode_paged_block_sparse(c.k_pool, c.v_pool, "bf16", c.block_tables,
                                               c.kv_lens, c.q, c.scale, keep.astype(bool),
                                               shared_q=True)
    assert_attention_close(out, o_ref, "bf16", "sparse out")
    assert_attention_close(lse, l_ref, "bf16", "sparse lse")
    check_rows_block_sparse(out, lse, c.k_pool, c.v_pool, "bf16", c.block_tables, c.kv_lens, c.q,
                            c.scale, keep.astype(bool), "mq sparse temporal")


@pytest.mark.parametrize("D,H_q,H_kv,n_q", [(32, 4, 4, 37), (64, 8, 2, 21), (128, 4, 4, 16)])
def test_mq_block_sparse_random_masks(D, H_q, H_kv, n_q):
    """Random masks (some query blocks keep nothing: zeros and -inf), a mask row stride larger
    than needed, GQA; and an all-kept mask gives the dense call's bits."""
    kv = [0, 1, 17, 300, 821, 1333]
    c = _random_mq(70 + D, kv, n_q, H_q, H_kv, D)
    rng = np.random.default_rng(71 + D)
    qb = (n_q + 15) // 16
    width = (max(kv) + 15) // 16 + 3
    keep = rng.random((len(kv), qb, width)) < 0.4
    keep[3, 0, :] = False  # a query block with no key at all
    desc = B.make_desc("paged", "bf16", H_kv, D, num_blocks=c.num_blocks)
    pool = B.alloc_pool(desc)
    pool.k.copy_(to_torch(c.k_pool, "bf16"))
    pool.v.copy_(to_torch(c.v_pool, "bf16"))
    bt = torch.from_numpy(c.block_tables).cuda()
    lens = torch.from_numpy(c.kv_lens).cuda()
    dq = to_torch(c.q, "bf16").cuda()
    bt_stride = c.block_tables.shape[1]
    shape = (len(kv), n_q, H_q, D)
    out, lse = _sparse_call(pool.pool, dq, 0, n_q, H_q, bt, bt_stride, lens, len(kv), max(kv),
                            c.scale, keep, shape)
    o_ref, l_ref = O.decode_paged_block_sparse(c.k_pool, c.v_pool, "bf16", c.block_tables,
                                               c.kv_lens, c.q, c.scale, keep, shared_q=True)
    assert_attention_close(out, o_ref, "bf16", "sparse out")
    assert_attention_close(lse, l_ref, "bf16", "sparse lse")
    check_rows_block_sparse(out, lse, c.k_pool, c.v_pool, "bf16", c.block_tables, c.kv_lens, c.q,
                            c.scale, keep, f"mq sparse random D={D}")
    assert np.all(out[3, :16] == 0) and np.all(np.isneginf(lse[3, :16]))
    # every tile kept: the dense multi-query call, bit for bit
    full = np.ones_like(keep)
    out_f, lse_f = _sparse_call(pool.pool, dq, 0, n_q, H_q, bt, bt_stride, lens, len(kv),
                                max(kv), c.scale, full, shape)
    out_d = torch.empty(shape, dtype=torch.float32, device="cuda")
    lse_d = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    B.pa_decode_attention(pool.pool, dq, 0, n_q, H_q, bt, bt_stride, lens, len(kv), max(kv),
                          c.scale, out=out_d, lse=lse_d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_f, out_d.cpu().numpy())
    np.testing.assert_array_equal(lse_f, lse_d.cpu().numpy())
