"""GPU parity of the fused spike tokenizer + K/V projection (pa_tokenize_kv) against the oracle,
through the C ABI: slots the call does not write keep their bits; written keys and values are
within the bound the arithmetic allows (one bf16 rounding step apart, plus the fp32 accumulation
of the matrix cores, whose order is unspecified); attention over the tokenized pool matches."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from paged_kv_cache_177_amd import binding as B
from paged_kv_cache_177_amd.runner import to_numpy, to_torch

from _parity import assert_attention_close, log

pytestmark = pytest.mark.gpu


def _run(c, max_events=None):
    desc = B.make_desc("paged", "bf16", c.num_heads, c.head_dim, num_blocks=c.num_blocks)
    pool = B.alloc_pool(desc)
    pool.k.copy_(to_torch(c.k_pool, "bf16"))
    pool.v.copy_(to_torch(c.v_pool, "bf16"))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    me = int(c.kv_lens.max(initial=0)) if max_events is None else max_events
    B.pa_tokenize_kv(pool.pool, d(c.n_emb), d(c.t_emb), d(c.v_emb),
                     B.pa_pack_projection(to_torch(c.w_k, "bf16").cuda()),
                     B.pa_pack_projection(to_torch(c.w_v, "bf16").cuda()),
                     d(c.offsets), d(c.neuron_ids), d(c.time_bins), d(c.value_ids),
                     d(c.block_tables), c.block_tables.shape[1], c.batch, me)
    torch.cuda.synchronize()
    return pool


def _check(c, pool, max_events=None):
    k2, v2, kx, vx, sabs = O.tokenize_kv(c.k_pool, c.v_pool, c.n_emb, c.t_emb, c.v_emb, c.w_k,
                                         c.w_v, c.offsets, c.neuron_ids, c.time_bins,
                                         c.value_ids, c.block_tables, max_events=max_events)
    kg, vg = to_numpy(pool.k, "bf16"), to_numpy(pool.v, "bf16")
    H, dh = c.num_heads, c.head_dim
    written = np.zeros(c.k_pool.shape[:1] + (16,), bool)
    exact = total = 0
    for b in range(c.batch):
        n = int(c.kv_lens[b]) if max_events is None else min(int(c.kv_lens[b]), max_events)
        for t in range(n):
            e = int(c.offsets[b]) + t
            blk, s = c.block_tables[b][t // 16], t % 16
            written[blk, s] = True
            for pool_gpu, ref_x in ((kg, kx), (vg, vx)):
                got = O.storage_to_f64(pool_gpu[blk, :, s, :], "bf16").reshape(-1)
                ref = ref_x[e]
                # two roundings to bf16 of values at most the accumulation error apart: one bf16
                # ulp (2^-7 relative) plus 256 terms of fp32 accumulation error (2^-16 sum|x w|)
                tol = 2.0 ** -7 * np.abs(ref) * 1.001 + 2.0 ** -16 * sabs[e] + 1e-30
                assert np.all(np.abs(got - ref) <= tol), f"row {b} token {t}"
                exact += int(np.sum(pool_gpu[blk, :, s, :].reshape(-1) ==
                                    O.f32_to_storage(ref.astype(np.float32), "bf16")))
                total += H * dh
    # slots not written keep their bits (NaN poison included)
    keep = ~written
    assert np.array_equal(kg.transpose(0, 2, 1, 3)[keep], c.k_pool.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(vg.transpose(0, 2, 1, 3)[keep], c.v_pool.transpose(0, 2, 1, 3)[keep])
    log(f"[tokenize] {total} values within bound, {exact / max(total, 1):.4f} identical to the "
        f"oracle's rounding")
    return k2, v2


def test_tokenize_mq_workload_and_attention():
    c = W.mq_tokenizer()
    log(f"[tokenize] B={c.batch} events={int(c.offsets[-1])} H={c.num_heads} dh={c.head_dim}")
    pool = _run(c)
    k2, v2 = _check(c, pool)
    # attention of the latents over the tokenized pool: the multi-query path vs the oracle on the
    # oracle's own tokenized pool
    bt = torch.from_numpy(c.block_tables).cuda()
    lens = torch.from_numpy(c.kv_lens).cuda()
    q = to_torch(c.q, "bf16").cuda()
    n_q = c.q.shape[0]
    out = torch.empty((c.batch, n_q, c.num_heads, c.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty(out.shape[:3], dtype=torch.float32, device="cuda")
    B.pa_decode_attention(pool.pool, q, 0, n_q, c.num_heads, bt, c.block_tables.shape[1], lens,
                          c.batch, int(c.kv_lens.max()), c.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = O.decode_paged(k2, v2, "bf16", c.block_tables, c.kv_lens, c.q, c.scale,
                                  shared_q=True)
    assert_attention_close(out.cpu().numpy(), o_ref, "bf16", "tokenized attention")
    assert_attention_close(lse.cpu().numpy(), l_ref, "bf16", "tokenized attention lse")


def test_tokenize_ragged_edges_and_truncation():
    """Rows of 0, 1, 16, 17, 31, 33 and 70 events (partial sub-blocks and workgroups), a second
    call with max_events = 20 that must ignore each row's later events."""
    c = W.mq_tokenizer(seed=9, batch=7, n_latents=16, model_dim=128, num_heads=2)
    # re-cut the events into the ragged counts wanted
    want = [0, 1, 16, 17, 31, 33, 70]
    E = int(c.offsets[-1])
    assert E >= sum(want)
    c.offsets = np.concatenate([[0], np.cumsum(want)]).astype(np.int32)
    nblk = [(n + 15) // 16 for n in want]
    perm = np.random.default_rng(91).permutation(c.num_blocks).astype(np.int32)
    bt = np.full((7, max(nblk)), perm[-1], dtype=np.int32)
    off = 0
    for b in range(7):
        bt[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    c.block_tables = bt
    pool = _run(c)
    _check(c, pool)
    pool = _run(c, max_events=20)
    _check(c, pool, max_events=20)


def test_pack_projection_layout():
    """pa_pack_projection is a bit-for-bit permutation into the documented fragment order: packed
    [((tile * (in / 32) + kc) * 64 + lane) * 8 + j] = w[16 tile + lane % 16][32 kc + 8 (lane / 16)
    + j]; checked against the same index map written with numpy reshapes (and two sizes)."""
    rng = np.random.default_rng(11)
    for out_f, in_f in ((256, 256), (48, 96)):
        w = rng.integers(0, 1 << 16, size=(out_f, in_f), dtype=np.uint16)
        got = B.pa_pack_projection(torch.from_numpy(w.view(np.int16)).cuda()).cpu().numpy()
        got = got.view(np.uint16).reshape(-1)
        # w[tile, r, kc, g, j] with row 16 tile + r, input 32 kc + 8 g + j -> [tile, kc, g, r, j]
        ref = w.reshape(out_f // 16, 16, in_f // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
        assert np.array_equal(got, ref), (out_f, in_f)


@pytest.mark.parametrize("model_dim,num_heads,head_dim", [
    (96, 3, 32),    # odd number of 32-input steps (a padding step); tiles dead inside a group
    (32, 1, 32),    # one step; four of the eight waves own no tile
    (64, 2, 64),
    (512, 8, 128),  # 16 steps per tile; four tile groups per wave
])
def test_tokenize_shapes(model_dim, num_heads, head_dim):
    """Other model widths and head shapes against the oracle: every written value within the
    bound, every other slot untouched."""
    c = W.mq_tokenizer(seed=31, batch=3, n_neurons=60, n_bins=80, model_dim=model_dim,
                       num_heads=num_heads, head_dim=head_dim)
    log(f"[tokenize] Dm={model_dim} H={num_heads} dh={head_dim} events={int(c.offsets[-1])}")
    pool = _run(c)
    _check(c, pool)


def test_tokenize_launch_larger_than_the_device_holds():
    """40 rows of ~800 events: about 560 workgroups, more than the device holds at once, so the
    launch takes the instance that keeps two weight steps in flight (smaller launches request all
    of a wave's steps up front). Its writes are held to the same bound, and the first three rows,
    tokenized alone by the other instance into the same pool, get the same bits."""
    import dataclasses

    c = W.mq_tokenizer(seed=12, batch=40)
    log(f"[tokenize] B={c.batch} events={int(c.offsets[-1])} (large launch)")
    pool = _run(c)
    _check(c, pool)
    kg, vg = to_numpy(pool.k, "bf16"), to_numpy(pool.v, "bf16")
    e3 = int(c.offsets[3])
    small = dataclasses.replace(c, offsets=c.offsets[:4].copy(), neuron_ids=c.neuron_ids[:e3],
                                time_bins=c.time_bins[:e3], value_ids=c.value_ids[:e3],
                                block_tables=c.block_tables[:3].copy())
    pool3 = _run(small)
    k3, v3 = to_numpy(pool3.k, "bf16"), to_numpy(pool3.v, "bf16")
    for b in range(3):
        n = int(c.offsets[b + 1] - c.offsets[b])
        for t in range(0, n, 16):
            blk = c.block_tables[b][t // 16]
            m = min(16, n - t)
            np.testing.assert_array_equal(k3[blk, :, :m], kg[blk, :, :m], err_msg=f"row {b}")
            np.testing.assert_array_equal(v3[blk, :, :m], vg[blk, :, :m], err_msg=f"row {b}")
