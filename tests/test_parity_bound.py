"""The GPU parity check can fail: the comparison helper of the GPU tests (tests/_parity.py
check_rows) run on the CPU, with the oracle's own results standing in for the GPU's. At the long
rows of the long-context workload (41k-113k tokens, D = 128) the acceptance tolerance (max-abs
2e-3, mean-abs 2e-4) is blind to a lost or doubled 16-token block; the bound derived from the
kernels' fp32 arithmetic is not. No GPU is used."""

import numpy as np
import pytest

import oracle as O
import workloads as W

from _parity import TOL, attention_bound, check_rows, check_rows_block_sparse, mq_wave_tokens

H_KV, G, D = 2, 4, 128


def _row_pool(n, seed):
    """One row of n tokens in a shuffled bf16 pool of N(0,1) values (the long-context recipe, with
    two of its eight KV heads), its block table, and four N(0,1) queries per KV head."""
    rng = np.random.default_rng(seed)
    nblk = (n + 15) // 16
    k = W.to_storage(rng.standard_normal((nblk, H_KV, 16, D), dtype=np.float32), "bf16")
    v = W.to_storage(rng.standard_normal((nblk, H_KV, 16, D), dtype=np.float32), "bf16")
    bt = rng.permutation(nblk).astype(np.int32)
    q = W.to_storage(rng.standard_normal((H_KV * G, D), dtype=np.float32), "bf16")
    return k, v, bt, q


def _oracle_as_gpu(k, v, bt, n, q, scale):
    """What a GPU would return for this row: the oracle's fp64 result rounded to fp32."""
    K, V = O.gather_paged(k, v, "bf16", bt, n)
    o, l = O.attend_two_pass(O.storage_to_f64(q, "bf16")[None], K, V, scale)
    return o[0].astype(np.float32)[None], l[0].astype(np.float32)[None]


@pytest.fixture(scope="module", params=[41188, 112543])
def long_row(request):
    n = request.param
    k, v, bt, q = _row_pool(n, 900 + n % 97)
    return n, k, v, bt, q


def _check(out, lse, k, v, bt, n, q, what):
    return check_rows(out, lse, k, v, "bf16", bt[None], np.array([n]), q[None],
                      W.fp32_scale(D), what)


def test_the_true_row_passes(long_row):
    n, k, v, bt, q = long_row
    out, lse = _oracle_as_gpu(k, v, bt, n, q, W.fp32_scale(D))
    rec = _check(out, lse, k, v, bt, n, q, f"true row n={n}")
    assert rec["ratio"] < 0.05  # rounding to fp32 alone is far inside the derived bound


@pytest.mark.parametrize("mutation", ["dropped", "doubled"])
def test_a_lost_or_doubled_block_fails(long_row, mutation):
    n, k, v, bt, q = long_row
    j = len(bt) // 2  # a full block in the middle of the row
    if mutation == "dropped":
        bt_m, n_m = np.delete(bt, j), n - 16
    else:
        bt_m, n_m = np.insert(bt, j, bt[j]), n + 16
    out, lse = _oracle_as_gpu(k, v, bt_m, n_m, q, W.fp32_scale(D))
    # the acceptance tolerance alone does not see it
    K, V = O.gather_paged(k, v, "bf16", bt, n)
    o_ref, l_ref = O.attend_two_pass(O.storage_to_f64(q, "bf16")[None], K, V, W.fp32_scale(D))
    shift = np.abs(out[0].astype(np.float64) - o_ref[0]).max()
    assert shift <= TOL["bf16"][0]
    with pytest.raises(AssertionError, match="derived fp32 bound"):
        _check(out, lse, k, v, bt, n, q, f"{mutation} block n={n}")


def test_bound_scales_with_the_arithmetic():
    """Closed cases of the bound: an empty row has bound 0; one key gives out = v exactly, and the
    bound stays a few ulps of |v| (no accumulation to speak of beyond the fixed chain count)."""
    q = np.ones((1, 4, D))
    K = np.zeros((0, 1, D))
    bo, bl = attention_bound(q, K, K, 0.088)
    assert np.all(bo == 0) and np.all(bl == 0)
    rng = np.random.default_rng(5)
    K = rng.standard_normal((1, 1, D))
    V = rng.standard_normal((1, 1, D))
    bo, bl = attention_bound(q, K, V, 0.088)
    assert np.all(bo > 0) and np.all(bo <= 3e-4 * np.abs(V[0, 0]) + 1e-12)


def test_block_sparse_check_accepts_the_oracle_and_rejects_a_dropped_block():
    """The block-sparse helper (check_rows_block_sparse) on the CPU: the oracle's own fp32-rounded
    result passes; a result in which one query block lost one of its kept key blocks fails; a
    query block that keeps nothing must be exactly 0 / -inf."""
    rng = np.random.default_rng(77)
    kv, n_q, H_q, H_kv, Dh = [0, 100, 900], 40, 4, 2, 32
    c = W.make_paged_case("sparse-pin", 77, [max(x - 1, 0) for x in kv], H_q, H_kv, Dh, "bf16")
    # the step's token appended, so row b holds exactly kv[b] keys
    kp, vp, _ = O.append_kv(c.k_pool, c.v_pool, "bf16", "paged", c.block_tables, c.positions,
                            c.dest, c.k_new, c.v_new)
    c.k_pool, c.v_pool, c.kv_lens = kp, vp, np.asarray(kv, np.int32)
    q = W.to_storage(rng.standard_normal((n_q, H_q, Dh), dtype=np.float32), "bf16")
    keep = rng.random((len(kv), 3, (max(kv) + 15) // 16 + 1)) < 0.5
    keep[2, 1, :] = False  # a query block of the long row keeps nothing
    o, l = O.decode_paged_block_sparse(c.k_pool, c.v_pool, "bf16", c.block_tables, c.kv_lens, q,
                                       c.scale, keep, shared_q=True)
    out, lse = o.astype(np.float32), l.astype(np.float32)
    rec = check_rows_block_sparse(out, lse, c.k_pool, c.v_pool, "bf16", c.block_tables, c.kv_lens,
                                  q, c.scale, keep, "sparse true")
    assert rec["ratio"] < 0.05
    # one kept key block of query block 0 of the long row dropped
    j = int(np.flatnonzero(keep[2, 0, :(kv[2] + 15) // 16])[3])
    keep_m = keep.copy()
    keep_m[2, 0, j] = False
    o_m, l_m = O.decode_paged_block_sparse(c.k_pool, c.v_pool, "bf16", c.block_tables, c.kv_lens,
                                           q, c.scale, keep_m, shared_q=True)
    with pytest.raises(AssertionError):
        check_rows_block_sparse(o_m.astype(np.float32), l_m.astype(np.float32), c.k_pool,
                                c.v_pool, "bf16", c.block_tables, c.kv_lens, q, c.scale, keep,
                                "sparse dropped block")
    # an empty query block that is not exactly 0 fails
    out_z = out.copy()
    out_z[2, 16, 0, 0] = 1e-30
    with pytest.raises(AssertionError, match="keeps nothing"):
        check_rows_block_sparse(out_z, lse, c.k_pool, c.v_pool, "bf16", c.block_tables, c.kv_lens,
                                q, c.scale, keep, "sparse empty block")


def test_mq_wave_tokens_counts_a_waves_blocks():
    """4 waves deal a row's 16-token blocks round-robin: a wave takes ceil(blocks / 4) blocks."""
    assert mq_wave_tokens(np.array([0])) == 0
    assert mq_wave_tokens(np.array([1])) == 16
    assert mq_wave_tokens(np.array([64])) == 16       # 4 blocks, one each
    assert mq_wave_tokens(np.array([65])) == 32       # 5 blocks: one wave takes two
    assert mq_wave_tokens(np.array([821, 17])) == 208  # 52 blocks of the longer row: 13 per wave
