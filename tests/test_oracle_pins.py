"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties one part of the oracle to a library routine, a closed form, an invariant of the
method, a high-precision evaluation or brute force, so that a dropped term, a wrong sign, index or
head mapping, or a transposed operand fails at least one of them.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------------------------
# Storage conversions
# ---------------------------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    """Oracle RNE fp32 -> bf16 equals torch's CPU conversion (a library routine), bit for bit."""
    rng = _rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    special_bits = np.array([
        0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F807FFF,  # ties to even / odd, just above/below
        0x00000001, 0x00008000, 0x00018000, 0x807F8000,  # subnormals and ties among them
        0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,  # overflow to inf, infinities
        0x00000000, 0x80000000, 0x3F800000, 0xC0490FDB,
    ], dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, special_bits, rng.uniform(-1e30, 1e30, 1000).astype(np.float32)])
    ours = O.f32_to_storage(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_widening_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    ours = O.storage_to_f64(bits[finite], "bf16")
    ref = torch.from_numpy(bits[finite].view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(ours, ref)


# ---------------------------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------------------------
def _ulp32(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


@pytest.mark.parametrize("theta,D", [(1e4, 64), (1e6, 64), (1e4, 128), (1e4, 32)])
def test_rope_table_against_high_precision(theta, D):
    """Every table entry is the fp32 rounding of cos/sin(p * theta**(-2i/D)), checked against a
    50-digit evaluation (pins the frequency formula, the cos/sin roles and the rounding)."""
    positions = [0, 1, 2, 3, 17, 255, 1000, 2047]
    cos, sin = O.rope_tables(theta, D, max(positions) + 1)
    mpmath.mp.dps = 50
    for p in positions:
        for i in range(D // 2):
            a = mpmath.mpf(p) * mpmath.power(mpmath.mpf(theta), mpmath.mpf(-2 * i) / D)
            c, s = float(mpmath.cos(a)), float(mpmath.sin(a))
            assert abs(float(cos[p, i]) - c) <= 0.5 * _ulp32(c) + 1e-12
            assert abs(float(sin[p, i]) - s) <= 0.5 * _ulp32(s) + 1e-12


def test_rope_position_zero_is_identity():
    cos, sin = O.rope_tables(1e4, 64, 4)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    x = _rng(2).standard_normal((3, 64)).astype(np.float32)
    r = O.rope_rotate_f32(x, cos[0][None], sin[0][None])
    np.testing.assert_array_equal(r, x)


def test_rotate_half_is_complex_rotation():
    """Pairs (x_i, x_{i+D/2}) rotate like x_i + j x_{i+D/2} multiplied by exp(j * angle): pins the
    rotate-half pairing and the sign of the rotation, within 2 fp32 ulp."""
    D, theta = 64, 1e4
    positions = np.array([0, 5, 123, 2000])
    cos, sin = O.rope_tables(theta, D, 2001)
    x = _rng(3).standard_normal((len(positions), D)).astype(np.float32)
    r = O.rope_rotate_f32(x, cos[positions], sin[positions])
    half = D // 2
    z = (x[:, :half].astype(np.float64) + 1j * x[:, half:].astype(np.float64))
    zr = z * (cos[positions].astype(np.float64) + 1j * sin[positions].astype(np.float64))
    tol_re = 2 * _ulp32(np.abs(x[:, :half]) + np.abs(x[:, half:]))
    assert np.all(np.abs(r[:, :half] - zr.real) <= tol_re)
    assert np.all(np.abs(r[:, half:] - zr.imag) <= tol_re)


def test_rotate_half_pairing_touches_i_and_i_plus_half():
    D = 64
    cos, sin = O.rope_tables(1e4, D, 8)
    for i in [0, 5, 31]:
        e = np.zeros((1, D), np.float32)
        e[0, i] = 1.0
        r = O.rope_rotate_f32(e, cos[7][None], sin[7][None])
        nz = set(np.nonzero(r[0])[0].tolist())
        assert nz == {i, i + D // 2}
        assert r[0, i] == cos[7, i] and r[0, i + D // 2] == sin[7, i]


def test_rotation_preserves_norm_and_relative_position():
    """|R x| = |x| and <R_{p+d} q, R_{t+d} k> = <R_p q, R_t k>: scores depend only on the offset,
    which is why a key stored post-RoPE is position-inert wherever it sits (helexa PR #121)."""
    D, theta = 64, 1e4
    cos, sin = O.rope_tables(theta, D, 4096)
    rng = _rng(4)
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    for p, t, d in [(10, 3, 0), (10, 3, 100), (700, 20, 1500), (0, 0, 3000)]:
        rq = O.rope_rotate_f32(q[None], cos[p + d][None], sin[p + d][None])[0].astype(np.float64)
        rk = O.rope_rotate_f32(k[None], cos[t + d][None], sin[t + d][None])[0].astype(np.float64)
        rq0 = O.rope_rotate_f32(q[None], cos[p][None], sin[p][None])[0].astype(np.float64)
        rk0 = O.rope_rotate_f32(k[None], cos[t][None], sin[t][None])[0].astype(np.float64)
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) <= 1e-5 * np.linalg.norm(q)
        assert abs(rq @ rk - rq0 @ rk0) <= 1e-4 * (np.linalg.norm(q) * np.linalg.norm(k))


# ---------------------------------------------------------------------------------------------
# append_kv
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_touches_exactly_the_closed_form_slots(dtype):
    c = W.tiny_edges(seed=5, dtype=dtype)
    cos, sin = O.rope_tables(c.rope_theta, c.head_dim, c.rope_max_pos)
    k2, v2, q2 = O.append_kv(c.k_pool, c.v_pool, dtype, "paged", c.block_tables, c.positions,
                             c.dest, c.k_new, c.v_new, cos, sin, q_in=c.q)
    view = (lambda a: a.view(np.uint32)) if dtype == "f32" else (lambda a: a)
    changed_k = view(k2) != view(c.k_pool)
    expect = np.zeros_like(changed_k)
    for b in range(c.batch):
        t = int(c.dest[b])
        expect[c.block_tables[b][t // 16], :, t % 16, :] = True
    # the slot was poison (NaN) before, so every element of it changes
    np.testing.assert_array_equal(changed_k, expect)
    np.testing.assert_array_equal(view(v2) != view(c.v_pool), expect)
    assert int(expect.sum()) == c.batch * c.num_kv_heads * c.head_dim
    # values are stored verbatim
    for b in range(c.batch):
        t = int(c.dest[b])
        np.testing.assert_array_equal(view(v2[c.block_tables[b][t // 16], :, t % 16, :]),
                                      view(c.v_new[b]))


def test_append_rotation_close_to_fp64_and_position0_exact():
    c = W.tiny(seed=6)
    cos, sin = O.rope_tables(c.rope_theta, c.head_dim, 64)
    pos = np.array([0, 17, 33], dtype=np.int32)
    k2, _, q2 = O.append_kv(c.k_pool, c.v_pool, "f32", "paged", c.block_tables, pos, c.dest,
                            c.k_new, c.v_new, cos, sin, q_in=c.q)
    for b in range(3):
        t = int(c.dest[b])
        stored = k2[c.block_tables[b][t // 16], :, t % 16, :].astype(np.float64)
        x = c.k_new[b].astype(np.float64)
        half = 32
        cc = cos[pos[b]].astype(np.float64)
        ss = sin[pos[b]].astype(np.float64)
        ref = np.concatenate([x[:, :half] * cc - x[:, half:] * ss,
                              x[:, half:] * cc + x[:, :half] * ss], axis=1)
        tol = 2 * _ulp32(np.abs(x[:, :half]) + np.abs(x[:, half:]))
        tol = np.concatenate([tol, tol], axis=1)
        assert np.all(np.abs(stored - ref) <= tol)
        if pos[b] == 0:
            np.testing.assert_array_equal(stored, x)
            np.testing.assert_array_equal(q2[b], c.q[b])


def test_append_padded_layout_writes_the_column():
    rng = _rng(7)
    B, H, S, D = 3, 2, 40, 64
    k = np.full((B, H, S, D), np.nan, np.float32)
    v = np.full((B, H, S, D), np.nan, np.float32)
    kn = rng.standard_normal((B, H, D)).astype(np.float32)
    vn = rng.standard_normal((B, H, D)).astype(np.float32)
    cos, sin = O.rope_tables(1e4, D, 64)
    pos = np.array([3, 9, 20], np.int32)
    dest = np.array([30, 30, 30], np.int32)  # lockstep: all rows write the same column
    k2, v2, _ = O.append_kv(k, v, "f32", "padded", None, pos, dest, kn, vn, cos, sin)
    changed = ~np.isnan(k2)
    assert changed.sum() == B * H * D and np.all(changed[:, :, 30, :])
    np.testing.assert_array_equal(v2[:, :, 30, :], vn)
    # the stored key is the one rotated at the logical position, whatever the column
    kp, _, _ = O.append_kv(k, v, "f32", "padded", None, pos, pos, kn, vn, cos, sin)
    for b in range(B):
        np.testing.assert_array_equal(k2[b, :, 30, :], kp[b, :, pos[b], :])


# ---------------------------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------------------------
def _rand_row(rng, n, H_q, H_kv, D, n_q=1):
    q = rng.standard_normal((n_q, H_q, D))
    K = rng.standard_normal((n, H_kv, D))
    V = rng.standard_normal((n, H_kv, D))
    return q, K, V


@pytest.mark.parametrize("n,H_q,H_kv,D,n_q", [(1, 4, 2, 64, 1), (37, 4, 2, 64, 1),
                                              (200, 32, 8, 64, 1), (150, 8, 8, 32, 5),
                                              (300, 8, 1, 128, 2)])
def test_attention_matches_torch_sdpa(n, H_q, H_kv, D, n_q):
    """Library routine: torch CPU scaled_dot_product_attention in fp64, KV heads repeated G times
    consecutively (query head h uses KV head h // G)."""
    rng = _rng(n)
    q, K, V = _rand_row(rng, n, H_q, H_kv, D, n_q)
    scale = W.fp32_scale(D)
    out, lse = O.attend_two_pass(q, K, V, scale)
    G = H_q // H_kv
    tq = torch.from_numpy(q).permute(1, 0, 2)               # (H_q, n_q, D)
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    s = scale * torch.einsum("hqd,hkd->hqk", tq, tk)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).permute(1, 0).numpy(),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s.numpy(), axis=-1).T,
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [1, 2, 5, 16, 17])
def test_attention_brute_force(n):
    rng = _rng(100 + n)
    q, K, V = _rand_row(rng, n, 4, 2, 8, n_q=2)
    o1, l1 = O.attend_two_pass(q, K, V, 0.37)
    o2, l2 = O.attend_brute_force(q, K, V, 0.37)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_attention_worked_example_fixture():
    with open(os.path.join(GOLDEN, "attention_worked_example.json")) as f:
        g = json.load(f)
    q = np.array(g["q"])[None]
    out, lse = O.attend_two_pass(q, np.array(g["k"]), np.array(g["v"]), g["scale"])
    np.testing.assert_allclose(out[0], np.array(g["out"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], np.array(g["lse"]), rtol=0, atol=1e-15)


def test_attention_closed_forms():
    rng = _rng(9)
    # one key: the output is that value exactly, lse is the score
    q, K, V = _rand_row(rng, 1, 4, 2, 64)
    out, lse = O.attend_two_pass(q, K, V, 0.125)
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], V[0, h // 2])
        assert lse[0, h] == pytest.approx(0.125 * q[0, h] @ K[0, h // 2], abs=1e-15)
    # zero query, or all keys equal: uniform weights, the mean of V
    q, K, V = _rand_row(rng, 50, 4, 2, 64)
    out, _ = O.attend_two_pass(np.zeros_like(q), K, V, 0.125)
    np.testing.assert_allclose(out[0, 3], V[:, 1].mean(axis=0), atol=1e-14)
    Keq = np.repeat(K[:1], 50, axis=0)
    out, lse = O.attend_two_pass(q, Keq, V, 0.125)
    np.testing.assert_allclose(out[0, 0], V[:, 0].mean(axis=0), atol=1e-14)
    assert lse[0, 0] == pytest.approx(0.125 * q[0, 0] @ K[0, 0] + math.log(50), abs=1e-12)
    # a dominant key wins
    K2 = K.copy()
    K2[7, 0] = 1e3 * q[0, 0] / np.linalg.norm(q[0, 0])
    out, _ = O.attend_two_pass(q, K2, V, 0.125)
    np.testing.assert_allclose(out[0, 0], V[7, 0], atol=1e-12)
    # no keys: zeros and -inf, no NaN
    out, lse = O.attend_two_pass(q, K[:0], V[:0], 0.125)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_gqa_equals_mha_with_repeated_heads():
    rng = _rng(10)
    q, K, V = _rand_row(rng, 40, 8, 2, 16)
    o_gqa, l_gqa = O.attend_two_pass(q, K, V, 0.25)
    Kr = np.repeat(K, 4, axis=1)
    Vr = np.repeat(V, 4, axis=1)
    o_mha, l_mha = O.attend_two_pass(q, Kr, Vr, 0.25)
    np.testing.assert_array_equal(o_gqa, o_mha)
    np.testing.assert_array_equal(l_gqa, l_mha)
    # and each head's output differs across KV groups (the mapping is not h % H_kv)
    o_alt = np.stack([O.attend_two_pass(q[:, h:h + 1], K[:, h % 2:h % 2 + 1],
                                        V[:, h % 2:h % 2 + 1], 0.25)[0][:, 0]
                      for h in range(8)], axis=1)
    assert not np.allclose(o_alt, o_gqa)


def test_online_softmax_equals_two_pass():
    rng = _rng(11)
    for n in [1, 15, 16, 17, 100, 513]:
        q, K, V = _rand_row(rng, n, 4, 2, 64, n_q=3)
        q *= 4.0  # sharp softmax: the running max changes often
        o1, l1 = O.attend_two_pass(q, K, V, 0.125)
        for tile in [1, 16, 64]:
            o2, l2 = O.attend_online_tiled(q, K, V, 0.125, tile=tile)
            np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-13)


def test_split_merge_equals_unsplit():
    rng = _rng(12)
    for n in [2, 40, 1000]:
        q, K, V = _rand_row(rng, n, 4, 2, 64)
        o1, l1 = O.attend_two_pass(q, K, V, 0.125)
        for _ in range(5):
            k = int(rng.integers(1, min(n, 8)))
            cuts = sorted(set(rng.integers(1, n, k).tolist()))
            o2, l2 = O.attend_split_merge(q, K, V, 0.125, cuts)
            np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(l2, l1, rtol=1e-13, atol=1e-13)
    # an empty chunk carries no weight; all-empty gives (0, -inf)
    o, l = O.merge_partials([np.ones((1, 2, 3)), np.zeros((1, 2, 3))],
                            [np.zeros((1, 2)), np.full((1, 2), -np.inf)])
    np.testing.assert_array_equal(o, np.ones((1, 2, 3)))
    np.testing.assert_array_equal(l, np.zeros((1, 2)))
    o, l = O.merge_partials([np.ones((1, 2, 3))], [np.full((1, 2), -np.inf)])
    assert np.all(o == 0) and np.all(np.isneginf(l))


# ---------------------------------------------------------------------------------------------
# Paged / padded / batched invariants
# ---------------------------------------------------------------------------------------------
def _identity_relayout(c):
    """The same logical tokens with every row's blocks laid out in logical order."""
    nblk = (c.kv_lens + 15) // 16
    total = int(nblk.sum()) + 1
    kp = np.full((total,) + c.k_pool.shape[1:], W.poison_value(c.dtype), c.k_pool.dtype)
    vp = kp.copy()
    bt = np.full_like(c.block_tables, total - 1)
    off = 0
    for b in range(c.batch):
        for j in range(nblk[b]):
            kp[off] = c.k_pool[c.block_tables[b][j]]
            vp[off] = c.v_pool[c.block_tables[b][j]]
            bt[b, j] = off
            off += 1
    return kp, vp, bt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_equals_contiguous_and_batched_equals_per_row(dtype):
    c = W.make_paged_case("t", 13, [0, 3, 16, 40, 77], 8, 2, 64, dtype)
    c.k_pool, c.v_pool, _ = O.append_kv(c.k_pool, c.v_pool, dtype, "paged", c.block_tables,
                                        c.positions, c.dest, c.k_new, c.v_new)
    o1, l1 = O.decode_paged(c.k_pool, c.v_pool, dtype, c.block_tables, c.kv_lens, c.q, c.scale)
    kp, vp, bt = _identity_relayout(c)
    o2, l2 = O.decode_paged(kp, vp, dtype, bt, c.kv_lens, c.q, c.scale)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    for b in range(c.batch):
        ob, lb = O.decode_paged(c.k_pool, c.v_pool, dtype, c.block_tables[b:b + 1],
                                c.kv_lens[b:b + 1], c.q[b:b + 1], c.scale)
        np.testing.assert_array_equal(ob[0], o1[b])
        np.testing.assert_array_equal(lb[0], l1[b])
    assert np.all(np.isfinite(o1))  # poison never reached the result


def test_padded_equals_paged_and_additive_mask_form():
    """Right-padded lockstep rows give the same attention as their paged form (same logical tokens);
    the literal additive -inf mask over a finite gap agrees with skipping the gap."""
    c = W.make_paged_case("t", 14, [5, 30, 18], 4, 2, 64, "f32")
    B, H, D = c.batch, c.num_kv_heads, c.head_dim
    hist = []
    for b in range(B):
        K, V = O.gather_paged(c.k_pool, c.v_pool, "f32", c.block_tables[b], c.n_ctx[b])
        hist.append((np.moveaxis(K, 0, 1).astype(np.float32), np.moveaxis(V, 0, 1).astype(np.float32)))
    seq_cap = 64
    kpad, vpad, prefix, padded_len = O.assemble_padded(hist, seq_cap, np.float32(np.nan))
    # the step: position = prefix_len, column = padded_len
    dest = np.full(B, padded_len, np.int32)
    kpad, vpad, _ = O.append_kv(kpad, vpad, "f32", "padded", None, c.positions, dest,
                                c.k_new, c.v_new)
    kp, vp, _ = O.append_kv(c.k_pool, c.v_pool, "f32", "paged", c.block_tables, c.positions,
                            c.dest, c.k_new, c.v_new)
    o_paged, l_paged = O.decode_paged(kp, vp, "f32", c.block_tables, c.kv_lens, c.q, c.scale)
    o_pad, l_pad = O.decode_padded(kpad, vpad, "f32", prefix, np.full(B, padded_len),
                                   padded_len + 1, c.q, c.scale)
    np.testing.assert_array_equal(o_pad, o_paged)
    np.testing.assert_array_equal(l_pad, l_paged)
    kz = np.where(np.isnan(kpad), 0, kpad)
    vz = np.where(np.isnan(vpad), 0, vpad)
    o_m, l_m = O.decode_padded_additive_mask(kz, vz, "f32", prefix, np.full(B, padded_len),
                                             padded_len + 1, c.q, c.scale)
    np.testing.assert_allclose(o_m, o_paged, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l_m, l_paged, rtol=0, atol=1e-14)
    # uniform lengths: no gap at all ("no mask when lengths are uniform")
    assert O.padded_valid_columns(7, 7, 9).tolist() == list(range(9))


def test_extract_then_assemble_keeps_one_gap_per_row():
    rng = _rng(15)
    H, D, cap = 2, 4, 32
    hist = [(rng.standard_normal((H, n, D)).astype(np.float32),) * 2 for n in [3, 7, 5]]
    kpad, vpad, prefix, plen = O.assemble_padded(hist, cap, np.float32(np.nan))
    assert plen == 7 and prefix.tolist() == [3, 7, 5]
    # two lockstep decode columns
    kpad[:, :, plen:plen + 2, :] = rng.standard_normal((3, H, 2, D))
    rows = [O.extract_row_padded(kpad, vpad, b, prefix[b], plen, 2) for b in range(3)]
    for b, (kr, _) in enumerate(rows):
        assert kr.shape[1] == prefix[b] + 2 and not np.isnan(kr).any()
        np.testing.assert_array_equal(kr[:, :prefix[b]], hist[b][0])
        np.testing.assert_array_equal(kr[:, prefix[b]:], kpad[b, :, plen:plen + 2])
    # a row leaves: re-assemble the survivors; each has exactly one gap again
    k2, _, prefix2, plen2 = O.assemble_padded([rows[0], rows[2]], cap, np.float32(np.nan))
    assert prefix2.tolist() == [5, 7] and plen2 == 7
    assert np.isnan(k2[0, :, 5:7]).all() and not np.isnan(k2[0, :, :5]).any()


def test_padding_is_position_inert():
    """A key appended at logical position p attends identically whether it sits in column p or in a
    later column after a gap: only the logical position enters through RoPE (helexa PR #121)."""
    rng = _rng(16)
    D, H_q, H = 64, 4, 2
    cos, sin = O.rope_tables(1e4, D, 64)
    n = 9
    hist = rng.standard_normal((H, n, D)).astype(np.float32)
    q = rng.standard_normal((1, H_q, D)).astype(np.float32)
    kn = rng.standard_normal((1, H, D)).astype(np.float32)
    vn = rng.standard_normal((1, H, D)).astype(np.float32)
    res = []
    for col in [n, n + 7, n + 20]:
        kpad = np.full((1, H, 40, D), np.nan, np.float32)
        vpad = kpad.copy()
        kpad[0, :, :n] = hist
        vpad[0, :, :n] = hist
        kpad, vpad, qo = O.append_kv(kpad, vpad, "f32", "padded", None, [n], [col], kn, vn,
                                     cos, sin, q_in=q)
        res.append(O.decode_padded(kpad, vpad, "f32", [n], [col], col + 1, qo, 0.125))
    for o, l in res[1:]:
        np.testing.assert_array_equal(o, res[0][0])
        np.testing.assert_array_equal(l, res[0][1])


# ---------------------------------------------------------------------------------------------
# Block-sparse cross-attention (query blocks of 16 x 16-token key blocks)
# ---------------------------------------------------------------------------------------------
def _keep(rng, n_q, n, p=0.5):
    return rng.random(((n_q + 15) // 16, (n + 15) // 16)) < p


@pytest.mark.parametrize("n,n_q,H_q,H_kv,D", [(40, 20, 4, 4, 32), (150, 37, 8, 2, 64),
                                              (64, 24, 8, 8, 16)])
def test_block_sparse_matches_torch_sdpa_with_bool_mask(n, n_q, H_q, H_kv, D):
    """Library routine: torch CPU scaled_dot_product_attention in fp64 with a boolean attn_mask
    built elementwise from the block mask (True = the pair takes part). Queries that keep no key
    are left out of torch's comparison (torch gives NaN there) and must be 0 / -inf here."""
    rng = _rng(500 + n)
    q, K, V = _rand_row(rng, n, H_q, H_kv, D, n_q)
    keep = _keep(rng, n_q, n)
    keep[0, :] = False  # the first query block keeps nothing
    scale = W.fp32_scale(D)
    out, lse = O.attend_block_sparse(q, K, V, scale, keep)
    G = H_q // H_kv
    pair = np.array([[keep[i // 16, t // 16] for t in range(n)] for i in range(n_q)])
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
    mask = torch.from_numpy(pair)[None].expand(H_q, n_q, n)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=scale).permute(1, 0, 2).numpy()
    live = pair.any(axis=1)
    assert live.any() and not live.all()
    np.testing.assert_allclose(out[live], ref[live], rtol=0, atol=1e-12)
    assert np.all(out[~live] == 0) and np.all(np.isneginf(lse[~live]))
    s = scale * np.einsum("hqd,hkd->hqk", tq.numpy(), tk.numpy())
    s = np.where(pair[None], s, -np.inf)
    ref_lse = scipy.special.logsumexp(s[:, live, :], axis=-1).T
    np.testing.assert_allclose(lse[live], ref_lse, rtol=0, atol=1e-12)


def test_block_sparse_special_cases():
    rng = _rng(510)
    q, K, V = _rand_row(rng, 70, 4, 2, 32, n_q=33)
    scale = 0.17
    # every block kept: the dense definition (per-query products sum in another order than the
    # batched one, so equal up to rounding)
    full = np.ones((3, 5), dtype=bool)
    o1, l1 = O.attend_block_sparse(q, K, V, scale, full)
    o2, l2 = O.attend_two_pass(q, K, V, scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)
    # nothing kept: zeros and -inf, no NaN
    o, l = O.attend_block_sparse(q, K, V, scale, ~full)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # 65 keys: key block 4 holds one token (key 64); with only that block kept, for the second
    # query block only, those queries get that value exactly and the others zeros
    one = np.zeros((3, 5), dtype=bool)
    one[1, 4] = True
    o, l = O.attend_block_sparse(q, K[:65], V[:65], scale, one)
    for i in range(16, 32):
        for h in range(4):
            np.testing.assert_array_equal(o[i, h], V[64, h // 2])
            assert l[i, h] == pytest.approx(scale * q[i, h] @ K[64, h // 2], abs=1e-14)
    assert np.all(o[:16] == 0) and np.all(o[32:] == 0)
    # the mask indexes queries (i // 16) and keys (t // 16), not the other way round: tile 0 keeps
    # only key block 1 and tile 1 only key block 0; each equals dense attention over that slice
    sw = np.zeros((3, 5), dtype=bool)
    sw[0, 1] = True
    sw[1, 0] = True
    o, _ = O.attend_block_sparse(q, K, V, scale, sw)
    d1, _ = O.attend_two_pass(q[:16], K[16:32], V[16:32], scale)
    d0, _ = O.attend_two_pass(q[16:32], K[:16], V[:16], scale)
    np.testing.assert_allclose(o[:16], d1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[16:32], d0, rtol=0, atol=1e-14)


def test_block_sparse_brute_force_and_additive_form():
    rng = _rng(520)
    for n, n_q in [(5, 3), (17, 18), (40, 33)]:
        q, K, V = _rand_row(rng, n, 4, 2, 8, n_q)
        keep = _keep(rng, n_q, n, 0.6)
        o1, l1 = O.attend_block_sparse(q, K, V, 0.31, keep)
        o3, l3 = O.attend_block_mask_additive(q, K, V, 0.31, keep)
        np.testing.assert_allclose(o1, o3, rtol=0, atol=1e-14)
        np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(l3))
        fin = np.isfinite(l1)
        np.testing.assert_allclose(l1[fin], l3[fin], rtol=0, atol=1e-14)
        # brute force, query by query over the kept keys written out by hand
        for i in range(n_q):
            cols = [t for t in range(n) if keep[i // 16, t // 16]]
            ob, lb = O.attend_brute_force(q[i:i + 1], K[cols], V[cols], 0.31)
            np.testing.assert_allclose(o1[i], ob[0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l1[i], lb[0], rtol=0, atol=1e-13)


def test_block_sparse_batched_equals_per_row():
    """Batched paged form vs each row alone on its gathered keys."""
    c = W.make_paged_case("bs-oracle", 530, [20, 47, 0, 33], 4, 2, 16, "bf16")
    rng = _rng(531)
    n_q = 20
    q = W.to_storage(rng.standard_normal((n_q, 4, 16), dtype=np.float32), "bf16")
    keep = rng.random((4, 2, 4)) < 0.5
    out, lse = O.decode_paged_block_sparse(c.k_pool, c.v_pool, "bf16", c.block_tables,
                                           c.kv_lens - 1, q, c.scale, keep, shared_q=True)
    for b in range(4):
        K, V = O.gather_paged(c.k_pool, c.v_pool, "bf16", c.block_tables[b], c.kv_lens[b] - 1)
        o, l = O.attend_block_sparse(O.storage_to_f64(q, "bf16"), K, V, c.scale, keep[b])
        np.testing.assert_array_equal(out[b], o)
        np.testing.assert_array_equal(lse[b], l)


# ---------------------------------------------------------------------------------------------
# Per-head QK RMSNorm (before RoPE)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("D", [32, 64, 128])
def test_rms_norm_close_to_fp64_and_torch(D):
    """Within a few fp32 ulp of the fp64 formula, and of torch's CPU rms_norm (a library routine
    with its own reduction order)."""
    rng = _rng(600 + D)
    x = (rng.standard_normal((40, 4, D)) * rng.uniform(0.01, 30, (40, 4, 1))).astype(np.float32)
    w = rng.uniform(0.5, 2.0, D).astype(np.float32)
    eps = 1e-5
    y = O.rms_norm_head_f32(x, w, eps)
    x64 = x.astype(np.float64)
    y64 = x64 / np.sqrt((x64 ** 2).mean(axis=-1, keepdims=True) + np.float64(np.float32(eps))) \
        * w.astype(np.float64)
    ulp = np.spacing(np.abs(y64).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(y - y64) <= 4 * ulp)
    yt = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(w), eps).numpy()
    assert np.all(np.abs(y - yt) <= 4 * ulp)
    # the RMS of the output (with unit weights) is 1 up to eps
    y1 = O.rms_norm_head_f32(x, np.ones(D, np.float32), 0.0)
    np.testing.assert_allclose(np.sqrt((y1.astype(np.float64) ** 2).mean(axis=-1)), 1.0,
                               rtol=1e-6)


def test_rms_norm_closed_forms():
    D = 64
    w = np.ones(D, np.float32)
    # a constant head c = +-2^k normalises to +-1 exactly (eps = 0)
    for c in [1.0, -4.0, 0.25, 1024.0]:
        y = O.rms_norm_head_f32(np.full(D, c, np.float32), w, 0.0)
        np.testing.assert_array_equal(y, np.full(D, np.sign(c), np.float32))
    # scaling the input by a power of two leaves the output unchanged bit for bit (eps = 0)
    rng = _rng(610)
    x = rng.standard_normal((10, D)).astype(np.float32)
    wr = rng.uniform(0.5, 2, D).astype(np.float32)
    np.testing.assert_array_equal(O.rms_norm_head_f32(x * np.float32(8.0), wr, 0.0),
                                  O.rms_norm_head_f32(x, wr, 0.0))
    # the weight multiplies each element: weight 2^k scales the output by 2^k exactly
    np.testing.assert_array_equal(O.rms_norm_head_f32(x, wr * np.float32(4.0), 1e-5),
                                  O.rms_norm_head_f32(x, wr, 1e-5) * np.float32(4.0))
    # a zero head gives zeros (eps > 0), never NaN
    assert np.all(O.rms_norm_head_f32(np.zeros(D, np.float32), wr, 1e-6) == 0)


def test_append_with_qk_norm_normalises_then_rotates():
    """The stored key is RoPE(RMSNorm(k)), the query the same with its own weight; the value is
    untouched; without tables the key is only normalised."""
    c = W.make_paged_case("qkn", 620, [5, 17, 33], 4, 2, 64, "bf16", rope_theta=1e4)
    rng = _rng(621)
    wq = rng.uniform(0.5, 2, 64).astype(np.float32)
    wk = rng.uniform(0.5, 2, 64).astype(np.float32)
    cos, sin = O.rope_tables(1e4, 64, c.rope_max_pos)
    k2, v2, q2 = O.append_kv(c.k_pool, c.v_pool, "bf16", "paged", c.block_tables, c.positions,
                             c.dest, c.k_new, c.v_new, cos, sin, q_in=c.q, q_norm_w=wq,
                             k_norm_w=wk, norm_eps=1e-5)
    for b in range(3):
        t = int(c.dest[b])
        blk = c.block_tables[b][t // 16]
        xk = O.storage_to_f64(c.k_new[b], "bf16").astype(np.float32)
        p = int(c.positions[b])
        want = O.f32_to_storage(O.rope_rotate_f32(O.rms_norm_head_f32(xk, wk, 1e-5),
                                                  cos[p][None], sin[p][None]), "bf16")
        np.testing.assert_array_equal(k2[blk, :, t % 16, :], want)
        np.testing.assert_array_equal(v2[blk, :, t % 16, :], c.v_new[b])
        xq = O.storage_to_f64(c.q[b], "bf16").astype(np.float32)
        np.testing.assert_array_equal(
            q2[b], O.f32_to_storage(O.rope_rotate_f32(O.rms_norm_head_f32(xq, wq, 1e-5),
                                                      cos[p][None], sin[p][None]), "bf16"))
    # normalised keys have RMS ~ |w| before rounding: with unit weights, RMS 1 within bf16
    k3, _, _ = O.append_kv(c.k_pool, c.v_pool, "bf16", "paged", c.block_tables, c.positions,
                           c.dest, c.k_new, c.v_new, k_norm_w=np.ones(64, np.float32),
                           norm_eps=0.0)
    t = int(c.dest[0])
    kk = O.storage_to_f64(k3[c.block_tables[0][t // 16], :, t % 16, :], "bf16")
    np.testing.assert_allclose(np.sqrt((kk ** 2).mean(axis=-1)), 1.0, rtol=1e-2)


# ---------------------------------------------------------------------------------------------
# Fused spike tokenizer + K/V projection
# ---------------------------------------------------------------------------------------------
def _tok_case(rng, E_rows, Dm=64, H=2, dh=32):
    n_emb = rng.normal(0, 0.5, (13, Dm)).astype(np.float32)
    t_emb = rng.normal(0, 0.5, (9, Dm)).astype(np.float32)
    v_emb = rng.normal(0, 0.5, (4, Dm)).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(E_rows)]).astype(np.int32)
    E = int(offsets[-1])
    nid = rng.integers(0, 13, E).astype(np.int32)
    tb = np.sort(rng.integers(0, 9, E)).astype(np.int32)
    vid = rng.integers(0, 4, E).astype(np.int32)
    wk = W.to_storage(rng.normal(0, 0.2, (H * dh, Dm)).astype(np.float32), "bf16")
    wv = W.to_storage(rng.normal(0, 0.2, (H * dh, Dm)).astype(np.float32), "bf16")
    return n_emb, t_emb, v_emb, offsets, nid, tb, vid, wk, wv


def test_spike_embedding_sums_three_rows_in_order():
    rng = _rng(800)
    n_emb, t_emb, v_emb, _, nid, tb, vid, _, _ = _tok_case(rng, [20])
    x = O.spike_embed_f32(n_emb, t_emb, v_emb, nid, tb, vid)
    ref = (n_emb[nid].astype(np.float64) + t_emb[tb] + v_emb[vid])
    np.testing.assert_allclose(x, ref, rtol=0, atol=1e-6)
    # the order is (n + t) + v: values where the other groupings round differently
    big = np.full((1, 4), 1.0, np.float32)
    x2 = O.spike_embed_f32(big, np.full((1, 4), 2.0 ** -24, np.float32),
                           np.full((1, 4), 2.0 ** -24, np.float32), [0], [0], [0])
    assert np.all(x2 == np.float32(1.0))  # 1 + 2^-24 rounds to 1, twice; n + (t + v) would not
    # library routine: torch embedding lookups in fp64
    te = (torch.nn.functional.embedding(torch.from_numpy(nid.astype(np.int64)),
                                        torch.from_numpy(n_emb.astype(np.float64)))
          + torch.nn.functional.embedding(torch.from_numpy(tb.astype(np.int64)),
                                          torch.from_numpy(t_emb.astype(np.float64)))
          + torch.nn.functional.embedding(torch.from_numpy(vid.astype(np.int64)),
                                          torch.from_numpy(v_emb.astype(np.float64))))
    np.testing.assert_allclose(x, te.numpy(), rtol=0, atol=1e-6)


def test_tokenize_kv_slots_projection_and_closed_forms():
    rng = _rng(810)
    E_rows = [5, 0, 37, 16]
    n_emb, t_emb, v_emb, off, nid, tb, vid, wk, wv = _tok_case(rng, E_rows)
    c = W.make_paged_case("tok", 811, [e - 1 if e else 0 for e in E_rows], 2, 2, 32, "bf16")
    k2, v2, kx, vx, sabs = O.tokenize_kv(c.k_pool, c.v_pool, n_emb, t_emb, v_emb, wk, wv, off,
                                         nid, tb, vid, c.block_tables)
    # exactly the events' slots changed (the pools hold NaN poison elsewhere: compare bits)
    changed = np.zeros(c.k_pool.shape[:1] + (16,), bool)
    for b in range(4):
        for t in range(E_rows[b]):
            changed[c.block_tables[b][t // 16], t % 16] = True
    same_k = np.all(k2 == c.k_pool, axis=(1, 3))  # (blocks, 16)
    assert np.array_equal(~same_k, changed)
    # library routine: torch linear in fp64 on the bf16-rounded embeddings
    x = O.spike_embed_f32(n_emb, t_emb, v_emb, nid, tb, vid)
    xb = torch.from_numpy(O.storage_to_f64(O.f32_to_storage(x, "bf16"), "bf16"))
    tk = torch.nn.functional.linear(xb, torch.from_numpy(O.storage_to_f64(wk, "bf16")))
    np.testing.assert_allclose(kx, tk.numpy(), rtol=0, atol=1e-12)
    # row 2, token 20 -> its block 1, slot 4; heads split the 64 outputs in order
    e = int(off[2]) + 20
    blk = c.block_tables[2][1]
    np.testing.assert_array_equal(k2[blk, 1, 4, :],
                                  O.f32_to_storage(kx[e, 32:].astype(np.float32), "bf16"))
    np.testing.assert_array_equal(v2[blk, 0, 4, :],
                                  O.f32_to_storage(vx[e, :32].astype(np.float32), "bf16"))
    # identity projection: the key is the bf16-rounded embedding itself; doubling the weights
    # doubles every key exactly
    eye = W.to_storage(np.eye(64, dtype=np.float32), "bf16")
    k3, _, kx3, _, _ = O.tokenize_kv(c.k_pool, c.v_pool, n_emb, t_emb, v_emb, eye, eye, off, nid,
                                     tb, vid, c.block_tables)
    np.testing.assert_array_equal(O.f32_to_storage(kx3.astype(np.float32), "bf16"),
                                  O.f32_to_storage(x, "bf16"))
    two = W.to_storage(2 * O.storage_to_f64(wk, "bf16").astype(np.float32), "bf16")
    _, _, kx4, _, _ = O.tokenize_kv(c.k_pool, c.v_pool, n_emb, t_emb, v_emb, two, wv, off, nid,
                                    tb, vid, c.block_tables)
    np.testing.assert_array_equal(kx4, 2 * kx)
    assert np.all(sabs >= np.abs(kx) - 1e-12)
