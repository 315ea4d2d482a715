"""Shared parity helpers for the GPU tests: run a step through the C ABI, run the oracle on the
same host inputs, compare."""

import sys

import numpy as np
import torch

import oracle as O
from paged_kv_cache_177_amd.runner import PagedStep, to_numpy

# attention tolerances against the fp64 oracle
TOL = {"bf16": (2e-3, 2e-4), "f32": (1e-5, 1e-5)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(a, dtype):
    return a.view(np.uint32) if dtype == "f32" else a.view(np.uint16)


def assert_attention_close(got, ref, dtype, what="out"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU result"
    d = np.abs(np.subtract(got, ref, out=np.zeros_like(got), where=~both_inf))
    max_tol, mean_tol = TOL[dtype]
    assert d.max() <= max_tol, f"{what}: max abs err {d.max():.3e} > {max_tol}"
    assert d.mean() <= mean_tol, f"{what}: mean abs err {d.mean():.3e} > {mean_tol}"
    return float(d.max()), float(d.mean())


def oracle_append(case):
    cos = sin = None
    if case.rope_max_pos > 0:
        cos, sin = O.rope_tables(case.rope_theta, case.head_dim, case.rope_max_pos)
    k2, v2, q2 = O.append_kv(case.k_pool, case.v_pool, case.dtype, "paged", case.block_tables,
                             case.positions, case.dest, case.k_new, case.v_new, cos, sin,
                             q_in=case.q if cos is not None else None)
    return k2, v2, (q2 if cos is not None else case.q), cos, sin


def run_and_check_paged(case, rows=None, check_pool=True, runner=None):
    """Append + decode on the GPU; compare pool bits, rotated queries, RoPE tables and attention
    (on ``rows`` only, default all) with the oracle. Returns (runner, max_err, mean_err)."""
    log(f"[parity] case={case.name} B={case.batch} D={case.head_dim} G="
        f"{case.num_q_heads // case.num_kv_heads} dtype={case.dtype} max_kv={case.max_kv_len}")
    r = runner or PagedStep(case)
    r.append()
    r.decode()
    torch.cuda.synchronize()
    k2, v2, q_used, cos, sin = oracle_append(case)
    if cos is not None:
        np.testing.assert_array_equal(r.kv.rope_cos.cpu().numpy().view(np.uint32),
                                      cos.view(np.uint32))
        np.testing.assert_array_equal(r.kv.rope_sin.cpu().numpy().view(np.uint32),
                                      sin.view(np.uint32))
        np.testing.assert_array_equal(bits(to_numpy(r.q_rot, case.dtype), case.dtype),
                                      bits(q_used, case.dtype))
    if check_pool:
        np.testing.assert_array_equal(bits(to_numpy(r.kv.k, case.dtype), case.dtype),
                                      bits(k2, case.dtype))
        np.testing.assert_array_equal(bits(to_numpy(r.kv.v, case.dtype), case.dtype),
                                      bits(v2, case.dtype))
    rows = np.arange(case.batch) if rows is None else np.asarray(rows)
    o_ref, l_ref = O.decode_paged(k2, v2, case.dtype, case.block_tables[rows],
                                  case.kv_lens[rows], q_used[rows], case.scale)
    out = r.out.cpu().numpy()[rows]
    lse = r.lse.cpu().numpy()[rows]
    mx, mean = assert_attention_close(out, o_ref[:, 0], case.dtype, "out")
    assert_attention_close(lse, l_ref[:, 0], case.dtype, "lse")
    log(f"[parity] ok case={case.name} max_err={mx:.2e} mean_err={mean:.2e}")
    return r, mx, mean
