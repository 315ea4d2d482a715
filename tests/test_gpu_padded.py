"""GPU parity of the right-padded lockstep form (append at the lockstep column + decode that skips
each row's padding gap) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from paged_kv_cache_177_amd.runner import PaddedLockstep, PagedStep, to_numpy, to_torch

from _parity import assert_attention_close, bits, check_rows, log

pytestmark = pytest.mark.gpu


def run_and_check_padded(pc, gap_override=None):
    """Append + padded decode on the GPU vs the oracle: the padded pool bit for bit, attention
    within tolerance. Returns (out, lse) of the GPU."""
    log(f"[padded] case={pc.name} B={pc.batch} D={pc.head_dim} padded_len={pc.padded_len} "
        f"seq_cap={pc.seq_cap} dtype={pc.dtype}")
    dev = "cuda"
    L = PaddedLockstep(pc.dtype, pc.num_q_heads, pc.num_kv_heads, pc.head_dim, pc.batch,
                       pc.seq_cap, rope_theta=pc.rope_theta, rope_max_pos=pc.rope_max_pos)
    L.kv.k.copy_(to_torch(pc.k_pad, pc.dtype))
    L.kv.v.copy_(to_torch(pc.v_pad, pc.dtype))
    pos = torch.from_numpy(pc.positions).to(dev)
    dest = torch.from_numpy(pc.dest).to(dev)
    k_new = to_torch(pc.k_new, pc.dtype).to(dev)
    v_new = to_torch(pc.v_new, pc.dtype).to(dev)
    q = to_torch(pc.q, pc.dtype).to(dev)
    rope = pc.rope_max_pos > 0
    q_rot = torch.empty_like(q) if rope else None
    L.append(pos, dest, k_new, v_new, q if rope else None, q_rot)
    gs_np = pc.prefix_lens.astype(np.int32)
    ge_np = np.full(pc.batch, pc.padded_len, np.int32)
    if gap_override is not None:
        gs_np, ge_np = gap_override
    gs = torch.from_numpy(gs_np).to(dev)
    ge = torch.from_numpy(ge_np).to(dev)
    out, lse = L.decode(q_rot if rope else q, gs, ge, pc.kv_cols, pc.scale)
    torch.cuda.synchronize()

    cos = sin = None
    if rope:
        cos, sin = O.rope_tables(pc.rope_theta, pc.head_dim, pc.rope_max_pos)
    k2, v2, q2 = O.append_kv(pc.k_pad, pc.v_pad, pc.dtype, "padded", None, pc.positions,
                             pc.dest, pc.k_new, pc.v_new, cos, sin,
                             q_in=pc.q if rope else None)
    q_used = q2 if rope else pc.q
    np.testing.assert_array_equal(bits(to_numpy(L.kv.k, pc.dtype), pc.dtype), bits(k2, pc.dtype))
    np.testing.assert_array_equal(bits(to_numpy(L.kv.v, pc.dtype), pc.dtype), bits(v2, pc.dtype))
    if rope:
        np.testing.assert_array_equal(bits(to_numpy(q_rot, pc.dtype), pc.dtype),
                                      bits(q2, pc.dtype))
    o_ref, l_ref = O.decode_padded(k2, v2, pc.dtype, gs_np, ge_np, pc.kv_cols, q_used, pc.scale)
    mx, mean = assert_attention_close(out.cpu().numpy(), o_ref[:, 0], pc.dtype, "out")
    assert_attention_close(lse.cpu().numpy(), l_ref[:, 0], pc.dtype, "lse")
    log(f"[padded] ok case={pc.name} max_err={mx:.2e} mean_err={mean:.2e}")
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("reading", ["A", "B"])
def test_tiny_padded(reading):
    run_and_check_padded(W.padded_from_paged(W.tiny(reading)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_edges_padded(dtype):
    run_and_check_padded(W.padded_from_paged(W.tiny_edges(dtype=dtype), seq_cap=48))


@pytest.mark.parametrize("D,G,dtype", [(64, 4, "bf16"), (128, 4, "bf16"), (64, 2, "f32"),
                                       (32, 1, "bf16")])
def test_ragged_padded_with_splits(D, G, dtype):
    """Gaps of every width, kv_cols spanning several chunks (split + merge), NaN in every gap."""
    n = [0, 5, 16, 700, 1023, 1500, 2100, 3000]
    c = W.make_paged_case(f"padded-D{D}-G{G}-{dtype}", 31, n, 2 * G, 2, D, dtype,
                          rope_theta=1e4 if dtype == "f32" else 0.0)
    run_and_check_padded(W.padded_from_paged(c, seq_cap=3100))


def test_padded_large_grid():
    """64 rows x 8 KV heads, up to 2 chunks each: a grid of a thousand workgroups, several per
    compute unit, with gaps of every width."""
    rng = np.random.default_rng(35)
    n = np.concatenate([[0, 1, 1023, 1024, 2046], rng.integers(1, 2047, 59)])
    c = W.make_paged_case("padded-wide", 35, n, 32, 8, 64, "bf16")
    run_and_check_padded(W.padded_from_paged(c, seq_cap=2100))


def test_uniform_lengths_have_no_gap():
    c = W.make_paged_case("uniform", 32, [300] * 6, 32, 8, 64, "bf16")
    pc = W.padded_from_paged(c)
    assert np.all(pc.prefix_lens == pc.padded_len)  # gap_start == gap_end
    run_and_check_padded(pc)


def test_padded_matches_paged():
    """The same logical tokens, paged vs right-padded: both within tolerance of the oracle and of
    each other."""
    c = W.make_paged_case("pvp", 33, [40, 900, 1100, 2500], 32, 8, 64, "bf16", rope_theta=1e6)
    out_pad, lse_pad = run_and_check_padded(W.padded_from_paged(c, seq_cap=2600))
    r = PagedStep(c)
    r.step()
    torch.cuda.synchronize()
    assert_attention_close(out_pad, r.out.cpu().numpy(), "bf16", "padded vs paged")
    assert_attention_close(lse_pad, r.lse.cpu().numpy(), "bf16", "padded vs paged lse")


def test_padded_long_rows_multiwave_merge():
    """Rows of 20 and 70 chunks (their merges run on 4 and 8 waves) next to a short one."""
    c = W.make_paged_case("padded-long", 34, [99, 20 * 1024 + 7, 70 * 1024 - 9], 8, 2, 64,
                          "bf16")
    run_and_check_padded(W.padded_from_paged(c))


@pytest.mark.parametrize("side_stream", [False, True])
def test_padded_runner_shares_its_workspace_across_batch_sizes(side_stream):
    """One PaddedLockstep keeps one workspace. Its finished-split counts sit at offsets set by
    batch x heads, so a smaller batch's partials land on a larger batch's counts; the runner
    zero-fills the workspace again when the batch changes. A call over the first 16 rows between
    two calls over all 64 (rows of up to 3 splits, merged inside the split grid) gives rows 0-15
    of the 64-row result, and the second 64-row call the bits of the first. On a side stream the
    runner's fills and allocations must be ordered with its launches on that stream: the three
    calls then give the default stream's bits."""
    rng = np.random.default_rng(37)
    n = rng.integers(1, 3000, 64)
    c = W.make_paged_case("padded-ws", 37, n, 8, 2, 64, "bf16")
    pc = W.padded_from_paged(c, seq_cap=3100)
    dev = "cuda"
    side = torch.cuda.Stream() if side_stream else None  # default priority
    L = PaddedLockstep(pc.dtype, pc.num_q_heads, pc.num_kv_heads, pc.head_dim, pc.batch,
                       pc.seq_cap, stream=side)
    L.kv.k.copy_(to_torch(pc.k_pad, pc.dtype))
    L.kv.v.copy_(to_torch(pc.v_pad, pc.dtype))
    L.append(torch.from_numpy(pc.positions).to(dev), torch.from_numpy(pc.dest).to(dev),
             to_torch(pc.k_new, pc.dtype).to(dev), to_torch(pc.v_new, pc.dtype).to(dev),
             None, None)
    q = to_torch(pc.q, pc.dtype).to(dev)
    gs = torch.from_numpy(pc.prefix_lens.astype(np.int32)).to(dev)
    ge = torch.from_numpy(np.full(pc.batch, pc.padded_len, np.int32)).to(dev)
    q16, gs16, ge16 = q[:16].contiguous(), gs[:16].contiguous(), ge[:16].contiguous()
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())  # inputs and pool were written here
    o1, l1 = L.decode(q, gs, ge, pc.kv_cols, pc.scale)
    o2, l2 = L.decode(q16, gs16, ge16, pc.kv_cols, pc.scale)
    o3, l3 = L.decode(q, gs, ge, pc.kv_cols, pc.scale)
    if side is not None:
        torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all()
    assert torch.equal(o2, o1[:16]) and torch.equal(l2, l1[:16])
    assert torch.equal(o3, o1) and torch.equal(l3, l1)
    # the same three calls on the default stream with a fresh runner: the same bits
    if side is not None:
        R = PaddedLockstep(pc.dtype, pc.num_q_heads, pc.num_kv_heads, pc.head_dim, pc.batch,
                           pc.seq_cap)
        R.kv.k.copy_(L.kv.k)
        R.kv.v.copy_(L.kv.v)
        r1, s1 = R.decode(q, gs, ge, pc.kv_cols, pc.scale)
        torch.cuda.synchronize()
        assert torch.equal(r1, o1) and torch.equal(s1, l1)


def test_b128_padded_full_size():
    """The B=128 workload laid out right-padded (128 rows x 8 KV heads x 8 140 columns, every row
    padded to the longest history, the step's token at the common column), in the launch the
    padded bench line times: one pa_append_decode_attention_padded call. The whole pool bit for bit
    (the step's column written, every other column untouched), every row and head within the
    acceptance tolerance and the derived fp32 bound, and the separate append + decode calls give
    the fused call's bits."""
    pc = W.padded_from_paged(W.b128())
    log(f"[padded] case={pc.name} B={pc.batch} padded_len={pc.padded_len} seq_cap={pc.seq_cap}")
    dev = "cuda"
    L = PaddedLockstep(pc.dtype, pc.num_q_heads, pc.num_kv_heads, pc.head_dim, pc.batch,
                       pc.seq_cap)
    L.kv.k.copy_(to_torch(pc.k_pad, pc.dtype))
    L.kv.v.copy_(to_torch(pc.v_pad, pc.dtype))
    pos = torch.from_numpy(pc.positions).to(dev)
    dest = torch.from_numpy(pc.dest).to(dev)
    k_new = to_torch(pc.k_new, pc.dtype).to(dev)
    v_new = to_torch(pc.v_new, pc.dtype).to(dev)
    q = to_torch(pc.q, pc.dtype).to(dev)
    gs_np = pc.prefix_lens.astype(np.int32)
    ge_np = np.full(pc.batch, pc.padded_len, np.int32)
    gs, ge = torch.from_numpy(gs_np).to(dev), torch.from_numpy(ge_np).to(dev)
    out, lse = L.append_decode(pos, dest, k_new, v_new, q, None, gs, ge, pc.kv_cols, pc.scale)
    torch.cuda.synchronize()

    k2, v2, _ = O.append_kv(pc.k_pad, pc.v_pad, pc.dtype, "padded", None, pc.positions, pc.dest,
                            pc.k_new, pc.v_new, None, None)
    np.testing.assert_array_equal(bits(to_numpy(L.kv.k, pc.dtype), pc.dtype), bits(k2, pc.dtype))
    np.testing.assert_array_equal(bits(to_numpy(L.kv.v, pc.dtype), pc.dtype), bits(v2, pc.dtype))

    def gather(b):
        cols = O.padded_valid_columns(gs_np[b], ge_np[b], pc.kv_cols)
        return O.gather_padded_columns(k2, v2, pc.dtype, b, cols)

    check_rows(out.cpu().numpy(), lse.cpu().numpy(), None, None, pc.dtype, None,
               pc.prefix_lens + 1, pc.q, pc.scale, "b128-padded fused", gather=gather)

    o2, l2 = L.decode(q, gs, ge, pc.kv_cols, pc.scale)
    torch.cuda.synchronize()
    assert torch.equal(o2, out) and torch.equal(l2, lse)
