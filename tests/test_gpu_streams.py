"""The calls run on the stream they are given: a step on a side stream gives the default stream's
bits, and two steps issued on two streams at once (each with its own workspace, as the ABI
requires for overlapping calls) give the bits of running them one after the other."""

import numpy as np
import pytest
import torch

import workloads as W
from paged_kv_cache_177_amd.runner import PagedStep, to_numpy

from _parity import bits

pytestmark = pytest.mark.gpu


def _same(a, b, dtype="bf16"):
    np.testing.assert_array_equal(a.out.cpu().numpy(), b.out.cpu().numpy())
    np.testing.assert_array_equal(a.lse.cpu().numpy(), b.lse.cpu().numpy())
    np.testing.assert_array_equal(bits(to_numpy(a.kv.k, dtype), dtype),
                                  bits(to_numpy(b.kv.k, dtype), dtype))


def test_a_step_on_a_side_stream():
    case = W.make_paged_case("stream-side", 61, [100, 2000, 5000, 40000], 16, 4, 64, "bf16",
                             rope_theta=1e4)
    ref = PagedStep(case)
    ref.step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    for fused in (False, True):
        r = PagedStep(case, stream=side)
        side.wait_stream(torch.cuda.current_stream())  # the pool copies ran on the current stream
        if fused:
            r.fused_step()
        else:
            r.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        _same(r, ref)


def test_two_streams_at_once():
    c1 = W.make_paged_case("stream-a", 62, [3000, 9000, 20000], 32, 8, 64, "bf16")
    c2 = W.make_paged_case("stream-b", 63, [700, 5000, 33000, 12], 16, 4, 128, "bf16",
                           rope_theta=1e4)
    refs = []
    for c in (c1, c2):
        r = PagedStep(c)
        for _ in range(3):
            r.fused_step()
        torch.cuda.synchronize()
        refs.append(r)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    r1, r2 = PagedStep(c1, stream=s1), PagedStep(c2, stream=s2)
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):  # issued interleaved, run concurrently
        r1.fused_step()
        r2.fused_step()
    torch.cuda.current_stream().wait_stream(s1)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    _same(r1, refs[0])
    _same(r2, refs[1])
