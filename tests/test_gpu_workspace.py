"""Kept partial buffers.  The query and the exact path keep their per-call partials
in buffers held across calls (per handle; per device and stream), grown when a
call needs more.  Calls made back to back, with no synchronisation between them,
on one stream or two, must give bit for bit the answers of the same calls made
one at a time (the kernels and their order of summation are the same)."""

import numpy as np
import pytest
import torch

import exp_density_sketching_amd as E
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _rand(rng, *shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).cuda()


# (h, n, d, dv, m): decode (m <= 8) and batched calls, sizes up and down so the
# buffers grow between calls and are then reused by smaller ones
EXACT_CASES = [(2, 3000, 16, 16, 1), (2, 70001, 16, 16, 4), (1, 5000, 32, 32, 300),
               (3, 20000, 64, 64, 2), (2, 2000, 16, 16, 2), (1, 40000, 16, 16, 700)]


def test_exact_attend_back_to_back_two_streams():
    rng = np.random.default_rng(11)
    inputs = []
    for (h, n, d, dv, m) in EXACT_CASES:
        inputs.append((_rand(rng, h, n, d, scale=0.2), _rand(rng, h, n, dv),
                       _rand(rng, h, m, d, scale=0.2)))
    # one at a time
    ref = []
    for K, V, Q in inputs:
        o, z = E.exact_attend(K, V, Q)
        torch.cuda.synchronize()
        ref.append((o.cpu(), z.cpu()))
    say("exact_attend: reference calls done; back to back on two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(2):
        for i, (K, V, Q) in enumerate(inputs):
            st = streams[(i + rep) % 2]
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                o = torch.empty(Q.shape[0], Q.shape[1], V.shape[2], device="cuda")
                z = torch.empty(Q.shape[0], Q.shape[1], device="cuda")
                E.exact_attend(K, V, Q, o, z)
            outs.append((i, o, z))
    torch.cuda.synchronize()
    for i, o, z in outs:
        assert torch.equal(o.cpu(), ref[i][0]), f"case {EXACT_CASES[i]}: out differs"
        assert torch.equal(z.cpu(), ref[i][1]), f"case {EXACT_CASES[i]}: Z differs"


@pytest.mark.parametrize("layout", ["full", "sym"])
def test_sketch_query_back_to_back(layout):
    rng = np.random.default_rng(12)
    d, dv, p, h = 16, 16, 3, 2
    sk = E.sketch_create(d, dv, p, h, layout)
    E.sketch_update(sk, _rand(rng, h, 5000, d, scale=0.25), _rand(rng, h, 5000, dv))
    qs = [_rand(rng, h, m, d, scale=0.25) for m in (1, 130, 7, 1000, 64, 257)]
    ref = []
    for Q in qs:
        o, z = E.sketch_query(sk, Q)
        torch.cuda.synchronize()
        ref.append((o.cpu(), z.cpu()))
    say(f"sketch_query ({layout}): reference calls done; back to back")
    outs = [E.sketch_query(sk, Q) for Q in qs for _ in range(2)]
    torch.cuda.synchronize()
    for k, (o, z) in enumerate(outs):
        assert torch.equal(o.cpu(), ref[k // 2][0]) and torch.equal(z.cpu(), ref[k // 2][1]), \
            f"query {k // 2} (m = {qs[k // 2].shape[1]}) differs"
    sk.destroy()
