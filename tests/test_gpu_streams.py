"""One handle driven from two torch streams without host synchronisation.

Every binding call re-points the handle at torch's current stream; the library
then makes the new stream wait for the old one, and a merge orders the two
handles' streams both ways.  The results must be bit-identical to the same call
sequence issued on one stream (every reduction runs in a fixed order).
"""

import numpy as np
import pytest
import torch

import exp_density_sketching_amd as E
from synthetic import WORKLOADS, generate
from tests.gpu_util import gpu, host, say

pytestmark = pytest.mark.gpu


def _sequence(w, Kg, Vg, Qg, streams, layout):
    """Two sketches fed in 1024-key calls (staged) and one 8192-key call (direct),
    merged, queried, stepped; the exact path beside them.  streams[i % 2] is made
    current for call i (the same stream twice for the serial run)."""
    outs = []
    with torch.cuda.stream(streams[0]):
        a = E.sketch_create(w.d, w.dv, w.p, w.h, layout)
        b = E.sketch_create(w.d, w.dv, w.p, w.h, layout)
    calls = [(c0, 1024) for c0 in range(0, 6144, 1024)] + [(6144, 8192)]
    # every input is made contiguous up front, before the streams start
    chunks = [(Kg[:, c0:c0 + c].contiguous(), Vg[:, c0:c0 + c].contiguous(),
               Kg[:, c0 + 7:c0 + 7 + c // 2].contiguous(),
               Vg[:, c0 + 7:c0 + 7 + c // 2].contiguous()) for c0, c in calls]
    k512, v512 = Kg[:, :512].contiguous(), Vg[:, :512].contiguous()
    steps = [(Kg[:, t].contiguous(), Vg[:, t].contiguous(), Qg[:, t].contiguous())
             for t in range(4)]
    torch.cuda.synchronize()
    i = 0
    for ka, va, kb, vb in chunks:
        with torch.cuda.stream(streams[i % 2]):
            E.sketch_update(a, ka, va)
        with torch.cuda.stream(streams[(i + 1) % 2]):
            E.sketch_update(b, kb, vb)
        i += 1
    with torch.cuda.stream(streams[1]):
        E.sketch_merge(a, b)
    with torch.cuda.stream(streams[0]):
        outs += list(E.sketch_query(a, Qg))
        E.sketch_update(b, k512, v512)       # b writes after the merge read it
    with torch.cuda.stream(streams[1]):
        outs += list(E.sketch_query(b, Qg))
        outs += list(E.exact_attend(Kg, Vg, Qg))
    for t in range(4):
        with torch.cuda.stream(streams[t % 2]):
            o = torch.empty((w.h, w.dv), device="cuda")
            z = torch.empty((w.h,), device="cuda")
            E.sketch_step(a, *steps[t], o, z)
            outs += [o, z]
    with torch.cuda.stream(streams[0]):
        outs.append(E.sketch_export(a))
    torch.cuda.synchronize()
    res = host(*outs)
    a.destroy()
    b.destroy()
    return res


@pytest.mark.parametrize("layout", ["full", "sym"])
@pytest.mark.parametrize("ident", [2, 4])
def test_two_streams_match_one(ident, layout):
    w = WORKLOADS[ident].scaled(n=16384, m=300, h=2)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    torch.cuda.synchronize()
    s0 = torch.cuda.current_stream()
    ref = _sequence(w, Kg, Vg, Qg, [s0, s0], layout)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got = _sequence(w, Kg, Vg, Qg, [s1, s2], layout)
    for k, (x, y) in enumerate(zip(got, ref)):
        assert np.array_equal(x, y, equal_nan=True), f"output {k} differs"
    say(f"workload {ident} {layout}: {len(ref)} outputs bit-identical on two streams")
