"""GPU parity of the streaming decode step (sketch_step) through the C ABI.

Each step appends one key/value pair per head and answers one query over the
stream including it; the answers are compared at every step with the oracle's
plain definition sum_i T_p(<q, k_i>) [1, v_i] over that prefix of the stream.
Bars as for sketch_query: rel <= 2e-4 on Zhat, abs <= 2e-4 on ohat.
"""

import numpy as np
import pytest
import torch

import oracle
import exp_density_sketching_amd as E
from synthetic import WORKLOADS, generate
from tests.gpu_util import SK_Z_REL, SK_O_ABS, gpu, host, say

pytestmark = pytest.mark.gpu

CASES = {
    "w2": dict(ident=2, n=3000, h=2),      # d=16, p=4
    "w4": dict(ident=4, n=2000, h=4),      # d=64, p=2, several heads
    "w5": dict(ident=5, n=1500, h=1),      # d=8, p=6
    "w1": dict(ident=1, n=500, h=1),       # d=4, p=3
}


def _case(key, steps):
    c = CASES[key]
    w = WORKLOADS[c["ident"]].scaled(n=c["n"] + steps, m=steps, h=c["h"], chunk=0,
                                   substreams=1)
    return w, c["n"]


@pytest.mark.parametrize("layout", ["full", "sym"])
@pytest.mark.parametrize("key", list(CASES))
def test_step_loop_matches_oracle(key, layout):
    steps = 40
    w, n0 = _case(key, steps)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    sk = E.sketch_create(w.d, w.dv, w.p, w.h, layout)
    E.sketch_update(sk, Kg[:, :n0].contiguous(), Vg[:, :n0].contiguous())
    worst_z = worst_o = 0.0
    for t in range(steps):
        i = n0 + t
        out, Z = E.sketch_step(sk, Kg[:, i].contiguous(), Vg[:, i].contiguous(),
                               Qg[:, t].contiguous())
        out, Z = host(out, Z)
        for hd in range(w.h):
            o_ref, z_ref = oracle.sketch_direct(K[hd, :i + 1], V[hd, :i + 1],
                                                Q[hd, t:t + 1], w.p)
            worst_z = max(worst_z, abs(Z[hd] - z_ref[0]) / abs(z_ref[0]))
            worst_o = max(worst_o, float(np.max(np.abs(out[hd] - o_ref[0]))))
    say(f"step {key} ({layout}): max rel Zhat err {worst_z:.3e}, max abs ohat err {worst_o:.3e}")
    assert sk.count == n0 + steps
    assert worst_z <= SK_Z_REL and worst_o <= SK_O_ABS
    sk.destroy()


@pytest.mark.parametrize("layout", ["full", "sym"])
def test_steps_equal_update(layout):
    """After T steps the state equals one sketch_update over the same keys."""
    steps = 25
    w, n0 = _case("w2", steps)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    a = E.sketch_create(w.d, w.dv, w.p, w.h, layout)
    b = E.sketch_create(w.d, w.dv, w.p, w.h, layout)
    E.sketch_update(a, Kg[:, :n0].contiguous(), Vg[:, :n0].contiguous())
    for t in range(steps):
        E.sketch_step(a, Kg[:, n0 + t].contiguous(), Vg[:, n0 + t].contiguous(),
                      Qg[:, t].contiguous())
    E.sketch_update(b, Kg, Vg)
    Sa, Sb = host(E.sketch_export(a), E.sketch_export(b))
    assert a.count == b.count == n0 + steps
    assert np.abs(Sa - Sb).max() <= 1e-5 * np.abs(Sb).max()
    # the step's answer equals sketch_query on the same state
    qa = Qg[:, :1].contiguous()
    o1, z1 = E.sketch_query(a, qa)
    o2, z2 = E.sketch_query(b, qa)
    o1, z1, o2, z2 = host(o1, z1, o2, z2)
    assert np.max(np.abs(z1 - z2) / np.abs(z2)) <= 1e-5
    a.destroy()
    b.destroy()


@pytest.mark.parametrize("layout", ["full", "sym"])
def test_step_from_empty_and_timing(layout):
    """First step on an empty sketch: Zhat = T_p(<q, k>), ohat = v."""
    sk = E.sketch_create(8, 4, 3, 2, layout)
    rng = np.random.default_rng(17)
    k, v, q = gpu((rng.standard_normal((2, 8)) * 0.3).astype(np.float32),
                  rng.standard_normal((2, 4)).astype(np.float32),
                  (rng.standard_normal((2, 8)) * 0.3).astype(np.float32))
    E.sketch_timing(sk, True)
    out, Z = host(*E.sketch_step(sk, k, v, q))
    kk, vv, qq = host(k, v, q)
    for hd in range(2):
        s = float(qq[hd] @ kk[hd])
        assert abs(Z[hd] - oracle.taylor_exp(s, 3)) <= 1e-6 * abs(Z[hd])
        # ohat = (T v) / T in fp32: a few ulps of each value
        assert np.all(np.abs(out[hd] - vv[hd]) <= 4 * 2.0 ** -23 * np.maximum(np.abs(vv[hd]), 1.0))
    assert len(E.sketch_kernel_times(sk, "step")) == 1
    assert sk.count == 1
    sk.destroy()
