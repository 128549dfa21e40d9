"""GPU parity of the sketch recentred at a fixed centre (sketch_set_center)
through the C ABI, against the oracle's plain definition
e^{<q,c>} sum_i T_p(<q, k_i - c>) [1, v_i].  Bars as for the plain sketch:
rel <= 2e-4 on Zhat, abs <= 2e-4 on ohat.
"""

import numpy as np
import pytest
import torch

import oracle
import exp_density_sketching_amd as E
from tests.gpu_util import SK_Z_REL, SK_O_ABS, gpu, host, say, zrel, oabs

pytestmark = pytest.mark.gpu


def _cluster(seed, h, n, m, d, dv, offset=1.2, spread=0.3):
    """Keys in one cluster per head away from the origin (fp32), queries of norm 1."""
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((h, 1, d))
    mu *= offset / np.linalg.norm(mu, axis=2, keepdims=True)
    K = (mu + spread * rng.standard_normal((h, n, d)) / np.sqrt(d)).astype(np.float32)
    V = rng.uniform(-1, 1, (h, n, dv)).astype(np.float32)
    Q = rng.standard_normal((h, m, d))
    Q = (Q / np.linalg.norm(Q, axis=2, keepdims=True)).astype(np.float32)
    c = K.astype(np.float64).mean(axis=1).astype(np.float32)        # [h, d]
    return K, V, Q, c


@pytest.mark.parametrize("layout", ["full", "sym"])
@pytest.mark.parametrize("d,dv,p,h,chunk", [(16, 16, 3, 2, 1000), (8, 8, 4, 1, 0),
                                            (64, 64, 2, 3, 0), (4, 4, 5, 1, 777)])
def test_centered_matches_oracle(layout, d, dv, p, h, chunk):
    n, m = 3001, 130
    K, V, Q, c = _cluster(7 + d + p, h, n, m, d, dv)
    Kg, Vg, Qg, cg = gpu(K, V, Q, c)
    sk = E.sketch_create(d, dv, p, h, layout)
    E.sketch_set_center(sk, cg)
    step = chunk or n
    for c0 in range(0, n, step):
        E.sketch_update(sk, Kg[:, c0:c0 + step].contiguous(), Vg[:, c0:c0 + step].contiguous())
    out, Z = host(*E.sketch_query(sk, Qg))
    wz = wo = 0.0
    for hd in range(h):
        o_ref, z_ref = oracle.sketch_direct_centered(K[hd], V[hd], Q[hd], p, c[hd])
        wz = max(wz, zrel(Z[hd], z_ref))
        wo = max(wo, oabs(out[hd], o_ref))
    say(f"centred d={d} p={p} ({layout}): max rel Zhat err {wz:.3e}, max abs ohat err {wo:.3e}")
    assert wz <= SK_Z_REL and wo <= SK_O_ABS
    sk.destroy()


@pytest.mark.parametrize("layout", ["full", "sym"])
def test_zero_centre_is_plain_and_rules(layout):
    K, V, Q, c = _cluster(3, 1, 2000, 50, 8, 8)
    Kg, Vg, Qg = gpu(K, V, Q)
    a = E.sketch_create(8, 8, 3, 1, layout)
    b = E.sketch_create(8, 8, 3, 1, layout)
    E.sketch_set_center(b, torch.zeros(1, 8, device="cuda"))
    for s_ in (a, b):
        E.sketch_update(s_, Kg, Vg)
    oa, za, ob, zb = host(*E.sketch_query(a, Qg), *E.sketch_query(b, Qg))
    assert np.array_equal(oa, ob) and np.array_equal(za, zb)
    # a centre only on an empty sketch; different centres do not merge
    with pytest.raises(E.SketchError) as ei:
        E.sketch_set_center(a, torch.ones(1, 8, device="cuda"))
    assert ei.value.code == -1
    cc = E.sketch_create(8, 8, 3, 1, layout)
    E.sketch_set_center(cc, torch.full((1, 8), 0.5, device="cuda"))
    with pytest.raises(E.SketchError) as ei:
        E.sketch_merge(a, cc)
    assert ei.value.code == -3
    # reset keeps the centre; removing it makes the sketch plain again
    E.sketch_reset(b)
    E.sketch_set_center(b, None)
    E.sketch_update(b, Kg, Vg)
    ob, zb = host(*E.sketch_query(b, Qg))
    assert np.array_equal(oa, ob) and np.array_equal(za, zb)
    for s_ in (a, b, cc):
        s_.destroy()


@pytest.mark.parametrize("layout", ["full", "sym"])
def test_centered_step(layout):
    K, V, Q, c = _cluster(11, 2, 830, 30, 16, 8)
    Kg, Vg, Qg, cg = gpu(K, V, Q, c)
    sk = E.sketch_create(16, 8, 3, 2, layout)
    E.sketch_set_center(sk, cg)
    E.sketch_update(sk, Kg[:, :800].contiguous(), Vg[:, :800].contiguous())
    wz = wo = 0.0
    for t in range(30):
        i = 800 + t
        out, Z = host(*E.sketch_step(sk, Kg[:, i].contiguous(), Vg[:, i].contiguous(),
                                     Qg[:, t].contiguous()))
        for hd in range(2):
            o_ref, z_ref = oracle.sketch_direct_centered(K[hd, :i + 1], V[hd, :i + 1],
                                                         Q[hd, t:t + 1], 3, c[hd])
            wz = max(wz, abs(Z[hd] - z_ref[0]) / z_ref[0])
            wo = max(wo, float(np.max(np.abs(out[hd] - o_ref[0]))))
    assert wz <= SK_Z_REL and wo <= SK_O_ABS
    sk.destroy()


def test_centring_shrinks_the_error():
    """On a cluster away from the origin the recentred sketch is far closer to
    the exact answers than the plain one, and within the Lagrange bound with the
    shifted radius."""
    d, dv, p = 16, 16, 3
    K, V, Q, c = _cluster(21, 1, 8192, 256, d, dv, offset=1.5, spread=0.3)
    Kg, Vg, Qg, cg = gpu(K, V, Q, c)
    plain = E.sketch_create(d, dv, p, 1, "sym")
    cent = E.sketch_create(d, dv, p, 1, "sym")
    E.sketch_set_center(cent, cg)
    E.sketch_update(plain, Kg, Vg)
    E.sketch_update(cent, Kg, Vg)
    o_p, z_p = host(*E.sketch_query(plain, Qg))
    o_c, z_c = host(*E.sketch_query(cent, Qg))
    o_e, z_e = host(*E.exact_attend(Kg, Vg, Qg))
    err_p = float(np.max(np.abs(z_p - z_e) / z_e))
    err_c = float(np.max(np.abs(z_c - z_e) / z_e))
    rho = float(np.max(np.linalg.norm(Q[0], axis=1)) *
                np.max(np.linalg.norm(K[0].astype(np.float64) - c[0], axis=1)))
    bound = oracle.kde_relative_bound(p, rho)
    say(f"cluster at 1.5: plain rel Z err {err_p:.3e}, centred {err_c:.3e} (bound {bound:.3e})")
    assert err_c <= bound + 4 * SK_Z_REL
    assert err_c < 0.1 * err_p
    plain.destroy()
    cent.destroy()
