"""Tail coreset on the GPU (coreset_* through the C ABI) against the float64 oracle.

The kept points are copies of input rows, so they are compared bit for bit (same
points, same order, same weights) with oracle.coreset.MergeReduceCoreset run on
the same fp32 inputs.  The walk decides in float64 on both sides; should a
uniform fall within rounding of its threshold the two kept sets may differ
there, so a mismatch is reported with the oracle's smallest decision margin of
the reduce where it starts.  Answers (head from sketch_query, tail from
coreset_query) are compared with the oracle's head + tail at the sketch's bars:
rel <= 2e-4 on Zhat, abs <= 2e-4 on ohat.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import coreset as ocs
import exp_density_sketching_amd as E
from synthetic import WORKLOADS, generate
from tests.gpu_util import SK_Z_REL, SK_O_ABS, gpu, host, zrel, oabs, say

pytestmark = pytest.mark.gpu

C0 = 0.25
SEED = 20240611


def _calls(n, chunk):
    step = chunk if chunk > 0 else n
    return [(c0, min(n, c0 + step)) for c0 in range(0, n, step)]


def _oracle(K, V, hd, d, dv, p, B, calls, heads, c0=C0, seed=SEED):
    oc = ocs.MergeReduceCoreset(d, dv, p, B, c0, seed, heads=heads, head=hd)
    for a, b in calls:
        oc.update(K[hd][a:b], V[hd][a:b])
    return oc


def _margins(K, V, hd, d, dv, p, B, calls, heads):
    """Smallest |U_t - P_t| of every reduce of the oracle's run (diagnostics)."""
    out = []
    real = ocs.halve

    def spy(Km, Vm, pp, c0, U):
        r = real(Km, Vm, pp, c0, U)
        out.append(float(np.min(np.abs(U - r["prob"]))))
        return r
    ocs.halve = spy
    try:
        _oracle(K, V, hd, d, dv, p, B, calls, heads)
    finally:
        ocs.halve = real
    return out


def _run_gpu(K, V, d, dv, p, h, B, calls):
    Kg, Vg = gpu(K, V)
    cs = E.coreset_create(d, dv, p, h, block=B, c0=C0, seed=SEED)
    for a, b in calls:
        E.coreset_update(cs, Kg[:, a:b].contiguous(), Vg[:, a:b].contiguous())
    return cs


def _check_points(cs, K, V, d, dv, p, h, B, calls, label, heads_checked=None):
    Kx, Vx, wx = host(*E.coreset_export(cs))
    pts, cnt, red = cs.info()
    for hd in (range(h) if heads_checked is None else heads_checked):
        oc = _oracle(K, V, hd, d, dv, p, B, calls, h)
        Ko, Vo, wo = oc.points()
        ok = (Ko.shape == Kx[hd].shape and np.array_equal(Ko, Kx[hd]) and
              np.array_equal(Vo, Vx[hd]) and np.array_equal(wo, wx[hd]))
        if not ok:
            m = _margins(K, V, hd, d, dv, p, B, calls, h)
            say(f"{label}: head {hd} differs; oracle reduces {len(m)}, smallest decision "
                f"margins {sorted(m)[:3]}")
        assert ok, f"{label}: kept points of head {hd} differ from the oracle's"
        assert oc.serial == red and oc.count == cnt
    say(f"{label}: {pts} points per head after {cnt} keys and {red} reduces match the oracle")


SHAPES = [  # d, dv, p, h, B, n, chunk, key radius
    (4, 4, 3, 1, 64, 1000, 0, 1.0),
    (16, 16, 4, 1, 128, 5000, 700, 1.0),
    (64, 64, 2, 3, 64, 3000, 0, 0.75),
    (8, 8, 6, 1, 64, 4113, 4096, 2.0),
    (32, 32, 3, 2, 192, 2000, 333, 1.5),
    (8, 128, 1, 1, 64, 700, 0, 1.0),
    (128, 8, 2, 2, 128, 900, 450, 1.0),
]


def _inputs(d, dv, n, m, h, r, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((h, n, d))
    K *= r / np.linalg.norm(K, axis=2, keepdims=True)
    Q = rng.standard_normal((h, m, d))
    Q *= r / np.linalg.norm(Q, axis=2, keepdims=True)
    V = rng.uniform(-1, 1, (h, n, dv))
    return K.astype(np.float32), V.astype(np.float32), Q.astype(np.float32)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"d{s[0]}dv{s[1]}p{s[2]}h{s[3]}B{s[4]}"
                                               for s in SHAPES])
def test_points_and_answers_match_oracle(shape):
    d, dv, p, h, B, n, chunk, r = shape
    K, V, Q = _inputs(d, dv, n, 37, h, r, seed=d * 7 + dv + p)
    calls = _calls(n, chunk)
    cs = _run_gpu(K, V, d, dv, p, h, B, calls)
    _check_points(cs, K, V, d, dv, p, h, B, calls, f"d={d} dv={dv} p={p} h={h} B={B}")
    # head (moments) + tail (coreset) against the oracle's head + tail
    Kg, Vg, Qg = gpu(K, V, Q)
    sk = E.sketch_create(d, dv, p, h)
    E.sketch_update(sk, Kg, Vg)
    out, Z = E.sketch_query(sk, Qg)
    E.coreset_query(cs, Qg, out, Z)
    out, Z = host(out, Z)
    wz, wo = 0.0, 0.0
    for hd in range(h):
        oh, zh = oracle.sketch_direct(K[hd], V[hd], Q[hd], p)
        tN, tZ = _oracle(K, V, hd, d, dv, p, B, calls, h).tail_query(Q[hd])
        o_ref, z_ref = ocs.answer_with_tail(oh, zh, tN, tZ)
        wz = max(wz, zrel(Z[hd], z_ref))
        wo = max(wo, oabs(out[hd], o_ref))
    say(f"  head + tail: max rel Z err {wz:.2e}, max abs o err {wo:.2e}")
    assert wz <= SK_Z_REL and wo <= SK_O_ABS
    sk.destroy()
    cs.destroy()


def test_tail_only_answer():
    """Zeros as the head answer: Z = the tail sum, out = tN / tZ."""
    d, dv, p, h, B = 16, 8, 1, 2, 64
    K, V, Q = _inputs(d, dv, 1500, 50, h, 1.2, seed=3)
    cs = _run_gpu(K, V, d, dv, p, h, B, [(0, 1500)])
    Qg = gpu(Q)[0]
    out = torch.zeros((h, 50, dv), device="cuda")
    Z = torch.zeros((h, 50), device="cuda")
    E.coreset_query(cs, Qg, out, Z)
    out, Z = host(out, Z)
    for hd in range(h):
        oc = _oracle(K, V, hd, d, dv, p, B, [(0, 1500)], h)
        tN, tZ = oc.tail_query(Q[hd])
        Kp, _, w = oc.points()
        mag = (np.abs(ocs.tail_exp(Q[hd].astype(np.float64) @ Kp.T, p)) * w).sum(axis=1)
        assert np.all(np.abs(Z[hd] - tZ) <= 2e-5 * mag)
        assert oabs(out[hd] * Z[hd][:, None], tN) <= 2e-5 * mag.max()
    cs.destroy()


def test_no_reduce_is_the_exact_answer():
    """A block larger than the stream: the coreset is the stream, and head + tail
    is the exact answer (against the exact path on the GPU and the oracle)."""
    d, dv, p, h = 16, 16, 2, 2
    K, V, Q = _inputs(d, dv, 900, 64, h, 1.0, seed=4)
    Kg, Vg, Qg = gpu(K, V, Q)
    cs = E.coreset_create(d, dv, p, h, block=1024)
    E.coreset_update(cs, Kg, Vg)
    assert cs.info() == (900, 900, 0)
    sk = E.sketch_create(d, dv, p, h)
    E.sketch_update(sk, Kg, Vg)
    out, Z = E.sketch_query(sk, Qg)
    E.coreset_query(cs, Qg, out, Z)
    out, Z = host(out, Z)
    for hd in range(h):
        o_ref, z_ref = oracle.exact_attention(K[hd], V[hd], Q[hd])
        assert zrel(Z[hd], z_ref) <= 1e-5 and oabs(out[hd], o_ref) <= 1e-5
    sk.destroy()
    cs.destroy()


def test_merge_matches_oracle():
    d, dv, p, h, B = 16, 16, 3, 2, 64
    K, V, _ = _inputs(d, dv, 3000, 1, h, 1.0, seed=5)
    parts = [(0, 1100), (1100, 1937), (1937, 3000)]
    Kg, Vg = gpu(K, V)
    hs = []
    for a, b in parts:
        c = E.coreset_create(d, dv, p, h, block=B, c0=C0, seed=SEED)
        E.coreset_update(c, Kg[:, a:b].contiguous(), Vg[:, a:b].contiguous())
        hs.append(c)
    E.coreset_merge(hs[0], hs[1])
    E.coreset_merge(hs[0], hs[2])
    Kx, Vx, wx = host(*E.coreset_export(hs[0]))
    for hd in range(h):
        ors = []
        for a, b in parts:
            ors.append(ocs.MergeReduceCoreset(d, dv, p, B, C0, SEED, heads=h, head=hd)
                       .update(K[hd][a:b], V[hd][a:b]))
        ors[0].merge(ors[1]).merge(ors[2])
        Ko, Vo, wo = ors[0].points()
        assert np.array_equal(Ko, Kx[hd]) and np.array_equal(Vo, Vx[hd])
        assert np.array_equal(wo, wx[hd])
    # the sources are unchanged
    K1, _, _ = host(*E.coreset_export(hs[1]))
    Ko1, _, _ = ocs.MergeReduceCoreset(d, dv, p, B, C0, SEED, heads=h, head=0).update(
        K[0][1100:1937], V[0][1100:1937]).points()
    assert np.array_equal(K1[0], Ko1)
    for c in hs:
        c.destroy()


def test_reset_and_errors():
    d, dv, p, h, B = 8, 8, 2, 1, 64
    K, V, _ = _inputs(d, dv, 500, 1, h, 1.0, seed=6)
    Kg, Vg = gpu(K, V)
    cs = E.coreset_create(d, dv, p, h, block=B, c0=C0, seed=SEED)
    E.coreset_update(cs, Kg, Vg)
    E.coreset_reset(cs)
    assert cs.info() == (0, 0, 0)
    E.coreset_update(cs, Kg, Vg)
    _check_points(cs, K, V, d, dv, p, h, B, [(0, 500)], "after reset")
    other = E.coreset_create(d, dv, p, h, block=128)
    with pytest.raises(E.SketchError):
        E.coreset_merge(cs, other)
    with pytest.raises(E.SketchError):
        E.coreset_create(d, dv, p, h, block=100)
    cs.destroy()
    other.destroy()


def test_full_size_workload2():
    """Workload 2 at full size (65,536 keys in 16 calls of 4096), blocks of 512:
    127 reduces; every kept point against the oracle."""
    w = WORKLOADS[2]
    K, V, Q = generate(w)
    calls = _calls(w.n, w.chunk)
    cs = _run_gpu(K, V, w.d, w.dv, w.p, w.h, 512, calls)
    _check_points(cs, K, V, w.d, w.dv, w.p, w.h, 512, calls, w.name)
    cs.destroy()


def test_32_heads_sampled():
    """The 32-head shape (d = dv = 64, p = 2) with 16,384 keys per head, blocks of
    512 (31 reduces per head, run as batches across heads): heads 0 and 31 against
    the oracle."""
    w = WORKLOADS[4].scaled(n=16384, m=8)
    K, V, Q = generate(w)
    calls = _calls(w.n, 0)
    cs = _run_gpu(K, V, w.d, w.dv, w.p, w.h, 512, calls)
    _check_points(cs, K, V, w.d, w.dv, w.p, w.h, 512, calls, "32 heads", heads_checked=[0, 31])
    cs.destroy()
