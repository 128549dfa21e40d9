"""GPU parity of the multiset storage layout ("sym") through the C ABI (MI355X only).

The answers are compared with the oracle's plain definition sum_i T_p(<q, k_i>)
(the same values the full layout reaches), the stored entries with the oracle's
multiset moments (oracle.SymMomentSketch, itself pinned against np.kron-built
Kronecker moments and brute force).  Bars as for the full layout: sketch rel
<= 2e-4 on Zhat and abs <= 2e-4 on ohat; entries within fp32 rounding of the sum
of absolute terms.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exp_density_sketching_amd as E
from exp_density_sketching_amd.workload import ingest, run_sketch
from synthetic import WORKLOADS, generate
from tests.gpu_util import SK_Z_REL, SK_O_ABS, gpu, host, oabs, say, zrel
from tests.test_gpu_parity import SMALL, _check_sketch, _small

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key", list(SMALL))
def test_sym_sketch_small(key):
    w = _small(key)
    K, V, Q = generate(w)
    _check_sketch(w, K, V, Q, label=f"small {key}", layout="sym")


@pytest.mark.parametrize("ident,n,h", [(1, 999, 1), (2, 700, 1), (3, 600, 1), (4, 300, 2),
                                       (5, 150, 1)])
def test_sym_state_matches_oracle(ident, n, h):
    """The exported multiset entries equal the oracle's, entry by entry, within
    fp32 rounding of the sum of absolute terms (oracle run on |K|, |V|)."""
    w = WORKLOADS[ident].scaled(n=n, m=1, h=h, chunk=256 if ident in (2, 3) else 0,
                              substreams=2 if ident == 3 else 1)
    K, V, Q = generate(w)
    Kg, Vg = gpu(K, V)
    sk, _ = ingest(w, Kg, Vg, layout="sym")
    S = host(E.sketch_export(sk))[0]
    rows = math.comb(w.d + w.p, w.p)
    assert E.sketch_layout(sk) == ("sym", rows)
    for hd in range(h):
        ref = oracle.SymMomentSketch(w.d, w.dv, w.p).update(K[hd], V[hd]).canonical_state()
        mag = oracle.SymMomentSketch(w.d, w.dv, w.p).update(
            np.abs(K[hd].astype(np.float64)), np.abs(V[hd].astype(np.float64))).canonical_state()
        assert S[hd].shape == ref.shape == (rows, 1 + w.dv)
        err = np.abs(S[hd] - ref)
        assert np.all(err <= 2e-6 * mag + 1e-30), float((err / (mag + 1e-30)).max())
    ptr, D, cols, cnt = E.sketch_state(sk)
    assert ptr and D == rows and cols == 1 + w.dv and cnt == n


# blocks of 64 or more columns with multisets of at most 2 indices (d <= 64) are
# queried by the last index: (4, 64, 2), (8, 64, 2), (16, 64, 2), (32, 64, 2) and
# (64, 128, 2) put 16, 8, 4, 2 and 1 slots of paired prefix runs in a stage
# ((16, 64, 3), (64, 32, 3): one block would qualify, so both take the row-range
# kernel)
@pytest.mark.parametrize("d,dv,p", [(8, 4, 0), (8, 4, 1), (16, 4, 3), (4, 32, 2),
                                    (128, 128, 1), (4, 4, 7), (32, 8, 2), (64, 128, 2),
                                    (128, 4, 2), (4, 64, 2), (8, 64, 2), (16, 64, 2),
                                    (32, 64, 2), (16, 64, 3), (64, 32, 3)])
def test_sym_other_shapes(d, dv, p):
    w = WORKLOADS[1].scaled(n=1537, m=129)
    w = type(w)(**{**w.__dict__, "d": d, "dv": dv, "p": p, "key_r": 0.8})
    K, V, Q = generate(w)
    _check_sketch(w, K, V, Q, label=f"d={d} dv={dv} p={p}", layout="sym")


def test_sym_equals_full_layout():
    """Both layouts answer the same queries to fp32 rounding."""
    w = WORKLOADS[2].scaled(n=3 * 4096 + 11, m=300)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    of, zf, a = run_sketch(w, Kg, Vg, Qg, layout="full")
    os_, zs, b = run_sketch(w, Kg, Vg, Qg, layout="sym")
    of, zf, os_, zs = host(of, zf, os_, zs)
    assert zrel(zs, zf) <= SK_Z_REL and oabs(os_, of) <= SK_O_ABS
    a.destroy()
    b.destroy()


def test_sym_empty_degenerate_and_merge():
    sk = E.sketch_create(8, 4, 3, layout="sym")
    rng = np.random.default_rng(6)
    Q = gpu(rng.standard_normal((5, 8)).astype(np.float32))[0]
    out, Z = host(*E.sketch_query(sk, Q))
    assert np.all(Z == 0.0) and np.all(np.isnan(out))
    E.sketch_update(sk, torch.empty(0, 8, device="cuda"), torch.empty(0, 4, device="cuda"))
    assert sk.count == 0
    # q = 0: Zhat = n, ohat = mean of the values
    K, V = gpu((rng.standard_normal((777, 8)) * 0.3).astype(np.float32),
               rng.standard_normal((777, 4)).astype(np.float32))
    E.sketch_update(sk, K, V)
    out, Z = host(*E.sketch_query(sk, torch.zeros(3, 8, device="cuda")))
    vbar = V.double().mean(0).cpu().numpy()
    assert np.all(np.abs(Z - 777) <= 777 * 1e-6)
    assert oabs(out, np.tile(vbar, (3, 1))) <= 1e-5
    # layouts do not merge with each other
    full = E.sketch_create(8, 4, 3)
    with pytest.raises(E.SketchError) as ei:
        E.sketch_merge(sk, full)
    assert ei.value.code == -3
    # merge of two halves == one stream; reset empties
    a = E.sketch_create(8, 4, 3, layout="sym")
    b = E.sketch_create(8, 4, 3, layout="sym")
    E.sketch_update(a, K[:400], V[:400])
    E.sketch_update(b, K[400:], V[400:])
    E.sketch_merge(a, b)
    S1, S2 = host(E.sketch_export(a), E.sketch_export(sk))
    assert np.abs(S1 - S2).max() <= 1e-6 * np.abs(S2).max()
    assert a.count == 777
    E.sketch_reset(sk)
    assert sk.count == 0 and np.all(host(E.sketch_export(sk))[0] == 0.0)
    for x in (sk, full, a, b):
        x.destroy()


def test_sym_deterministic():
    w = WORKLOADS[5].scaled(n=20000, m=100)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    outs = []
    for _ in range(2):
        o, z, sk = run_sketch(w, Kg, Vg, Qg, layout="sym")
        outs.append(host(o, z, E.sketch_export(sk)))
        sk.destroy()
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("ident", [1, 2, 3, 4, 5])
def test_sym_full_size_sampled(ident):
    w = WORKLOADS[ident]
    say(f"full workload {ident}: {w.name} (multiset layout) generating inputs")
    K, V, Q = generate(w)
    rng = np.random.default_rng(4321 + ident)
    ns = min(w.m, 96 if w.h == 1 else 8)
    qidx = np.sort(rng.choice(w.m, size=ns, replace=False))
    qidx[0] = 0
    qidx[-1] = w.m - 1
    _check_sketch(w, K, V, Q, qidx=qidx, label=f"full {ident}", layout="sym")


def test_sym_kernel_timing_events():
    w = WORKLOADS[2].scaled(n=3 * 4096, m=200)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    sk = E.sketch_create(w.d, w.dv, w.p, layout="sym")
    E.sketch_set_staging(sk, 0)         # one update launch per call
    E.sketch_timing(sk, True)
    for c0 in range(0, w.n, 4096):
        E.sketch_update(sk, Kg[:, c0:c0 + 4096], Vg[:, c0:c0 + 4096])
    E.sketch_query(sk, Qg)
    ups = E.sketch_kernel_times(sk, "update")
    qs = E.sketch_kernel_times(sk, "query")
    assert len(ups) == 3 and all(t > 0 for t in ups)
    assert len(qs) == 1 and qs[0] > 0
    sk.destroy()


@pytest.mark.parametrize("layout", ["full", "sym"])
@pytest.mark.parametrize("d,dv,p,h,n,m,chunk", [
    (128, 128, 2, 1, 2000, 130, 0),      # wide rows, large state
    (4, 4, 2, 64, 700, 33, 0),           # many heads
    (16, 8, 3, 2, 50, 127, 1),           # one key per call: no splits
    (8, 16, 2, 1, 3000, 1, 1000),        # a single query
    (8, 8, 3, 1, 2500, 128, 0),          # exactly one query tile
    (8, 8, 3, 1, 2500, 129, 0),          # one query past a tile
])
def test_edge_shapes(layout, d, dv, p, h, n, m, chunk):
    w = WORKLOADS[1].scaled(n=n, m=m, h=h, chunk=chunk)
    w = type(w)(**{**w.__dict__, "d": d, "dv": dv, "p": p, "key_r": 0.8})
    K, V, Q = generate(w)
    _check_sketch(w, K, V, Q, label=f"edge d={d} dv={dv} p={p} h={h} n={n} m={m}",
                  layout=layout)
