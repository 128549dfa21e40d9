"""GPU parity through the C ABI against the float64 oracle (MI355X only).

Small cases compare every output; they span several tiles and a ragged tail of
keys, chunks and queries.  Full-size cases run each workload exactly as the
benchmark does and compare every query, which the oracle answers by its direct
route over the whole stream.  Bars: sketch rel <= 2e-4 on Zhat and abs <= 2e-4 on ohat;
exact rel <= 1e-5 on Z and abs <= 1e-5 on o.
"""

import numpy as np
import pytest
import torch

import oracle
import exp_density_sketching_amd as E
from exp_density_sketching_amd.workload import ingest, run_sketch
from synthetic import WORKLOADS, generate
from tests.gpu_util import (SK_Z_REL, SK_O_ABS, EX_Z_REL, EX_O_ABS, gpu, host, zrel,
                            oabs, say)

pytestmark = pytest.mark.gpu


def _queries(qidx, hd, m):
    """Query indices checked on head hd: all (None), one array for every head, or
    a list with one entry (array or None) per head."""
    sel = qidx[hd] if isinstance(qidx, list) else qidx
    return np.arange(m) if sel is None else sel


def _check_sketch(w, K, V, Q, qidx=None, label="", layout="full"):
    Kg, Vg, Qg = gpu(K, V, Q)
    out, Z, sk = run_sketch(w, Kg, Vg, Qg, layout=layout)
    out, Z = host(out, Z)
    worst_z, worst_o = 0.0, 0.0
    for hd in range(w.h):
        qi = _queries(qidx, hd, Q.shape[1])
        o_ref, z_ref = oracle.sketch_direct(K[hd], V[hd], Q[hd][qi], w.p)
        worst_z = max(worst_z, zrel(Z[hd][qi], z_ref))
        worst_o = max(worst_o, oabs(out[hd][qi], o_ref))
    say(f"{label} sketch ({layout}): max rel Zhat err {worst_z:.3e}, "
        f"max abs ohat err {worst_o:.3e}")
    assert worst_z <= SK_Z_REL
    assert worst_o <= SK_O_ABS
    sk.destroy()


def _check_exact(w, K, V, Q, qidx=None, label=""):
    Kg, Vg, Qg = gpu(K, V, Q)
    out, Z = E.exact_attend(Kg, Vg, Qg)
    out, Z = host(out, Z)
    worst_z, worst_o = 0.0, 0.0
    for hd in range(w.h):
        qi = _queries(qidx, hd, Q.shape[1])
        o_ref, z_ref = oracle.exact_attention(K[hd], V[hd], Q[hd][qi])
        worst_z = max(worst_z, zrel(Z[hd][qi], z_ref))
        worst_o = max(worst_o, oabs(out[hd][qi], o_ref))
    say(f"{label} exact: max rel Z err {worst_z:.3e}, max abs o err {worst_o:.3e}")
    assert worst_z <= EX_Z_REL
    assert worst_o <= EX_O_ABS


# Small versions: every output compared.  Ragged n, chunk and m on purpose.
SMALL = {
    1: dict(n=4096, m=64),
    "1r": dict(n=4097, m=65, chunk=1000),
    2: dict(n=2 * 4096 + 37, m=200),
    3: dict(n=8192 + 5, m=300),
    4: dict(n=5000, m=70, h=3),
    5: dict(n=3001, m=130),
}


def _small(key):
    ident = key if isinstance(key, int) else int(str(key)[0])
    return WORKLOADS[ident].scaled(**SMALL[key])


@pytest.mark.parametrize("key", list(SMALL))
def test_sketch_small(key):
    w = _small(key)
    K, V, Q = generate(w)
    _check_sketch(w, K, V, Q, label=f"small {key}")


@pytest.mark.parametrize("key", list(SMALL))
def test_exact_small(key):
    w = _small(key)
    K, V, Q = generate(w)
    _check_exact(w, K, V, Q, label=f"small {key}")


@pytest.mark.parametrize("ident,n,h", [(1, 999, 1), (2, 700, 1), (3, 600, 1), (4, 300, 2),
                                       (5, 150, 1), (2, 2501, 2), (3, 1601, 2)])
def test_state_matches_oracle_moments(ident, n, h):
    """The exported [M | N] equals the oracle's moments entry by entry, within
    fp32 rounding of the sum of absolute terms (oracle run on |K|, |V|)."""
    w = WORKLOADS[ident].scaled(n=n, m=1, h=h, chunk=256 if ident in (2, 3) else 0,
                              substreams=2 if ident == 3 else 1)
    K, V, Q = generate(w)
    Kg, Vg = gpu(K, V)
    sk, _ = ingest(w, Kg, Vg)
    S = host(E.sketch_export(sk))[0]
    for hd in range(h):
        ref = oracle.MomentSketch(w.d, w.dv, w.p).update(K[hd], V[hd]).canonical_state()
        mag = oracle.MomentSketch(w.d, w.dv, w.p).update(
            np.abs(K[hd].astype(np.float64)), np.abs(V[hd].astype(np.float64))).canonical_state()
        err = np.abs(S[hd] - ref)
        assert S[hd].shape == ref.shape
        assert np.all(err <= 2e-6 * mag + 1e-30), float((err / (mag + 1e-30)).max())
    ptr, D, cols, cnt = E.sketch_state(sk)
    assert ptr and D == w.D and cols == 1 + w.dv and cnt == n


# (16, 64, 3) .. (4, 64, 4) put 64 or more columns (d + dv, or dv at the top) on
# levels j >= 1, where the query contracts the whole level without folding a
# digit; (32, 32, 2) .. (16, 16, 3) have levels of 8, 16 or 32 columns, whose last
# digit the query moves to the column side for d >= 16 (d C = 128 up to 2048
# columns; 32-column levels from j = 2 on: (32, 32, 2) and (64, 32, 2) at the top,
# (16, 16, 3) below it, (32, 32, 3) both) and contracts with folded
# trailing digits for d <= 8
@pytest.mark.parametrize("d,dv,p", [(8, 4, 0), (8, 4, 1), (16, 4, 3), (4, 32, 2),
                                    (128, 128, 1), (32, 8, 2), (32, 16, 2),
                                    (64, 16, 1), (128, 16, 1),
                                    (16, 64, 3), (8, 64, 3), (4, 64, 4), (32, 32, 2),
                                    (4, 4, 7), (64, 8, 2), (8, 8, 4), (16, 16, 3),
                                    (64, 32, 2), (32, 32, 3)])
def test_other_shapes(d, dv, p):
    w = WORKLOADS[1].scaled(n=1537, m=129)
    w = type(w)(**{**w.__dict__, "d": d, "dv": dv, "p": p, "key_r": 0.8})
    K, V, Q = generate(w)
    _check_sketch(w, K, V, Q, label=f"d={d} dv={dv} p={p}")
    _check_exact(w, K, V, Q, label=f"d={d} dv={dv} p={p}")


@pytest.mark.parametrize("d,dv,p,n", [(16, 16, 6, 1024), (32, 8, 5, 768)])
def test_deep_levels_digit_kernel(d, dv, p, n):
    """Levels with two and three leading digits on the digit-organised kernel
    (d = 16 up to degree 6, d = 32 up to degree 5; the states are 1.2 GB), against
    the oracle's direct route."""
    w = WORKLOADS[1].scaled(n=n, m=64)
    w = type(w)(**{**w.__dict__, "d": d, "dv": dv, "p": p, "key_r": 0.8})
    s = E.sketch_create(d, dv, p, 1)
    try:
        assert E.sketch_update_path(s) == "digits"
    finally:
        s.destroy()
    K, V, Q = generate(w)
    _check_sketch(w, K, V, Q, label=f"d={d} dv={dv} p={p}")


def test_decode_mode_exact():
    """m = 1..8 queries per head takes the streaming kernel."""
    for m in (1, 2, 3, 5, 8):
        w = WORKLOADS[4].scaled(n=9001, m=m, h=4)
        K, V, Q = generate(w)
        _check_exact(w, K, V, Q, label=f"decode m={m}")


def test_empty_and_degenerate():
    sk = E.sketch_create(8, 4, 3)
    rng = np.random.default_rng(5)
    Q = gpu(rng.standard_normal((5, 8)).astype(np.float32))[0]
    out, Z = E.sketch_query(sk, Q)
    out, Z = host(out, Z)
    assert np.all(Z == 0.0) and np.all(np.isnan(out))
    # n = 0 update is a no-op
    E.sketch_update(sk, torch.empty(0, 8, device="cuda"), torch.empty(0, 4, device="cuda"))
    assert sk.count == 0
    # exact over an empty stream
    o, z = E.exact_attend(torch.empty(1, 0, 8, device="cuda"),
                          torch.empty(1, 0, 4, device="cuda"), Q[None])
    o, z = host(o, z)
    assert np.all(z == 0.0) and np.all(np.isnan(o))
    # q = 0: Zhat = Z = n, outputs = mean of the values
    K, V = gpu((rng.standard_normal((777, 8)) * 0.3).astype(np.float32),
               rng.standard_normal((777, 4)).astype(np.float32))
    E.sketch_update(sk, K, V)
    q0 = torch.zeros(3, 8, device="cuda")
    out, Z = host(*E.sketch_query(sk, q0))
    vbar = V.double().mean(0).cpu().numpy()
    assert np.all(np.abs(Z - 777) <= 777 * 1e-6)
    assert oabs(out, np.tile(vbar, (3, 1))) <= 1e-5
    # reset empties the sketch
    E.sketch_reset(sk)
    assert sk.count == 0
    S = host(E.sketch_export(sk))[0]
    assert np.all(S == 0.0)
    sk.destroy()


def test_merge_mismatch_and_determinism():
    a = E.sketch_create(8, 8, 3)
    b = E.sketch_create(8, 8, 2)
    with pytest.raises(E.SketchError) as ei:
        E.sketch_merge(a, b)
    assert ei.value.code == -3
    w = WORKLOADS[5].scaled(n=20000, m=100)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    outs = []
    for _ in range(2):
        o, z, sk = run_sketch(w, Kg, Vg, Qg)
        outs.append(host(o, z, E.sketch_export(sk)))
        sk.destroy()
    for x, y in zip(*outs):
        assert np.array_equal(x, y)
    a.destroy()
    b.destroy()


def test_merge_equals_single_stream():
    w = WORKLOADS[2].scaled(n=9000, m=64, chunk=1024)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    whole, _ = ingest(w, Kg, Vg)
    parts, _ = ingest(w.scaled(substreams=3), Kg, Vg)
    S1, S2 = host(E.sketch_export(whole), E.sketch_export(parts))
    mag = np.abs(S1).max()
    assert np.abs(S1 - S2).max() <= 1e-6 * mag
    assert parts.count == whole.count == 9000


# Full-size workloads, run as the benchmark runs them.  Every query of workloads
# 1 and 2; the others, whose oracle takes minutes over all queries, a sample that
# keeps the first and last query: 256 of workload 3's 4096, 512 of workload 5's
# 2048, and on the 32-head workload all 256 queries of heads 0, 1, 30 and 31 and
# 8 queries of every other head.
FULL_SAMPLE = {1: None, 2: None, 3: 256, 4: None, 5: 512}


@pytest.mark.parametrize("ident", [1, 2, 3, 4, 5])
def test_full_size(ident):
    w = WORKLOADS[ident]
    say(f"full workload {ident}: {w.name} generating inputs")
    K, V, Q = generate(w)
    ns = FULL_SAMPLE[ident]
    qidx = None
    if ns is not None:
        rng = np.random.default_rng(1234 + ident)
        qidx = np.sort(rng.choice(w.m, size=ns, replace=False))
        qidx[0] = 0
        qidx[-1] = w.m - 1
    if w.h > 4:
        # all queries of the first two and last two heads, 8 of each other head
        rng = np.random.default_rng(1234 + ident)
        few = np.sort(rng.choice(w.m, size=8, replace=False))
        full_heads = {0, 1, w.h - 2, w.h - 1}
        qidx = [None if hd in full_heads else few for hd in range(w.h)]
    _check_sketch(w, K, V, Q, qidx=qidx, label=f"full {ident}")
    _check_exact(w, K, V, Q, qidx=qidx, label=f"full {ident}")


def test_full_size_decode_exact():
    """Decode shape of the 32-head workload: one query per head over 128K keys."""
    w = WORKLOADS[4].scaled(m=1)
    K, V, Q = generate(w)
    _check_exact(w, K, V, Q, label="decode 32x128K")


def test_full_size_single_head_decode_exact():
    """Decode over one long head (d = dv = 32, 1M keys): hundreds of slices folded
    per query, m = 1 and 3."""
    for m in (1, 3):
        w = WORKLOADS[3].scaled(m=m)
        K, V, Q = generate(w)
        _check_exact(w, K, V, Q, label=f"decode 1x1M m={m}")


def test_sketch_error_within_bound():
    """GPU sketch against GPU exact, against the truncation bound (high-temperature
    workloads, where the bound is informative)."""
    for ident in (1, 2, 4):
        w = WORKLOADS[ident].scaled(n=16384, m=128, h=min(WORKLOADS[ident].h, 2))
        K, V, Q = generate(w)
        Kg, Vg, Qg = gpu(K, V, Q)
        o_s, z_s, sk = run_sketch(w, Kg, Vg, Qg)
        o_e, z_e = E.exact_attend(Kg, Vg, Qg)
        o_s, z_s, o_e, z_e = host(o_s, z_s, o_e, z_e)
        for hd in range(w.h):
            rho = oracle.measured_radius(K[hd], Q[hd])
            bound = oracle.kde_relative_bound(w.p, rho)
            err = np.abs(z_s[hd] - z_e[hd]) / z_e[hd]
            say(f"workload {ident}: sketch-vs-exact max rel Z err {err.max():.3e} "
                f"(bound {bound:.3e})")
            assert np.all(err <= bound + 4 * SK_Z_REL)
        sk.destroy()


def test_kernel_timing_events():
    """sketch_timing records one event pair per update/query kernel launch."""
    w = WORKLOADS[2].scaled(n=3 * 4096, m=200)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    sk = E.sketch_create(w.d, w.dv, w.p)
    E.sketch_set_staging(sk, 0)         # one update launch per call
    E.sketch_timing(sk, True)
    for c0 in range(0, w.n, 4096):
        E.sketch_update(sk, Kg[:, c0:c0 + 4096], Vg[:, c0:c0 + 4096])
    E.sketch_query(sk, Qg)
    ups = E.sketch_kernel_times(sk, "update")
    qs = E.sketch_kernel_times(sk, "query")
    assert len(ups) == 3 and all(t > 0 for t in ups)
    assert len(qs) == 1 and qs[0] > 0
    assert E.sketch_kernel_times(sk, "update") == []
    E.sketch_timing(sk, False)
    E.sketch_update(sk, Kg[:, :4096], Vg[:, :4096])
    assert E.sketch_kernel_times(sk, "update") == []
    sk.destroy()


@pytest.mark.parametrize("staging", [0, None])
@pytest.mark.parametrize("layout", ["full", "sym"])
def test_pending_partials_are_always_added(layout, staging):
    """Split update calls leave their partials for the next launch to add; every
    reader (export, query, merge) and reset must see the right state.  Calls of
    4096 keys (split) alternate with calls of 100 keys (one split, added in
    place); a reset drops what is pending; a merge takes pending partials of
    both sides."""
    w = WORKLOADS[2].scaled(n=25000, m=8)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    sizes = [4096, 4096, 100, 4096, 257, 4096, 4096]
    bounds = np.cumsum([0] + sizes)
    a = E.sketch_create(w.d, w.dv, w.p, 1, layout)
    if staging is not None:
        E.sketch_set_staging(a, staging)     # 0: every call launches (split partials)
    # garbage that the reset must drop, pending at the time of the reset
    E.sketch_update(a, Kg[:, :4096], Vg[:, :4096])
    E.sketch_update(a, Kg[:, 4096:8192], Vg[:, 4096:8192])
    E.sketch_reset(a)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        E.sketch_update(a, Kg[:, lo:hi], Vg[:, lo:hi])
    n_a = int(bounds[-1])
    # a second sketch with its own pending partials, merged into the first
    b = E.sketch_create(w.d, w.dv, w.p, 1, layout)
    if staging is not None:
        E.sketch_set_staging(b, staging)
    E.sketch_update(b, Kg[:, n_a:n_a + 4096 + 2], Vg[:, n_a:n_a + 4096 + 2])
    E.sketch_merge(a, b)
    n = n_a + 4096 + 2
    S = host(E.sketch_export(a))[0][0]
    Ref = oracle.SymMomentSketch if layout == "sym" else oracle.MomentSketch
    ref = Ref(w.d, w.dv, w.p).update(K[0, :n], V[0, :n]).canonical_state()
    mag = Ref(w.d, w.dv, w.p).update(np.abs(K[0, :n].astype(np.float64)),
                                     np.abs(V[0, :n].astype(np.float64))).canonical_state()
    assert a.count == n
    assert np.all(np.abs(S - ref) <= 2e-6 * mag + 1e-30)
    out, Z = host(*E.sketch_query(a, Qg))
    o_ref, z_ref = oracle.sketch_direct(K[0, :n], V[0, :n], Q[0], w.p)
    assert zrel(Z[0], z_ref) <= SK_Z_REL and oabs(out[0], o_ref) <= SK_O_ABS
    a.destroy()
    b.destroy()


@pytest.mark.parametrize("layout", ["full", "sym"])
def test_staged_calls_equal_direct_calls(layout):
    """Staged small calls (default staging) give the moments of the same keys as
    one direct call; staged keys are contracted before every reader, dropped by
    reset, and kept in order around a large call and a staging change."""
    w = WORKLOADS[2].scaled(n=40000, m=16, h=2)
    K, V, Q = generate(w)
    Kg, Vg, Qg = gpu(K, V, Q)
    st = E.sketch_create(w.d, w.dv, w.p, 2, layout)
    E.sketch_update(st, Kg[:, :300].contiguous(), Vg[:, :300].contiguous())
    E.sketch_reset(st)                             # staged keys dropped
    cuts = [0, 1000, 1001, 4097, 20000, 20033, 24000, 40000]
    for i, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        if i == 4:
            E.sketch_set_staging(st, 2048)         # change of size mid-stream
        E.sketch_update(st, Kg[:, lo:hi].contiguous(), Vg[:, lo:hi].contiguous())
    assert st.count == 40000
    ref = E.sketch_create(w.d, w.dv, w.p, 2, layout)
    E.sketch_set_staging(ref, 0)
    E.sketch_update(ref, Kg, Vg)
    o1, z1 = host(*E.sketch_query(st, Qg))
    o2, z2 = host(*E.sketch_query(ref, Qg))
    assert zrel(z1, z2) <= 1e-5 and oabs(o1, o2) <= 1e-5
    S1, S2 = host(E.sketch_export(st), E.sketch_export(ref))
    assert np.abs(S1 - S2).max() <= 1e-5 * np.abs(S2).max()
    # merge and decode step with keys still staged on both sides
    a = E.sketch_create(w.d, w.dv, w.p, 2, layout)
    b = E.sketch_create(w.d, w.dv, w.p, 2, layout)
    E.sketch_update(a, Kg[:, :3000].contiguous(), Vg[:, :3000].contiguous())
    E.sketch_update(b, Kg[:, 3000:6000].contiguous(), Vg[:, 3000:6000].contiguous())
    E.sketch_merge(a, b)
    out, Z = host(*E.sketch_step(a, Kg[:, 6000].contiguous(), Vg[:, 6000].contiguous(),
                                 Qg[:, 0].contiguous()))
    for hd in range(2):
        o_ref, z_ref = oracle.sketch_direct(K[hd, :6001], V[hd, :6001], Q[hd, :1], w.p)
        assert abs(Z[hd] - z_ref[0]) / z_ref[0] <= SK_Z_REL
        assert np.max(np.abs(out[hd] - o_ref[0])) <= SK_O_ABS
    for x in (st, ref, a, b):
        x.destroy()


@pytest.mark.gpu
@pytest.mark.parametrize("d,layout,want", [(16, "full", "digits"), (32, "full", "digits"),
                                           (64, "full", "digits"), (8, "full", "tiles"),
                                           (128, "full", "tiles"), (16, "sym", "multiset")])
def test_update_path(d, layout, want):
    """Key widths 16, 32 and 64 run the digit-organised kernel, the others the
    tile kernel (both checked against the oracle above); the multiset layout its
    own."""
    s = E.sketch_create(d, d, 2, 1, layout)
    try:
        assert E.sketch_update_path(s) == want
    finally:
        s.destroy()


# Levels of nine or more digits: the query's split keeps at most eight digits on
# its row side and folds the rest in the epilogue (d = 4 with wide value rows, so
# the plain split would put every digit on the row side).
@pytest.mark.parametrize("d,dv,p", [(4, 64, 9), (4, 32, 10), (4, 8, 11), (4, 4, 12)])
def test_deep_levels(d, dv, p):
    w = WORKLOADS[1].scaled(n=333, m=45)
    w = type(w)(**{**w.__dict__, "d": d, "dv": dv, "p": p, "key_r": 0.9})
    K, V, Q = generate(w)
    _check_sketch(w, K, V, Q, label=f"deep d={d} dv={dv} p={p}")
