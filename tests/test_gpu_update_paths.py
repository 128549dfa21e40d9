"""The two full-layout update kernels agree: at d = 16, 32 and 64 the digit-organised
kernel runs by default and the tile kernel only with EXPSKETCH_UPDATE_KR=0, a
setting read once per process, so the tile kernel runs in one child process on
the same seeded inputs and both are checked against the float64 oracle and each
other.  Likewise the digit kernel's cut of long calls into several launches
(EXPSKETCH_UPDATE_MAXKEYS lowers the cut to a few hundred keys)."""

import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import exp_density_sketching_amd as E
from exp_density_sketching_amd.workload import run_sketch
from synthetic import generate
from tests.gpu_util import SK_Z_REL, SK_O_ABS, gpu, host, oabs, say, zrel
from tests.test_gpu_parity import _small

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# child: same workloads under the environment it is given; writes <outdir>/<tag>_<key>.npz
_CHILD = r"""
import os, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import exp_density_sketching_amd as E
from exp_density_sketching_amd.workload import run_sketch
from synthetic import generate
from tests.gpu_util import gpu, host
from tests.test_gpu_parity import _small
for key in sys.argv[4:]:
    w = _small(int(key))
    K, V, Q = generate(w)
    out, Z, sk = run_sketch(w, *gpu(K, V, Q))
    S, out, Z = host(E.sketch_export(sk), out, Z)
    np.savez(os.path.join(sys.argv[2], "%s_%s.npz" % (sys.argv[3], key)), S=S, out=out, Z=Z,
             path=np.array(E.sketch_update_path(sk)))
    print("child: workload", key, "done", flush=True)
    sk.destroy()
"""


def _child(tmp_path, tag, keys, **env):
    say(f"child process ({tag}, {env}): workloads {keys} (small sizes)")
    res = subprocess.run([sys.executable, "-u", "-c", _CHILD, ROOT, str(tmp_path), tag] +
                         [str(k) for k in keys],
                         env=dict(os.environ, **env), cwd=ROOT, capture_output=True, text=True,
                         timeout=180)
    assert res.returncode == 0, res.stderr[-2000:]


def _compare(tmp_path, tag, keys, path):
    for key in keys:
        w = _small(key)
        K, V, Q = generate(w)
        out_d, Z_d, sk = run_sketch(w, *gpu(K, V, Q))
        assert E.sketch_update_path(sk) == "digits"
        S_d, out_d, Z_d = host(E.sketch_export(sk), out_d, Z_d)
        sk.destroy()
        c = np.load(tmp_path / f"{tag}_{key}.npz")
        assert str(c["path"]) == path
        S_t, out_t, Z_t = c["S"], c["out"], c["Z"]
        # the moments agree to fp32 summation order
        diff = np.abs(S_t - S_d).max() / np.abs(S_d).max()
        say(f"workload {key}: {tag} vs default state max rel diff {diff:.2e}")
        assert diff <= 1e-5
        for hd in range(w.h):
            o_ref, z_ref = oracle.sketch_direct(K[hd], V[hd], Q[hd], w.p)
            for o, z in ((out_d[hd], Z_d[hd]), (out_t[hd], Z_t[hd])):
                assert zrel(z, z_ref) <= SK_Z_REL and oabs(o, o_ref) <= SK_O_ABS


def test_tile_and_digit_kernels_agree(tmp_path):
    keys = [2, 3, 4]                    # d = 16 (p = 4), 32 (p = 3), 64 (p = 2, 3 heads)
    _child(tmp_path, "tiles", keys, EXPSKETCH_UPDATE_KR="0")
    _compare(tmp_path, "tiles", keys, "tiles")


def test_digit_kernel_long_call_cut(tmp_path):
    # the small cases stream 4096-key calls through staging; with a 300-key cut
    # every flush runs as several launches, the last one ragged and odd
    keys = [2, 3]
    _child(tmp_path, "cut", keys, EXPSKETCH_UPDATE_MAXKEYS="300")
    _compare(tmp_path, "cut", keys, "digits")


def test_digit_kernel_split_cap_large_state():
    """A 64-head state of 69 MB (d = dv = 64, p = 2) with 8192 keys per head: the
    update takes its waves in many rounds per SIMD, where the split chooser's cost
    is lowest at 16 to 24 key splits, whose partials (1.1-1.7 GB) would not fit
    the kept partial buffers (1 GiB each); the chooser then keeps to the split
    counts that fit (at most 15), so the call keeps the deferred reduce.  Sampled
    heads against the float64 oracle's direct route."""
    from synthetic import WORKLOADS
    w = WORKLOADS[4].scaled(n=8192, m=32, h=64)
    K, V, Q = generate(w)
    say(f"split cap: h={w.h} d={w.d} dv={w.dv} p={w.p} n={w.n} m={w.m}")
    out, Z, sk = run_sketch(w, *gpu(K, V, Q))
    out, Z = host(out, Z)
    sk.destroy()
    for hh in (0, 29, 63):
        o_ref, z_ref = oracle.sketch_direct(K[hh], V[hh], Q[hh], w.p)
        ez, eo = zrel(Z[hh], z_ref), oabs(out[hh], o_ref)
        say(f"  head {hh}: rel Z {ez:.2e} abs o {eo:.2e}")
        assert ez <= SK_Z_REL and eo <= SK_O_ABS
