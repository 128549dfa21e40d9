"""The allocation-free exact path (exact_attend_noalloc) against exact_attend.

Two calls in a row on the library's fixed scratch, the second with a smaller
input, each compared with exact_attend on the same inputs to the exact path's
bars (rel 1e-5 on Z, abs 1e-5 on o); a shape whose partials must use fewer
slices to fit; a shape beyond the scratch (refused with SK_ESCRATCH).
"""

import numpy as np
import pytest
import torch

import exp_density_sketching_amd as E
from tests.gpu_util import EX_Z_REL, EX_O_ABS, gpu, host, zrel, oabs, say

pytestmark = pytest.mark.gpu


def _inputs(h, n, m, d, dv, seed):
    rng = np.random.default_rng(seed)
    K = (rng.standard_normal((h, n, d)) * 0.8 / np.sqrt(d)).astype(np.float32)
    V = rng.standard_normal((h, n, dv)).astype(np.float32)
    Q = (rng.standard_normal((h, m, d)) * 0.8 / np.sqrt(d)).astype(np.float32)
    return gpu(K, V, Q)


def _compare(h, n, m, d, dv, seed, label):
    Kg, Vg, Qg = _inputs(h, n, m, d, dv, seed)
    out = torch.full((h, m, dv), float("nan"), device="cuda")
    Z = torch.full((h, m), float("nan"), device="cuda")
    say(f"{label}: h={h} n={n} m={m} d={d} dv={dv}")
    E.exact_attend_noalloc(Kg, Vg, Qg, out, Z)
    o_ref, z_ref = E.exact_attend(Kg, Vg, Qg)
    o, z, o_ref, z_ref = host(out, Z, o_ref, z_ref)
    ez, eo = zrel(z, z_ref), oabs(o, o_ref)
    say(f"{label}: rel Z {ez:.2e}, abs o {eo:.2e}")
    assert ez <= EX_Z_REL and eo <= EX_O_ABS


def test_two_calls_second_smaller():
    _compare(3, 40000, 200, 32, 32, 1, "first call (batched)")
    _compare(2, 5000, 5, 16, 16, 2, "second call (decode, smaller)")


def test_fewer_slices_to_fit():
    # 8 heads x 4096 queries x 34 floats per slice: at most 3 slices fit
    _compare(8, 8192, 4096, 32, 32, 3, "slices lowered to fit the scratch")
    _compare(1, 300, 7, 8, 8, 4, "small call after it")


def test_beyond_the_scratch_is_refused():
    Kg, Vg, Qg = _inputs(32, 64, 2048, 4, 64, 5)
    out = torch.empty((32, 2048, 64), device="cuda")
    Z = torch.empty((32, 2048), device="cuda")
    with pytest.raises(E.SketchError) as err:
        E.exact_attend_noalloc(Kg, Vg, Qg, out, Z)
    assert err.value.code == -5


def test_decode_calls_in_a_row():
    """Decode calls (m <= 8) with other head counts, key counts and query counts
    in a row on the one scratch array: each must match exact_attend."""
    for i, (h, n, m) in enumerate([(3, 9000, 1), (7, 4000, 8), (2, 70000, 3), (3, 9000, 1)]):
        _compare(h, n, m, 16, 32, 10 + i, f"decode call {i}")
