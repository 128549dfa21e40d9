"""Helpers shared by the GPU parity tests: tolerances and comparisons."""

import numpy as np
import torch

# Acceptance bars: sketch vs the float64 oracle, exact path vs the float64 oracle.
SK_Z_REL = 2e-4
SK_O_ABS = 2e-4
EX_Z_REL = 1e-5
EX_O_ABS = 1e-5


def gpu(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]


def host(*tensors):
    torch.cuda.synchronize()
    return [t.detach().cpu().numpy().astype(np.float64) for t in tensors]


def zrel(z, zref):
    zref = np.asarray(zref, np.float64)
    return float(np.max(np.abs(np.asarray(z, np.float64) - zref) / np.abs(zref)))


def oabs(o, oref):
    return float(np.max(np.abs(np.asarray(o, np.float64) - np.asarray(oref, np.float64))))


def say(*a):
    print(*a, flush=True)
