"""ctypes binding of libexpsketch.so: argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI declared in
include/expsketch.h.  PyTorch supplies device memory (CUDA/HIP tensors) and the
current stream.  There is no CPU path: if the library is not built, loading it
raises immediately.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libexpsketch.so")

SK_OK, SK_EINVAL, SK_ENOMEM, SK_EMISMATCH, SK_EHIP, SK_ESCRATCH = 0, -1, -2, -3, -4, -5
LAYOUTS = {"full": 0, "sym": 1}

EXPORTED = ("sketch_create", "sketch_create_ex", "sketch_layout", "sketch_update_path",
            "sketch_destroy",
            "sketch_set_stream", "sketch_reset", "sketch_update", "sketch_merge",
            "sketch_query", "sketch_step", "sketch_set_center", "sketch_set_staging",
            "exact_attend", "exact_attend_noalloc", "exact_release_workspaces",
            "exact_timing", "exact_kernel_times",
            "sketch_state", "sketch_export", "sketch_info", "sketch_timing",
            "sketch_kernel_times", "sk_strerror", "sk_version",
            "coreset_create", "coreset_destroy", "coreset_set_stream", "coreset_reset",
            "coreset_update", "coreset_merge", "coreset_query", "coreset_info",
            "coreset_export")


class SketchError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        msg = _lib().sk_strerror(code).decode() if _LIB is not None else str(code)
        super().__init__(f"{where}: {msg} (status {code})")


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m exp_density_sketching_amd.build` (there is no CPU fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        c_int, c_i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        sig = {
            "sketch_create": (c_int, [c_int, c_int, c_int, c_int, vp, ctypes.POINTER(vp)]),
            "sketch_create_ex": (c_int, [c_int, c_int, c_int, c_int, c_int, vp,
                                         ctypes.POINTER(vp)]),
            "sketch_layout": (c_int, [vp, ctypes.POINTER(c_int), ctypes.POINTER(c_i64)]),
            "sketch_update_path": (c_int, [vp, ctypes.POINTER(c_int)]),
            "sketch_destroy": (c_int, [vp]),
            "sketch_set_stream": (c_int, [vp, vp]),
            "sketch_reset": (c_int, [vp]),
            "sketch_update": (c_int, [vp, vp, vp, c_i64]),
            "sketch_merge": (c_int, [vp, vp]),
            "sketch_query": (c_int, [vp, vp, c_i64, vp, vp]),
            "sketch_step": (c_int, [vp, vp, vp, vp, vp, vp]),
            "sketch_set_center": (c_int, [vp, vp]),
            "sketch_set_staging": (c_int, [vp, c_i64]),
            "exact_attend": (c_int, [vp, vp, c_i64, c_int, c_int, c_int, vp, c_i64, vp,
                                     vp, vp]),
            "exact_attend_noalloc": (c_int, [vp, vp, c_i64, c_int, c_int, c_int, vp, c_i64,
                                             vp, vp, vp]),
            "exact_release_workspaces": (c_int, []),
            "exact_timing": (c_int, [c_int]),
            "exact_kernel_times": (c_int, [ctypes.POINTER(ctypes.c_float), c_int,
                                           ctypes.POINTER(c_int)]),
            "sketch_state": (c_int, [vp, ctypes.POINTER(vp), ctypes.POINTER(c_i64),
                                     ctypes.POINTER(c_int), ctypes.POINTER(c_i64)]),
            "sketch_export": (c_int, [vp, vp]),
            "sketch_info": (c_int, [vp, ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                    ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                    ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]),
            "sketch_timing": (c_int, [vp, c_int]),
            "sketch_kernel_times": (c_int, [vp, c_int, ctypes.POINTER(ctypes.c_float), c_int,
                                            ctypes.POINTER(c_int)]),
            "coreset_create": (c_int, [c_int, c_int, c_int, c_int, c_int, ctypes.c_double,
                                       ctypes.c_uint64, vp, ctypes.POINTER(vp)]),
            "coreset_destroy": (c_int, [vp]),
            "coreset_set_stream": (c_int, [vp, vp]),
            "coreset_reset": (c_int, [vp]),
            "coreset_update": (c_int, [vp, vp, vp, c_i64]),
            "coreset_merge": (c_int, [vp, vp]),
            "coreset_query": (c_int, [vp, vp, c_i64, vp, vp]),
            "coreset_info": (c_int, [vp, ctypes.POINTER(c_i64), ctypes.POINTER(c_i64),
                                     ctypes.POINTER(c_i64)]),
            "coreset_export": (c_int, [vp, vp, vp, vp]),
            "sk_strerror": (ctypes.c_char_p, [c_int]),
            "sk_version": (c_int, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(code, where):
    if code != SK_OK:
        raise SketchError(code, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dims):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous float32")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _heads(t, name):
    """Accept [n, x] (one head) or [h, n, x]; return the 3-d view."""
    if t.dim() == 2:
        return t.unsqueeze(0)
    if t.dim() != 3:
        raise ValueError(f"{name} must be [n, x] or [h, n, x]")
    return t


class Sketch:
    """A handle of the C library (sketch_create_ex ... sketch_destroy).

    layout "full" keeps every Kronecker index tuple (D = sum_j d^j rows); "sym"
    keeps one entry per multiset of indices (C(d + p, p) rows, same answers)."""

    def __init__(self, d, dv, p, h=1, layout="full"):
        lib = _lib()
        if layout not in LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
        handle = ctypes.c_void_p()
        _check(lib.sketch_create_ex(d, dv, p, h, LAYOUTS[layout], _stream(),
                                    ctypes.byref(handle)), "sketch_create_ex")
        self._h = handle
        self.d, self.dv, self.p, self.h = d, dv, p, h
        self.layout = layout
        rows = ctypes.c_int64()
        _check(lib.sketch_layout(handle, None, ctypes.byref(rows)), "sketch_layout")
        self.rows = rows.value

    def _handle(self):
        if self._h is None:
            raise RuntimeError("sketch destroyed")
        _check(_lib().sketch_set_stream(self._h, _stream()), "sketch_set_stream")
        return self._h

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            h, self._h = self._h, None
            _check(_lib().sketch_destroy(h), "sketch_destroy")

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    @property
    def D(self):
        return sum(self.d ** j for j in range(self.p + 1))

    @property
    def count(self):
        c = ctypes.c_int64()
        _check(_lib().sketch_info(self._h, None, None, None, None, None, ctypes.byref(c)),
               "sketch_info")
        return c.value


def sketch_create(d, dv, p, h=1, layout="full"):
    return Sketch(d, dv, p, h, layout)


def sketch_layout(s):
    """(layout name, rows of the canonical view)."""
    lay = ctypes.c_int()
    rows = ctypes.c_int64()
    _check(_lib().sketch_layout(s._handle(), ctypes.byref(lay), ctypes.byref(rows)),
           "sketch_layout")
    return {v: k for k, v in LAYOUTS.items()}[lay.value], rows.value


UPDATE_PATHS = {0: "tiles", 1: "digits", 2: "multiset"}
UPDATE_KERNELS = {"tiles": "sk_update_kernel", "digits": "sk_update_kr_kernel",
                  "multiset": "sk_sym_update_kernel"}


def sketch_update_path(s):
    """Name of the kernel family the handle's updates launch: "tiles", "digits"
    or "multiset"."""
    kind = ctypes.c_int()
    _check(_lib().sketch_update_path(s._handle(), ctypes.byref(kind)), "sketch_update_path")
    return UPDATE_PATHS[kind.value]


def sketch_destroy(s):
    s.destroy()


def sketch_reset(s):
    _check(_lib().sketch_reset(s._handle()), "sketch_reset")


def sketch_update(s, K, V):
    """K [h, n, d] (or [n, d]), V [h, n, dv] (or [n, dv]) float32 GPU tensors."""
    K, V = _heads(K, "K"), _heads(V, "V")
    if K.shape[0] != s.h or V.shape[0] != s.h or K.shape[2] != s.d or V.shape[2] != s.dv \
            or K.shape[1] != V.shape[1]:
        raise ValueError(f"shape mismatch: K {tuple(K.shape)}, V {tuple(V.shape)} for "
                         f"h={s.h}, d={s.d}, dv={s.dv}")
    n = K.shape[1]
    _check(_lib().sketch_update(s._handle(), _dev(K, "K", 3), _dev(V, "V", 3), n),
           "sketch_update")


def sketch_merge(dst, src):
    _check(_lib().sketch_merge(dst._handle(), src._handle()), "sketch_merge")


def sketch_query(s, Q, out=None, Z=None):
    """Q [h, m, d] (or [m, d]) -> (out [h, m, dv], Z [h, m]) float32 GPU tensors."""
    squeeze = Q.dim() == 2
    Q = _heads(Q, "Q")
    if Q.shape[0] != s.h or Q.shape[2] != s.d:
        raise ValueError(f"Q {tuple(Q.shape)} does not match h={s.h}, d={s.d}")
    m = Q.shape[1]
    if out is None:
        out = torch.empty((s.h, m, s.dv), dtype=torch.float32, device=Q.device)
    if Z is None:
        Z = torch.empty((s.h, m), dtype=torch.float32, device=Q.device)
    _check(_lib().sketch_query(s._handle(), _dev(Q, "Q", 3), m, _dev(out, "out", 3),
                               _dev(Z, "Z", 2)), "sketch_query")
    return (out[0], Z[0]) if squeeze else (out, Z)


def sketch_set_center(s, c):
    """Recentre an empty sketch at c [h, d] (or [d] for one head); None removes it."""
    if c is None:
        _check(_lib().sketch_set_center(s._handle(), None), "sketch_set_center")
        return
    if c.dim() == 1:
        c = c.unsqueeze(0)
    if tuple(c.shape) != (s.h, s.d):
        raise ValueError(f"c {tuple(c.shape)} does not match h={s.h}, d={s.d}")
    _check(_lib().sketch_set_center(s._handle(), _dev(c.contiguous(), "c", 2)),
           "sketch_set_center")


def sketch_set_staging(s, keys):
    """Staging size of sketch_update in keys per head (0: off)."""
    _check(_lib().sketch_set_staging(s._handle(), int(keys)), "sketch_set_staging")


def sketch_step(s, k, v, q, out=None, Z=None):
    """One decode step per head: append (k, v), answer q over the stream with it.

    k [h, d], v [h, dv], q [h, d] (or 1-d for one head) -> (out [h, dv], Z [h])."""
    squeeze = k.dim() == 1
    if squeeze:
        k, v, q = k.unsqueeze(0), v.unsqueeze(0), q.unsqueeze(0)
    if tuple(k.shape) != (s.h, s.d) or tuple(v.shape) != (s.h, s.dv) or \
            tuple(q.shape) != (s.h, s.d):
        raise ValueError(f"k {tuple(k.shape)}, v {tuple(v.shape)}, q {tuple(q.shape)} do "
                         f"not match h={s.h}, d={s.d}, dv={s.dv}")
    if out is None:
        out = torch.empty((s.h, s.dv), dtype=torch.float32, device=k.device)
    if Z is None:
        Z = torch.empty((s.h,), dtype=torch.float32, device=k.device)
    _check(_lib().sketch_step(s._handle(), _dev(k, "k", 2), _dev(v, "v", 2), _dev(q, "q", 2),
                              _dev(out, "out", 2), _dev(Z, "Z", 1)), "sketch_step")
    return (out[0], Z[0]) if squeeze else (out, Z)


def sketch_export(s, dst=None, device=None):
    """Canonical [M | N] view into a new (or given) tensor [h, rows, 1 + dv]
    (rows = D for the full layout, C(d + p, p) for the multiset layout)."""
    if dst is None:
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        dst = torch.empty((s.h, s.rows, 1 + s.dv), dtype=torch.float32, device=dev)
    elif tuple(dst.shape) != (s.h, s.rows, 1 + s.dv):
        raise ValueError(f"dst must be [{s.h}, {s.rows}, {1 + s.dv}]")
    _check(_lib().sketch_export(s._handle(), _dev(dst, "dst", 3)), "sketch_export")
    return dst


def sketch_state(s):
    """(device pointer, D, cols, count) of the library-owned canonical view."""
    ptr = ctypes.c_void_p()
    D = ctypes.c_int64()
    cols = ctypes.c_int()
    cnt = ctypes.c_int64()
    _check(_lib().sketch_state(s._handle(), ctypes.byref(ptr), ctypes.byref(D),
                               ctypes.byref(cols), ctypes.byref(cnt)), "sketch_state")
    return ptr.value, D.value, cols.value, cnt.value


def sketch_timing(s, enable=True):
    _check(_lib().sketch_timing(s._h, 1 if enable else 0), "sketch_timing")


def sketch_kernel_times(s, kind):
    """Milliseconds of each recorded kernel of `kind` ("update", "query", "step")."""
    k = {"update": 0, "query": 1, "step": 2}[kind]
    cap = 256
    buf = (ctypes.c_float * cap)()
    cnt = ctypes.c_int()
    _check(_lib().sketch_kernel_times(s._h, k, buf, cap, ctypes.byref(cnt)),
           "sketch_kernel_times")
    return [buf[i] for i in range(min(cnt.value, cap))]


def exact_attend(K, V, Q, out=None, Z=None):
    """Exact KDE normaliser and softmax attention: K [h,n,d], V [h,n,dv], Q [h,m,d]."""
    squeeze = Q.dim() == 2
    K, V, Q = _heads(K, "K"), _heads(V, "V"), _heads(Q, "Q")
    h, n, d = K.shape
    dv = V.shape[2]
    m = Q.shape[1]
    if V.shape[:2] != (h, n) or Q.shape[0] != h or Q.shape[2] != d:
        raise ValueError(f"shape mismatch: K {tuple(K.shape)}, V {tuple(V.shape)}, "
                         f"Q {tuple(Q.shape)}")
    if out is None:
        out = torch.empty((h, m, dv), dtype=torch.float32, device=Q.device)
    if Z is None:
        Z = torch.empty((h, m), dtype=torch.float32, device=Q.device)
    _check(_lib().exact_attend(_dev(K, "K", 3), _dev(V, "V", 3), n, d, dv, h,
                               _dev(Q, "Q", 3), m, _dev(out, "out", 3), _dev(Z, "Z", 2),
                               _stream()), "exact_attend")
    return (out[0], Z[0]) if squeeze else (out, Z)


def exact_attend_noalloc(K, V, Q, out, Z):
    """exact_attend with its partials in the library's fixed scratch array (nothing
    allocated by the library); out [h,m,dv] and Z [h,m] are the caller's."""
    K, V, Q = _heads(K, "K"), _heads(V, "V"), _heads(Q, "Q")
    h, n, d = K.shape
    dv = V.shape[2]
    m = Q.shape[1]
    if V.shape[:2] != (h, n) or Q.shape[0] != h or Q.shape[2] != d:
        raise ValueError(f"shape mismatch: K {tuple(K.shape)}, V {tuple(V.shape)}, "
                         f"Q {tuple(Q.shape)}")
    _check(_lib().exact_attend_noalloc(_dev(K, "K", 3), _dev(V, "V", 3), n, d, dv, h,
                                       _dev(Q, "Q", 3), m, _dev(out, "out", 3),
                                       _dev(Z, "Z", 2), _stream()), "exact_attend_noalloc")
    return out, Z


def exact_timing(enable=True):
    _check(_lib().exact_timing(1 if enable else 0), "exact_timing")


def exact_kernel_times():
    """Milliseconds of the recorded slice kernels of exact_attend calls."""
    cap = 256
    buf = (ctypes.c_float * cap)()
    cnt = ctypes.c_int()
    _check(_lib().exact_kernel_times(buf, cap, ctypes.byref(cnt)), "exact_kernel_times")
    return [buf[i] for i in range(min(cnt.value, cap))]


def exact_release_workspaces():
    """Free the partials buffers exact_attend keeps per (device, stream)."""
    _check(_lib().exact_release_workspaces(), "exact_release_workspaces")


class Coreset:
    """Tail coreset handle (coreset_create ... coreset_destroy): Merge-and-Reduce
    blocks of `block` points per head, each reduce a discrepancy halving."""

    def __init__(self, d, dv, p, h=1, block=512, c0=0.25, seed=0):
        handle = ctypes.c_void_p()
        _check(_lib().coreset_create(d, dv, p, h, block, float(c0), int(seed) & (2**64 - 1),
                                     _stream(), ctypes.byref(handle)), "coreset_create")
        self._h = handle
        self.d, self.dv, self.p, self.h, self.block = d, dv, p, h, block

    def _handle(self):
        if self._h is None:
            raise RuntimeError("coreset destroyed")
        _check(_lib().coreset_set_stream(self._h, _stream()), "coreset_set_stream")
        return self._h

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            h, self._h = self._h, None
            _check(_lib().coreset_destroy(h), "coreset_destroy")

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def info(self):
        """(points per head, points ingested per head, reduces done)."""
        pts, cnt, red = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(_lib().coreset_info(self._handle(), ctypes.byref(pts), ctypes.byref(cnt),
                                   ctypes.byref(red)), "coreset_info")
        return pts.value, cnt.value, red.value


def coreset_create(d, dv, p, h=1, block=512, c0=0.25, seed=0):
    return Coreset(d, dv, p, h, block, c0, seed)


def coreset_reset(c):
    _check(_lib().coreset_reset(c._handle()), "coreset_reset")


def coreset_update(c, K, V):
    """K [h, n, d] (or [n, d]), V [h, n, dv]: n more points per head."""
    K, V = _heads(K, "K"), _heads(V, "V")
    if K.shape[0] != c.h or K.shape[2] != c.d or V.shape[:2] != K.shape[:2] or V.shape[2] != c.dv:
        raise ValueError(f"shape mismatch: K {tuple(K.shape)}, V {tuple(V.shape)}")
    _check(_lib().coreset_update(c._handle(), _dev(K, "K", 3), _dev(V, "V", 3), K.shape[1]),
           "coreset_update")


def coreset_merge(dst, src):
    _check(_lib().coreset_merge(dst._handle(), src._handle()), "coreset_merge")


def coreset_query(c, Q, out, Z):
    """Adds the tail to the head answer (out [h, m, dv], Z [h, m]) in place."""
    Q = _heads(Q, "Q")
    if Q.shape[0] != c.h or Q.shape[2] != c.d:
        raise ValueError(f"Q must be [{c.h}, m, {c.d}]")
    _check(_lib().coreset_query(c._handle(), _dev(Q, "Q", 3), Q.shape[1], _dev(out, "out", 3),
                                _dev(Z, "Z", 2)), "coreset_query")
    return out, Z


def coreset_export(c):
    """(K [h, P, d], V [h, P, dv], w [h, P]) of the coreset's points."""
    pts = c.info()[0]
    dev = torch.device("cuda", torch.cuda.current_device())
    K = torch.empty((c.h, pts, c.d), dtype=torch.float32, device=dev)
    V = torch.empty((c.h, pts, c.dv), dtype=torch.float32, device=dev)
    w = torch.empty((c.h, pts), dtype=torch.float32, device=dev)
    if pts > 0:
        _check(_lib().coreset_export(c._handle(), _dev(K, "K", 3), _dev(V, "V", 3),
                                     _dev(w, "w", 2)), "coreset_export")
    return K, V, w


def raw():
    """The loaded ctypes library (for tests of the C ABI itself)."""
    return _lib()
