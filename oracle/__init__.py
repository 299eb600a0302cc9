"""ctypes front end of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users; the product path (``selective_scan_amd``)
never imports it. It shares no code with the HIP library.

Every function upcasts its inputs to contiguous float64 (exact for bf16 and fp32
storage) and returns float64 arrays. Shapes and meaning follow the C header:

* ``scan``        Mamba-1 sequential recurrence         -> (y [B,L,D], h_final [B,D,N])
* ``scan_unroll`` the same, by brute-force unrolling     -> (y, h_final)
* ``ssd_seq``     SSD recurrence, scalar decay per head  -> (y [B,L,H,P], h_final [B,H,N,P])
* ``ssd_chunked`` SSD in chunked decayed-attention form  -> (y, h_final)
* ``ssd_unroll``  SSD by brute-force unrolling           -> (y, h_final)
* ``step``        one decode step                        -> (y [B,D], new state [B,D,N])
* ``ssd_step``    one SSD decode step                    -> (y [B,H,P], new state [B,H,N,P])
* ``scan_bwd``    gradient of ``scan`` for the loss sum(dy*y) + sum(dh_final*h_final)
                  -> dict of dx, ddelta, dA, dBm, dCm, dD, dz, dh0
* ``scan_disc``, ``step_disc``  ``scan`` / ``step`` with disc = "euler" | "zoh" and
                  Delta = softplus(delta + delta_bias) preprocessing
* ``scan3``       Mamba-3: complex transitions Are + i theta, exponential-trapezoidal
                  rule weighted by lam -> (y [B,L,D], h_final complex [B,D,N])
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


class Oracle:
    """Bindings to one build of the oracle library (the default one, or a test variant)."""

    def __init__(self, path=DEFAULT_LIB):
        if not os.path.exists(path):
            from . import build as _b
            _b.build(out=path)
        self.path = path
        self.lib = ctypes.CDLL(path)
        i, d = ctypes.c_int, _dp
        sig_scan = [i, i, i, i] + [d] * 10
        sig_ssd = [i, i, i, i, i] + [d] * 10
        for name, args in [("oracle_scan", sig_scan), ("oracle_scan_unroll", sig_scan),
                           ("oracle_ssd_seq", sig_ssd), ("oracle_ssd_unroll", sig_ssd),
                           ("oracle_ssd_chunked", [i] * 6 + [d] * 10),
                           ("oracle_step", [i, i, i] + [d] * 9),
                           ("oracle_ssd_step", [i, i, i, i] + [d] * 9),
                           ("oracle_scan_bwd", [i, i, i, i] + [d] * 18),
                           ("oracle_scan_disc", [i, i, i, i, i, d, i] + [d] * 10),
                           ("oracle_step_disc", [i, i, i, i, d, i] + [d] * 9),
                           ("oracle_scan3", [i, i, i, i] + [d] * 14)]:
            fn = getattr(self.lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        self.lib.oracle_set_threads.argtypes = [ctypes.c_int]
        self.lib.oracle_set_threads.restype = None
        self.lib.oracle_get_threads.argtypes = []
        self.lib.oracle_get_threads.restype = ctypes.c_int

    # -- threads ---------------------------------------------------------
    def set_threads(self, n):
        self.lib.oracle_set_threads(int(n))

    def get_threads(self):
        return int(self.lib.oracle_get_threads())

    # -- Mamba-1 -----------------------------------------------------------
    def _scan_like(self, fn, x, delta, A, Bm, Cm, D=None, z=None, h0=None):
        x, delta, A, Bm, Cm = map(_f64, (x, delta, A, Bm, Cm))
        D, z, h0 = _f64(D), _f64(z), _f64(h0)
        Bb, L, Dd = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and A.shape == (Dd, N)
        assert Bm.shape == (Bb, L, N) and Cm.shape == (Bb, L, N)
        assert D is None or D.shape == (Dd,)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (Bb, Dd, N)
        y = np.empty_like(x)
        hf = np.empty((Bb, Dd, N))
        rc = fn(Bb, L, Dd, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hf))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, hf

    def scan(self, *a, **k):
        return self._scan_like(self.lib.oracle_scan, *a, **k)

    def scan_unroll(self, *a, **k):
        return self._scan_like(self.lib.oracle_scan_unroll, *a, **k)

    def scan_bwd(self, x, delta, A, Bm, Cm, dy, D=None, z=None, h0=None, dh_final=None,
                 want_dh0=True):
        """Gradients of ``scan`` for l = sum(dy * y) + sum(dh_final * h_final).

        Returns a dict with dx, ddelta [B,L,D], dA [D,N], dBm, dCm [B,L,N],
        dD [D] (None without D), dz [B,L,D] (None without z), dh0 [B,D,N]
        (None unless want_dh0)."""
        x, delta, A, Bm, Cm, dy = map(_f64, (x, delta, A, Bm, Cm, dy))
        D, z, h0, dhf = _f64(D), _f64(z), _f64(h0), _f64(dh_final)
        Bb, L, Dd = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and dy.shape == x.shape and A.shape == (Dd, N)
        assert Bm.shape == (Bb, L, N) and Cm.shape == (Bb, L, N)
        assert D is None or D.shape == (Dd,)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (Bb, Dd, N)
        assert dhf is None or dhf.shape == (Bb, Dd, N)
        out = dict(dx=np.empty_like(x), ddelta=np.empty_like(x), dA=np.empty((Dd, N)),
                   dBm=np.empty((Bb, L, N)), dCm=np.empty((Bb, L, N)),
                   dD=None if D is None else np.empty(Dd),
                   dz=None if z is None else np.empty_like(x),
                   dh0=np.empty((Bb, Dd, N)) if want_dh0 else None)
        rc = self.lib.oracle_scan_bwd(Bb, L, Dd, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                                      _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dhf),
                                      *(_ptr(out[k]) for k in ("dx", "ddelta", "dA", "dBm", "dCm",
                                                               "dD", "dz", "dh0")))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    _DISC = {"euler": 0, "zoh": 1}

    def scan_disc(self, x, delta, A, Bm, Cm, D=None, z=None, h0=None, disc="euler", delta_bias=None,
                  delta_softplus=False):
        """``scan`` with discretisation ``disc`` and Delta = [softplus](delta + delta_bias)."""
        x, delta, A, Bm, Cm = map(_f64, (x, delta, A, Bm, Cm))
        D, z, h0, bias = _f64(D), _f64(z), _f64(h0), _f64(delta_bias)
        Bb, L, Dd = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and A.shape == (Dd, N)
        assert Bm.shape == (Bb, L, N) and Cm.shape == (Bb, L, N)
        assert bias is None or bias.shape == (Dd,)
        y = np.empty_like(x)
        hf = np.empty((Bb, Dd, N))
        rc = self.lib.oracle_scan_disc(Bb, L, Dd, N, self._DISC[disc], _ptr(bias), int(bool(delta_softplus)),
                                       _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z),
                                       _ptr(h0), _ptr(y), _ptr(hf))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, hf

    def scan3(self, x, delta, lam, Are, theta, Bm, Cm, D=None, z=None, h0=None, x_prev=None, B_prev=None):
        """Mamba-3 scan (O8). h0: complex [B,D,N] or None; x_prev [B,D] and B_prev [B,N]:
        the token before the sequence (both None: zero). Returns (y, h_final complex)."""
        x, delta, lam, Are, theta, Bm, Cm = map(_f64, (x, delta, lam, Are, theta, Bm, Cm))
        D, z, xp, bp = _f64(D), _f64(z), _f64(x_prev), _f64(B_prev)
        Bb, L, Dd = x.shape
        N = Are.shape[1]
        assert delta.shape == x.shape and lam.shape == x.shape
        assert Are.shape == (Dd, N) and theta.shape == (Dd, N)
        assert Bm.shape == (Bb, L, N) and Cm.shape == (Bb, L, N)
        h0r = None
        if h0 is not None:
            h0 = np.asarray(h0, dtype=np.complex128)
            assert h0.shape == (Bb, Dd, N)
            h0r = np.ascontiguousarray(np.stack([h0.real, h0.imag], axis=-1))
        y = np.empty_like(x)
        hf = np.empty((Bb, Dd, N, 2))
        rc = self.lib.oracle_scan3(Bb, L, Dd, N, _ptr(x), _ptr(delta), _ptr(lam), _ptr(Are), _ptr(theta),
                                   _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(h0r), _ptr(xp), _ptr(bp),
                                   _ptr(y), _ptr(hf))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, hf[..., 0] + 1j * hf[..., 1]

    def step_disc(self, state, x, delta, A, Bm, Cm, D=None, z=None, disc="euler", delta_bias=None,
                  delta_softplus=False):
        """``step`` with discretisation ``disc`` and Delta = [softplus](delta + delta_bias)."""
        st = _f64(state).copy()
        x, delta, A, Bm, Cm = map(_f64, (x, delta, A, Bm, Cm))
        D, z, bias = _f64(D), _f64(z), _f64(delta_bias)
        Bb, Dd, N = st.shape
        assert x.shape == (Bb, Dd) and delta.shape == (Bb, Dd) and A.shape == (Dd, N)
        y = np.empty((Bb, Dd))
        rc = self.lib.oracle_step_disc(Bb, Dd, N, self._DISC[disc], _ptr(bias), int(bool(delta_softplus)),
                                       _ptr(st), _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D),
                                       _ptr(z), _ptr(y))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, st

    # -- SSD ---------------------------------------------------------------
    def _ssd_args(self, x, delta, A, Bm, Cm, D, z, h0):
        x, delta, A, Bm, Cm = map(_f64, (x, delta, A, Bm, Cm))
        D, z, h0 = _f64(D), _f64(z), _f64(h0)
        Bb, L, H, P = x.shape
        N = Bm.shape[2]
        assert delta.shape == (Bb, L, H) and A.shape == (H,)
        assert Bm.shape == (Bb, L, N) and Cm.shape == (Bb, L, N)
        assert D is None or D.shape == (H,)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (Bb, H, N, P)
        return (x, delta, A, Bm, Cm, D, z, h0), (Bb, L, H, P, N)

    def _ssd_call(self, fn, dims, arrs, extra=()):
        x, delta, A, Bm, Cm, D, z, h0 = arrs
        Bb, L, H, P, N = dims
        y = np.empty_like(x)
        hf = np.empty((Bb, H, N, P))
        rc = fn(Bb, L, H, P, N, *extra, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hf))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, hf

    def ssd_seq(self, x, delta, A, Bm, Cm, D=None, z=None, h0=None):
        arrs, dims = self._ssd_args(x, delta, A, Bm, Cm, D, z, h0)
        return self._ssd_call(self.lib.oracle_ssd_seq, dims, arrs)

    def ssd_unroll(self, x, delta, A, Bm, Cm, D=None, z=None, h0=None):
        arrs, dims = self._ssd_args(x, delta, A, Bm, Cm, D, z, h0)
        return self._ssd_call(self.lib.oracle_ssd_unroll, dims, arrs)

    def ssd_chunked(self, x, delta, A, Bm, Cm, D=None, z=None, h0=None, chunk=256):
        arrs, dims = self._ssd_args(x, delta, A, Bm, Cm, D, z, h0)
        return self._ssd_call(self.lib.oracle_ssd_chunked, dims, arrs, extra=(int(chunk),))

    # -- decode --------------------------------------------------------------
    def step(self, state, x, delta, A, Bm, Cm, D=None, z=None):
        st = _f64(state).copy()
        x, delta, A, Bm, Cm = map(_f64, (x, delta, A, Bm, Cm))
        D, z = _f64(D), _f64(z)
        Bb, Dd, N = st.shape
        assert x.shape == (Bb, Dd) and delta.shape == (Bb, Dd) and A.shape == (Dd, N)
        assert Bm.shape == (Bb, N) and Cm.shape == (Bb, N)
        y = np.empty((Bb, Dd))
        rc = self.lib.oracle_step(Bb, Dd, N, _ptr(st), _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm),
                                  _ptr(Cm), _ptr(D), _ptr(z), _ptr(y))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, st

    def ssd_step(self, state, x, delta, A, Bm, Cm, D=None, z=None):
        st = _f64(state).copy()
        x, delta, A, Bm, Cm = map(_f64, (x, delta, A, Bm, Cm))
        D, z = _f64(D), _f64(z)
        Bb, H, N, P = st.shape
        assert x.shape == (Bb, H, P) and delta.shape == (Bb, H) and A.shape == (H,)
        y = np.empty((Bb, H, P))
        rc = self.lib.oracle_ssd_step(Bb, H, P, N, _ptr(st), _ptr(x), _ptr(delta), _ptr(A),
                                      _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(z), _ptr(y))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, st


_default = None


def get():
    """The oracle built from ``oracle.c`` (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def scan(*a, **k):
    return get().scan(*a, **k)


def scan_unroll(*a, **k):
    return get().scan_unroll(*a, **k)


def scan_bwd(*a, **k):
    return get().scan_bwd(*a, **k)


def scan_disc(*a, **k):
    return get().scan_disc(*a, **k)


def step_disc(*a, **k):
    return get().step_disc(*a, **k)


def scan3(*a, **k):
    return get().scan3(*a, **k)


def ssd_seq(*a, **k):
    return get().ssd_seq(*a, **k)


def ssd_chunked(*a, **k):
    return get().ssd_chunked(*a, **k)


def ssd_unroll(*a, **k):
    return get().ssd_unroll(*a, **k)


def step(*a, **k):
    return get().step(*a, **k)


def ssd_step(*a, **k):
    return get().ssd_step(*a, **k)
