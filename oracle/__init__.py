"""fp64 CPU oracle for Parallax attention (Python side).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It never imports
the GPU library, and the GPU library never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
independent queries); this module only builds that file with gcc, converts
inputs to contiguous float64 arrays and calls it through ctypes.

Definition followed (zubnet.ai news item on Parallax, second paragraph):
the output is softmax attention minus the key-value covariance contracted
with the probe rho_i = W_R x_i; W_R = 0 gives plain softmax attention.
Per query:  o = vbar - C rho, with C = sum_j p_j (v_j - vbar)(k_j - kbar)^T
and p the softmax of scale * q.k over the visible keys.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
import tempfile
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)


# A library path in this variable replaces the default build (used to run
# the pins against a sanitizer build of oracle.c).
LIBRARY_ENV = "PARALLAX_ORACLE_LIB"
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]


def compile_library(output: str = LIBRARY, mutant: int = 0, sanitize: bool = False) -> str:
    """Compile oracle.c with gcc into ``output`` (atomically) and return it.
    ``sanitize`` adds AddressSanitizer and UndefinedBehaviorSanitizer
    (the process that loads it needs the sanitizer runtimes preloaded)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Werror", SOURCE, "-o", output + ".tmp", "-lm"]
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    if sanitize:
        cmd[1:1] = SANITIZE_FLAGS
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(output + ".tmp", output)
    return output


def build(force: bool = True) -> str:
    """Build liboracle.so next to the source."""
    if force or not os.path.exists(LIBRARY):
        compile_library(LIBRARY)
    return LIBRARY


def _declare(lib):
    lib.oracle_decode_f64.argtypes = [_dp, _dp, _dp, _dp, _ip, _dp,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_long, ctypes.c_double,
                                      ctypes.c_int]
    lib.oracle_fwd_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, ctypes.c_int,
                                   ctypes.c_int]
    lib.oracle_fwd_rows_f64.argtypes = [_dp, _dp, _dp, _dp, _lp,
                                        ctypes.c_long, _dp, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_double,
                                        ctypes.c_int, ctypes.c_int]
    lib.oracle_decode_partial_f64.argtypes = [_dp, _dp, _dp, _dp,
                                              ctypes.c_long, ctypes.c_long,
                                              ctypes.c_int, ctypes.c_double,
                                              ctypes.c_long, _dp]
    lib.oracle_merge_f64.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp]
    lib.oracle_decode_onepass_f64.argtypes = [_dp, _dp, _dp, _dp, _ip, _dp,
                                              ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_long,
                                              ctypes.c_double, ctypes.c_long,
                                              ctypes.c_int]
    lib.oracle_bwd_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                   _dp, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                   ctypes.c_int, ctypes.c_int]
    lib.oracle_lla_probe_f64.argtypes = [_dp, _dp, _dp, _ip, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_int]
    lib.oracle_max_threads.argtypes = []
    for name in ("oracle_decode_f64", "oracle_fwd_f64", "oracle_fwd_rows_f64",
                 "oracle_decode_partial_f64", "oracle_merge_f64",
                 "oracle_decode_onepass_f64", "oracle_bwd_f64",
                 "oracle_lla_probe_f64", "oracle_max_threads"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None):
    """Load (building first if absent) and return the ctypes library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        override = os.environ.get(LIBRARY_ENV)
        if override:
            _lib = _declare(ctypes.CDLL(override))
            return _lib
        if not os.path.exists(LIBRARY):
            build()
        _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def load_mutant(mutant: int, directory: Optional[str] = None):
    """Build and load a deliberately wrong variant (for the mutation test)."""
    directory = directory or tempfile.mkdtemp(prefix="oracle_mutant_")
    path = os.path.join(directory, f"liboracle_m{mutant}.so")
    compile_library(path, mutant=mutant)
    return _declare(ctypes.CDLL(path))


def max_threads() -> int:
    return int(load().oracle_max_threads())


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch  # local: torch is optional for the oracle
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


class Oracle:
    """Thin caller over one loaded library (the real one or a mutant)."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    def decode(self, q, rho, k, v, seqlens=None, scale: Optional[float] = None,
               threads: int = 0) -> np.ndarray:
        """Decode: q, rho [B,H,D]; k, v [B,H,L,D]; seqlens int [B] or None."""
        q, rho, k, v = _f64(q), _f64(rho), _f64(k), _f64(v)
        B, H, L, D = k.shape
        assert q.shape == (B, H, D) and rho.shape == (B, H, D)
        assert v.shape == (B, H, L, D)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        out = np.zeros((B, H, D), dtype=np.float64)
        sl = None
        if seqlens is not None:
            if hasattr(seqlens, "detach"):
                seqlens = seqlens.detach().cpu().numpy()
            sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
            assert sl.shape == (B,)
        rc = self.lib.oracle_decode_f64(
            _ptr(q), _ptr(rho), _ptr(k), _ptr(v),
            sl.ctypes.data_as(_ip) if sl is not None else None, _ptr(out),
            B, H, D, L, scale, int(threads))
        _check(rc, "decode")
        return out

    def fwd(self, q, k, v, rho, scale: Optional[float] = None,
            causal: bool = True, threads: int = 0) -> np.ndarray:
        """Prefill over [B,N,H,D] tensors; returns [B,N,H,D] float64."""
        q, k, v, rho = _f64(q), _f64(k), _f64(v), _f64(rho)
        B, N, H, D = q.shape
        for t in (k, v, rho):
            assert t.shape == (B, N, H, D)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        out = np.zeros((B, N, H, D), dtype=np.float64)
        rc = self.lib.oracle_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(rho),
                                     _ptr(out), B, N, H, D, scale,
                                     1 if causal else 0, int(threads))
        _check(rc, "fwd")
        return out

    def bwd(self, q, k, v, rho, dout, scale: Optional[float] = None,
            causal: bool = True, threads: int = 0):
        """Gradients (dq, dk, dv, drho) of sum(dout * fwd(q, k, v, rho)),
        all [B,N,H,D] float64."""
        q, k, v, rho, dout = _f64(q), _f64(k), _f64(v), _f64(rho), _f64(dout)
        B, N, H, D = q.shape
        for t in (k, v, rho, dout):
            assert t.shape == (B, N, H, D)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        outs = [np.zeros((B, N, H, D), dtype=np.float64) for _ in range(4)]
        rc = self.lib.oracle_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(rho),
                                     _ptr(dout), *(_ptr(o) for o in outs),
                                     B, N, H, D, scale, 1 if causal else 0,
                                     int(threads))
        _check(rc, "bwd")
        return tuple(outs)

    def lla_probe(self, q, k, scale: Optional[float] = None, causal: bool = True,
                  lam: float = 1.0, maxit: int = 500, tol: float = 1e-12,
                  threads: int = 0, allow_unconverged: bool = False):
        """Exact local-linear probe by conjugate gradient: returns
        (rho [B,N,H,D] float64, iterations [B,N,H] int32)."""
        q, k = _f64(q), _f64(k)
        B, N, H, D = q.shape
        assert k.shape == (B, N, H, D)
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        rho = np.zeros((B, N, H, D), dtype=np.float64)
        its = np.zeros((B, N, H), dtype=np.int32)
        rc = self.lib.oracle_lla_probe_f64(
            _ptr(q), _ptr(k), _ptr(rho), its.ctypes.data_as(_ip), B, N, H, D, scale,
            1 if causal else 0, float(lam), int(maxit), float(tol), int(threads))
        if not (rc == 3 and allow_unconverged):
            _check(rc, "lla_probe")
        return rho, its

    def fwd_rows(self, q, k, v, rho, rows, scale: Optional[float] = None,
                 causal: bool = True, threads: int = 0) -> np.ndarray:
        """Selected prefill rows; rows: sequence of (b, i, h)."""
        q, k, v, rho = _f64(q), _f64(k), _f64(v), _f64(rho)
        B, N, H, D = q.shape
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        out = np.zeros((r.shape[0], D), dtype=np.float64)
        rc = self.lib.oracle_fwd_rows_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(rho), r.ctypes.data_as(_lp),
            r.shape[0], _ptr(out), B, N, H, D, scale, 1 if causal else 0,
            int(threads))
        _check(rc, "fwd_rows")
        return out

    def decode_partial(self, q_row, rho_row, K, V, j0: int, j1: int,
                       scale: float, chunk: int = 1) -> np.ndarray:
        """One-pass state [m, l, A_r, A_v(D), A_rv(D)] over keys [j0, j1)."""
        q_row, rho_row, K, V = _f64(q_row), _f64(rho_row), _f64(K), _f64(V)
        D = q_row.shape[-1]
        st = np.zeros(3 + 2 * D, dtype=np.float64)
        rc = self.lib.oracle_decode_partial_f64(
            _ptr(q_row), _ptr(rho_row), _ptr(K), _ptr(V), int(j0), int(j1), D,
            float(scale), int(chunk), _ptr(st))
        _check(rc, "decode_partial")
        return st

    def merge(self, states: Sequence[np.ndarray]) -> np.ndarray:
        st = np.ascontiguousarray(np.stack([_f64(s) for s in states]))
        D = (st.shape[1] - 3) // 2
        out = np.zeros(D, dtype=np.float64)
        _check(self.lib.oracle_merge_f64(_ptr(st), st.shape[0], D, _ptr(out)),
               "merge")
        return out

    def decode_onepass(self, q, rho, k, v, seqlens=None,
                       scale: Optional[float] = None, chunk: int = 64,
                       threads: int = 0) -> np.ndarray:
        q, rho, k, v = _f64(q), _f64(rho), _f64(k), _f64(v)
        B, H, L, D = k.shape
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        out = np.zeros((B, H, D), dtype=np.float64)
        sl = None
        if seqlens is not None:
            if hasattr(seqlens, "detach"):
                seqlens = seqlens.detach().cpu().numpy()
            sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
        rc = self.lib.oracle_decode_onepass_f64(
            _ptr(q), _ptr(rho), _ptr(k), _ptr(v),
            sl.ctypes.data_as(_ip) if sl is not None else None, _ptr(out),
            B, H, D, L, scale, int(chunk), int(threads))
        _check(rc, "decode_onepass")
        return out


_default: Optional[Oracle] = None


def _o() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def decode(*a, **kw):
    return _o().decode(*a, **kw)


def fwd(*a, **kw):
    return _o().fwd(*a, **kw)


def bwd(*a, **kw):
    return _o().bwd(*a, **kw)


def project(x, w) -> np.ndarray:
    """Fused input projection y = x W^T (x [M, K], W [N, K]) in fp64: the
    layer's q, k, v and probe rho = W_R x (zubnet.ai item, second paragraph)
    as one product with the weights stacked along the output features. A
    library matrix product is the whole definition."""
    return _f64(x) @ _f64(w).T


def lla_probe(*a, **kw):
    return _o().lla_probe(*a, **kw)


def fwd_rows(*a, **kw):
    return _o().fwd_rows(*a, **kw)


def decode_partial(*a, **kw):
    return _o().decode_partial(*a, **kw)


def merge(*a, **kw):
    return _o().merge(*a, **kw)


def decode_onepass(*a, **kw):
    return _o().decode_onepass(*a, **kw)
