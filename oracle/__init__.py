"""Python access to the float64 parity oracle -- TEST INFRASTRUCTURE ONLY.

The oracle is a plain sequential per-token implementation of the gated delta
rule in C (``gdn_oracle.c``), built into ``liboracle.so`` next to this file.
Only the tests, the smoke check and the benchmark's CPU-baseline leg use it;
the HIP library and its binding never import this package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdn_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE double: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
           "-Wall", "-Wextra", *extra_flags, "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


_P = ctypes.c_void_p
_F = ctypes.c_float
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double


class Oracle:
    """ctypes wrapper of one built oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built; run oracle.build()")
        self.path = path
        self._lib = ctypes.CDLL(path)
        self._lib.gdn_oracle_prefill.restype = _I
        self._lib.gdn_oracle_prefill.argtypes = [_I, _I, _I, _I, _I, _I, _I, _D,
                                                 _P, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _I]
        self._lib.gdn_oracle_decode.restype = _I
        self._lib.gdn_oracle_decode.argtypes = [_I, _I, _I, _I, _I, _I, _D,
                                                _P, _P, _P, _P, _P, _P, _I64, _P, _P, _I]
        self._lib.gdn_oracle_kda_prefill.restype = _I
        self._lib.gdn_oracle_kda_prefill.argtypes = [_I, _I, _I, _I, _I, _I, _I, _D,
                                                     _P, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _I]
        self._lib.gdn_oracle_kda_decode.restype = _I
        self._lib.gdn_oracle_kda_decode.argtypes = [_I, _I, _I, _I, _I, _I, _D,
                                                    _P, _P, _P, _P, _P, _P, _I64, _P, _P, _I]
        self._lib.gdn_oracle_gated_rmsnorm.restype = _I
        self._lib.gdn_oracle_gated_rmsnorm.argtypes = [_I64, _I, _P, _P, _P, _D, _P, _I]
        self._lib.gdn_oracle_qkv_prologue.restype = _I
        self._lib.gdn_oracle_qkv_prologue.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _D, _I]
        self._lib.gdn_oracle_max_threads.restype = _I
        self._lib.gdn_oracle_max_threads.argtypes = []

    def max_threads(self) -> int:
        return int(self._lib.gdn_oracle_max_threads())

    @staticmethod
    def _f32(x):
        return np.ascontiguousarray(x, dtype=np.float32)

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    def prefill(self, q, k, v, g, beta, s0=None, scale: float = 1.0, head_map: int = 0,
                pairs: Optional[Sequence[int]] = None, threads: Optional[int] = None):
        """Sequential float64 prefill.

        q, k [B][Hk][T][dk]; v [B][Hv][T][dv]; g, beta [B][Hv][T]; s0 [B][Hv][dv][dk] or None.
        Returns (o, s_final) as float64: o [B][Hv][T][dv] and s_final [B][Hv][dv][dk] when
        pairs is None, else compact [npairs][T][dv] and [npairs][dv][dk] over the listed
        flattened (b * Hv + h) pairs.
        """
        return self._prefill(self._lib.gdn_oracle_prefill, False, q, k, v, g, beta, s0, scale, head_map,
                             pairs, threads)

    def kda_prefill(self, q, k, v, g, beta, s0=None, scale: float = 1.0, head_map: int = 0,
                    pairs: Optional[Sequence[int]] = None, threads: Optional[int] = None):
        """Sequential float64 prefill with one log-decay per key channel: as ``prefill`` with
        g [B][Hv][T][dk]."""
        return self._prefill(self._lib.gdn_oracle_kda_prefill, True, q, k, v, g, beta, s0, scale, head_map,
                             pairs, threads)

    def _prefill(self, fn, per_channel, q, k, v, g, beta, s0, scale, head_map, pairs, threads):
        q, k, v, g, beta = (self._f32(x) for x in (q, k, v, g, beta))
        B, Hk, T, dk = q.shape
        Hv, dv = v.shape[1], v.shape[3]
        gshape = (B, Hv, T, dk) if per_channel else (B, Hv, T)
        if k.shape != q.shape or v.shape[:3] != (B, Hv, T) or g.shape != gshape \
                or beta.shape != (B, Hv, T):
            raise ValueError("inconsistent prefill input shapes")
        s0c = None
        if s0 is not None:
            s0c = np.ascontiguousarray(s0, dtype=np.float64)
            if s0c.shape != (B, Hv, dv, dk):
                raise ValueError("s0 must be [B][Hv][dv][dk]")
        if pairs is None:
            n, pa = B * Hv, None
        else:
            pa = np.ascontiguousarray(pairs, dtype=np.int64)
            n = len(pa)
        o = np.empty((n, T, dv), dtype=np.float64)
        s = np.empty((n, dv, dk), dtype=np.float64)
        threads = threads or self.max_threads()
        rc = fn(B, T, Hk, Hv, dk, dv, head_map, float(scale),
                self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(g),
                self._ptr(beta), self._ptr(s0c), self._ptr(pa), n,
                self._ptr(o), self._ptr(s), int(threads))
        if rc != 0:
            raise ValueError(f"oracle prefill rejected its arguments (code {rc})")
        if pairs is None:
            return o.reshape(B, Hv, T, dv), s.reshape(B, Hv, dv, dk)
        return o, s

    def decode_step(self, q, k, v, g, beta, state, scale: float = 1.0, head_map: int = 0,
                    pairs: Optional[Sequence[int]] = None, threads: Optional[int] = None):
        """One float64 decode step; updates ``state`` (float64, C-contiguous) in place.

        q, k [B][Hk][dk]; v [B][Hv][dv]; g, beta [B][Hv]. state is [B][Hv][dv][dk] when pairs
        is None, else [npairs][dv][dk]. Returns o ([B][Hv][dv] or [npairs][dv]).
        """
        return self._decode(self._lib.gdn_oracle_decode, False, q, k, v, g, beta, state, scale, head_map,
                            pairs, threads)

    def kda_decode_step(self, q, k, v, g, beta, state, scale: float = 1.0, head_map: int = 0,
                        pairs: Optional[Sequence[int]] = None, threads: Optional[int] = None):
        """One float64 decode step with one log-decay per key channel: as ``decode_step`` with
        g [B][Hv][dk]."""
        return self._decode(self._lib.gdn_oracle_kda_decode, True, q, k, v, g, beta, state, scale, head_map,
                            pairs, threads)

    def _decode(self, fn, per_channel, q, k, v, g, beta, state, scale, head_map, pairs, threads):
        q, k, v, g, beta = (self._f32(x) for x in (q, k, v, g, beta))
        B, Hk, dk = q.shape
        Hv, dv = v.shape[1], v.shape[2]
        if g.shape != ((B, Hv, dk) if per_channel else (B, Hv)) or beta.shape != (B, Hv):
            raise ValueError("inconsistent decode input shapes")
        if state.dtype != np.float64 or not state.flags["C_CONTIGUOUS"]:
            raise ValueError("state must be a C-contiguous float64 array")
        if pairs is None:
            n, pa = B * Hv, None
        else:
            pa = np.ascontiguousarray(pairs, dtype=np.int64)
            n = len(pa)
        if state.size != n * dv * dk:
            raise ValueError("state has the wrong size")
        o = np.empty((n, dv), dtype=np.float64)
        threads = threads or self.max_threads()
        rc = fn(B, Hk, Hv, dk, dv, head_map, float(scale),
                self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(g),
                self._ptr(beta), self._ptr(pa), n, self._ptr(state),
                self._ptr(o), int(threads))
        if rc != 0:
            raise ValueError(f"oracle decode rejected its arguments (code {rc})")
        return o.reshape(B, Hv, dv) if pairs is None else o


    def gated_rmsnorm(self, x, weight, gate=None, eps: float = 1e-6, threads: Optional[int] = None):
        """Gated RMSNorm over the last axis in float64: x / sqrt(mean(x^2) + eps) * weight *
        silu(gate) (gate None: no gate factor). x is widened to float64, weight and gate to
        float32 then float64; returns a new float64 array of x's shape."""
        xc = np.ascontiguousarray(x, dtype=np.float64)
        n = xc.shape[-1]
        w = self._f32(weight)
        if w.shape != (n,):
            raise ValueError("weight must have the last-axis length of x")
        gc = None
        if gate is not None:
            gc = self._f32(gate)
            if gc.shape != xc.shape:
                raise ValueError("gate must have the shape of x")
        y = np.empty_like(xc)
        rc = self._lib.gdn_oracle_gated_rmsnorm(xc.size // n, n, self._ptr(xc), self._ptr(gc), self._ptr(w),
                                                float(eps), self._ptr(y), int(threads or self.max_threads()))
        if rc != 0:
            raise ValueError(f"oracle gated_rmsnorm rejected its arguments (code {rc})")
        return y


    def qkv_prologue(self, x, w, Hk: int, Hv: int, d: int, state=None, eps: float = 1e-6,
                     threads: Optional[int] = None):
        """Causal depthwise conv (K = w.shape[1] taps) + SiLU, then the q | k | v split with
        per-head L2 normalisation of q and k, in float64. x [B][T][(2 Hk + Hv) d] (float32
        values), w [(2 Hk + Hv) d][K], state [B][K-1][channels] or None (zero rows). Returns
        (q [B][Hk][T][d], k [B][Hk][T][d], v [B][Hv][T][d], new state [B][K-1][channels])."""
        xc = self._f32(x)
        B, T, C = xc.shape
        wc = self._f32(w)
        K = wc.shape[1]
        if C != (2 * Hk + Hv) * d or wc.shape != (C, K):
            raise ValueError("x must be [B][T][(2 Hk + Hv) d] and w [channels][K]")
        sc = None
        if state is not None:
            sc = np.ascontiguousarray(state, dtype=np.float64)
            if sc.shape != (B, K - 1, C):
                raise ValueError("state must be [B][K-1][channels]")
        q = np.empty((B, Hk, T, d))
        k = np.empty((B, Hk, T, d))
        v = np.empty((B, Hv, T, d))
        st = np.empty((B, K - 1, C))
        rc = self._lib.gdn_oracle_qkv_prologue(B, T, Hk, Hv, d, K, self._ptr(xc), self._ptr(wc), self._ptr(sc),
                                               self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(st),
                                               float(eps), int(threads or self.max_threads()))
        if rc != 0:
            raise ValueError(f"oracle qkv_prologue rejected its arguments (code {rc})")
        return q, k, v, st


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The oracle built next to this file (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default
