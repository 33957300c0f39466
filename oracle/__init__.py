"""fp64 CPU oracle of the KDA layer core (prologue, recurrence, epilogue).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does and
shares no code with it.  The arithmetic lives in ``kda_oracle.c`` (plain
sequential fp64 loops); this module only marshals numpy arrays into that
library through ctypes and builds it with gcc when it is missing.

The recurrence follows the step list of the OpenModelAtlas page "Kimi K3 -
KDA layer" and the five-step order of "Inside Kimi K3: How KDA, AttnRes, and
896 Experts Work" (section "KDA writes corrections into a recurrent matrix").
Every input is converted exactly to float64 (bf16 and fp32 values are exact
in fp64), so the oracle sees the same numbers the GPU sees.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple, Union

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "_kda_oracle.so")

CONV_HIST = 3


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE semantics, no fast-math)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-o", out + ".tmp", src,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


_D = ctypes.POINTER(ctypes.c_double)


class Oracle:
    """Handle on one compiled oracle library (the default one, or a test build)."""

    def __init__(self, path: Optional[str] = None):
        if path is None:
            path = _LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build()
        self.path = path
        lib = ctypes.CDLL(path)
        f = lib.kda_oracle_run
        f.restype = ctypes.c_int
        f.argtypes = ([ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_int64)] + [_D] * 14 +
                      [ctypes.c_double] * 3 + [ctypes.c_int] * 2 + [_D] * 5 + [ctypes.c_int])
        self._run = f
        g = lib.kda_oracle_lowrank_log_alpha
        g.restype = ctypes.c_int
        g.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [_D] * 5
        self._gate = g
        g2 = lib.kda_oracle_softplus_log_alpha
        g2.restype = ctypes.c_int
        g2.argtypes = g.argtypes
        self._gate_softplus = g2
        b = lib.kda_oracle_beta_from_logit
        b.restype = ctypes.c_int
        b.argtypes = [ctypes.c_int64, _D, _D]
        self._beta = b

    def beta_from_logit(self, w):
        """beta = sigma(w) of the "Kimi K3 - KDA layer" step list, elementwise, from the
        pre-activation w (any shape)."""
        w = _f64(w)
        out = np.zeros_like(w)
        if self._beta(w.size, _p(w), _p(out)) != 0:
            raise ValueError("beta_from_logit failed")
        return out

    def lowrank_log_alpha(self, z, w, bias, a):
        """log alpha [T, H, d] of the low-rank gate of the "Kimi K3 - KDA layer" step list,
        alpha = exp(-5 sigmoid(e^{A_h} (z_down W_up + b_alpha))), from z_down [T, r],
        W_up stored output-major [H*d, r], b_alpha [H*d] and A [H]."""
        return self._lowrank(self._gate, z, w, bias, a)

    def softplus_log_alpha(self, z, w, bias, a):
        """log alpha [T, H, d] of Kimi Linear's unbounded gate,
        log alpha = -e^{A_h} softplus(z_down W_up + b_alpha) (any value below 0), from the
        same factors as lowrank_log_alpha."""
        return self._lowrank(self._gate_softplus, z, w, bias, a)

    @staticmethod
    def _lowrank(fn, z, w, bias, a):
        z, w, bias, a = (_f64(x) for x in (z, w, bias, a))
        T, r = z.shape
        H = a.shape[0]
        d = w.shape[0] // H
        assert w.shape == (H * d, r) and bias.shape == (H * d,)
        out = np.zeros((T, H, d), np.float64)
        rc = fn(T, H, d, r, _p(z), _p(w), _p(bias), _p(a), _p(out))
        if rc != 0:
            raise ValueError(f"low-rank gate failed ({rc})")
        return out

    # ------------------------------------------------------------------ prefill
    def prefill(self, q, k, v, log_alpha, beta, cu_seqlens, *, g=None, conv_w=None,
                conv_in=None, rms_w=None, state_in=None, scale: Optional[float] = None,
                l2_eps: float = 1e-6, rms_eps: float = 1e-6, prologue: Optional[bool] = None,
                epilogue: Optional[bool] = None, threads: Optional[int] = None):
        """Run the recurrence over packed variable-length sequences.

        q, k: [T, H, dk]; v: [T, H, dv]; log_alpha: [T, H, dk]; beta: [T, H];
        g: [T, H, dv]; cu_seqlens: [N+1] token offsets.  conv_w is either a
        [3, H*d, 4] array (streams q, k, v; tap j multiplies x_{t-j}) when
        dk == dv, or a tuple (wq, wk, wv) of [H*dk|dv, 4] arrays.  conv_in is
        [N, 3, 3, H*d] (stream, oldest-first history, channel) or a tuple of
        three [N, 3, H*d] arrays.  state_in: [N, H, dk, dv], S[i][j] with i the
        key channel.  Defaults: scale = 1/sqrt(dk), prologue on iff conv_w is
        given, epilogue on iff g is given.

        Returns (o [T,H,dv], state_out [N,H,dk,dv], conv_out) with conv_out in
        the same form as conv_in was given (array form when conv_w is an
        array), or None when the prologue is off.
        """
        q = _f64(q); k = _f64(k); v = _f64(v)
        la = _f64(log_alpha); b = _f64(beta)
        if q.ndim != 3 or k.shape != q.shape or la.shape != q.shape:
            raise ValueError("q, k, log_alpha must share shape [T, H, dk]")
        T, H, dk = q.shape
        if v.ndim != 3 or v.shape[:2] != (T, H):
            raise ValueError("v must be [T, H, dv]")
        dv = v.shape[2]
        if b.shape != (T, H):
            raise ValueError("beta must be [T, H]")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        if N < 0 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
        if prologue is None:
            prologue = conv_w is not None
        if epilogue is None:
            epilogue = g is not None
        if scale is None:
            scale = 1.0 / np.sqrt(dk)
        gg = _f64(g) if epilogue else None
        if epilogue and gg.shape != (T, H, dv):
            raise ValueError("g must be [T, H, dv]")

        array_form = conv_w is not None and not isinstance(conv_w, (tuple, list))
        wq = wk = wv = None
        ciq = cik = civ = None
        if prologue:
            if array_form:
                cw = _f64(conv_w)
                if dk != dv or cw.shape != (3, H * dk, 4):
                    raise ValueError("conv_w array form must be [3, H*d, 4] with dk == dv")
                wq, wk, wv = (np.ascontiguousarray(cw[s]) for s in range(3))
            else:
                wq, wk, wv = (_f64(x) for x in conv_w)
            if wq.shape != (H * dk, 4) or wk.shape != (H * dk, 4) or wv.shape != (H * dv, 4):
                raise ValueError("conv weights have the wrong shape")
            if conv_in is not None:
                if isinstance(conv_in, (tuple, list)):
                    ciq, cik, civ = (_f64(x) for x in conv_in)
                else:
                    ci = _f64(conv_in)
                    if dk != dv or ci.shape != (N, 3, CONV_HIST, H * dk):
                        raise ValueError("conv_in array form must be [N, 3, 3, H*d]")
                    ciq, cik, civ = (np.ascontiguousarray(ci[:, s]) for s in range(3))
                if (ciq.shape != (N, CONV_HIST, H * dk) or cik.shape != ciq.shape
                        or civ.shape != (N, CONV_HIST, H * dv)):
                    raise ValueError("conv_in has the wrong shape")
        rw = _f64(rms_w) if rms_w is not None else None
        if rw is not None and rw.shape != (dv,):
            raise ValueError("rms_w must be [dv]")
        s_in = _f64(state_in) if state_in is not None else None
        if s_in is not None and s_in.shape != (N, H, dk, dv):
            raise ValueError("state_in must be [N, H, dk, dv]")

        o = np.zeros((T, H, dv), np.float64)
        s_out = np.zeros((N, H, dk, dv), np.float64)
        coq = np.zeros((N, CONV_HIST, H * dk)) if prologue else None
        cok = np.zeros((N, CONV_HIST, H * dk)) if prologue else None
        cov = np.zeros((N, CONV_HIST, H * dv)) if prologue else None
        rc = self._run(N, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                       _p(q), _p(k), _p(v), _p(gg), _p(la), _p(b), _p(wq), _p(wk), _p(wv),
                       _p(ciq), _p(cik), _p(civ), _p(rw), _p(s_in),
                       float(scale), float(l2_eps), float(rms_eps), int(bool(prologue)),
                       int(bool(epilogue)), _p(o), _p(s_out), _p(coq), _p(cok), _p(cov),
                       int(threads or _default_threads()))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_run failed with code {rc}")
        conv_out = None
        if prologue:
            conv_out = np.stack([coq, cok, cov], axis=1) if (array_form and dk == dv) else (coq, cok, cov)
        return o, s_out, conv_out

    # ------------------------------------------------------------------- decode
    def decode_step(self, q, k, v, log_alpha, beta, state, *, g=None, conv_w=None,
                    conv_state=None, rms_w=None, scale=None, l2_eps=1e-6, rms_eps=1e-6,
                    prologue=None, epilogue=None, threads=None):
        """One token per request: q, k, log_alpha [B,H,dk]; v, g [B,H,dv]; beta [B,H];
        state [B,H,dk,dv]; conv_state [B,3,3,H*d].  Returns (o, new_state, new_conv_state);
        the inputs are not modified (the GPU entry point updates in place)."""
        q = _f64(q)
        B = q.shape[0]
        cu = np.arange(B + 1, dtype=np.int64)
        return self.prefill(q, k, v, log_alpha, beta, cu, g=g, conv_w=conv_w,
                            conv_in=conv_state, rms_w=rms_w, state_in=state, scale=scale,
                            l2_eps=l2_eps, rms_eps=rms_eps, prologue=prologue,
                            epilogue=epilogue, threads=threads)


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, _D)
    return a.ctypes.data_as(_D)


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def prefill(*args, **kwargs):
    return default().prefill(*args, **kwargs)


def lowrank_log_alpha(*args, **kwargs):
    return default().lowrank_log_alpha(*args, **kwargs)


def softplus_log_alpha(*args, **kwargs):
    return default().softplus_log_alpha(*args, **kwargs)


def decode_step(*args, **kwargs):
    return default().decode_step(*args, **kwargs)


def beta_from_logit(*args, **kwargs):
    return default().beta_from_logit(*args, **kwargs)
