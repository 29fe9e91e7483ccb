"""fp64 CPU oracle for PagedWeight's fused mixed-precision MoE expert path.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the bench's
CPU-baseline leg may import this package.  It shares no code with the HIP
library (any_precision_expert_amd) and never imports it.

The arithmetic lives in pw_oracle.c (plain C, fp64, sums in ascending index
order).  This wrapper only marshals numpy arrays: fp16 inputs are widened to
fp64 with numpy before the call.  See pw_oracle.c for the definition each
function follows and the passages of the PagedWeight pages it rests on.

Every function here is pinned by tests/test_oracle_*.py against brute force,
closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pw_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile pw_oracle.c with gcc (no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


class _Block(ctypes.Structure):
    _fields_ = [("code8", ctypes.c_void_p), ("lut", ctypes.c_void_p),
                ("R", ctypes.c_int32), ("K", ctypes.c_int32), ("q", ctypes.c_int32)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.pwo_route_topk.argtypes = [vp, i64, i32, i32, vp, vp]
        L.pwo_permute.argtypes = [vp, i64, i32, i32, vp, vp]
        L.pwo_decode_codes.argtypes = [vp, i64, i32, vp]
        L.pwo_decode_block.argtypes = [ctypes.POINTER(_Block), vp]
        L.pwo_moe_layer.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp,
                                    ctypes.POINTER(_Block), ctypes.POINTER(_Block),
                                    ctypes.POINTER(_Block), ctypes.POINTER(_Block),
                                    vp, i64, vp]
        L.pwo_num_threads.restype = ctypes.c_int
        L.pwo_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def set_threads(n: int) -> None:
    lib().pwo_set_threads(int(n))


def num_threads() -> int:
    return int(lib().pwo_num_threads())


def route_topk(logits: np.ndarray, k: int):
    """idx int32 [T][k], w float64 [T][k] (route: value desc, index asc; softmax over k)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    rc = lib().pwo_route_topk(_p(lg), T, E, k, _p(idx), _p(w))
    if rc:
        raise ValueError("oracle route_topk: invalid arguments")
    return idx, w


def permute(idx: np.ndarray, E: int):
    """offsets int32 [E+1], sorted int32 [T*k]: stable sort of assignments by expert."""
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = ix.shape
    offsets = np.empty(E + 1, dtype=np.int32)
    srt = np.empty(T * k, dtype=np.int32)
    rc = lib().pwo_permute(_p(ix), T, k, E, _p(offsets), _p(srt))
    if rc:
        raise ValueError("oracle permute: invalid arguments")
    return offsets, srt


def decode_codes(code8: np.ndarray, q: int) -> np.ndarray:
    c = np.ascontiguousarray(code8, dtype=np.uint8)
    out = np.empty_like(c)
    if lib().pwo_decode_codes(_p(c), c.size, int(q), _p(out)):
        raise ValueError("oracle decode_codes: bad q")
    return out


class _Held:
    """Keeps widened arrays alive while ctypes structs point at them."""

    def __init__(self):
        self.keep = []

    def block(self, b) -> _Block:
        code8 = np.ascontiguousarray(b.code8, dtype=np.uint8)
        lut = np.ascontiguousarray(b.luts[b.q], dtype=np.float16).astype(np.float64)
        self.keep += [code8, lut]
        return _Block(_p(code8), _p(lut), code8.shape[0], code8.shape[1], int(b.q))


def decode_block(b) -> np.ndarray:
    h = _Held()
    blk = h.block(b)
    W = np.empty((b.R, b.K), dtype=np.float64)
    if lib().pwo_decode_block(ctypes.byref(blk), _p(W)):
        raise ValueError("oracle decode_block: bad q")
    return W


class PreparedLayer:
    """A layer's blocks widened once, so repeated oracle calls (and the timed
    CPU baseline) exclude the fp16 -> fp64 input conversion."""

    def __init__(self, weights):
        s = weights.shape
        self.shape = s
        self._h = _Held()
        E = s.E
        self.gu = (_Block * E)()
        self.dn = (_Block * E)()
        for e in range(E):
            if weights.gate_up[e] is not None:
                self.gu[e] = self._h.block(weights.gate_up[e])
                self.dn[e] = self._h.block(weights.down[e])
        self.sgu = self.sdn = None
        if s.I_shared:
            self.sgu = self._h.block(weights.shared_gate_up)
            self.sdn = self._h.block(weights.shared_down)

    def ffn(self, x: np.ndarray, idx: np.ndarray, w: np.ndarray,
            tokens: Optional[Sequence[int]] = None) -> np.ndarray:
        s = self.shape
        xd = np.ascontiguousarray(x, dtype=np.float16).astype(np.float64)
        T = xd.shape[0]
        ix = np.ascontiguousarray(idx, dtype=np.int32)
        wd = np.ascontiguousarray(w, dtype=np.float64)
        if tokens is None:
            tk, nt, tp = None, T, None
        else:
            tk = np.ascontiguousarray(tokens, dtype=np.int32)
            nt, tp = tk.size, _p(tk)
        y = np.empty((nt, s.H), dtype=np.float64)
        sg = ctypes.byref(self.sgu) if self.sgu is not None else None
        sd = ctypes.byref(self.sdn) if self.sdn is not None else None
        rc = lib().pwo_moe_layer(T, s.H, s.I, s.E, s.top_k, s.I_shared, _p(xd), _p(ix), _p(wd),
                                 self.gu, self.dn, sg, sd, tp, nt, _p(y))
        if rc:
            raise ValueError("oracle moe_layer: invalid arguments (rc=%d)" % rc)
        return y


def moe_layer(weights, acts, tokens: Optional[Sequence[int]] = None, prepared=None):
    """Full oracle pass: route -> permute -> decode -> FFN -> combine.

    Returns dict(y [n][H] fp64, idx, w, offsets, sorted)."""
    s = weights.shape
    idx, w = route_topk(acts.logits, s.top_k)
    offsets, srt = permute(idx, s.E)
    P = prepared if prepared is not None else PreparedLayer(weights)
    y = P.ffn(acts.x, idx, w, tokens)
    return dict(y=y, idx=idx, w=w, offsets=offsets, sorted=srt)


def timed_layer(prepared: PreparedLayer, acts, tokens: Optional[Sequence[int]] = None):
    """Route + permute + FFN timed with a monotonic clock (input widening excluded).

    Returns (seconds, y)."""
    s = prepared.shape
    xd = np.ascontiguousarray(acts.x, dtype=np.float16)
    t0 = time.perf_counter()
    idx, w = route_topk(acts.logits, s.top_k)
    permute(idx, s.E)
    y = prepared.ffn(xd, idx, w, tokens)
    return time.perf_counter() - t0, y
