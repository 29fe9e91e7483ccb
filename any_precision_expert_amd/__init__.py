"""MI355X-native fused mixed-precision MoE expert path (PagedWeight hot path).

Thin ctypes binding of libpw.so, the C ABI declared in include/pw.h.  This
module only marshals arguments (device pointers from torch tensors, stream
handles, host numpy buffers); every step of the path runs in the library's
HIP kernels.  Importing it does not need a GPU; calling into a missing
library raises immediately -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpw.so")

PW_OK, PW_ERR_INVALID, PW_ERR_OOM, PW_ERR_HIP, PW_ERR_STATE = 0, 1, 2, 3, 4
QMIN, QMAX = 3, 8
MODULE_GATE_UP, MODULE_DOWN = 0, 1
EXPERT_SHARED = -1
MAX_TOKENS = 65536
STATIC_SCRATCH_BYTES = 16 << 20
LUT_HALVES_PER_ROW = sum(1 << k for k in range(QMIN, QMAX + 1))

# every function declared in include/pw.h
EXPORTS = (
    "pw_last_error", "pw_create", "pw_destroy", "pw_pack_bitplanes", "pw_plane_words",
    "pw_register_block", "pw_workspace_size", "pw_decode_tokens_per_pass", "pw_set_tokens_per_pass", "pw_route_topk", "pw_permute_by_expert", "pw_route_permute",
    "pw_moe_ffn_bitplane", "pw_moe_layer", "pw_moe_layer_noalloc", "pw_routing_mass_enable", "pw_routing_mass_reset",
    "pw_routing_mass_read", "pw_plan_widths", "pw_request_widths", "pw_commit_ready", "pw_block_state",
    "pw_set_committed_bits", "pw_get_committed_bits", "pw_block_id", "pw_plane_states", "pw_committed_widths",
    "pw_routing_mass_copy", "pw_plan_event", "pw_retarget", "pw_trim", "pw_pool_stats",
    "pw_resident_bytes", "pw_debug_decode", "pw_debug_decode_codes", "pw_debug_dequant", "pw_profile_enable",
    "pw_profile_read",
)


PAGE_RESIDENT, PAGE_IN_TRANSFER, PAGE_READY = 0, 1, 2
PLANE_GPU, PLANE_IN_TRANSFER, PLANE_READY, PLANE_CPU, PLANE_ABSENT = 0, 1, 2, 3, 4
DECODE_PATH_TILE128, DECODE_PATH_TILE64, DECODE_PATH_PREFILL, DECODE_PATH_TILE64_WIDE = 0, 1, 2, 3


class PlanParams(ctypes.Structure):
    """pw_plan_params: width floors, hot-expert threshold and multiplier."""
    _fields_ = [("q_min", ctypes.c_int), ("q_max", ctypes.c_int), ("hot_floor", ctypes.c_int),
                ("hot_share", ctypes.c_double), ("hot_mult", ctypes.c_double), ("mass_eps", ctypes.c_double)]


class PwError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("pw status %d: %s" % (status, msg))
        self.status = status


class ModelDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("inter_shared", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("keep_host_masters", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpw.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libpw.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.pw_last_error.restype = ctypes.c_char_p
        L.pw_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(ModelDesc)]
        L.pw_destroy.argtypes = [vp]
        L.pw_pack_bitplanes.argtypes = [vp, i64, i64, vp]
        L.pw_plane_words.argtypes = [i64, i64]
        L.pw_plane_words.restype = i64
        L.pw_register_block.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int]
        L.pw_workspace_size.argtypes = [vp, ctypes.c_int]
        L.pw_workspace_size.restype = sz
        L.pw_decode_tokens_per_pass.argtypes = [ctypes.c_int] * 4
        L.pw_decode_tokens_per_pass.restype = i32
        L.pw_set_tokens_per_pass.argtypes = [vp, ctypes.c_int]
        L.pw_route_topk.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp]
        L.pw_permute_by_expert.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp]
        L.pw_route_permute.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp]
        L.pw_moe_ffn_bitplane.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pw_moe_layer.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pw_moe_layer_noalloc.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp]
        L.pw_request_widths.argtypes = [vp, ctypes.c_int, vp, vp, vp]
        L.pw_commit_ready.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int)]
        L.pw_block_state.argtypes = [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.pw_routing_mass_enable.argtypes = [vp, ctypes.c_int]
        L.pw_routing_mass_reset.argtypes = [vp, vp]
        L.pw_routing_mass_read.argtypes = [vp, vp, vp]
        L.pw_plan_widths.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                     ctypes.POINTER(PlanParams), i64, vp, ctypes.POINTER(i64)]
        L.pw_set_committed_bits.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp]
        L.pw_plane_states.argtypes = [vp, i32, vp]
        L.pw_committed_widths.argtypes = [vp, vp]
        L.pw_routing_mass_copy.argtypes = [vp, vp, vp]
        L.pw_plan_event.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp,
                                    ctypes.POINTER(ctypes.c_int)]
        L.pw_retarget.argtypes = [vp, i64, vp, vp, ctypes.POINTER(PlanParams), vp, ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(i64)]
        L.pw_trim.argtypes = [vp, ctypes.POINTER(i64)]
        L.pw_pool_stats.argtypes = [vp] + [ctypes.POINTER(i64)] * 6
        L.pw_get_committed_bits.argtypes = [vp, i32, ctypes.POINTER(i32)]
        L.pw_block_id.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.pw_block_id.restype = i32
        L.pw_resident_bytes.argtypes = [vp]
        L.pw_resident_bytes.restype = i64
        L.pw_debug_decode.argtypes = [vp, i32, ctypes.c_int, vp, vp, vp]
        L.pw_debug_decode_codes.argtypes = [vp, i32, vp, vp]
        L.pw_debug_dequant.argtypes = [vp, i32, vp, vp]
        L.pw_profile_enable.argtypes = [vp, ctypes.c_int]
        L.pw_profile_read.argtypes = [vp, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(i64)]
        for name in EXPORTS:
            if name not in ("pw_last_error", "pw_plane_words", "pw_workspace_size", "pw_block_id",
                            "pw_resident_bytes", "pw_decode_tokens_per_pass"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().pw_last_error().decode()


def _check(st: int) -> None:
    if st != PW_OK:
        raise PwError(st, last_error())


def _ptr(t) -> int:
    """Device or host address of a torch tensor, numpy array or int (0 = NULL)."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    assert t.is_contiguous(), "tensor must be contiguous"
    return t.data_ptr()


def _stream(s) -> int:
    """hipStream_t of a torch stream (None = torch's current stream)."""
    if isinstance(s, int):
        return s
    if s is None:
        import torch
        s = torch.cuda.current_stream()
    return s.cuda_stream


# ---------------------------------------------------------------- host helpers

def plane_words(R: int, K: int) -> int:
    return int(lib().pw_plane_words(R, K))


def pack_bitplanes(code8: np.ndarray) -> np.ndarray:
    """uint8 [R][K] parent codes -> uint32 [8][plane_words] bit-planes (library packer)."""
    c = np.ascontiguousarray(code8, dtype=np.uint8)
    R, K = c.shape
    out = np.empty((8, plane_words(R, K)), dtype=np.uint32)
    _check(lib().pw_pack_bitplanes(_ptr(c), R, K, _ptr(out)))
    return out


def concat_luts(luts: Dict[int, np.ndarray]) -> np.ndarray:
    """LUT_3..LUT_8 (fp16 [R][2^k] each) -> uint16 [R * 504] in the ABI's order."""
    parts = [np.ascontiguousarray(luts[k], dtype=np.float16).view(np.uint16).reshape(-1)
             for k in range(QMIN, QMAX + 1)]
    return np.concatenate(parts)


class Context:
    """Owns a pw_ctx: the weight page table, device slabs and host masters."""

    def __init__(self, device: int, num_layers: int, num_experts: int, hidden: int, inter: int,
                 top_k: int, inter_shared: int = 0, keep_host_masters: bool = True):
        self.desc = ModelDesc(num_layers, num_experts, hidden, inter, inter_shared, top_k,
                              1 if keep_host_masters else 0)
        h = ctypes.c_void_p()
        _check(lib().pw_create(ctypes.byref(h), device, ctypes.byref(self.desc)))
        self.h = h

    def close(self) -> None:
        if self.h:
            _check(lib().pw_destroy(self.h))
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # page table ---------------------------------------------------------
    def block_id(self, layer: int, expert: int, module: int) -> int:
        return int(lib().pw_block_id(self.h, layer, expert, module))

    def register_block(self, layer: int, expert: int, module: int, planes: np.ndarray,
                       luts: np.ndarray, q: int) -> None:
        p = np.ascontiguousarray(planes, dtype=np.uint32)
        l_ = np.ascontiguousarray(luts, dtype=np.uint16)
        _check(lib().pw_register_block(self.h, layer, expert, module, _ptr(p), _ptr(l_), int(q)))

    def register_code_block(self, layer: int, expert: int, module: int, code8: np.ndarray,
                            luts: Dict[int, np.ndarray], q: int) -> None:
        self.register_block(layer, expert, module, pack_bitplanes(code8), concat_luts(luts), q)

    def committed_bits(self, block_id: int) -> int:
        q = ctypes.c_int32()
        _check(lib().pw_get_committed_bits(self.h, block_id, ctypes.byref(q)))
        return int(q.value)

    def set_committed_bits(self, block_ids: Sequence[int], q_new: Sequence[int],
                           compute=None, copy=None) -> None:
        ids = np.ascontiguousarray(block_ids, dtype=np.int32)
        qs = np.ascontiguousarray(q_new, dtype=np.uint8)
        assert ids.size == qs.size
        _check(lib().pw_set_committed_bits(self.h, ids.size, _ptr(ids), _ptr(qs), _stream(compute),
                                           _stream(copy) if copy is not None else _stream(compute)))

    def resident_bytes(self) -> int:
        return int(lib().pw_resident_bytes(self.h))

    # hot path -----------------------------------------------------------
    def workspace_size(self, T: int) -> int:
        return int(lib().pw_workspace_size(self.h, T))

    def set_tokens_per_pass(self, tokens: int) -> None:
        """pw_set_tokens_per_pass: 8, 16 or 32 tokens per decode pass for this
        context's later calls, 0 for the per-call choice."""
        _check(lib().pw_set_tokens_per_pass(self.h, tokens))

    def route_topk(self, logits, T: int, topk_idx, topk_w, stream=None) -> None:
        _check(lib().pw_route_topk(self.h, _ptr(logits), T, _ptr(topk_idx), _ptr(topk_w), _stream(stream)))

    def permute_by_expert(self, topk_idx, T: int, offsets, sorted_assign, stream=None) -> None:
        _check(lib().pw_permute_by_expert(self.h, _ptr(topk_idx), T, _ptr(offsets), _ptr(sorted_assign),
                                          _stream(stream)))

    def route_permute(self, logits, T: int, topk_idx, topk_w, offsets, sorted_assign, stream=None) -> None:
        _check(lib().pw_route_permute(self.h, _ptr(logits), T, _ptr(topk_idx), _ptr(topk_w), _ptr(offsets),
                                      _ptr(sorted_assign), _stream(stream)))

    def moe_ffn_bitplane(self, layer: int, x, T: int, topk_idx, topk_w, offsets, sorted_assign, y,
                         workspace, ws_bytes: Optional[int] = None, stream=None) -> None:
        if ws_bytes is None:
            ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib().pw_moe_ffn_bitplane(self.h, layer, _ptr(x), T, _ptr(topk_idx), _ptr(topk_w),
                                         _ptr(offsets), _ptr(sorted_assign), _ptr(y), _ptr(workspace),
                                         ws_bytes, _stream(stream)))

    def moe_layer(self, layer: int, logits, x, T: int, topk_idx, topk_w, offsets, sorted_assign, y,
                  workspace, ws_bytes: Optional[int] = None, stream=None) -> None:
        if ws_bytes is None:
            ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib().pw_moe_layer(self.h, layer, _ptr(logits), _ptr(x), T, _ptr(topk_idx), _ptr(topk_w),
                                  _ptr(offsets), _ptr(sorted_assign), _ptr(y), _ptr(workspace), ws_bytes,
                                  _stream(stream)))

    def moe_layer_noalloc(self, layer: int, logits, x, T: int, topk_idx, topk_w, offsets, sorted_assign, y,
                          stream=None) -> None:
        _check(lib().pw_moe_layer_noalloc(self.h, layer, _ptr(logits), _ptr(x), T, _ptr(topk_idx), _ptr(topk_w),
                                          _ptr(offsets), _ptr(sorted_assign), _ptr(y), _stream(stream)))

    def request_widths(self, block_ids, q_desired, copy_stream=None) -> None:
        ids = np.ascontiguousarray(block_ids, dtype=np.int32)
        q = np.ascontiguousarray(q_desired, dtype=np.uint8)
        assert ids.shape == q.shape
        _check(lib().pw_request_widths(self.h, int(ids.size), ids.ctypes.data_as(ctypes.c_void_p),
                                       q.ctypes.data_as(ctypes.c_void_p), _stream(copy_stream)))

    def commit_ready(self, compute_stream=None) -> int:
        n = ctypes.c_int(0)
        _check(lib().pw_commit_ready(self.h, _stream(compute_stream), ctypes.byref(n)))
        return n.value

    def block_state(self, block_id: int):
        """(committed q, desired q, state) with state PAGE_RESIDENT / PAGE_IN_TRANSFER / PAGE_READY."""
        qc, qd, st = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pw_block_state(self.h, block_id, ctypes.byref(qc), ctypes.byref(qd), ctypes.byref(st)))
        return qc.value, qd.value, st.value

    def plane_states(self, block_id: int) -> np.ndarray:
        """int32 [9]: state of bit-planes 0..7 and of the desired width's LUT (PLANE_*)."""
        out = np.zeros(9, dtype=np.int32)
        _check(lib().pw_plane_states(self.h, block_id, out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def committed_widths(self) -> np.ndarray:
        """uint8 [L][E + 1][2]: committed width of every block (slot E = shared expert; 0 = not registered)."""
        d = self.desc
        out = np.zeros((d.num_layers, d.num_experts + 1, 2), dtype=np.uint8)
        _check(lib().pw_committed_widths(self.h, out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def routing_mass_copy(self, dst, stream=None) -> None:
        """Enqueue a copy of the routing mass into dst (device tensor or pinned host tensor of L*E fp64)."""
        _check(lib().pw_routing_mass_copy(self.h, _ptr(dst), _stream(stream)))

    def retarget(self, byte_target: int, mass: np.ndarray, sensitivity: np.ndarray, copy_stream=None,
                 q_min: int = 3, q_max: int = 8, hot_floor: int = 6, hot_share: float = 0.1,
                 hot_mult: float = 4.0, mass_eps: float = 1e-3):
        """pw_retarget: (blocks requested, planned routed bytes)."""
        d = self.desc
        m = np.ascontiguousarray(mass, dtype=np.float64).reshape(d.num_layers, d.num_experts)
        s = np.ascontiguousarray(sensitivity, dtype=np.float32).reshape(d.num_layers, d.num_experts, 2)
        p = PlanParams(q_min, q_max, hot_floor, hot_share, hot_mult, mass_eps)
        n, total = ctypes.c_int(0), ctypes.c_int64(0)
        _check(lib().pw_retarget(self.h, int(byte_target), m.ctypes.data_as(ctypes.c_void_p),
                                 s.ctypes.data_as(ctypes.c_void_p), ctypes.byref(p), _stream(copy_stream),
                                 ctypes.byref(n), ctypes.byref(total)))
        return n.value, total.value

    def trim(self) -> int:
        freed = ctypes.c_int64(0)
        _check(lib().pw_trim(self.h, ctypes.byref(freed)))
        return freed.value

    def pool_stats(self) -> dict:
        v = [ctypes.c_int64(0) for _ in range(6)]
        _check(lib().pw_pool_stats(self.h, *[ctypes.byref(x) for x in v]))
        keys = ("resident", "cached", "waiting", "held", "device_allocs", "events")
        return {k: x.value for k, x in zip(keys, v)}

    def routing_mass_enable(self, on: bool = True) -> None:
        _check(lib().pw_routing_mass_enable(self.h, 1 if on else 0))

    def routing_mass_reset(self, stream=None) -> None:
        _check(lib().pw_routing_mass_reset(self.h, _stream(stream)))

    def routing_mass(self, stream=None) -> np.ndarray:
        """The accumulated routing mass [L][E] (fp64) after the work on `stream`."""
        d = self.desc
        out = np.zeros((d.num_layers, d.num_experts), dtype=np.float64)
        _check(lib().pw_routing_mass_read(self.h, out.ctypes.data_as(ctypes.c_void_p), _stream(stream)))
        return out

    # test exports and profiling ----------------------------------------
    def debug_decode(self, block_id: int, path: int, codes_out=None, w_out=None, stream=None) -> None:
        _check(lib().pw_debug_decode(self.h, block_id, int(path), _ptr(codes_out), _ptr(w_out), _stream(stream)))

    def debug_decode_codes(self, block_id: int, out, stream=None) -> None:
        _check(lib().pw_debug_decode_codes(self.h, block_id, _ptr(out), _stream(stream)))

    def debug_dequant(self, block_id: int, out, stream=None) -> None:
        _check(lib().pw_debug_dequant(self.h, block_id, _ptr(out), _stream(stream)))

    def profile_enable(self, on: bool = True) -> None:
        _check(lib().pw_profile_enable(self.h, 1 if on else 0))

    def profile_read(self, kernel: str):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        _check(lib().pw_profile_read(self.h, kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
        return float(ms.value), int(n.value)


def decode_tokens_per_pass(T: int, top_k: int, E: int, I_shared: int = 0) -> int:
    """pw_decode_tokens_per_pass: 8, 16 or 32 tokens per decode pass for a
    call of T tokens (0: no decode call, or the prefill path)."""
    return int(lib().pw_decode_tokens_per_pass(T, top_k, E, I_shared))


def plan_event(q_cur: np.ndarray, mass: np.ndarray, lower: bool, n_change: int, skip: Optional[np.ndarray] = None):
    """pw_plan_event: (block ids int32, new widths uint8) of one fixed-fraction
    commit event.  q_cur: [L][E][2]; mass: [L][E]; skip: [L][E][2] or None."""
    q = np.ascontiguousarray(q_cur, dtype=np.uint8)
    L, E = q.shape[0], q.shape[1]
    m = np.ascontiguousarray(mass, dtype=np.float64).reshape(L, E)
    sk = None if skip is None else np.ascontiguousarray(skip, dtype=np.uint8).reshape(L, E, 2)
    ids = np.zeros(max(n_change, 1), dtype=np.int32)
    qs = np.zeros(max(n_change, 1), dtype=np.uint8)
    n = ctypes.c_int(0)
    _check(lib().pw_plan_event(L, E, q.ctypes.data_as(ctypes.c_void_p), m.ctypes.data_as(ctypes.c_void_p),
                               None if sk is None else sk.ctypes.data_as(ctypes.c_void_p), 1 if lower else 0,
                               int(n_change), ids.ctypes.data_as(ctypes.c_void_p), qs.ctypes.data_as(ctypes.c_void_p),
                               ctypes.byref(n)))
    return ids[:n.value].copy(), qs[:n.value].copy()


def plan_widths(H: int, I: int, q_cur: np.ndarray, mass: np.ndarray, sensitivity: np.ndarray,
                byte_target: int, q_min: int = 3, q_max: int = 8, hot_floor: int = 6, hot_share: float = 0.1,
                hot_mult: float = 4.0, mass_eps: float = 1e-3):
    """pw_plan_widths: new widths [L][E][2] (uint8) and the routed blocks'
    bytes at those widths.  q_cur: [L][E][2]; mass: [L][E]; sensitivity:
    [L][E][2]."""
    q_cur = np.ascontiguousarray(q_cur, dtype=np.uint8)
    L, E = q_cur.shape[0], q_cur.shape[1]
    mass = np.ascontiguousarray(mass, dtype=np.float64).reshape(L, E)
    sens = np.ascontiguousarray(sensitivity, dtype=np.float32).reshape(L, E, 2)
    out = np.zeros_like(q_cur)
    total = ctypes.c_int64(0)
    p = PlanParams(q_min, q_max, hot_floor, hot_share, hot_mult, mass_eps)
    _check(lib().pw_plan_widths(L, E, H, I, q_cur.ctypes.data_as(ctypes.c_void_p), mass.ctypes.data_as(ctypes.c_void_p),
                                sens.ctypes.data_as(ctypes.c_void_p), ctypes.byref(p), int(byte_target),
                                out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(total)))
    return out, int(total.value)
