"""fp64 CPU oracle of the mixture-of-experts FFN block -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU path never calls it, and it
shares no code with the GPU path: the arithmetic lives in ``moe_oracle.c``
(plain fp64 loops, compiled by gcc), and this module only marshals numpy
arrays into it.

What it computes, and the passages it follows (archdiff.com comparison pages):

* ``router_logits`` -- "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro", component
  table, router row, Qwen3.5 cell: each expert's logit is a linear function
  of the token vector, x . W_r.
* ``route`` -- same row: softmax, top-k, renormalise, no selection bias
  (Qwen3.5 cell); sqrt-softplus affinities with a selection-only per-expert
  bias, selected scores normalised and scaled by 2.5 (DeepSeek-V4-Pro cell);
  the blueprint router box (sigma or sqrt-softplus, balanced by a bias) for the
  sigmoid score.  Ties at the top-k boundary go to the lower expert index
  (the pages are silent; this is the reading taken).
* ``route_hashed`` -- same row, DeepSeek-V4-Pro cell: in its first three
  MoE layers a fixed hash of the token id, not the router, picks the experts.  Read as a fixed table of k
  expert ids per token id; the combine weights stay the router's (the same
  formulas as ``route``, on the table's experts).
* ``bias_update`` -- same cell: auxiliary-loss-free balancing with bias speed
  0.001; each selection bias moves by the speed towards balance, by the sign of
  (mean load - the expert's load) over the batch's assignments.
* ``permute`` -- expert-contiguous order of the (token, slot) assignments,
  stable in token order (a counting sort; the pages imply the grouping by
  selecting routed experts per token).
* ``quant_rows`` / ``e4m3_*`` -- blueprint training box (FP8 with block scales):
  E4M3FN, one fp32 scale (group max / 448) per 128-value group.
* ``e2m1_value`` / ``e8m0_value`` and ``ExpertSet(fmt="mxfp4")`` -- the same box names
  MXFP4: OCP MX E2M1 elements with one E8M0 (power-of-two) scale per 32 values along
  the reduction axis.
* ``moe_tokens`` -- "Qwen3.5-397B-A17B vs Gemma 4 31B", component table,
  routed-experts row (SwiGLU experts) and shared-expert row (the shared
  expert's output is added to the routed sum; in the Qwen3.5 cell scaled
  first by a per-token sigmoid gate of a learned vector); blueprint
  shared-expert box (one or two shared experts used by every token).

Parity status per function is listed in the module docstrings of the tests
that pin it (``tests/test_oracle_*.py``).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, E4M3, MXFP4 = 0, 1, 2, 3
SOFTMAX, SIGMOID, SQRT_SOFTPLUS = 0, 1, 2

_LIB = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)
_up = ctypes.POINTER(ctypes.c_uint8)


class _ExpertSet(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("n", ctypes.c_int),
                ("gate", ctypes.POINTER(ctypes.c_void_p)),
                ("up", ctypes.POINTER(ctypes.c_void_p)),
                ("down", ctypes.POINTER(ctypes.c_void_p)),
                ("gate_scales", ctypes.POINTER(ctypes.c_void_p)),
                ("up_scales", ctypes.POINTER(ctypes.c_void_p)),
                ("down_scales", ctypes.POINTER(ctypes.c_void_p))]


class _FfnCfg(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("f", ctypes.c_int), ("k", ctypes.c_int),
                ("f_shared", ctypes.c_int), ("quant", ctypes.c_int), ("block", ctypes.c_int),
                ("shared_gate", ctypes.POINTER(ctypes.c_double))]


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_round.restype = ctypes.c_double
        L.orc_e4m3_round.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
        L.orc_quant_rows.restype = None
        L.orc_quant_rows.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _up, _fp, _dp]
        L.orc_router_logits.restype = None
        L.orc_router_logits.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp,
                                        ctypes.c_int, ctypes.c_void_p, _fp, _dp]
        L.orc_score.restype = ctypes.c_double
        L.orc_score.argtypes = [ctypes.c_int, ctypes.c_double]
        L.orc_route.restype = ctypes.c_int
        L.orc_route.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_double, _dp, _fp, _ip, _dp, _dp]
        L.orc_permute.restype = ctypes.c_int
        L.orc_permute.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _ip, _ip, _ip, _ip]
        L.orc_route_hashed.restype = ctypes.c_int
        L.orc_route_hashed.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_double, _dp, _ip, ctypes.c_int,
                                       _ip, _ip, _dp]
        L.orc_bias_update.restype = ctypes.c_int
        L.orc_bias_update.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _ip,
                                      ctypes.c_float, _fp]
        L.orc_moe_tokens.restype = ctypes.c_int
        L.orc_moe_tokens.argtypes = [ctypes.POINTER(_FfnCfg), ctypes.c_int, _dp, _ip, _dp,
                                     ctypes.POINTER(_ExpertSet), ctypes.POINTER(_ExpertSet), _dp]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_num_threads.argtypes = []
        _LIB = L
    return _LIB


def _ptr(a, t):
    return a.ctypes.data_as(t)


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use."""
    return int(lib().orc_num_threads())


# --------------------------------------------------------------------------- formats

def bf16_value(bits):
    """Exact fp64 values of bfloat16 bit patterns (uint16 array)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return np.array([lib().orc_bf16_value(int(b)) for b in bits.ravel()]).reshape(bits.shape)


def e4m3_value(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib().orc_e4m3_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e4m3_round(values):
    values = np.asarray(values, dtype=np.float64)
    return np.array([lib().orc_e4m3_round(float(v)) for v in values.ravel()]).reshape(values.shape)


def e4m3_encode(values):
    values = np.asarray(values, dtype=np.float64)
    return np.array([lib().orc_e4m3_encode(float(v)) for v in values.ravel()],
                    dtype=np.uint8).reshape(values.shape)


def e2m1_value(codes):
    """fp64 values of 4-bit E2M1 codes (MXFP4 elements)."""
    return np.array([lib().orc_e2m1_value(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def e8m0_value(codes):
    """fp64 values of E8M0 scale codes (2^(code - 127))."""
    return np.array([lib().orc_e8m0_value(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def quant_rows(x, group=128):
    """Block-scaled FP8 quantisation of each row in groups of ``group`` values.

    Returns (codes uint8 [R,C], scales float32 [R,C/group], dequantised fp64 [R,C])."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    R, C = x.shape
    assert C % group == 0
    codes = np.empty((R, C), np.uint8)
    scales = np.empty((R, C // group), np.float32)
    xdq = np.empty((R, C), np.float64)
    lib().orc_quant_rows(_ptr(x, _dp), R, C, group, _ptr(codes, _up), _ptr(scales, _fp),
                         _ptr(xdq, _dp))
    return codes, scales, xdq


# --------------------------------------------------------------------------- storage

def storage_dtype(arr) -> int:
    """Oracle dtype code of a stored weight array (numpy)."""
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.uint8:
        return E4M3
    raise TypeError(f"unsupported storage dtype {arr.dtype}")


# --------------------------------------------------------------------------- router

def router_logits(x, w_router, logit_bias=None):
    """l = x W_r (+ z).  x: fp64 [T,d]; w_router: stored [d,E] (float32 or bf16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    w_router = np.ascontiguousarray(w_router)
    T, d = x.shape
    d2, E = w_router.shape
    assert d == d2
    out = np.empty((T, E), np.float64)
    lb = None
    if logit_bias is not None:
        lb = np.ascontiguousarray(logit_bias, dtype=np.float32)
    lib().orc_router_logits(T, d, E, _ptr(x, _dp), storage_dtype(w_router),
                            w_router.ctypes.data_as(ctypes.c_void_p),
                            _ptr(lb, _fp) if lb is not None else None, _ptr(out, _dp))
    return out


def score(kind, l):
    return lib().orc_score(int(kind), float(l))


def route(logits, k, score_kind=SOFTMAX, renormalize=True, gamma=1.0, select_bias=None):
    """Top-k ids (key desc, lower index on ties), combine weights, selected scores."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    s = np.empty((T, k), np.float64)
    sb = None
    if select_bias is not None:
        sb = np.ascontiguousarray(select_bias, dtype=np.float32)
    rc = lib().orc_route(T, E, k, int(score_kind), int(bool(renormalize)), float(gamma),
                         _ptr(logits, _dp), _ptr(sb, _fp) if sb is not None else None,
                         _ptr(ids, _ip), _ptr(w, _dp), _ptr(s, _dp))
    if rc != 0:
        raise ValueError("oracle route: k out of range")
    return ids, w, s


def route_hashed(logits, token_ids, table, score_kind=SOFTMAX, renormalize=True, gamma=1.0):
    """Experts from a fixed token-id table (ids[t] = table[token_ids[t]]) and the router's
    combine weights for them."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    token_ids = np.ascontiguousarray(token_ids, dtype=np.int32)
    table = np.ascontiguousarray(table, dtype=np.int32)
    T, E = logits.shape
    vocab, k = table.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = lib().orc_route_hashed(T, E, k, int(score_kind), int(bool(renormalize)), float(gamma),
                                _ptr(logits, _dp), _ptr(token_ids, _ip), vocab,
                                _ptr(table, _ip), _ptr(ids, _ip), _ptr(w, _dp))
    if rc != 0:
        raise ValueError("oracle route_hashed: token id or table entry out of range")
    return ids, w


def bias_update(bias, ids, num_experts, speed=0.001):
    """One balancing step of the fp32 selection bias from the batch's expert ids [T, k]."""
    b = np.array(bias, dtype=np.float32, copy=True)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    rc = lib().orc_bias_update(T, k, num_experts, _ptr(ids, _ip), float(np.float32(speed)),
                               _ptr(b, _fp))
    if rc != 0:
        raise ValueError("oracle bias_update: expert id out of range")
    return b


def permute(ids, num_experts):
    """(off[E+1], perm_token[T*k], inv_perm[T*k]) of the stable expert-contiguous order."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    off = np.empty(num_experts + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    rc = lib().orc_permute(T, k, num_experts, _ptr(ids, _ip), _ptr(off, _ip), _ptr(perm, _ip),
                           _ptr(inv, _ip))
    if rc != 0:
        raise ValueError("oracle permute: expert id out of range")
    return off, perm, inv


# --------------------------------------------------------------------------- experts

class ExpertSet:
    """Per-expert stored weights for the oracle.

    ``gate[e]``, ``up[e]``: [d, f]; ``down[e]``: [f, d] -- float32, bf16 bits
    (uint16) or E4M3 codes (uint8) with ``*_scales[e]`` float32
    [rows/128, cols/128].  ``fmt="mxfp4"``: stored transposed, ``gate[e]``/``up[e]``
    uint8 [f, d/2] and ``down[e]`` [d, f/2], two E2M1 codes per byte (lower K index in the
    low nibble), with E8M0 scale bytes ``*_scales[e]`` [f, d/32] / [d, f/32].  Entries may be
    ``None`` for experts no token uses."""

    def __init__(self, n, gate, up, down, gate_scales=None, up_scales=None, down_scales=None,
                 fmt=None):
        self.n = n
        self.fmt = fmt
        self.gate, self.up, self.down = gate, up, down
        self.gate_scales, self.up_scales, self.down_scales = gate_scales, up_scales, down_scales

    def _c(self):
        keep = []

        def arr(lst):
            ptrs = (ctypes.c_void_p * max(self.n, 1))()
            for i in range(self.n):
                a = lst[i] if lst is not None else None
                if a is not None:
                    a = np.ascontiguousarray(a)
                    keep.append(a)
                    ptrs[i] = a.ctypes.data
            keep.append(ptrs)
            return ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))

        dtype = MXFP4 if self.fmt == "mxfp4" else None
        for lst in (() if dtype is not None else (self.gate, self.up, self.down)):
            for a in lst:
                if a is not None:
                    dtype = storage_dtype(np.asarray(a))
                    break
            if dtype is not None:
                break
        s = _ExpertSet(dtype if dtype is not None else F32, self.n, arr(self.gate),
                       arr(self.up), arr(self.down), arr(self.gate_scales),
                       arr(self.up_scales), arr(self.down_scales))
        return s, keep


def moe_tokens(x, ids, w, routed: ExpertSet, shared: ExpertSet, d, f, f_shared, quant=False,
               block=128, shared_gate=None):
    """Block output for the given token rows: G * shared SwiGLU(s) + sum_j w_j SwiGLU_{ids_j},
    G = sigmoid(x~ . shared_gate) when a gate vector [d] is given (exact values), else 1."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    n, k = ids.shape
    assert x.shape == (n, d)
    gate = None
    if shared_gate is not None:
        gate = np.ascontiguousarray(shared_gate, dtype=np.float64)
        assert gate.shape == (d,)
    cfg = _FfnCfg(d, f, k, f_shared, int(bool(quant)), block,
                  None if gate is None else _ptr(gate, _dp))
    rs, keep_r = routed._c()
    if shared is not None and shared.n > 0:
        ss, keep_s = shared._c()
        sp = ctypes.pointer(ss)
    else:
        keep_s, sp = [], None
    out = np.empty((n, d), np.float64)
    rc = lib().orc_moe_tokens(ctypes.byref(cfg), n, _ptr(x, _dp), _ptr(ids, _ip), _ptr(w, _dp),
                              ctypes.byref(rs), sp, _ptr(out, _dp))
    del keep_r, keep_s
    if rc != 0:
        raise ValueError("oracle moe_tokens: an expert was not supplied or an id is out of range")
    return out
