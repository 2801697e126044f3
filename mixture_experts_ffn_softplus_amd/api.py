"""Python binding of the C ABI in include/moe.h (ctypes; argument marshalling only).

Every step of the block runs in the HIP library ``libmoe_mi355x.so``; this module passes
torch tensors' device pointers and torch's current HIP stream to it.  Importing it without
the built library raises: there is no fallback path.
"""
import ctypes
import os

import torch

from .configs import BF16, F32, FP8_E4M3, MXFP4, MoEConfig

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED = 0, 1, 2
MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = 3, 4

(PACK_ROUTER, PACK_GATE_UP, PACK_GATE_UP_SCALES, PACK_DOWN, PACK_DOWN_SCALES,
 PACK_SHARED_GATE_UP, PACK_SHARED_GATE_UP_SCALES, PACK_SHARED_DOWN,
 PACK_SHARED_DOWN_SCALES) = range(9)
PACK_COUNT = 9

EXPORTED = ["moe_status_string", "moe_workspace_size", "moe_packed_size", "moe_pack_weights",
            "moe_route", "moe_route_from_logits", "moe_route_hashed", "moe_update_bias",
            "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_forward_noalloc"]

# bytes of the library's own workspace behind moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class moe_config_t(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("num_shared", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("score", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("quant_block", ctypes.c_int32),
                ("shared_gate", ctypes.c_int32), ("out_f32", ctypes.c_int32)]


_vp = ctypes.c_void_p


class moe_logical_weights_t(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "w_router", "w_gate", "w_up", "w_down", "w_gate_scales", "w_up_scales",
        "w_down_scales", "ws_gate", "ws_up", "ws_down", "ws_gate_scales", "ws_up_scales",
        "ws_down_scales")]


class moe_weights_t(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "w_router", "logit_bias", "select_bias", "w_gate_up", "w_gate_up_scales", "w_down",
        "w_down_scales", "ws_gate_up", "ws_gate_up_scales", "ws_down", "ws_down_scales",
        "ws_gate_vec")]


NUM_STAGE_EVENTS = 8
STAGES = ["route", "permute", "tile_list", "gate_up", "down", "shared_gate_up", "combine"]


class moe_debug_t(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "logits", "topk_ids", "topk_w", "expert_offsets", "perm_token", "inv_perm", "y_perm",
        "stage_events")]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)}")
        self.status = status


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        cp = ctypes.POINTER(moe_config_t)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_workspace_size.restype = ctypes.c_size_t
        L.moe_workspace_size.argtypes = [cp]
        L.moe_packed_size.restype = ctypes.c_size_t
        L.moe_packed_size.argtypes = [cp, ctypes.c_int]
        L.moe_pack_weights.restype = ctypes.c_int
        L.moe_pack_weights.argtypes = [cp, ctypes.POINTER(moe_logical_weights_t),
                                       ctypes.POINTER(_vp), _vp]
        wp = ctypes.POINTER(moe_weights_t)
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [cp, _vp, wp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moe_route_from_logits.restype = ctypes.c_int
        L.moe_route_from_logits.argtypes = [cp, _vp, _vp, _vp, _vp, _vp]
        L.moe_route_hashed.restype = ctypes.c_int
        L.moe_route_hashed.argtypes = [cp, _vp, wp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                       _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moe_update_bias.restype = ctypes.c_int
        L.moe_update_bias.argtypes = [cp, _vp, ctypes.c_float, _vp, _vp]
        L.moe_permute.restype = ctypes.c_int
        L.moe_permute.argtypes = [cp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [cp, _vp, _vp, _vp, _vp, wp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [cp, _vp, _vp, _vp, _vp, _vp, wp, _vp, _vp, ctypes.c_size_t,
                                  _vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward.argtypes = [cp, _vp, wp, _vp, ctypes.POINTER(moe_debug_t), _vp,
                                  ctypes.c_size_t, _vp]
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = [cp, _vp, wp, _vp, ctypes.POINTER(moe_debug_t), _vp]
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def _p(t):
    """Device pointer of a tensor (None -> NULL); ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def config_struct(cfg: MoEConfig, **override) -> moe_config_t:
    c = moe_config_t(cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k, cfg.d_ff,
                     cfg.num_shared, cfg.d_ff_shared, cfg.score, cfg.renormalize,
                     cfg.routed_scale, cfg.act_dtype, cfg.expert_dtype, cfg.router_dtype,
                     cfg.quant_block, cfg.shared_gate, cfg.out_f32)
    for k, v in override.items():
        setattr(c, k, v)
    return c


def _cfg(cfg):
    return ctypes.byref(cfg if isinstance(cfg, moe_config_t) else config_struct(cfg))


def _tokens(c: MoEConfig) -> int:
    return c.num_tokens


def _assignments(c: MoEConfig) -> int:
    return c.assignments


def _need(t, cfg, rows_of, dtype_of, where, what):
    """A tensor the library writes must be a contiguous [rows_of(cfg), d] buffer of the dtype
    the config implies: the C entry points take bare pointers and cannot check it.  (Checked
    for a MoEConfig and a torch tensor; raw structs and pointers pass through.)"""
    if not isinstance(t, torch.Tensor) or not isinstance(cfg, MoEConfig):
        return
    n, dt = rows_of(cfg) * cfg.d_model, dtype_of(cfg)
    if t.dtype != dt or t.numel() < n or not t.is_contiguous():
        raise ValueError(f"{where}: {what} must be a contiguous {dt} tensor of at least {n} "
                         f"elements, got {t.dtype} with {t.numel()}")


# ------------------------------------------------------------------ the C entry points

def moe_workspace_size(cfg) -> int:
    return int(lib().moe_workspace_size(_cfg(cfg)))


def moe_packed_size(cfg, which: int) -> int:
    return int(lib().moe_packed_size(_cfg(cfg), int(which)))


def moe_pack_weights(cfg, logical: moe_logical_weights_t, packed, stream=None):
    arr = (_vp * PACK_COUNT)(*[_p(t) for t in packed])
    _check(lib().moe_pack_weights(_cfg(cfg), ctypes.byref(logical), arr, _stream(stream)),
           "moe_pack_weights")


def moe_route(cfg, x, weights: moe_weights_t, logits, topk_ids, topk_w, xq=None,
              xq_scales=None, ws=None, stream=None):
    _check(lib().moe_route(_cfg(cfg), _p(x), ctypes.byref(weights), _p(logits), _p(topk_ids),
                           _p(topk_w), _p(xq), _p(xq_scales), _p(ws),
                           ws.numel() * ws.element_size() if ws is not None else 0,
                           _stream(stream)), "moe_route")


def moe_route_from_logits(cfg, logits, select_bias, topk_ids, topk_w, stream=None):
    _check(lib().moe_route_from_logits(_cfg(cfg), _p(logits), _p(select_bias), _p(topk_ids),
                                       _p(topk_w), _stream(stream)), "moe_route_from_logits")


def moe_route_hashed(cfg, x, weights, token_ids, hash_table, logits, topk_ids, topk_w, xq=None,
                     xq_scales=None, ws=None, stream=None):
    """hash_table: int32 [vocab, k] on the device; token_ids: int32 [T]."""
    _check(lib().moe_route_hashed(_cfg(cfg), _p(x), ctypes.byref(weights), _p(token_ids),
                                  _p(hash_table), int(hash_table.shape[0]), _p(logits),
                                  _p(topk_ids), _p(topk_w), _p(xq), _p(xq_scales), _p(ws),
                                  ws.numel() * ws.element_size() if ws is not None else 0,
                                  _stream(stream)), "moe_route_hashed")


def moe_update_bias(cfg, expert_offsets, select_bias, speed=0.001, stream=None):
    """One balancing step of the fp32 selection bias [E], in place."""
    _check(lib().moe_update_bias(_cfg(cfg), _p(expert_offsets), float(speed), _p(select_bias),
                                 _stream(stream)), "moe_update_bias")


def moe_permute(cfg, topk_ids, expert_offsets, perm_token, inv_perm, ws, stream=None):
    _check(lib().moe_permute(_cfg(cfg), _p(topk_ids), _p(expert_offsets), _p(perm_token),
                             _p(inv_perm), _p(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "moe_permute")


def moe_expert_ffn(cfg, x_or_xq, xq_scales, expert_offsets, perm_token, weights, y_perm, ws,
                   stream=None):
    _need(y_perm, cfg, _assignments, y_dtype, "moe_expert_ffn", "y_perm")
    _check(lib().moe_expert_ffn(_cfg(cfg), _p(x_or_xq), _p(xq_scales), _p(expert_offsets),
                                _p(perm_token), ctypes.byref(weights), _p(y_perm), _p(ws),
                                ws.numel() * ws.element_size(), _stream(stream)),
           "moe_expert_ffn")


def moe_combine(cfg, x_or_xq, xq_scales, y_perm, inv_perm, topk_w, weights, out, ws,
                stream=None):
    _need(out, cfg, _tokens, out_dtype, "moe_combine", "out")
    _check(lib().moe_combine(_cfg(cfg), _p(x_or_xq), _p(xq_scales), _p(y_perm), _p(inv_perm),
                             _p(topk_w), ctypes.byref(weights), _p(out), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "moe_combine")


def moe_forward(cfg, x, weights, out, ws, dbg: dict = None, stream=None):
    _need(out, cfg, _tokens, out_dtype, "moe_forward", "out")
    if dbg:
        _need(dbg.get("y_perm"), cfg, _assignments, y_dtype, "moe_forward", "dbg['y_perm']")
    d = None
    if dbg:
        d = moe_debug_t(*[_p(dbg.get(n)) for n, _ in moe_debug_t._fields_])
    _check(lib().moe_forward(_cfg(cfg), _p(x), ctypes.byref(weights), _p(out),
                             ctypes.byref(d) if d is not None else None, _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")


def moe_forward_noalloc(cfg, x, weights, out, dbg: dict = None, stream=None):
    """moe_forward on the library's own static device workspace (no workspace argument)."""
    _need(out, cfg, _tokens, out_dtype, "moe_forward_noalloc", "out")
    if dbg:
        _need(dbg.get("y_perm"), cfg, _assignments, y_dtype, "moe_forward_noalloc",
              "dbg['y_perm']")
    d = None
    if dbg:
        d = moe_debug_t(*[_p(dbg.get(n)) for n, _ in moe_debug_t._fields_])
    _check(lib().moe_forward_noalloc(_cfg(cfg), _p(x), ctypes.byref(weights), _p(out),
                                     ctypes.byref(d) if d is not None else None,
                                     _stream(stream)), "moe_forward_noalloc")


# ------------------------------------------------------------------ memory plumbing

_TORCH_ACT = {F32: torch.float32, BF16: torch.bfloat16}


def y_dtype(cfg: MoEConfig):
    """Element type of y_perm: fp32 for fp32 experts, fp16 for bf16 experts, bf16 for FP8 /
    MXFP4 experts (E4M3 activations)."""
    if cfg.expert_dtype in (FP8_E4M3, MXFP4):
        return torch.bfloat16
    return torch.float32 if cfg.expert_dtype == F32 else torch.float16


def out_dtype(cfg: MoEConfig):
    return torch.float32 if cfg.out_f32 else _TORCH_ACT[cfg.act_dtype]


def workspace(cfg: MoEConfig, device="cuda") -> torch.Tensor:
    n = moe_workspace_size(cfg)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARGUMENT, "moe_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


class PackedWeights:
    """Packed device buffers of one layer plus the per-expert biases."""

    def __init__(self, cfg: MoEConfig, buffers, logit_bias=None, select_bias=None,
                 shared_gate=None):
        self.cfg = cfg
        self.buffers = buffers
        self.logit_bias = logit_bias
        self.select_bias = select_bias
        self.shared_gate = shared_gate

    def struct(self) -> moe_weights_t:
        b = self.buffers
        return moe_weights_t(
            _p(b[PACK_ROUTER]), _p(self.logit_bias), _p(self.select_bias),
            _p(b[PACK_GATE_UP]), _p(b[PACK_GATE_UP_SCALES]), _p(b[PACK_DOWN]),
            _p(b[PACK_DOWN_SCALES]), _p(b[PACK_SHARED_GATE_UP]),
            _p(b[PACK_SHARED_GATE_UP_SCALES]), _p(b[PACK_SHARED_DOWN]),
            _p(b[PACK_SHARED_DOWN_SCALES]), _p(self.shared_gate))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.buffers if t is not None)


def pack(cfg: MoEConfig, w_router, routed: dict, shared: dict = None, logit_bias=None,
         select_bias=None, stream=None, shared_gate=None) -> PackedWeights:
    """Allocate the packed buffers and fill them with moe_pack_weights."""
    dev = w_router.device
    bufs = []
    for i in range(PACK_COUNT):
        n = moe_packed_size(cfg, i)
        bufs.append(torch.empty(n, dtype=torch.uint8, device=dev) if n else None)
    sh = shared or {}
    lw = moe_logical_weights_t(
        _p(w_router), _p(routed["gate"]), _p(routed["up"]), _p(routed["down"]),
        _p(routed.get("gate_scales")), _p(routed.get("up_scales")),
        _p(routed.get("down_scales")), _p(sh.get("gate")), _p(sh.get("up")), _p(sh.get("down")),
        _p(sh.get("gate_scales")), _p(sh.get("up_scales")), _p(sh.get("down_scales")))
    moe_pack_weights(cfg, lw, bufs, stream)
    return PackedWeights(cfg, bufs, logit_bias, select_bias, shared_gate)
