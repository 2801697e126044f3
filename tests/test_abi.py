"""The C ABI without a GPU: the library loads, exports every symbol include/moe.h declares, the
ctypes structs match the header's layout, and bad arguments return their status codes from
the host-side checks (nothing is launched on these paths)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

from mixture_experts_ffn_softplus_amd import PRESETS, api
from mixture_experts_ffn_softplus_amd.configs import BF16, F32, FP8_E4M3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert set(syms) == set(api.EXPORTED)
    L = api.lib()
    for s in syms:
        assert hasattr(L, s), s
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(syms) <= exported
    # internal kernels and helpers stay hidden
    assert not any(s.startswith("_ZN3moe") for s in exported)


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(moe_config_t), offsetof(moe_config_t, routed_scale),
         offsetof(moe_config_t, quant_block), sizeof(moe_logical_weights_t),
         sizeof(moe_weights_t), sizeof(moe_debug_t));
  return 0;
}''')
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.dirname(HEADER)}",
                        "-I/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot compile the header with gcc here: " + r.stderr[:200])
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(api.moe_config_t), api.moe_config_t.routed_scale.offset,
            api.moe_config_t.quant_block.offset, ctypes.sizeof(api.moe_logical_weights_t),
            ctypes.sizeof(api.moe_weights_t), ctypes.sizeof(api.moe_debug_t)]
    assert got == want


def test_status_strings():
    assert api.status_string(0) == "MOE_OK"
    assert api.status_string(3) == "MOE_ERR_WORKSPACE_TOO_SMALL"
    assert api.status_string(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("field,value,status", [
    ("num_tokens", -1, api.MOE_ERR_INVALID_ARGUMENT),
    ("top_k", 0, api.MOE_ERR_INVALID_ARGUMENT),
    ("top_k", 17, api.MOE_ERR_INVALID_ARGUMENT),        # k > E
    ("num_experts", 0, api.MOE_ERR_INVALID_ARGUMENT),
    ("score", 7, api.MOE_ERR_INVALID_ARGUMENT),
    ("renormalize", 2, api.MOE_ERR_INVALID_ARGUMENT),
    ("routed_scale", float("nan"), api.MOE_ERR_INVALID_ARGUMENT),
    ("d_model", 200, api.MOE_ERR_UNSUPPORTED),           # not a multiple of 128
    ("d_ff", 96, api.MOE_ERR_UNSUPPORTED),
    ("expert_dtype", BF16, api.MOE_ERR_UNSUPPORTED),     # f32 activations with bf16 experts
    ("expert_dtype", 3, api.MOE_ERR_UNSUPPORTED),        # MXFP4 experts need bf16 activations
    ("expert_dtype", 4, api.MOE_ERR_INVALID_ARGUMENT),   # no such format
    ("router_dtype", 3, api.MOE_ERR_UNSUPPORTED),        # MXFP4 is for expert weights only
    ("act_dtype", 5, api.MOE_ERR_INVALID_ARGUMENT),
    ("out_f32", 2, api.MOE_ERR_INVALID_ARGUMENT),
])
def test_config_errors_return_status_without_launch(field, value, status):
    cfg = api.config_struct(PRESETS["tiny_fp32"], **{field: value})
    assert api.moe_workspace_size(cfg) == 0
    L = api.lib()
    w = api.moe_weights_t()
    rc = L.moe_forward(ctypes.byref(cfg), 1, ctypes.byref(w), 1, None, 1, 1 << 40, None)
    assert rc == status


@pytest.mark.parametrize("out_f32, dtype", [(1, torch.bfloat16), (0, torch.float32)])
def test_binding_rejects_an_output_of_another_dtype(out_f32, dtype):
    # the C entry points take bare pointers: a bf16 buffer for an fp32 output would be
    # overrun, so the binding refuses it before anything is launched
    cfg = PRESETS["softmax_bf16"].with_(num_tokens=4, out_f32=out_f32)
    out = torch.empty(4, cfg.d_model, dtype=dtype)
    ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out must be"):
        api.moe_forward(cfg, None, api.moe_weights_t(), out, ws)
    with pytest.raises(ValueError, match="out must be"):
        api.moe_combine(cfg, None, None, None, None, None, api.moe_weights_t(), out, ws)
    y = torch.empty(cfg.assignments, cfg.d_model, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="y_perm must be"):
        api.moe_expert_ffn(cfg, None, None, None, None, api.moe_weights_t(), y, ws)


@pytest.mark.parametrize("preset, y_dtype", [("tiny_fp32", torch.float32),
                                              ("softmax_bf16", torch.float16),
                                              ("fp8_block", torch.bfloat16),
                                              ("mxfp4_decode", torch.bfloat16)])
def test_y_perm_element_type_per_expert_format(preset, y_dtype):
    # y_perm rows: fp32 for fp32 experts, IEEE fp16 for bf16 experts, bf16 for E4M3
    # activations; a buffer of any other element type is refused before a launch (the kernels
    # would write 2-byte rows into a 4-byte buffer's first half, or overrun a 2-byte one)
    cfg = PRESETS[preset].with_(num_tokens=4)
    assert api.y_dtype(cfg) == y_dtype
    ws = torch.empty(16, dtype=torch.uint8)
    for other in (torch.float32, torch.float16, torch.bfloat16):
        if other == y_dtype:
            continue
        y = torch.empty(cfg.assignments, cfg.d_model, dtype=other)
        with pytest.raises(ValueError, match="y_perm must be"):
            api.moe_expert_ffn(cfg, None, None, None, None, api.moe_weights_t(), y, ws)


def test_large_and_fp8_constraints():
    c = api.config_struct(PRESETS["fp8_block"], quant_block=64)
    assert api.lib().moe_workspace_size(ctypes.byref(c)) == 0
    # the limits themselves are accepted, one past either is not
    for over, E, k in [(False, 1024, 64), (True, 1025, 64), (True, 1024, 65), (True, 2048, 8)]:
        c = api.config_struct(PRESETS["softmax_bf16"], num_experts=E, top_k=k)
        assert (api.lib().moe_workspace_size(ctypes.byref(c)) == 0) == over, (E, k)
        if over:
            assert api.lib().moe_route_from_logits(ctypes.byref(c), 1, None, 1, 1, None) == \
                api.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,over,ok", [
    # h = [T*k, d_ff] bf16 = 65536 * 8 * 4096 * 2 B = 4 GiB exactly
    ("softmax_bf16", dict(num_tokens=65536, top_k=8, d_ff=4096), dict(num_tokens=65535)),
    # x = [T, d] bf16 = 4 GiB
    ("softmax_bf16", dict(num_tokens=1 << 19, top_k=1, d_model=4096),
     dict(num_tokens=(1 << 19) - 1)),
    # the shared experts' h = [T, S*f_s] bf16 = 4 GiB
    ("softplus_bf16", dict(num_tokens=1 << 18, top_k=1, num_shared=2, d_ff_shared=4096),
     dict(num_tokens=(1 << 18) - 1)),
    # one routed expert's gate/up weights [2f, d] fp32 = 4 GiB
    ("tiny_fp32", dict(num_tokens=1, d_model=32768, d_ff=16384, d_ff_shared=128),
     dict(d_ff=16384 - 128)),
    # the FP8 h = [T*k, d_ff] E4M3 = 4 GiB
    ("fp8_block", dict(num_tokens=1 << 18, top_k=32, d_ff=512), dict(top_k=31)),
    # T*k = 2^30 assignments: the permutation's row count
    ("softmax_bf16", dict(num_tokens=1 << 27, top_k=8, d_model=128, d_ff=128, d_ff_shared=128),
     dict(num_tokens=1 << 20)),
    # the largest int32 widths: the products of the size arithmetic would overflow 64 bits
    ("softmax_bf16", dict(num_tokens=0, d_model=2**31 - 128, d_ff=2**31 - 128),
     dict(d_model=1 << 20, d_ff=128, d_ff_shared=128)),
])
def test_configs_beyond_32_bit_operands_are_refused(name, over, ok):
    # every GEMM operand goes through a 32-bit buffer resource: a config with an operand of
    # 4 GiB or more is refused before anything is launched, instead of reading wrapped rows
    c = api.config_struct(PRESETS[name], **over)
    L = api.lib()
    assert L.moe_workspace_size(ctypes.byref(c)) == 0
    w = api.moe_weights_t()
    assert L.moe_forward(ctypes.byref(c), 1, ctypes.byref(w), 1, None, 1, 1 << 40, None) == \
        api.MOE_ERR_UNSUPPORTED
    # just inside the limits the same shape is accepted
    c = api.config_struct(PRESETS[name], **{**over, **ok})
    assert L.moe_workspace_size(ctypes.byref(c)) > 0


def test_null_pointers_and_small_workspace():
    L = api.lib()
    cfg = api.config_struct(PRESETS["tiny_fp32"])
    ws_need = api.moe_workspace_size(cfg)
    assert ws_need > 0
    w_ok = api.moe_weights_t(*([8] * 12))
    cp = ctypes.byref(cfg)
    # NULL x / out / weights / ws
    assert L.moe_forward(cp, None, ctypes.byref(w_ok), 8, None, 8, ws_need, None) == 1
    assert L.moe_forward(cp, 8, ctypes.byref(w_ok), None, None, 8, ws_need, None) == 1
    assert L.moe_forward(cp, 8, None, 8, None, 8, ws_need, None) == 1
    assert L.moe_forward(cp, 8, ctypes.byref(w_ok), 8, None, None, ws_need, None) == 1
    # missing router / expert weights
    w_bad = api.moe_weights_t(*([8] * 12))
    w_bad.w_router = None
    assert L.moe_forward(cp, 8, ctypes.byref(w_bad), 8, None, 8, ws_need, None) == 1
    w_bad = api.moe_weights_t(*([8] * 12))
    w_bad.ws_down = None
    assert L.moe_forward(cp, 8, ctypes.byref(w_bad), 8, None, 8, ws_need, None) == 1
    # a gated shared expert needs its gate vector; the gate flag is 0 or 1
    gated = api.config_struct(PRESETS["qwen_gated_bf16"])
    w_bad = api.moe_weights_t(*([8] * 12))
    w_bad.ws_gate_vec = None
    n = api.moe_workspace_size(gated)
    assert L.moe_forward(ctypes.byref(gated), 8, ctypes.byref(w_bad), 8, None, 8, n, None) == 1
    assert L.moe_combine(ctypes.byref(gated), 8, None, 8, 8, 8, ctypes.byref(w_bad), 8, 8, n,
                         None) == 1
    assert api.moe_workspace_size(api.config_struct(PRESETS["qwen_gated_bf16"],
                                                    shared_gate=2)) == 0
    # workspace one byte short
    assert L.moe_forward(cp, 8, ctypes.byref(w_ok), 8, None, 8, ws_need - 1, None) == 3
    assert L.moe_permute(cp, 8, 8, 8, 8, 8, ws_need - 1, None) == 3
    assert L.moe_permute(cp, None, 8, 8, 8, 8, ws_need, None) == 1
    assert L.moe_expert_ffn(cp, 8, None, 8, 8, ctypes.byref(w_ok), 8, 8, ws_need - 1, None) == 3
    assert L.moe_combine(cp, 8, None, 8, None, 8, ctypes.byref(w_ok), 8, 8, ws_need, None) == 1
    assert L.moe_route(cp, 8, ctypes.byref(w_ok), None, None, 8, None, None, None, 0, None) == 1
    assert L.moe_pack_weights(cp, None, None, None) == 1


def test_zero_tokens_is_a_valid_noop():
    L = api.lib()
    cfg = api.config_struct(PRESETS["softmax_bf16"], num_tokens=0)
    n = api.moe_workspace_size(cfg)
    assert n > 0
    w = api.moe_weights_t(*([8] * 12))
    assert L.moe_forward(ctypes.byref(cfg), 8, ctypes.byref(w), 8, None, 8, n, None) == 0
    assert L.moe_route_from_logits(ctypes.byref(cfg), 8, None, 8, 8, None) == 0


def test_packed_sizes():
    c = PRESETS["softmax_bf16"]
    d, f, E = c.d_model, c.d_ff, c.num_experts
    assert api.moe_packed_size(c, api.PACK_GATE_UP) == E * 2 * f * d * 2
    assert api.moe_packed_size(c, api.PACK_DOWN) == E * f * d * 2
    assert api.moe_packed_size(c, api.PACK_GATE_UP_SCALES) == 0
    assert api.moe_packed_size(c, api.PACK_ROUTER) == 512 * d * 2
    q = PRESETS["fp8_block"]
    assert api.moe_packed_size(q, api.PACK_GATE_UP) == 896 * 2 * 512 * 4096
    assert api.moe_packed_size(q, api.PACK_ROUTER) == 1024 * 4096 * 4     # bf16 hi + lo planes, 256-padded
    assert api.moe_packed_size(q, api.PACK_DOWN_SCALES) == 896 * (4096 // 16) * (512 // 128) * 4
    t = PRESETS["tiny_fp32"]
    assert api.moe_packed_size(t, api.PACK_SHARED_DOWN) == 256 * 256 * 4
    assert api.moe_packed_size(t, 42) == 0
    assert FP8_E4M3 == 2 and F32 == 0


def test_hashed_route_and_bias_update_argument_checks():
    L = api.lib()
    cfg = api.config_struct(PRESETS["tiny_fp32"])
    cp = ctypes.byref(cfg)
    n = api.moe_workspace_size(cfg)
    w = api.moe_weights_t(*([8] * 12))
    wp = ctypes.byref(w)
    # moe_route_hashed: token ids, table and a positive vocab are required
    assert L.moe_route_hashed(cp, 8, wp, None, 8, 4, None, 8, 8, None, None, 8, n, None) == 1
    assert L.moe_route_hashed(cp, 8, wp, 8, None, 4, None, 8, 8, None, None, 8, n, None) == 1
    assert L.moe_route_hashed(cp, 8, wp, 8, 8, 0, None, 8, 8, None, None, 8, n, None) == 1
    assert L.moe_route_hashed(cp, 8, wp, 8, 8, 4, None, 8, 8, None, None, 8, n - 1, None) == 3
    c0 = api.config_struct(PRESETS["tiny_fp32"], num_tokens=0)
    assert L.moe_route_hashed(ctypes.byref(c0), 8, wp, 8, 8, 4, None, 8, 8, None, None, 8, n,
                              None) == 0
    # moe_update_bias: offsets and bias required; speed finite and >= 0
    assert L.moe_update_bias(cp, None, 0.001, 8, None) == 1
    assert L.moe_update_bias(cp, 8, 0.001, None, None) == 1
    assert L.moe_update_bias(cp, 8, float("nan"), 8, None) == 1
    assert L.moe_update_bias(cp, 8, -0.001, 8, None) == 1
    bad = api.config_struct(PRESETS["tiny_fp32"], top_k=0)
    assert L.moe_update_bias(ctypes.byref(bad), 8, 0.001, 8, None) == 1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: any other --gpus value exits with status 2 and a message,
    before anything touches a GPU."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_noalloc_forward_refuses_configs_beyond_its_scratch():
    # the allocation-free forward has a fixed workspace: a config that needs more is refused
    # on the host, before any HIP call
    L = api.lib()
    # placeholder pointers: the checks below return before anything is dereferenced
    w = api.moe_weights_t(*([1] * len(api.moe_weights_t._fields_)))
    big = api.config_struct(PRESETS["softmax_bf16"])
    assert L.moe_workspace_size(ctypes.byref(big)) > api.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(big), 1, ctypes.byref(w), 1, None, None) == \
        api.MOE_ERR_WORKSPACE_TOO_SMALL
    # the decode workload fits; argument errors still come first
    dec = api.config_struct(PRESETS["decode_bf16"])
    assert 0 < L.moe_workspace_size(ctypes.byref(dec)) <= api.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(dec), None, ctypes.byref(w), 1, None, None) == \
        api.MOE_ERR_INVALID_ARGUMENT
    bad = api.config_struct(PRESETS["decode_bf16"], top_k=0)
    assert L.moe_forward_noalloc(ctypes.byref(bad), 1, ctypes.byref(w), 1, None, None) == \
        api.MOE_ERR_INVALID_ARGUMENT


def test_c_example_program_runs_on_the_host(tmp_path):
    # the plain C++ driver of the ABI (no GPU call before these checks): usage without a
    # directory, and a refused config reported before any device memory is touched
    from mixture_experts_ffn_softplus_amd import build as hip_build
    if not os.path.exists(hip_build.EXAMPLE):
        pytest.skip("forward_c is not built")
    r = subprocess.run([hip_build.EXAMPLE], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    bad = api.config_struct(PRESETS["fp8_block"], quant_block=64)
    (tmp_path / "config.bin").write_bytes(bytes(bad))
    r = subprocess.run([hip_build.EXAMPLE, str(tmp_path)], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "not supported" in r.stderr
    (tmp_path / "config.bin").write_bytes(bytes(bad)[:-4])
    r = subprocess.run([hip_build.EXAMPLE, str(tmp_path)], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "moe_config_t is" in r.stderr
