"""The block driven from a plain C++ program through the C ABI alone.

`forward_c` (built next to the library from `mixture_experts_ffn_softplus_amd/examples/`) is host
code linked only against the library and the HIP runtime: it reads the config struct and the
logical weights as raw bytes, allocates with hipMalloc, packs with moe_pack_weights and runs one
moe_forward on the default stream.  No Python or PyTorch is in that process.  Its output must
equal, bit for bit, the output of the same forward called through the Python binding on the same
inputs (the parity of that path against the oracle is what the other GPU tests check).
"""
import os
import subprocess

import numpy as np
import pytest
import torch

from mixture_experts_ffn_softplus_amd import PRESETS, api, synth
from mixture_experts_ffn_softplus_amd import build as hip_build

pytestmark = pytest.mark.gpu

BF = PRESETS["softmax_bf16"]
CASES = {
    "bf16_softmax_ragged": BF.with_(name="c_bf16_softmax_ragged", num_tokens=300, d_model=256,
                                    num_experts=24, top_k=4, d_ff=128, num_shared=1,
                                    d_ff_shared=256, seed=61),
    "bf16_sqrt_softplus_biases": PRESETS["softplus_bf16"].with_(
        name="c_bf16_sqrt_softplus", num_tokens=200, d_model=384, num_experts=20, top_k=3,
        d_ff=256, num_shared=2, d_ff_shared=128, seed=62),
    "fp8_f32_router_gated": PRESETS["fp8_block"].with_(
        name="c_fp8_gated", num_tokens=150, d_model=256, num_experts=10, top_k=3, d_ff=512,
        num_shared=1, d_ff_shared=512, shared_gate=1, seed=63),
    "mxfp4_decode": PRESETS["mxfp4_decode"].with_(name="c_mxfp4_decode", num_tokens=24,
                                                  d_model=512, num_experts=32, top_k=4,
                                                  d_ff=512, num_shared=1, d_ff_shared=512,
                                                  seed=64),
}


def _dump(t, path):
    if t is not None:
        t.detach().contiguous().view(-1).view(torch.uint8).cpu().numpy().tofile(path)


@pytest.mark.parametrize("name", list(CASES))
def test_c_program_matches_the_python_binding(name, tmp_path):
    assert os.path.exists(hip_build.EXAMPLE), "forward_c is built with the library"
    cfg = CASES[name]
    print(f"[c-abi] {name}", flush=True)
    inp = synth.inputs(cfg, "cuda")
    pw = api.pack(cfg, inp["w_router"], inp["routed"], inp["shared"], inp["logit_bias"],
                  inp["select_bias"], shared_gate=inp["shared_gate"])
    ws = api.workspace(cfg)
    out = torch.empty(cfg.num_tokens, cfg.d_model, dtype=api.out_dtype(cfg), device="cuda")
    api.moe_forward(cfg, inp["x"], pw.struct(), out, ws)
    torch.cuda.synchronize()

    (tmp_path / "config.bin").write_bytes(bytes(api.config_struct(cfg)))
    _dump(inp["x"], tmp_path / "x.bin")
    _dump(inp["w_router"], tmp_path / "w_router.bin")
    for key in ("gate", "up", "down", "gate_scales", "up_scales", "down_scales"):
        _dump(inp["routed"].get(key), tmp_path / f"w_{key}.bin")
        if inp["shared"]:
            _dump(inp["shared"].get(key), tmp_path / f"ws_{key}.bin")
    _dump(inp["logit_bias"], tmp_path / "logit_bias.bin")
    _dump(inp["select_bias"], tmp_path / "select_bias.bin")
    if cfg.shared_gate:
        _dump(inp["shared_gate"], tmp_path / "gate_vec.bin")

    r = subprocess.run([hip_build.EXAMPLE, str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr + r.stdout
    got = np.fromfile(tmp_path / "out.bin", dtype=np.uint8)
    want = out.contiguous().view(-1).view(torch.uint8).cpu().numpy()
    assert got.shape == want.shape
    assert np.array_equal(got, want)
