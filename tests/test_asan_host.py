"""Host-side AddressSanitizer run of the library's argument checks (CPU only).

The library's sources are compiled for the host alone (no device code) with AddressSanitizer
instrumentation, and a small C driver, itself built with AddressSanitizer, calls every entry
point on its error paths -- bad configs, NULL pointers, short workspaces, oversized operands,
zero tokens -- plus the size queries on every named workload.  Nothing reaches a kernel launch;
the run must end with every status as expected and no sanitizer report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mixture_experts_ffn_softplus_amd import PRESETS
from mixture_experts_ffn_softplus_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = hip_build.HIPCC
CLANG = "/opt/rocm/llvm/bin/clang"

DRIVER = r'''
#include <stdio.h>
#include <string.h>
#include "moe.h"

static int fails = 0;
#define EXPECT(call, want) do { int got_ = (int)(call); if (got_ != (int)(want)) { \
  fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
  ++fails; } } while (0)

static moe_config_t preset(int i);

int main(void) {
  char buf[4096];
  void* P = buf;  /* a placeholder pointer: never dereferenced on these paths */
  moe_weights_t w, w0;
  memset(&w0, 0, sizeof w0);
  void** wp = (void**)&w;
  for (size_t i = 0; i < sizeof w / sizeof(void*); ++i) wp[i] = P;
  moe_logical_weights_t lw;
  void** lp = (void**)&lw;
  for (size_t i = 0; i < sizeof lw / sizeof(void*); ++i) lp[i] = P;
  void* packed[MOE_PACK_COUNT];
  for (int i = 0; i < MOE_PACK_COUNT; ++i) packed[i] = P;

  for (int s = -1; s <= 5; ++s) EXPECT(moe_status_string((moe_status_t)s) != NULL, 1);
  EXPECT(moe_workspace_size(NULL), 0);
  EXPECT(moe_packed_size(NULL, 0), 0);

  for (int p = 0; p < NUM_PRESETS; ++p) {
    moe_config_t c = preset(p);
    size_t ws = moe_workspace_size(&c);
    EXPECT(ws > 0, 1);
    for (int i = -1; i <= MOE_PACK_COUNT; ++i) (void)moe_packed_size(&c, i);
    /* NULL required pointers */
    EXPECT(moe_forward(&c, NULL, &w, P, NULL, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_forward(&c, P, NULL, P, NULL, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_forward(&c, P, &w0, P, NULL, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_forward(&c, P, &w, P, NULL, NULL, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_forward(&c, P, &w, P, NULL, P, ws - 1, 0), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_route(&c, P, &w, NULL, NULL, P, NULL, NULL, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_route(&c, P, &w, NULL, P, P, NULL, NULL, P, 0, 0), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_route_hashed(&c, P, &w, NULL, P, 1, NULL, P, P, NULL, NULL, P, ws, 0),
           MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_route_hashed(&c, P, &w, P, P, 0, NULL, P, P, NULL, NULL, P, ws, 0),
           MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_route_from_logits(&c, NULL, NULL, P, P, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_update_bias(&c, P, -1.0f, P, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_update_bias(&c, NULL, 0.001f, P, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_permute(&c, P, P, NULL, P, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_permute(&c, P, P, P, P, P, 16, 0), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_expert_ffn(&c, P, P, NULL, P, &w, P, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_expert_ffn(&c, P, P, P, P, &w0, P, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_combine(&c, P, P, P, NULL, P, &w, P, P, ws, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_combine(&c, P, P, P, P, P, &w, P, P, 1, 0), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_pack_weights(&c, NULL, packed, 0), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_forward_noalloc(&c, NULL, &w, P, NULL, 0), MOE_ERR_INVALID_ARGUMENT);
    if (ws > MOE_NOALLOC_SCRATCH_BYTES)
      EXPECT(moe_forward_noalloc(&c, P, &w, P, NULL, 0), MOE_ERR_WORKSPACE_TOO_SMALL);
    /* zero tokens: valid, launches nothing */
    moe_config_t z = c;
    z.num_tokens = 0;
    size_t wz = moe_workspace_size(&z);
    EXPECT(moe_forward(&z, P, &w, P, NULL, P, wz, 0), MOE_OK);
    EXPECT(moe_route(&z, P, &w, NULL, P, P, NULL, NULL, P, wz, 0), MOE_OK);
    EXPECT(moe_permute(&z, P, P, P, P, P, wz, 0), MOE_OK);
    EXPECT(moe_expert_ffn(&z, P, P, P, P, &w, P, P, wz, 0), MOE_OK);
    EXPECT(moe_combine(&z, P, P, P, P, P, &w, P, P, wz, 0), MOE_OK);
    EXPECT(moe_route_from_logits(&z, P, NULL, P, P, 0), MOE_OK);
    EXPECT(moe_forward_noalloc(&z, P, &w, P, NULL, 0), MOE_OK);
    /* bad and unsupported configs: every field pushed out of range */
    int32_t* f = (int32_t*)&c;
    for (size_t i = 0; i < sizeof c / sizeof(int32_t); ++i) {
      const int32_t vals[] = {-1, 0, 3, 7, 1 << 30, -2147483647 - 1, 2147483647};
      for (size_t v = 0; v < sizeof vals / sizeof vals[0]; ++v) {
        moe_config_t b = c;
        ((int32_t*)&b)[i] = vals[v];
        size_t n = moe_workspace_size(&b);
        if (n == 0) {
          int st = moe_forward(&b, P, &w, P, NULL, P, (size_t)1 << 40, 0);
          if (st != MOE_ERR_INVALID_ARGUMENT && st != MOE_ERR_UNSUPPORTED) {
            fprintf(stderr, "field %zu = %d: status %d\n", i, vals[v], st);
            ++fails;
          }
        }
        (void)moe_packed_size(&b, MOE_PACK_GATE_UP);
      }
      (void)f;
    }
  }
  if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
  printf("asan driver: all checks passed\n");
  return 0;
}
'''


def _preset_table():
    rows = []
    for cfg in PRESETS.values():
        rows.append("{%d, %d, %d, %d, %d, %d, %d, %d, %d, %.9ef, %d, %d, %d, %d, %d, %d}" % (
            cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k, cfg.d_ff, cfg.num_shared,
            cfg.d_ff_shared, cfg.score, cfg.renormalize, cfg.routed_scale, cfg.act_dtype,
            cfg.expert_dtype, cfg.router_dtype, cfg.quant_block, cfg.shared_gate, cfg.out_f32))
    return ("#define NUM_PRESETS %d\nstatic const moe_config_t kPresets[] = {\n  %s};\n"
            "static moe_config_t preset(int i) { return kPresets[i]; }\n"
            % (len(rows), ",\n  ".join(rows)))


def _asan_library():
    """The library built with AddressSanitizer on its host half (device code as usual, so the
    code object is complete), cached under the package's _build/ by a hash of the sources and
    flags."""
    import hashlib
    csrc = os.path.join(ROOT, "mixture_experts_ffn_softplus_amd", "csrc")
    flags = [f"--offload-arch={hip_build.ARCH}", "-O1", "-std=c++17", "-fPIC",
             "-fvisibility=hidden", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    h = hashlib.sha256(" ".join(flags).encode())
    for src in sorted(os.listdir(csrc)) + ["../../include/moe.h"]:
        with open(os.path.join(csrc, src), "rb") as fh:
            h.update(src.encode() + fh.read())
    out = os.path.join(hip_build.BUILD, "asan", h.hexdigest()[:16])
    lib = os.path.join(out, "libmoe_asan.so")
    if os.path.exists(lib):
        return lib
    os.makedirs(out, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([HIPCC, *flags, "-c", os.path.join(csrc, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 2)) as ex:
        objs = list(ex.map(compile_one, hip_build.SOURCES))
    r = subprocess.run([HIPCC, f"--offload-arch={hip_build.ARCH}", "-shared", "-fPIC", *objs,
                        "-o", lib + ".tmp"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    os.replace(lib + ".tmp", lib)
    return lib


@pytest.mark.skipif(not (shutil.which(HIPCC) or os.path.exists(HIPCC)) or
                    not os.path.exists(CLANG), reason="needs hipcc and ROCm's clang")
def test_argument_checks_under_address_sanitizer(tmp_path):
    lib = _asan_library()
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER.replace("static moe_config_t preset(int i);", _preset_table()))
    exe = str(tmp_path / "driver")
    r = subprocess.run([CLANG, "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1",
                        "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
                        "-I/opt/rocm/include", str(drv), lib, "-L/opt/rocm/lib", "-lamdhip64",
                        f"-Wl,-rpath,{os.path.dirname(lib)}", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "all checks passed" in r.stdout
