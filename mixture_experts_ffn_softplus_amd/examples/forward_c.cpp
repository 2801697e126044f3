// forward_c -- the whole block through the C ABI alone: no Python, no PyTorch.
//
// Usage: forward_c DIR
//   DIR/config.bin     the moe_config_t struct, raw bytes
//   DIR/x.bin          x [T, d] in act_dtype
//   DIR/<name>.bin     each logical weight of moe_logical_weights_t that the config uses
//                      (w_router, w_gate, w_up, w_down, their *_scales, ws_gate, ws_up, ws_down,
//                      ws_*_scales), raw bytes in the layout include/moe.h documents
//   DIR/logit_bias.bin, DIR/select_bias.bin, DIR/gate_vec.bin   optional
// writes DIR/out.bin (the block output [T, d]) and exits 0, or prints the failing call and
// exits 1.  Every buffer is allocated here with hipMalloc, the weights are packed once with
// moe_pack_weights, and one moe_forward runs on the default stream.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "moe.h"

namespace {

std::vector<char> read_file(const std::string& path, bool required) {
  std::vector<char> data;
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) {
    if (required) {
      std::fprintf(stderr, "forward_c: cannot open %s\n", path.c_str());
      std::exit(1);
    }
    return data;
  }
  std::fseek(f, 0, SEEK_END);
  const long n = std::ftell(f);
  std::fseek(f, 0, SEEK_SET);
  data.resize(static_cast<size_t>(n));
  if (n > 0 && std::fread(data.data(), 1, data.size(), f) != data.size()) {
    std::fprintf(stderr, "forward_c: short read of %s\n", path.c_str());
    std::exit(1);
  }
  std::fclose(f);
  return data;
}

void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "forward_c: %s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

void check_moe(moe_status_t s, const char* what) {
  if (s != MOE_OK) {
    std::fprintf(stderr, "forward_c: %s: %s\n", what, moe_status_string(s));
    std::exit(1);
  }
}

// Device copy of DIR/name.bin, or nullptr when the file is absent and optional.
std::vector<void*> g_allocs;
void* upload(const std::string& dir, const char* name, bool required = false) {
  const std::vector<char> host = read_file(dir + "/" + name + ".bin", required);
  if (host.empty()) return nullptr;
  void* dev = nullptr;
  check_hip(hipMalloc(&dev, host.size()), name);
  g_allocs.push_back(dev);
  check_hip(hipMemcpy(dev, host.data(), host.size(), hipMemcpyHostToDevice), name);
  return dev;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: forward_c DIR\n");
    return 1;
  }
  const std::string dir = argv[1];
  const std::vector<char> cfg_bytes = read_file(dir + "/config.bin", true);
  if (cfg_bytes.size() != sizeof(moe_config_t)) {
    std::fprintf(stderr, "forward_c: config.bin holds %zu bytes, moe_config_t is %zu\n",
                 cfg_bytes.size(), sizeof(moe_config_t));
    return 1;
  }
  moe_config_t cfg;
  std::memcpy(&cfg, cfg_bytes.data(), sizeof cfg);

  const size_t ws_bytes = moe_workspace_size(&cfg);
  if (ws_bytes == 0) {
    std::fprintf(stderr, "forward_c: the config is not supported\n");
    return 1;
  }

  moe_logical_weights_t lw = {};
  lw.w_router = upload(dir, "w_router", true);
  lw.w_gate = upload(dir, "w_gate", true);
  lw.w_up = upload(dir, "w_up", true);
  lw.w_down = upload(dir, "w_down", true);
  lw.w_gate_scales = upload(dir, "w_gate_scales");
  lw.w_up_scales = upload(dir, "w_up_scales");
  lw.w_down_scales = upload(dir, "w_down_scales");
  lw.ws_gate = upload(dir, "ws_gate");
  lw.ws_up = upload(dir, "ws_up");
  lw.ws_down = upload(dir, "ws_down");
  lw.ws_gate_scales = upload(dir, "ws_gate_scales");
  lw.ws_up_scales = upload(dir, "ws_up_scales");
  lw.ws_down_scales = upload(dir, "ws_down_scales");

  void* packed[MOE_PACK_COUNT] = {};
  for (int i = 0; i < MOE_PACK_COUNT; ++i) {
    const size_t n = moe_packed_size(&cfg, i);
    if (n == 0) continue;
    check_hip(hipMalloc(&packed[i], n), "hipMalloc(packed)");
    g_allocs.push_back(packed[i]);
  }
  check_moe(moe_pack_weights(&cfg, &lw, packed, nullptr), "moe_pack_weights");

  moe_weights_t w = {};
  w.w_router = packed[MOE_PACK_ROUTER];
  w.logit_bias = static_cast<const float*>(upload(dir, "logit_bias"));
  w.select_bias = static_cast<const float*>(upload(dir, "select_bias"));
  w.w_gate_up = packed[MOE_PACK_GATE_UP];
  w.w_gate_up_scales = packed[MOE_PACK_GATE_UP_SCALES];
  w.w_down = packed[MOE_PACK_DOWN];
  w.w_down_scales = packed[MOE_PACK_DOWN_SCALES];
  w.ws_gate_up = packed[MOE_PACK_SHARED_GATE_UP];
  w.ws_gate_up_scales = packed[MOE_PACK_SHARED_GATE_UP_SCALES];
  w.ws_down = packed[MOE_PACK_SHARED_DOWN];
  w.ws_down_scales = packed[MOE_PACK_SHARED_DOWN_SCALES];
  w.ws_gate_vec = upload(dir, "gate_vec");

  const void* x = upload(dir, "x", cfg.num_tokens > 0);
  const size_t out_elem = cfg.out_f32 || cfg.act_dtype == MOE_F32 ? 4 : 2;
  const size_t out_bytes = static_cast<size_t>(cfg.num_tokens) * cfg.d_model * out_elem;
  void* out = nullptr;
  void* ws = nullptr;
  check_hip(hipMalloc(&out, out_bytes > 0 ? out_bytes : 1), "hipMalloc(out)");
  check_hip(hipMalloc(&ws, ws_bytes), "hipMalloc(workspace)");
  g_allocs.push_back(out);
  g_allocs.push_back(ws);

  check_moe(moe_forward(&cfg, x, &w, out, nullptr, ws, ws_bytes, nullptr), "moe_forward");
  check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");
  check_hip(hipGetLastError(), "kernels");

  std::vector<char> host(out_bytes);
  if (out_bytes > 0) check_hip(hipMemcpy(host.data(), out, out_bytes, hipMemcpyDeviceToHost), "copy out");
  FILE* f = std::fopen((dir + "/out.bin").c_str(), "wb");
  if (!f || std::fwrite(host.data(), 1, host.size(), f) != host.size()) {
    std::fprintf(stderr, "forward_c: cannot write out.bin\n");
    return 1;
  }
  std::fclose(f);
  for (void* p : g_allocs) check_hip(hipFree(p), "hipFree");
  std::printf("forward_c: ok, %zu output bytes\n", out_bytes);
  return 0;
}
