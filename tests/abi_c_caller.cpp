// A plain C++ caller of the TSP library: one rank's layer forward driven
// through include/tsp.h alone (device memory from hipMalloc, no Python), for
// tests/test_gpu_c_caller.py, which loads it as a shared library, calls
//
//   int tsp_c_caller_run(const char* dir)
//
// and compares its output with the Python binding's.
//
// DIR/dims.txt   ten integers: batch seq degree rank hidden q_heads kv_heads
//                head_dim ffn partition
// DIR/x.bin      bf16 bits [B][S][h], the whole sequence in position order
// DIR/w_qkv.bin, w_o.bin, w_gate.bin, w_up.bin, w_down.bin
//                bf16 bits in the ABI layouts
// writes DIR/y.bin: float32 [B][S/D][h], the rank's layer output.
// The other ranks' K/V all-gather slots are filled with tsp_qkv_proj from
// their rows (the stand-in for the all-gather), then tsp_layer_fwd runs.
// Returns 0 on success; otherwise 1, with the failing call and
// tsp_last_error() on stderr.
#include <cstdint>
#include <cstdio>
#include <stdexcept>
#include <string>
#include <vector>

#include "tsp.h"

namespace {

[[noreturn]] void die(const std::string& what) { throw std::runtime_error(what); }

void check_tsp(int rc, const char* call) {
  if (rc != TSP_OK) die(std::string(call) + " returned " + std::to_string(rc) + ": " + tsp_last_error());
}

void check_hip(hipError_t e, const char* call) {
  if (e != hipSuccess) die(std::string(call) + ": " + hipGetErrorString(e));
}

std::vector<uint16_t> read_u16(const std::string& path, size_t count) {
  std::vector<uint16_t> v(count);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (f == nullptr) die("cannot open " + path);
  const size_t got = std::fread(v.data(), 2, count, f);
  std::fclose(f);
  if (got != count) die(path + ": expected " + std::to_string(count) + " 16-bit values");
  return v;
}

template <typename T>
T* device_copy(const std::vector<T>& host) {
  T* d = nullptr;
  check_hip(hipMalloc(&d, host.size() * sizeof(T)), "hipMalloc");
  check_hip(hipMemcpy(d, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy to device");
  return d;
}

void* device_alloc(size_t bytes) {
  void* d = nullptr;
  check_hip(hipMalloc(&d, bytes > 0 ? bytes : 1), "hipMalloc");
  return d;
}

int run(const std::string& dir) {
  tsp_dims_t d{};
  {
    FILE* f = std::fopen((dir + "/dims.txt").c_str(), "r");
    if (f == nullptr) die("cannot open dims.txt");
    int v[10];
    for (int i = 0; i < 10; ++i)
      if (std::fscanf(f, "%d", &v[i]) != 1) die("dims.txt: expected ten integers");
    std::fclose(f);
    d.batch = v[0], d.seq = v[1], d.degree = v[2], d.rank = v[3], d.hidden = v[4];
    d.n_q_heads = v[5], d.n_kv_heads = v[6], d.head_dim = v[7], d.ffn = v[8], d.partition = v[9];
  }
  const size_t B = d.batch, S = d.seq, D = d.degree, T = S / D, h = d.hidden;
  const size_t nqkv = (size_t)(d.n_q_heads + 2 * d.n_kv_heads) / D * d.head_dim;
  const size_t qs = (size_t)d.n_q_heads / D * d.head_dim, fs = (size_t)d.ffn / D;

  const std::vector<uint16_t> x = read_u16(dir + "/x.bin", B * S * h);
  uint16_t* w_qkv = device_copy(read_u16(dir + "/w_qkv.bin", D * nqkv * h));
  uint16_t* w_o = device_copy(read_u16(dir + "/w_o.bin", D * h * qs));
  uint16_t* w_gate = device_copy(read_u16(dir + "/w_gate.bin", D * fs * h));
  uint16_t* w_up = device_copy(read_u16(dir + "/w_up.bin", D * fs * h));
  uint16_t* w_down = device_copy(read_u16(dir + "/w_down.bin", D * h * fs));

  // the K/V all-gather buffer, zeroed, then every other rank's slot
  const size_t kv_bytes = tsp_workspace_bytes(&d, TSP_FN_KV_GATHERED);
  if (kv_bytes == 0) die(std::string("tsp_workspace_bytes: ") + tsp_last_error());
  uint16_t* kv = static_cast<uint16_t*>(device_alloc(kv_bytes));
  check_hip(hipMemset(kv, 0, kv_bytes), "hipMemset");
  int32_t* l2g_dev = static_cast<int32_t*>(device_alloc(T * sizeof(int32_t)));
  std::vector<int32_t> l2g(T);
  std::vector<uint16_t> rows(B * T * h);
  uint16_t* x_local = static_cast<uint16_t*>(device_alloc(rows.size() * 2));
  // the other ranks first, the rank's own rows last (they stay in x_local)
  for (int i = 0; i < (int)D; ++i) {
    const int r = i == (int)D - 1 ? d.rank : (i < d.rank ? i : i + 1);
    tsp_dims_t dr = d;
    dr.rank = r;
    check_tsp(tsp_zigzag_index(&dr, l2g_dev, nullptr, nullptr), "tsp_zigzag_index");
    check_hip(hipMemcpy(l2g.data(), l2g_dev, T * sizeof(int32_t), hipMemcpyDeviceToHost), "hipMemcpy l2g");
    for (size_t b = 0; b < B; ++b)
      for (size_t t = 0; t < T; ++t) {
        const size_t p = (size_t)l2g[t];
        if (p >= S) die("local_to_global out of range");
        for (size_t c = 0; c < h; ++c) rows[(b * T + t) * h + c] = x[(b * S + p) * h + c];
      }
    check_hip(hipMemcpy(x_local, rows.data(), rows.size() * 2, hipMemcpyHostToDevice), "hipMemcpy rows");
    if (r != d.rank) {
      check_tsp(tsp_qkv_proj(&dr, r, x_local, w_qkv, nullptr, kv, nullptr), "tsp_qkv_proj");
      check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");  // before x_local is refilled
    }
  }
  const size_t ws_bytes = tsp_workspace_bytes(&d, TSP_FN_LAYER);
  if (ws_bytes == 0) die(std::string("tsp_workspace_bytes: ") + tsp_last_error());
  void* ws = device_alloc(ws_bytes);
  float* y = static_cast<float*>(device_alloc(B * T * h * sizeof(float)));
  check_tsp(tsp_layer_fwd(&d, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv, y, ws, ws_bytes, nullptr),
            "tsp_layer_fwd");
  check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");
  std::vector<float> y_host(B * T * h);
  check_hip(hipMemcpy(y_host.data(), y, y_host.size() * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy y");
  FILE* f = std::fopen((dir + "/y.bin").c_str(), "wb");
  if (f == nullptr || std::fwrite(y_host.data(), sizeof(float), y_host.size(), f) != y_host.size())
    die("cannot write y.bin");
  std::fclose(f);
  for (void* p : {(void*)w_qkv, (void*)w_o, (void*)w_gate, (void*)w_up, (void*)w_down, (void*)kv, (void*)l2g_dev,
                  (void*)x_local, ws, (void*)y})
    check_hip(hipFree(p), "hipFree");
  std::printf("abi_c_caller: rank %d of %d, %zu rows written\n", d.rank, d.degree, B * T);
  return 0;
}

}  // namespace

extern "C" int tsp_c_caller_run(const char* dir) {
  try {
    return run(dir);
  } catch (const std::exception& e) {
    std::fprintf(stderr, "abi_c_caller: %s\n", e.what());
    return 1;
  }
}
