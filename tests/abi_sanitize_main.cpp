// Drives every entry point of the C ABI through its argument checks and its
// workspace arithmetic, for a grid of shapes, under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; the kernel launchers are
// stand-ins and no GPU is present).  Exits non-zero on the first unexpected
// return code; the sanitizers abort on a memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "tsp.h"

static int failures = 0;

#define EXPECT(call, want)                                                                              \
  do {                                                                                                  \
    const int _rc = (call);                                                                             \
    if (_rc != (want)) {                                                                                \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, _rc, (int)(want), \
                   tsp_last_error());                                                                   \
      ++failures;                                                                                       \
    }                                                                                                   \
  } while (0)

int main() {
  // aligned and misaligned stand-in pointers: never dereferenced (the checks
  // fail before any use, or no device is present)
  void* P = reinterpret_cast<void*>(uintptr_t(0x10000));
  void* Q = reinterpret_cast<void*>(uintptr_t(0x10008));
  auto u16 = [](void* p) { return static_cast<uint16_t*>(p); };
  auto f32 = [](void* p) { return static_cast<float*>(p); };
  auto i32 = [](void* p) { return static_cast<int32_t*>(p); };
  const size_t BIG = size_t(1) << 40;

  // a grid of shapes, valid and not: every selector of tsp_workspace_bytes
  const int32_t Bs[] = {0, 1, 2}, Ss[] = {2, 16, 96, 250, 256, 8192, 131072}, Ds[] = {0, 1, 2, 3, 8};
  const int32_t hs[] = {64, 200, 4096}, Fs[] = {64, 768, 11008, 28672}, dhs[] = {64, 96, 128};
  long long valid = 0;
  for (int32_t b : Bs)
    for (int32_t S : Ss)
      for (int32_t D : Ds)
        for (int32_t h : hs)
          for (int32_t F : Fs)
            for (int32_t dh : dhs)
              for (int32_t part = -1; part <= 2; ++part) {
                tsp_dims_t d{b, S, D, D > 1 ? D - 1 : 0, h, 4 * (D > 0 ? D : 1), 2 * (D > 0 ? D : 1), dh, F, part};
                size_t ws[15];
                for (int fn = 0; fn <= 14; ++fn) ws[fn] = tsp_workspace_bytes(&d, fn);
                if (ws[3] > 0) {
                  ++valid;
                  if (ws[0] != 0 || ws[1] == 0 || ws[2] == 0 || ws[6] == 0 || ws[3] < ws[1] || ws[7] == 0 ||
                      ws[8] == 0 || ws[9] == 0 || ws[10] == 0 || ws[11] == 0 || ws[11] > ws[7] || ws[12] == 0 ||
                      ws[13] == 0 || ws[13] > ws[6] || ws[14] == 0) {
                    std::fprintf(stderr, "inconsistent workspace sizes\n");
                    ++failures;
                  }
                  // valid shape, stand-in pointers: stops at the missing device
                  EXPECT(tsp_layer_fwd(&d, u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), f32(P), P, ws[3],
                                       nullptr),
                         TSP_ERR_HIP);
                  EXPECT(tsp_mlp_ring_bwd(&d, P, TSP_F32, f32(P), u16(P), u16(P), u16(P), nullptr, f32(P), f32(P),
                                          f32(P), f32(P), P, ws[6], nullptr),
                         TSP_ERR_HIP);
                  EXPECT(tsp_mlp_ring_fwd_keep(&d, P, TSP_F32, u16(P), u16(P), u16(P), nullptr, f32(P), f32(P), P,
                                               ws[2], nullptr),
                         TSP_ERR_HIP);
                  EXPECT(tsp_mlp_ring_bwd_kept(&d, P, TSP_F32, f32(P), u16(P), u16(P), u16(P), f32(P), nullptr,
                                               f32(P), f32(P), f32(P), f32(P), P, ws[13], nullptr),
                         TSP_ERR_HIP);
                  EXPECT(tsp_attn_fwd_keep(&d, u16(P), u16(P), u16(P), u16(P), nullptr, f32(P), u16(P), u16(P),
                                           f32(P), P, ws[10], nullptr),
                         TSP_ERR_HIP);
                  EXPECT(tsp_attn_bwd_kept(&d, u16(P), u16(P), u16(P), u16(P), f32(P), f32(P), f32(P), f32(P),
                                           f32(P), P, ws[11], nullptr),
                         TSP_ERR_HIP);
                  EXPECT(tsp_kv_reorder(&d, u16(P), u16(P), S, nullptr), TSP_ERR_HIP);
                  EXPECT(tsp_attn_bwd(&d, u16(P), u16(P), u16(P), u16(P), f32(P), f32(P), f32(P), f32(P), P, ws[7],
                                      nullptr),
                         TSP_ERR_HIP);
                  EXPECT(tsp_attn_bwd_proj(&d, u16(P), u16(P), f32(P), f32(P), nullptr, f32(P), f32(P), P, ws[8],
                                           nullptr),
                         TSP_ERR_HIP);
                }
              }
  if (valid < 100) {
    std::fprintf(stderr, "too few valid shapes (%lld)\n", valid);
    ++failures;
  }

  tsp_dims_t d{1, 256, 2, 0, 256, 4, 4, 64, 768, 0};
  const size_t wl = tsp_workspace_bytes(&d, TSP_FN_LAYER), wa = tsp_workspace_bytes(&d, TSP_FN_ATTN),
               wm = tsp_workspace_bytes(&d, TSP_FN_MLP), wb = tsp_workspace_bytes(&d, TSP_FN_MLP_BWD);
  // every entry point: NULL and misaligned pointers, bad codes, small workspace
  EXPECT(tsp_zigzag_index(nullptr, i32(P), nullptr, nullptr), TSP_ERR_NULL_POINTER);
  EXPECT(tsp_zigzag_index(&d, nullptr, nullptr, nullptr), TSP_ERR_NULL_POINTER);
  EXPECT(tsp_qkv_proj(&d, 2, u16(P), u16(P), nullptr, u16(P), nullptr), TSP_ERR_RANK);
  EXPECT(tsp_qkv_proj(&d, 0, u16(Q), u16(P), nullptr, u16(P), nullptr), TSP_ERR_MISALIGNED);
  EXPECT(tsp_kv_reorder(&d, u16(P), u16(P), -1, nullptr), TSP_ERR_KMAX);
  EXPECT(tsp_kv_reorder(&d, u16(P), u16(P), 257, nullptr), TSP_ERR_KMAX);
  EXPECT(tsp_attn_fwd(&d, u16(P), u16(P), u16(P), u16(P), f32(Q), f32(P), P, BIG, nullptr), TSP_ERR_MISALIGNED);
  EXPECT(tsp_attn_fwd(&d, u16(P), u16(P), u16(P), u16(P), nullptr, f32(P), P, wa - 1, nullptr), TSP_ERR_WORKSPACE);
  EXPECT(tsp_mlp_ring_fwd(&d, P, 5, u16(P), u16(P), u16(P), nullptr, f32(P), P, BIG, nullptr), TSP_ERR_DTYPE);
  EXPECT(tsp_mlp_ring_fwd(&d, P, TSP_BF16, u16(P), u16(P), u16(P), nullptr, f32(P), P, wm - 1, nullptr),
         TSP_ERR_WORKSPACE);
  EXPECT(tsp_layer_fwd(&d, u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), f32(P), P, wl - 1, nullptr),
         TSP_ERR_WORKSPACE);
  EXPECT(tsp_layer_fwd(&d, u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), nullptr, f32(P), P, wl, nullptr),
         TSP_ERR_NULL_POINTER);
  EXPECT(tsp_mlp_ring_bwd(&d, P, TSP_BF16, f32(P), u16(P), u16(P), u16(P), nullptr, f32(P), f32(P), f32(P), nullptr,
                          P, wb, nullptr),
         TSP_ERR_NULL_POINTER);
  EXPECT(tsp_mlp_ring_bwd(&d, P, TSP_BF16, f32(P), u16(P), u16(P), u16(P), nullptr, f32(P), f32(P), f32(P), f32(P),
                          P, wb - 1, nullptr),
         TSP_ERR_WORKSPACE);
  const size_t w13 = tsp_workspace_bytes(&d, TSP_FN_MLP_BWD_KEPT);
  EXPECT(tsp_mlp_ring_fwd_keep(&d, P, TSP_BF16, u16(P), u16(P), u16(P), nullptr, f32(P), nullptr, P, wm, nullptr),
         TSP_ERR_NULL_POINTER);
  EXPECT(tsp_mlp_ring_fwd_keep(&d, P, TSP_BF16, u16(P), u16(P), u16(P), nullptr, f32(P), f32(Q), P, wm, nullptr),
         TSP_ERR_MISALIGNED);
  EXPECT(tsp_mlp_ring_bwd_kept(&d, P, TSP_BF16, f32(P), u16(P), u16(P), u16(P), nullptr, nullptr, f32(P), f32(P),
                               f32(P), f32(P), P, w13, nullptr),
         TSP_ERR_NULL_POINTER);
  EXPECT(tsp_mlp_ring_bwd_kept(&d, P, TSP_BF16, f32(P), u16(P), u16(P), u16(P), f32(P), nullptr, f32(P), f32(P),
                               f32(P), f32(P), P, w13 - 1, nullptr),
         TSP_ERR_WORKSPACE);
  EXPECT(tsp_layer_fwd_noalloc(&d, u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), nullptr, nullptr),
         TSP_ERR_NULL_POINTER);
  const size_t w7 = tsp_workspace_bytes(&d, TSP_FN_ATTN_BWD), w8 = tsp_workspace_bytes(&d, TSP_FN_ATTN_BWD_PROJ);
  EXPECT(tsp_attn_bwd(&d, u16(P), u16(P), u16(P), u16(P), f32(P), f32(P), nullptr, f32(P), P, w7, nullptr),
         TSP_ERR_NULL_POINTER);
  EXPECT(tsp_attn_bwd(&d, u16(P), u16(P), u16(P), u16(P), f32(Q), f32(P), f32(P), f32(P), P, w7, nullptr),
         TSP_ERR_MISALIGNED);
  EXPECT(tsp_attn_bwd(&d, u16(P), u16(P), u16(P), u16(P), f32(P), f32(P), f32(P), f32(P), P, w7 - 1, nullptr),
         TSP_ERR_WORKSPACE);
  EXPECT(tsp_attn_bwd_proj(&d, u16(P), u16(P), f32(P), f32(P), f32(Q), f32(P), f32(P), P, w8, nullptr),
         TSP_ERR_MISALIGNED);
  EXPECT(tsp_attn_bwd_proj(&d, u16(P), u16(P), f32(P), f32(P), nullptr, f32(P), f32(P), P, w8 - 1, nullptr),
         TSP_ERR_WORKSPACE);
  tsp_dims_t big{2, 16384, 8, 3, 4096, 32, 8, 128, 14336, 0};
  EXPECT(tsp_layer_fwd_noalloc(&big, u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), f32(P), nullptr),
         TSP_ERR_SCRATCH);
  EXPECT(tsp_set_tuning(TSP_TUNE_COUNT, 1), TSP_ERR_INVALID_ARG);
  EXPECT(tsp_set_tuning(TSP_TUNE_ATTN_PAIR, 0), TSP_OK);
  EXPECT(tsp_set_tuning(TSP_TUNE_ATTN_PAIR, -5), TSP_OK);
  EXPECT(tsp_profile_kernel(TSP_K_COUNT, 1), TSP_ERR_INVALID_ARG);
  EXPECT(tsp_profile_kernel(TSP_K_QKV, 0), TSP_ERR_INVALID_ARG);
  EXPECT(tsp_profile_kernel(TSP_K_NONE, 0), TSP_OK);
  EXPECT(tsp_profile_result(nullptr, nullptr), TSP_ERR_NULL_POINTER);
  // a very long error message is cut, not overrun
  tsp_dims_t odd{1, 256, 2, 0, 256, 4, 4, 64, 768, 123456789};
  EXPECT(tsp_layer_fwd(&odd, u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), u16(P), f32(P), P, wl, nullptr),
         TSP_ERR_PARTITION);
  if (std::strlen(tsp_last_error()) == 0) ++failures;

  std::printf("abi sanitize: %lld valid shapes, %d failures\n", valid, failures);
  return failures == 0 ? 0 : 1;
}
