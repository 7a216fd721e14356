// libtsp C ABI: argument validation, workspace carving and kernel dispatch.
// Every check runs before the first launch; nothing here allocates device
// memory or synchronises.
#include "../../include/tsp.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(TSP_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = int64_t(1) << 24;

// Validates dims and fills the derived shape.  Returns TSP_OK or an error code.
int make_shape(const tsp_dims_t* d, tsp::Shape* s) {
  if (d == nullptr) return fail(TSP_ERR_NULL_POINTER, "dims is NULL");
  if (d->batch < 1) return fail(TSP_ERR_BATCH, "batch must be >= 1 (got %d)", d->batch);
  if (d->degree < 1) return fail(TSP_ERR_DEGREE, "degree must be >= 1 (got %d)", d->degree);
  if (d->rank < 0 || d->rank >= d->degree)
    return fail(TSP_ERR_RANK, "rank %d not in [0, degree=%d)", d->rank, d->degree);
  if (d->seq < 2 * d->degree || d->seq % (2 * d->degree) != 0)
    return fail(TSP_ERR_SEQ, "seq %d must be a positive multiple of 2*degree=%d", d->seq, 2 * d->degree);
  if (d->n_q_heads < 1 || d->n_kv_heads < 1) return fail(TSP_ERR_HEADS, "head counts must be >= 1");
  if (d->n_q_heads % d->degree != 0 || d->n_kv_heads % d->degree != 0)
    return fail(TSP_ERR_HEADS, "n_q_heads %d and n_kv_heads %d must be multiples of degree %d", d->n_q_heads,
                d->n_kv_heads, d->degree);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(TSP_ERR_GQA, "n_q_heads %d must be a multiple of n_kv_heads %d", d->n_q_heads, d->n_kv_heads);
  if (d->hidden < 64 || d->hidden % 64 != 0)
    return fail(TSP_ERR_HIDDEN, "hidden %d must be a positive multiple of 64", d->hidden);
  if (d->ffn < 64 || d->ffn % 64 != 0 || (d->ffn / d->degree) * d->degree != d->ffn ||
      (d->ffn / d->degree) % 8 != 0)
    return fail(TSP_ERR_FFN, "ffn %d must be a positive multiple of 64 with ffn/degree a multiple of 8", d->ffn);
  if (d->partition != TSP_PARTITION_ZIGZAG && d->partition != TSP_PARTITION_STRIPED)
    return fail(TSP_ERR_PARTITION, "partition %d unknown (0 zigzag, 1 striped)", d->partition);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(TSP_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if ((int64_t)d->seq > kMaxDim || (int64_t)d->batch * d->seq / d->degree > kMaxDim ||
      d->hidden > 65536 || d->ffn > 1048576 || (int64_t)d->n_q_heads * d->head_dim > 65536)
    return fail(TSP_ERR_UNSUPPORTED, "shape exceeds the supported index range");
  tsp::Shape& x = *s;
  x.B = d->batch;
  x.S = d->seq;
  x.D = d->degree;
  x.r = d->rank;
  x.h = d->hidden;
  x.Hq = d->n_q_heads;
  x.Hkv = d->n_kv_heads;
  x.dh = d->head_dim;
  x.F = d->ffn;
  x.part = d->partition;
  x.T = x.S / x.D;
  x.c = x.S / (2 * x.D);
  x.M = x.B * x.T;
  x.Hq_s = x.Hq / x.D;
  x.Hkv_s = x.Hkv / x.D;
  x.F_s = x.F / x.D;
  x.kmax = x.part == TSP_PARTITION_STRIPED ? (x.T - 1) * x.D + x.r + 1 : (2 * x.D - x.r) * x.c;
  x.kmax_pad = (x.kmax + 63) / 64 * 64;
  x.nqkv_s = (x.Hq_s + 2 * x.Hkv_s) * x.dh;
  return TSP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int need_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(TSP_ERR_NULL_POINTER, "%s is NULL", name);
  if (!aligned16(p)) return fail(TSP_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return TSP_OK;
}

int opt_ptr(const void* p, const char* name) {
  if (p != nullptr && !aligned16(p)) return fail(TSP_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return TSP_OK;
}

// Process-wide kernel-choice overrides (tsp_set_tuning); -1 = default.
std::atomic<int> g_tune[TSP_TUNE_COUNT] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1};

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t bytes_q(const tsp::Shape& s) { return (size_t)s.M * s.Hq * s.dh * 2; }
size_t bytes_kvnat(const tsp::Shape& s) { return (size_t)2 * s.Hkv * s.B * s.kmax_pad * s.dh * 2; }
size_t bytes_knat(const tsp::Shape& s) { return bytes_kvnat(s) / 2; }
size_t bytes_o(const tsp::Shape& s) { return (size_t)s.M * s.Hq * s.dh * 2; }
size_t bytes_h32(const tsp::Shape& s) { return (size_t)s.M * s.h * 4; }
size_t bytes_h16(const tsp::Shape& s) { return (size_t)s.M * s.h * 2; }
size_t bytes_act(const tsp::Shape& s) { return (size_t)s.M * s.F * 2; }
size_t bytes_gathered(const tsp::Shape& s) {
  return (size_t)s.D * s.D * 2 * s.B * s.T * s.Hkv_s * s.dh * 2;
}

// Scratch for partial results: the split-K partial sums of the output and
// down projections, or the attention pieces; never live at the same time.
size_t bytes_partial(const tsp::Shape& s) {
  const int p = tsp::gemm_split_plan(s);
  const size_t gemm = p > 1 ? (size_t)p * s.M * s.h * 4 : 0;
  const size_t attn = tsp::attn_partial_bytes(s);
  return gemm > attn ? gemm : attn;
}

// Backward of the MLP ring: M rows padded to 64 on the transposed copies.
int mpad(const tsp::Shape& s) { return (s.M + 63) / 64 * 64; }

// Sequential 256-byte aligned pieces of a workspace (base may be null to
// only add up the size).
struct Carve {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* p = base != nullptr ? reinterpret_cast<T*>(base + off) : nullptr;
    off += up(bytes);
    return p;
  }
};

// The backward products that take a weight as their second operand read it
// as stored (K-major) unless TSP_TUNE_BWD_WEIGHTS asks for transposed copies
// or the shape does not suit the K-major kernel; only then does the
// workspace hold the copies.
bool kmajor(const tsp::Shape& s, int use) { return tsp::tune_get(TSP_TUNE_BWD_WEIGHTS) != 1 && tsp::kmajor_ok(s, use); }

struct MlpBwdWs {
  uint16_t *x16, *xT, *dy16, *dyT, *wdT, *wguT, *act, *dgu, *actT, *dguT;
  float *da, *partial;
};

// [(x16) | xT | dy16 | dyT | (wdT) | (wguT) | (da) | act | dgu | actT | dguT | split-K partials]
// (kept: g and u come from tsp_mlp_ring_fwd_keep, so neither the f16 copy of
// a float32 x for their recomputation nor dA is stored)
size_t ws_mlp_bwd(const tsp::Shape& s, MlpBwdWs* w = nullptr, char* base = nullptr, bool kept = false) {
  MlpBwdWs tmp;
  MlpBwdWs& x = w != nullptr ? *w : tmp;
  const size_t M = s.M, h = s.h, F = s.F, Mp = mpad(s);
  Carve c{base};
  x.x16 = kept ? nullptr : c.take<uint16_t>(M * h * 2);
  x.xT = c.take<uint16_t>(h * Mp * 2);
  x.dy16 = c.take<uint16_t>(M * h * 2);
  x.dyT = c.take<uint16_t>(h * Mp * 2);
  x.wdT = kmajor(s, tsp::KMAJ_DA) ? nullptr : c.take<uint16_t>(F * h * 2);
  x.wguT = kmajor(s, tsp::KMAJ_DX_MLP) ? nullptr : c.take<uint16_t>(h * 2 * F * 2);
  x.da = kept ? nullptr : c.take<float>(M * F * 4);
  x.act = c.take<uint16_t>(M * F * 2);
  x.dgu = c.take<uint16_t>(M * 2 * F * 2);
  x.actT = c.take<uint16_t>(F * Mp * 2);
  x.dguT = c.take<uint16_t>(2 * F * Mp * 2);
  const int p = tsp::gemm_split_plan(s);
  x.partial = p > 1 ? c.take<float>((size_t)p * M * h * 4) : nullptr;
  return c.off;
}

// Backward of the attention, part 1:
// [q | o | lse | delta | dh16 | dh^T | (Wo^T) | dO | O^T | attention pieces]
// (kept: the caller holds q, o and lse from tsp_attn_fwd_keep; they are not
// in the workspace)
struct AttnBwdWs {
  uint16_t *q, *o, *dh16, *dhT, *woT, *dout, *oT;
  float *lse, *delta, *partial;
};
size_t ws_attn_bwd(const tsp::Shape& s, AttnBwdWs* w = nullptr, char* base = nullptr, bool kept = false) {
  AttnBwdWs tmp;
  AttnBwdWs& x = w != nullptr ? *w : tmp;
  const size_t M = s.M, h = s.h, qd = (size_t)s.Hq * s.dh, Mp = mpad(s), rows = (size_t)s.B * s.Hq * s.T;
  Carve c{base};
  x.q = kept ? nullptr : c.take<uint16_t>(M * qd * 2);
  x.o = kept ? nullptr : c.take<uint16_t>(M * qd * 2);
  x.lse = kept ? nullptr : c.take<float>(rows * 4);
  x.delta = c.take<float>(rows * 4);
  x.dh16 = c.take<uint16_t>(M * h * 2);
  x.dhT = c.take<uint16_t>(h * Mp * 2);
  x.woT = kmajor(s, tsp::KMAJ_DO) ? nullptr : c.take<uint16_t>(qd * h * 2);
  x.dout = c.take<uint16_t>(M * qd * 2);
  x.oT = c.take<uint16_t>(qd * Mp * 2);
  const size_t part = tsp::attn_partial_bytes(s);
  x.partial = part > 0 ? c.take<float>(part) : nullptr;
  return c.off;
}

// Part 2: [G | G^T | (Wqkv^T) | x^T | split-K partials]
struct AttnBwdProjWs {
  uint16_t *g16, *gT, *wqkvT, *xT;
  float* partial;
};
size_t ws_attn_bwd_proj(const tsp::Shape& s, AttnBwdProjWs* w = nullptr, char* base = nullptr) {
  AttnBwdProjWs tmp;
  AttnBwdProjWs& x = w != nullptr ? *w : tmp;
  const size_t M = s.M, h = s.h, Nall = (size_t)s.D * s.nqkv_s, Mp = mpad(s);
  Carve c{base};
  x.g16 = c.take<uint16_t>(M * Nall * 2);
  x.gT = c.take<uint16_t>(Nall * Mp * 2);
  x.wqkvT = kmajor(s, tsp::KMAJ_DX_ATTN) ? nullptr : c.take<uint16_t>(h * Nall * 2);
  x.xT = c.take<uint16_t>(h * Mp * 2);
  const int p = tsp::gemm_split_plan(s);
  x.partial = p > 1 ? c.take<float>((size_t)p * M * h * 4) : nullptr;
  return c.off;
}

size_t bytes_dkv(const tsp::Shape& s) { return (size_t)s.D * s.D * 2 * s.M * s.Hkv_s * s.dh * 4; }

struct AttnWs {
  uint16_t *q, *o;
  float* partial;
};
struct MlpWs {
  uint16_t *h16, *act;
  float* partial;
};

// Workspace layouts (256-byte aligned pieces):
//   attention  [q | o | split-K partials]
//   MLP        [h16 | act | split-K partials]
//   layer      [q | o | h32 | h16 | act | split-K partials]
// (attention reads K/V straight from the all-gathered buffer)
size_t ws_attn(const tsp::Shape& s) { return up(bytes_q(s)) + up(bytes_o(s)) + up(bytes_partial(s)); }
// tsp_attn_fwd_keep: q and o go to the caller's buffers; at least one
// aligned piece so that the size is never 0
size_t ws_attn_keep(const tsp::Shape& s) { return bytes_partial(s) > 0 ? up(bytes_partial(s)) : kAlign; }
size_t ws_mlp(const tsp::Shape& s) { return up(bytes_h16(s)) + up(bytes_act(s)) + up(bytes_partial(s)); }
size_t ws_layer(const tsp::Shape& s) {
  return up(bytes_q(s)) + up(bytes_o(s)) + up(bytes_h32(s)) + up(bytes_h16(s)) + up(bytes_act(s)) +
         up(bytes_partial(s));
}

char* carve_attn(const tsp::Shape& s, char* p, AttnWs* w) {
  w->q = reinterpret_cast<uint16_t*>(p);
  p += up(bytes_q(s));
  w->o = reinterpret_cast<uint16_t*>(p);
  p += up(bytes_o(s));
  return p;
}

char* carve_mlp(const tsp::Shape& s, char* p, MlpWs* w) {
  w->h16 = reinterpret_cast<uint16_t*>(p);
  p += up(bytes_h16(s));
  w->act = reinterpret_cast<uint16_t*>(p);
  p += up(bytes_act(s));
  return p;
}

float* partial_or_null(const tsp::Shape& s, char* p) {
  return bytes_partial(s) > 0 ? reinterpret_cast<float*>(p) : nullptr;
}

// ---- fixed scratch array (tsp_layer_fwd_noalloc) ---------------------------
// The workspace of the entry point that allocates nothing.  Each GPU the
// library runs on holds its own copy for the life of the process.  In host
// code `scratch` is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress, looked up once per device and kept here.
static __device__ __align__(256) unsigned char scratch[TSP_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "tsp_layer_fwd_noalloc");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TSP_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "tsp_layer_fwd_noalloc: scratch address");
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
      return fail(TSP_ERR_HIP, "tsp_layer_fwd_noalloc: scratch address %p unusable", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TSP_OK;
}

// ---- live per-kernel timing (see tsp_profile_kernel) -----------------------
struct Profile {
  int kernel = TSP_K_NONE;
  int used = 0;
  std::vector<hipEvent_t> ev;  // 2 per launch
};
thread_local Profile g_prof;

void prof_release() {
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.kernel = TSP_K_NONE;
  g_prof.used = 0;
}

// Records the opening event when `id` is being profiled; returns the slot or -1.
int prof_open(int id, hipStream_t st) {
  if (g_prof.kernel != id || 2 * (g_prof.used + 1) > (int)g_prof.ev.size()) return -1;
  const int slot = g_prof.used++;
  (void)hipEventRecord(g_prof.ev[2 * slot], st);
  return slot;
}
void prof_close(int slot, hipStream_t st) {
  if (slot >= 0) (void)hipEventRecord(g_prof.ev[2 * slot + 1], st);
}

int check_device(const char* where) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, where);
  return TSP_OK;
}

#define TSP_TRY(expr)            \
  do {                           \
    int _rc = (expr);            \
    if (_rc != TSP_OK) return _rc; \
  } while (0)

#define TSP_LAUNCH(expr, where)                   \
  do {                                            \
    hipError_t _e = (expr);                       \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// A launch of kernel `id`, bracketed by profiling events when armed.
#define TSP_KLAUNCH(id, st, expr, where)          \
  do {                                            \
    const int _slot = prof_open(id, st);          \
    hipError_t _e = (expr);                       \
    prof_close(_slot, st);                        \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// out = resid + attention branch; resid is x_resid (bf16, the layer's own
// input), else resid_f32, else nothing.
// lse (optional): each row's log2 softmax normaliser, for the backward.
int run_attention(const tsp::Shape& s, const uint16_t* x_local, const uint16_t* w_qkv,
                  const uint16_t* w_o, uint16_t* kv_gathered, const uint16_t* x_resid, const float* resid_f32,
                  float* out, uint16_t* out16, const AttnWs& w, hipStream_t st, float* lse = nullptr) {
  TSP_KLAUNCH(TSP_K_QKV, st, tsp::launch_qkv_gemm(s, s.r, x_local, w_qkv, w.q, kv_gathered, st),
              "qkv projection");
  TSP_KLAUNCH(TSP_K_ATTN, st, tsp::launch_flash_attn(s, w.q, kv_gathered, w.o, w.partial, st, lse),
              "flash attention");
  TSP_KLAUNCH(TSP_K_OPROJ, st,
              tsp::launch_oproj_gemm(s, w.o, w_o, x_resid, resid_f32, out, out16, w.partial, st),
              "output projection");
  return TSP_OK;
}

// gu_keep (optional): g and u kept for the backward.
int run_mlp(const tsp::Shape& s, const uint16_t* x16, bool x_bf16, const float* resid, const uint16_t* w_gate,
            const uint16_t* w_up, const uint16_t* w_down, float* y, const MlpWs& w, hipStream_t st,
            float* gu_keep = nullptr) {
  TSP_KLAUNCH(TSP_K_GATEUP, st, tsp::launch_gateup_gemm(s, x16, x_bf16, w_gate, w_up, w.act, st, gu_keep),
              "mlp gate/up");
  TSP_KLAUNCH(TSP_K_DOWN, st, tsp::launch_down_gemm(s, w.act, w_down, resid, y, w.partial, st),
              "mlp down ring");
  return TSP_OK;
}

}  // namespace

namespace tsp {
int tune_get(int knob) {
  return knob >= 0 && knob < TSP_TUNE_COUNT ? g_tune[knob].load(std::memory_order_relaxed) : -1;
}
}  // namespace tsp

extern "C" {

const char* tsp_last_error(void) { return g_last_error.c_str(); }

int tsp_set_tuning(int32_t knob, int32_t value) {
  if (knob < 0 || knob >= TSP_TUNE_COUNT) return fail(TSP_ERR_INVALID_ARG, "unknown tuning knob %d", knob);
  g_tune[knob].store(value < 0 ? -1 : value, std::memory_order_relaxed);
  return TSP_OK;
}

int tsp_profile_kernel(int32_t kernel_id, int32_t max_launches) {
  if (kernel_id < TSP_K_NONE || kernel_id >= TSP_K_COUNT)
    return fail(TSP_ERR_INVALID_ARG, "unknown kernel id %d", kernel_id);
  prof_release();
  if (kernel_id == TSP_K_NONE) return TSP_OK;
  if (max_launches < 1 || max_launches > 100000)
    return fail(TSP_ERR_INVALID_ARG, "max_launches %d not in [1, 100000]", max_launches);
  TSP_TRY(check_device("tsp_profile_kernel"));
  g_prof.ev.resize(2 * (size_t)max_launches, nullptr);
  // timing-only events: no system-scope release/acquire (an L2 write-back
  // per record), which would stall the stream between the bracketed kernel
  // and its neighbours
  for (hipEvent_t& e : g_prof.ev) {
    hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (err != hipSuccess) {
      prof_release();
      return hip_fail(err, "tsp_profile_kernel");
    }
  }
  g_prof.kernel = kernel_id;
  return TSP_OK;
}

int tsp_profile_result(int32_t* launches, float* total_ms) {
  if (launches == nullptr || total_ms == nullptr)
    return fail(TSP_ERR_NULL_POINTER, "launches and total_ms must not be NULL");
  float sum = 0.0f;
  for (int i = 0; i < g_prof.used; ++i) {
    hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "tsp_profile_result");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "tsp_profile_result");
    sum += ms;
  }
  *launches = g_prof.used;
  *total_ms = sum;
  g_prof.used = 0;
  return TSP_OK;
}

size_t tsp_workspace_bytes(const tsp_dims_t* dims, int32_t fn) {
  tsp::Shape s;
  if (make_shape(dims, &s) != TSP_OK) return 0;
  switch (fn) {
    case TSP_FN_ATTN: return ws_attn(s);
    case TSP_FN_MLP: return ws_mlp(s);
    case TSP_FN_LAYER: return ws_layer(s);
    case TSP_FN_KV_NATURAL: return bytes_kvnat(s);
    case TSP_FN_KV_GATHERED: return bytes_gathered(s);
    case TSP_FN_MLP_BWD: return ws_mlp_bwd(s);
    case TSP_FN_ATTN_BWD: return ws_attn_bwd(s);
    case TSP_FN_ATTN_BWD_PROJ: return ws_attn_bwd_proj(s);
    case TSP_FN_DKV: return bytes_dkv(s);
    case TSP_FN_ATTN_KEEP: return ws_attn_keep(s);
    case TSP_FN_ATTN_BWD_KEPT: return ws_attn_bwd(s, nullptr, nullptr, true);
    case TSP_FN_LSE: return (size_t)s.B * s.Hq * s.T * 4;
    case TSP_FN_MLP_BWD_KEPT: return ws_mlp_bwd(s, nullptr, nullptr, true);
    case TSP_FN_GU: return (size_t)2 * s.M * s.F * 4;
    default: fail(TSP_ERR_INVALID_ARG, "unknown workspace selector %d", fn); return 0;
  }
}

int tsp_zigzag_index(const tsp_dims_t* dims, int32_t* local_to_global, int32_t* global_to_slot,
                     hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  if (local_to_global == nullptr) return fail(TSP_ERR_NULL_POINTER, "local_to_global is NULL");
  TSP_TRY(check_device("tsp_zigzag_index"));
  TSP_LAUNCH(tsp::launch_zigzag_index(s, local_to_global, global_to_slot, stream), "zigzag index");
  return TSP_OK;
}

int tsp_qkv_proj(const tsp_dims_t* dims, int32_t src_rank, const uint16_t* x_shard,
                 const uint16_t* w_qkv, uint16_t* q_out, uint16_t* kv_gathered, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  if (src_rank < 0 || src_rank >= s.D)
    return fail(TSP_ERR_RANK, "src_rank %d not in [0, %d)", src_rank, s.D);
  TSP_TRY(need_ptr(x_shard, "x_shard"));
  TSP_TRY(need_ptr(w_qkv, "w_qkv"));
  TSP_TRY(opt_ptr(q_out, "q_out"));
  TSP_TRY(need_ptr(kv_gathered, "kv_gathered"));
  TSP_TRY(check_device("tsp_qkv_proj"));
  TSP_KLAUNCH(TSP_K_QKV, stream,
              tsp::launch_qkv_gemm(s, src_rank, x_shard, w_qkv, q_out, kv_gathered, stream),
              "qkv projection");
  return TSP_OK;
}

int tsp_kv_reorder(const tsp_dims_t* dims, const uint16_t* kv_gathered, uint16_t* kv_natural, int32_t kmax,
                   hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  if (kmax < 0 || kmax > s.S) return fail(TSP_ERR_KMAX, "kmax %d not in [0, seq=%d]", kmax, s.S);
  TSP_TRY(need_ptr(kv_gathered, "kv_gathered"));
  TSP_TRY(need_ptr(kv_natural, "kv_natural"));
  TSP_TRY(check_device("tsp_kv_reorder"));
  if (kmax > 0) {
    s.kmax = kmax;
    s.kmax_pad = (kmax + 63) / 64 * 64;
  }
  uint16_t* vnat = kv_natural + bytes_knat(s) / 2;
  TSP_KLAUNCH(TSP_K_REORDER, stream, tsp::launch_kv_reorder(s, kv_gathered, kv_natural, vnat, stream),
              "kv reorder");
  return TSP_OK;
}

int tsp_attn_fwd(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                 const uint16_t* w_o, uint16_t* kv_gathered, const float* residual, float* out, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  TSP_TRY(need_ptr(x_local, "x_local"));
  TSP_TRY(need_ptr(w_qkv, "w_qkv"));
  TSP_TRY(need_ptr(w_o, "w_o"));
  TSP_TRY(need_ptr(kv_gathered, "kv_gathered"));
  TSP_TRY(opt_ptr(residual, "residual"));
  TSP_TRY(need_ptr(out, "out"));
  TSP_TRY(need_ptr(ws, "ws"));
  if (ws_bytes < ws_attn(s))
    return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws_attn(s));
  TSP_TRY(check_device("tsp_attn_fwd"));
  AttnWs w;
  w.partial = partial_or_null(s, carve_attn(s, static_cast<char*>(ws), &w));
  return run_attention(s, x_local, w_qkv, w_o, kv_gathered, nullptr, residual, out, nullptr, w, stream);
}

// tsp_mlp_ring_fwd, and tsp_mlp_ring_fwd_keep when gu_keep != nullptr.
static int mlp_ring_fwd(const char* fn, const tsp_dims_t* dims, const void* x, int32_t x_dtype,
                        const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down, const float* residual,
                        float* y, float* gu_keep, void* ws, size_t ws_bytes, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  if (x_dtype != TSP_BF16 && x_dtype != TSP_F16 && x_dtype != TSP_F32)
    return fail(TSP_ERR_DTYPE, "x_dtype %d unknown (0 bf16, 1 f16, 2 f32)", x_dtype);
  TSP_TRY(need_ptr(x, "x"));
  TSP_TRY(need_ptr(w_gate, "w_gate"));
  TSP_TRY(need_ptr(w_up, "w_up"));
  TSP_TRY(need_ptr(w_down, "w_down"));
  TSP_TRY(opt_ptr(residual, "residual"));
  TSP_TRY(need_ptr(y, "y"));
  TSP_TRY(need_ptr(ws, "ws"));
  if (ws_bytes < ws_mlp(s))
    return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws_mlp(s));
  TSP_TRY(check_device(fn));
  MlpWs w;
  w.partial = partial_or_null(s, carve_mlp(s, static_cast<char*>(ws), &w));
  const uint16_t* x16 = static_cast<const uint16_t*>(x);
  if (x_dtype == TSP_F32) {
    TSP_LAUNCH(tsp::launch_f32_to_f16(static_cast<const float*>(x), w.h16, (int64_t)s.M * s.h, stream),
               "mlp input rounding");
    x16 = w.h16;
  }
  return run_mlp(s, x16, x_dtype == TSP_BF16, residual, w_gate, w_up, w_down, y, w, stream, gu_keep);
}

int tsp_mlp_ring_fwd(const tsp_dims_t* dims, const void* x, int32_t x_dtype, const uint16_t* w_gate,
                     const uint16_t* w_up, const uint16_t* w_down, const float* residual, float* y, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  return mlp_ring_fwd("tsp_mlp_ring_fwd", dims, x, x_dtype, w_gate, w_up, w_down, residual, y, nullptr, ws,
                      ws_bytes, stream);
}

int tsp_mlp_ring_fwd_keep(const tsp_dims_t* dims, const void* x, int32_t x_dtype, const uint16_t* w_gate,
                          const uint16_t* w_up, const uint16_t* w_down, const float* residual, float* y,
                          float* gu_keep, void* ws, size_t ws_bytes, hipStream_t stream) {
  TSP_TRY(need_ptr(gu_keep, "gu_keep"));
  return mlp_ring_fwd("tsp_mlp_ring_fwd_keep", dims, x, x_dtype, w_gate, w_up, w_down, residual, y, gu_keep, ws,
                      ws_bytes, stream);
}

// tsp_mlp_ring_bwd, and tsp_mlp_ring_bwd_kept when gu_keep != nullptr.
static int mlp_ring_bwd(const char* fn, const tsp_dims_t* dims, const void* x, int32_t x_dtype, const float* dy,
                        const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down, const float* gu_keep,
                        const float* dx_residual, float* dx, float* dw_gate, float* dw_up, float* dw_down, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  if (x_dtype != TSP_BF16 && x_dtype != TSP_F16 && x_dtype != TSP_F32)
    return fail(TSP_ERR_DTYPE, "x_dtype %d unknown (0 bf16, 1 f16, 2 f32)", x_dtype);
  TSP_TRY(need_ptr(x, "x"));
  TSP_TRY(need_ptr(dy, "dy"));
  TSP_TRY(need_ptr(w_gate, "w_gate"));
  TSP_TRY(need_ptr(w_up, "w_up"));
  TSP_TRY(need_ptr(w_down, "w_down"));
  TSP_TRY(opt_ptr(dx_residual, "dx_residual"));
  TSP_TRY(need_ptr(dx, "dx"));
  TSP_TRY(need_ptr(dw_gate, "dw_gate"));
  TSP_TRY(need_ptr(dw_up, "dw_up"));
  TSP_TRY(need_ptr(dw_down, "dw_down"));
  TSP_TRY(need_ptr(ws, "ws"));
  const bool kept = gu_keep != nullptr;
  const size_t need = ws_mlp_bwd(s, nullptr, nullptr, kept);
  if (ws_bytes < need) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  TSP_TRY(check_device(fn));
  MlpBwdWs w;
  ws_mlp_bwd(s, &w, static_cast<char*>(ws), kept);
  const int Mp = mpad(s), h = s.h, F = s.F, Fs = s.F_s;
  const int tin = x_dtype == TSP_BF16 ? tsp::TR_BF16 : x_dtype == TSP_F16 ? tsp::TR_F16 : tsp::TR_F32;
  // recomputation input: x itself (bf16 or f16), or x rounded to f16
  const uint16_t* xg = static_cast<const uint16_t*>(x);
  if (!kept && x_dtype == TSP_F32) {
    TSP_LAUNCH(tsp::launch_f32_to_f16(static_cast<const float*>(x), w.x16, (int64_t)s.M * h, stream),
               "mlp bwd: x to f16");
    xg = w.x16;
  }
  // transposed / converted operands
  TSP_LAUNCH(tsp::launch_transpose_bf16(tin, x, h, 0, w.xT, Mp, 0, s.M, h, Mp, 1, stream), "mlp bwd: x^T");
  TSP_LAUNCH(tsp::launch_f32_to_bf16(dy, w.dy16, (int64_t)s.M * h, stream), "mlp bwd: dy to bf16");
  TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_F32, dy, h, 0, w.dyT, Mp, 0, s.M, h, Mp, 1, stream),
             "mlp bwd: dy^T");
  // dA = dy W_down and dx = sum dG_j W_gate,j + dU_j W_up,j read the weights
  // as stored; the workspace holds transposed copies (wdT, wguT) only where
  // the K-major products do not apply.  Kept g and u: dA stays in registers
  // and its epilogue forms a, dG and dU (no recomputation of g and u).
  if (w.wdT == nullptr) {
    if (kept)
      TSP_LAUNCH(tsp::launch_bwd_da_kept_kmajor(s, w.dy16, w_down, gu_keep, w.act, w.dgu, stream),
                 "mlp bwd: dA, dG, dU");
    else
      TSP_LAUNCH(tsp::launch_bwd_da_kmajor(s, w.dy16, w_down, w.da, stream), "mlp bwd: dA");
  } else {
    // Wd_j [h][Fs] -> WdT rows j Fs .. : [Fs][h]
    TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w_down, Fs, (int64_t)h * Fs, w.wdT, h, (int64_t)Fs * h, h,
                                          Fs, h, s.D, stream),
               "mlp bwd: Wd^T");
    if (kept)
      TSP_LAUNCH(tsp::launch_bwd_da_kept(s, w.dy16, w.wdT, gu_keep, w.act, w.dgu, stream), "mlp bwd: dA, dG, dU");
    else
      TSP_LAUNCH(tsp::launch_bwd_da(s, w.dy16, w.wdT, w.da, stream), "mlp bwd: dA");
  }
  if (!kept)
    TSP_LAUNCH(tsp::launch_bwd_gu(s, xg, x_dtype == TSP_BF16, w_gate, w_up, w.da, w.act, w.dgu, stream),
               "mlp bwd: gate/up recompute");
  if (w.wguT == nullptr) {
    TSP_LAUNCH(tsp::launch_bwd_dx_kmajor(s, w.dgu, w_gate, w_up, dx_residual, dx, w.partial, stream), "mlp bwd: dx");
  } else {
    // Wg_j, Wu_j [Fs][h] -> WguT [h][D][2][Fs]
    TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w_gate, h, (int64_t)Fs * h, w.wguT, 2 * (int64_t)F,
                                          2 * (int64_t)Fs, Fs, h, Fs, s.D, stream),
               "mlp bwd: Wg^T");
    TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w_up, h, (int64_t)Fs * h, w.wguT + Fs, 2 * (int64_t)F,
                                          2 * (int64_t)Fs, Fs, h, Fs, s.D, stream),
               "mlp bwd: Wu^T");
    TSP_LAUNCH(tsp::launch_bwd_dx(s, w.dgu, w.wguT, dx_residual, dx, w.partial, stream), "mlp bwd: dx");
  }
  TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w.act, F, 0, w.actT, Mp, 0, s.M, F, Mp, 1, stream),
             "mlp bwd: a^T");
  TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w.dgu, 2 * (int64_t)F, 0, w.dguT, Mp, 0, s.M, 2 * F, Mp, 1,
                                        stream),
             "mlp bwd: dGU^T");
  TSP_LAUNCH(tsp::launch_bwd_dwd(s, Mp, w.dyT, w.actT, dw_down, stream), "mlp bwd: dW_down");
  TSP_LAUNCH(tsp::launch_bwd_dwgu(s, Mp, w.dguT, w.xT, dw_gate, dw_up, stream), "mlp bwd: dW_gate, dW_up");
  return TSP_OK;
}

int tsp_mlp_ring_bwd(const tsp_dims_t* dims, const void* x, int32_t x_dtype, const float* dy,
                     const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                     const float* dx_residual, float* dx, float* dw_gate, float* dw_up, float* dw_down, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  return mlp_ring_bwd("tsp_mlp_ring_bwd", dims, x, x_dtype, dy, w_gate, w_up, w_down, nullptr, dx_residual, dx,
                      dw_gate, dw_up, dw_down, ws, ws_bytes, stream);
}

int tsp_mlp_ring_bwd_kept(const tsp_dims_t* dims, const void* x, int32_t x_dtype, const float* dy,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down, const float* gu_keep,
                          const float* dx_residual, float* dx, float* dw_gate, float* dw_up, float* dw_down,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  TSP_TRY(need_ptr(gu_keep, "gu_keep"));
  return mlp_ring_bwd("tsp_mlp_ring_bwd_kept", dims, x, x_dtype, dy, w_gate, w_up, w_down, gu_keep, dx_residual,
                      dx, dw_gate, dw_up, dw_down, ws, ws_bytes, stream);
}

// The attention backward from the forward's Q, O and row normalisers (w.q,
// w.o, w.lse) on: dO = dh W_O, Delta, dQ, the K/V-gradient send buffer and
// the dW_O share.
static int attn_bwd_from_forward(const tsp::Shape& s, const uint16_t* w_o, const uint16_t* kv_gathered,
                                 const float* dh, float* dq, float* dkv_send, float* dw_o, AttnBwdWs& w,
                                 hipStream_t stream) {
  const int Mp = mpad(s), h = s.h, qs = s.Hq_s * s.dh;
  // dO = dh W_O: W_O read as stored, or through the copy WoT (W_O_j
  // [h][qs] -> WoT rows j qs ..: [qs][h]) where the workspace holds one
  TSP_LAUNCH(tsp::launch_f32_to_bf16(dh, w.dh16, (int64_t)s.M * h, stream), "attn bwd: dh to bf16");
  if (w.woT == nullptr) {
    TSP_LAUNCH(tsp::launch_attn_bwd_do_kmajor(s, w.dh16, w_o, w.dout, stream), "attn bwd: dO");
  } else {
    TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w_o, qs, (int64_t)h * qs, w.woT, h, (int64_t)qs * h, h, qs,
                                          h, s.D, stream),
               "attn bwd: W_O^T");
    TSP_LAUNCH(tsp::launch_attn_bwd_do(s, w.dh16, w.woT, w.dout, stream), "attn bwd: dO");
  }
  {
    const int slot = prof_open(TSP_K_ATTN_BWD, stream);
    hipError_t e = tsp::launch_attn_bwd_core(s, w.q, kv_gathered, w.o, w.dout, w.lse, w.delta, dq, dkv_send,
                                             w.partial, stream);
    prof_close(slot, stream);
    if (e != hipSuccess) return hip_fail(e, "attn bwd: dQ, dK, dV");
  }
  // dW_O = dh^T O
  TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_F32, dh, h, 0, w.dhT, Mp, 0, s.M, h, Mp, 1, stream),
             "attn bwd: dh^T");
  TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_F16, w.o, (int64_t)s.Hq * s.dh, 0, w.oT, Mp, 0, s.M, s.Hq * s.dh,
                                        Mp, 1, stream),
             "attn bwd: O^T");
  TSP_LAUNCH(tsp::launch_attn_bwd_dwo(s, Mp, w.dhT, w.oT, dw_o, stream), "attn bwd: dW_O");
  return TSP_OK;
}

int tsp_attn_bwd(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv, const uint16_t* w_o,
                 const uint16_t* kv_gathered, const float* dh, float* dq, float* dkv_send, float* dw_o, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  TSP_TRY(need_ptr(x_local, "x_local"));
  TSP_TRY(need_ptr(w_qkv, "w_qkv"));
  TSP_TRY(need_ptr(w_o, "w_o"));
  TSP_TRY(need_ptr(kv_gathered, "kv_gathered"));
  TSP_TRY(need_ptr(dh, "dh"));
  TSP_TRY(need_ptr(dq, "dq"));
  TSP_TRY(need_ptr(dkv_send, "dkv_send"));
  TSP_TRY(need_ptr(dw_o, "dw_o"));
  TSP_TRY(need_ptr(ws, "ws"));
  if (ws_bytes < ws_attn_bwd(s))
    return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws_attn_bwd(s));
  TSP_TRY(check_device("tsp_attn_bwd"));
  AttnBwdWs w;
  ws_attn_bwd(s, &w, static_cast<char*>(ws));
  // recomputation: Q (from the Q rows of every shard of W_QKV, read in
  // place), then the attention output with its row normalisers
  TSP_LAUNCH(tsp::launch_q_gemm(s, x_local, static_cast<const uint16_t*>(w_qkv), w.q, stream), "attn bwd: Q");
  TSP_LAUNCH(tsp::launch_flash_attn(s, w.q, kv_gathered, w.o, w.partial, stream, w.lse), "attn bwd: attention");
  return attn_bwd_from_forward(s, w_o, kv_gathered, dh, dq, dkv_send, dw_o, w, stream);
}

int tsp_attn_bwd_kept(const tsp_dims_t* dims, const uint16_t* w_o, const uint16_t* kv_gathered,
                      const uint16_t* q_keep, const uint16_t* o_keep, const float* lse_keep, const float* dh,
                      float* dq, float* dkv_send, float* dw_o, void* ws, size_t ws_bytes, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  TSP_TRY(need_ptr(w_o, "w_o"));
  TSP_TRY(need_ptr(kv_gathered, "kv_gathered"));
  TSP_TRY(need_ptr(q_keep, "q_keep"));
  TSP_TRY(need_ptr(o_keep, "o_keep"));
  TSP_TRY(need_ptr(lse_keep, "lse_keep"));
  TSP_TRY(need_ptr(dh, "dh"));
  TSP_TRY(need_ptr(dq, "dq"));
  TSP_TRY(need_ptr(dkv_send, "dkv_send"));
  TSP_TRY(need_ptr(dw_o, "dw_o"));
  TSP_TRY(need_ptr(ws, "ws"));
  const size_t need = ws_attn_bwd(s, nullptr, nullptr, true);
  if (ws_bytes < need) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  TSP_TRY(check_device("tsp_attn_bwd_kept"));
  AttnBwdWs w;
  ws_attn_bwd(s, &w, static_cast<char*>(ws), true);
  w.q = const_cast<uint16_t*>(q_keep);
  w.o = const_cast<uint16_t*>(o_keep);
  w.lse = const_cast<float*>(lse_keep);
  return attn_bwd_from_forward(s, w_o, kv_gathered, dh, dq, dkv_send, dw_o, w, stream);
}

int tsp_attn_fwd_keep(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                      const uint16_t* w_o, uint16_t* kv_gathered, const float* residual, float* out,
                      uint16_t* q_keep, uint16_t* o_keep, float* lse_keep, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  TSP_TRY(need_ptr(x_local, "x_local"));
  TSP_TRY(need_ptr(w_qkv, "w_qkv"));
  TSP_TRY(need_ptr(w_o, "w_o"));
  TSP_TRY(need_ptr(kv_gathered, "kv_gathered"));
  TSP_TRY(opt_ptr(residual, "residual"));
  TSP_TRY(need_ptr(out, "out"));
  TSP_TRY(need_ptr(q_keep, "q_keep"));
  TSP_TRY(need_ptr(o_keep, "o_keep"));
  TSP_TRY(need_ptr(lse_keep, "lse_keep"));
  TSP_TRY(need_ptr(ws, "ws"));
  const size_t need = ws_attn_keep(s);
  if (ws_bytes < need) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  TSP_TRY(check_device("tsp_attn_fwd_keep"));
  AttnWs w;
  w.q = q_keep;
  w.o = o_keep;
  w.partial = partial_or_null(s, static_cast<char*>(ws));
  return run_attention(s, x_local, w_qkv, w_o, kv_gathered, nullptr, residual, out, nullptr, w, stream, lse_keep);
}

int tsp_attn_bwd_proj(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv, const float* dq,
                      const float* dkv_own, const float* dx_residual, float* dx, float* dw_qkv, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(make_shape(dims, &s));
  TSP_TRY(need_ptr(x_local, "x_local"));
  TSP_TRY(need_ptr(w_qkv, "w_qkv"));
  TSP_TRY(need_ptr(dq, "dq"));
  TSP_TRY(need_ptr(dkv_own, "dkv_own"));
  TSP_TRY(opt_ptr(dx_residual, "dx_residual"));
  TSP_TRY(need_ptr(dx, "dx"));
  TSP_TRY(need_ptr(dw_qkv, "dw_qkv"));
  TSP_TRY(need_ptr(ws, "ws"));
  if (ws_bytes < ws_attn_bwd_proj(s))
    return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws_attn_bwd_proj(s));
  TSP_TRY(check_device("tsp_attn_bwd_proj"));
  AttnBwdProjWs w;
  ws_attn_bwd_proj(s, &w, static_cast<char*>(ws));
  const int Mp = mpad(s), h = s.h, qs = s.Hq_s * s.dh, kvs = s.Hkv_s * s.dh, n = s.nqkv_s;
  const int64_t nall = (int64_t)s.D * n, own = (int64_t)s.M * kvs;
  // G [M][D][dQ_j | dK_j | dV_j] in bf16
  TSP_LAUNCH(tsp::launch_copy_bf16(tsp::TR_F32, dq, (int64_t)s.Hq * s.dh, qs, w.g16, nall, n, s.M, qs, s.D, stream),
             "attn bwd proj: G (dQ)");
  TSP_LAUNCH(tsp::launch_copy_bf16(tsp::TR_F32, dkv_own, kvs, 2 * own, w.g16 + qs, nall, n, s.M, kvs, s.D, stream),
             "attn bwd proj: G (dK)");
  TSP_LAUNCH(tsp::launch_copy_bf16(tsp::TR_F32, dkv_own + own, kvs, 2 * own, w.g16 + qs + kvs, nall, n, s.M, kvs,
                                   s.D, stream),
             "attn bwd proj: G (dV)");
  TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w.g16, nall, 0, w.gT, Mp, 0, s.M, (int)nall, Mp, 1, stream),
             "attn bwd proj: G^T");
  TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, x_local, h, 0, w.xT, Mp, 0, s.M, h, Mp, 1, stream),
             "attn bwd proj: x^T");
  // dx = dx_resid + G W_QKV: W_QKV read as stored, or through its transposed
  // copy where the workspace holds one
  if (w.wqkvT == nullptr) {
    TSP_LAUNCH(tsp::launch_attn_bwd_dx_kmajor(s, w.g16, w_qkv, dx_residual, dx, w.partial, stream),
               "attn bwd proj: dx");
  } else {
    TSP_LAUNCH(tsp::launch_transpose_bf16(tsp::TR_BF16, w_qkv, h, 0, w.wqkvT, nall, 0, (int)nall, h, (int)nall, 1,
                                          stream),
               "attn bwd proj: W_QKV^T");
    TSP_LAUNCH(tsp::launch_attn_bwd_dx(s, w.g16, w.wqkvT, dx_residual, dx, w.partial, stream), "attn bwd proj: dx");
  }
  TSP_LAUNCH(tsp::launch_attn_bwd_dwqkv(s, Mp, w.gT, w.xT, dw_qkv, stream), "attn bwd proj: dW_QKV");
  return TSP_OK;
}

// Checks of tsp_layer_fwd's arguments other than the workspace.
int check_layer_args(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                     const uint16_t* w_o, const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                     const uint16_t* kv_gathered, const float* y, tsp::Shape* s) {
  TSP_TRY(make_shape(dims, s));
  TSP_TRY(need_ptr(x_local, "x_local"));
  TSP_TRY(need_ptr(w_qkv, "w_qkv"));
  TSP_TRY(need_ptr(w_o, "w_o"));
  TSP_TRY(need_ptr(w_gate, "w_gate"));
  TSP_TRY(need_ptr(w_up, "w_up"));
  TSP_TRY(need_ptr(w_down, "w_down"));
  TSP_TRY(need_ptr(kv_gathered, "kv_gathered"));
  TSP_TRY(need_ptr(y, "y"));
  return TSP_OK;
}

int run_layer(const tsp::Shape& s, const uint16_t* x_local, const uint16_t* w_qkv, const uint16_t* w_o,
              const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down, uint16_t* kv_gathered,
              float* y, void* ws, hipStream_t stream) {
  AttnWs aw;
  MlpWs mw;
  char* p = carve_attn(s, static_cast<char*>(ws), &aw);
  float* h32 = reinterpret_cast<float*>(p);
  p += up(bytes_h32(s));
  p = carve_mlp(s, p, &mw);
  aw.partial = mw.partial = partial_or_null(s, p);
  TSP_TRY(run_attention(s, x_local, w_qkv, w_o, kv_gathered, x_local, nullptr, h32, mw.h16, aw, stream));
  return run_mlp(s, mw.h16, false, h32, w_gate, w_up, w_down, y, mw, stream);
}

int tsp_layer_fwd(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                  const uint16_t* w_o, const uint16_t* w_gate, const uint16_t* w_up,
                  const uint16_t* w_down, uint16_t* kv_gathered, float* y, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(check_layer_args(dims, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv_gathered, y, &s));
  TSP_TRY(need_ptr(ws, "ws"));
  if (ws_bytes < ws_layer(s))
    return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, ws_layer(s));
  TSP_TRY(check_device("tsp_layer_fwd"));
  return run_layer(s, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv_gathered, y, ws, stream);
}

int tsp_layer_fwd_noalloc(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                          const uint16_t* w_o, const uint16_t* w_gate, const uint16_t* w_up,
                          const uint16_t* w_down, uint16_t* kv_gathered, float* y, hipStream_t stream) {
  tsp::Shape s;
  TSP_TRY(check_layer_args(dims, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv_gathered, y, &s));
  if (ws_layer(s) > (size_t)TSP_SCRATCH_BYTES)
    return fail(TSP_ERR_SCRATCH, "layer needs %zu bytes of workspace, more than the %zu-byte scratch array",
                ws_layer(s), (size_t)TSP_SCRATCH_BYTES);
  void* ws = nullptr;
  TSP_TRY(scratch_ptr(&ws));
  return run_layer(s, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv_gathered, y, ws, stream);
}

}  // extern "C"
