// h3q_api.cpp -- the C ABI of libh3q (declared in include/h3q.h): handles, the resident adapter
// registry, argument validation, per-stream workspaces and kernel launch sequencing.
//
// Per call (FL2VA Turbo, "Implementation" and "Hot API"):
//   adapter none, or strength 0   -> [prescale x*pqs] -> GEMM over the K base columns only
//   adapter id                    -> LoRA-down (writes t' and x*pqs) -> GEMM over K + r_pad columns
//   W4A4 (H3Q_ACT_NVFP4)          -> activation NVFP4 quantizer first; LoRA-down still reads raw x
// Selecting or switching an adapter is a host-side map lookup: no device work, and the packed
// weight is never written.
#include "h3q.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "h3q_kernels.hpp"

using namespace h3q;

namespace {

constexpr int64_t kMaxDim = int64_t{1} << 20;
constexpr int64_t kMaxS = int64_t{1} << 24;
constexpr int32_t kMaxRank = 512;

thread_local std::string g_error;

h3q_status fail(h3q_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
h3q_status fail(h3q_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

h3q_status ok() {
  g_error.clear();
  return H3Q_OK;
}

#define H3Q_HIP_TRY(expr)                                                                   \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(H3Q_E_HIP, "%s: %s", #expr, hipGetErrorString(e_));   \
  } while (0)

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- device allocation, with a test hook: while H3Q_TEST_FAIL_ALLOC_AFTER=n is set, the first n
// allocations after the variable took its current value succeed and every later one fails ----
std::mutex g_alloc_mu;
std::string g_alloc_hook;
long g_alloc_count = 0;

hipError_t dev_alloc(void** p, size_t bytes) {
  {
    std::lock_guard<std::mutex> lk(g_alloc_mu);
    const char* hook = std::getenv("H3Q_TEST_FAIL_ALLOC_AFTER");
    if (hook) {
      if (g_alloc_hook != hook) {
        g_alloc_hook = hook;
        g_alloc_count = 0;
      }
      if (g_alloc_count++ >= std::atol(hook)) return hipErrorOutOfMemory;
    } else {
      g_alloc_hook.clear();
    }
  }
  return hipMalloc(p, bytes);
}

// ---- device check (gfx950 only), cached per device ----
h3q_status check_device(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(H3Q_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  static std::mutex mu;
  static std::map<int, bool> cache;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(H3Q_E_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    it = cache.emplace(dev, std::strncmp(prop.gcnArchName, "gfx950", 6) == 0).first;
  }
  if (!it->second) return fail(H3Q_E_UNSUPPORTED, "device %d is not gfx950", dev);
  *dev_out = dev;
  return H3Q_OK;
}

// ---- timing ----
struct TimingRec {
  int kind;
  hipEvent_t begin, end;
};
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<TimingRec> pending;
  std::vector<hipEvent_t> pool;
  double ms[4] = {0, 0, 0, 0};
  int64_t launches[4] = {0, 0, 0, 0};
} g_timing;

hipEvent_t take_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launches `fn` on `stream`, bracketed by events of `kind` when timing is on.
template <class F>
hipError_t timed(int kind, hipStream_t stream, F&& fn) {
  TimingRec rec{kind, nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.on) {
      rec.begin = take_event();
      rec.end = take_event();
    }
  }
  if (rec.begin && rec.end) {
    hipError_t e = hipEventRecord(rec.begin, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t err = fn();
  if (rec.begin && rec.end) {
    hipError_t e = hipEventRecord(rec.end, stream);
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (e == hipSuccess && err == hipSuccess) {
      g_timing.pending.push_back(rec);
    } else {
      g_timing.pool.push_back(rec.begin);
      g_timing.pool.push_back(rec.end);
    }
    if (err == hipSuccess) err = e;
  }
  return err;
}

// ---- per-(device, stream) grow-only workspace ----
// Under stream capture a call bakes the workspace's address into the graph, so a buffer that a
// capture has seen is never freed: when it must grow later, it is retired (kept until the process
// ends) and a new one is allocated. Growing it during a capture is refused (the allocation and the
// synchronization it needs cannot be captured): run the call once outside the capture first, on the
// same stream, with the same or a larger S.
struct Workspace {
  void* buf = nullptr;
  size_t bytes = 0;
  bool captured = false;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<void*> g_ws_retired;

h3q_status workspace(int dev, hipStream_t stream, size_t need, uint8_t** out) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace& ws = g_ws[{dev, stream}];
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  H3Q_HIP_TRY(hipStreamIsCapturing(stream, &cs));
  const bool capturing = cs != hipStreamCaptureStatusNone;
  if (ws.bytes < need) {
    if (capturing)
      return fail(H3Q_E_ARG, "workspace of %zu bytes needed during stream capture (have %zu): make the same call once "
                  "outside the capture on this stream first", need, ws.bytes);
    if (ws.buf) {
      H3Q_HIP_TRY(hipStreamSynchronize(stream));  // in-flight work may still read the old buffer
      if (ws.captured) {
        g_ws_retired.push_back(ws.buf);  // a captured graph may still use it
      } else {
        H3Q_HIP_TRY(hipFree(ws.buf));
      }
      ws.buf = nullptr;
      ws.bytes = 0;
      ws.captured = false;
    }
    const size_t bytes = static_cast<size_t>(round_up(static_cast<int64_t>(need), int64_t{1} << 21));
    if (dev_alloc(&ws.buf, bytes) != hipSuccess) {
      (void)hipGetLastError();
      ws.buf = nullptr;
      return fail(H3Q_E_NOMEM, "workspace allocation of %zu bytes failed", bytes);
    }
    ws.bytes = bytes;
  }
  if (capturing) ws.captured = true;
  // test hook: while H3Q_TEST_POISON_WORKSPACE is set, every call outside a capture first fills the
  // part of the workspace it uses with all-ones bytes (bf16 NaN), so that a kernel reading a part
  // that the call did not write shows up in the output
  if (!capturing && std::getenv("H3Q_TEST_POISON_WORKSPACE")) H3Q_HIP_TRY(hipMemsetAsync(ws.buf, 0xFF, need, stream));
  *out = static_cast<uint8_t*>(ws.buf);
  return H3Q_OK;
}

// ---- the fixed scratch of h3q_linear_ex_noalloc ----
// A file-scope device array: every GPU the library runs on holds its own copy from the time the
// library's code is loaded there until the process ends. In host code `scratch` is only a stand-in
// for the symbol, never a device address: the address is looked up once per device, with that device
// current (when the first weight is packed there, else on the first no-allocation call), and only
// that pointer is handed to kernels.
static_assert(H3Q_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[H3Q_NOALLOC_SCRATCH_BYTES];

h3q_status scratch_on_device(int dev, uint8_t** out) {
  static std::mutex mu;
  static std::map<int, uint8_t*> ptrs;
  std::lock_guard<std::mutex> lk(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(H3Q_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    it = ptrs.emplace(dev, static_cast<uint8_t*>(p)).first;
  }
  *out = it->second;
  return H3Q_OK;
}

}  // namespace

// ---- handles ----
struct Adapter {
  int32_t rank = 0, r_pad = 0;
  float alpha = 0.0f;
  uint16_t* A = nullptr;  // [r_pad][K_pad]
  uint16_t* B = nullptr;  // [n_tiles][r_pad/32][256][32]
};

struct h3q_weight_s {
  int device = -1;
  int64_t N = 0, K = 0, K_pad = 0;
  uint32_t flags = 0;
  float ts = 1.0f;
  int32_t n_tiles = 0, k_tiles = 0;
  uint8_t* codes = nullptr;   // [n_tiles][k_tiles][256][32]
  uint8_t* scales = nullptr;  // [n_tiles][k_tiles][256][4]
  size_t codes_bytes = 0, scales_bytes = 0;
  std::mutex mu;
  std::map<int32_t, Adapter> adapters;
};

namespace {

std::mutex g_handles_mu;
std::unordered_set<h3q_weight> g_handles;

bool live(h3q_weight w) {
  std::lock_guard<std::mutex> lk(g_handles_mu);
  return w && g_handles.count(w) != 0;
}

bool gate_up(const h3q_weight_s* w) { return (w->flags & H3Q_PACK_GATE_UP) != 0; }

void free_adapter(Adapter& a) {
  if (a.A) (void)hipFree(a.A);
  if (a.B) (void)hipFree(a.B);
  a.A = a.B = nullptr;
}

h3q_status copy_to_device(void** dst, const void* src, size_t bytes) {
  if (dev_alloc(dst, bytes) != hipSuccess) {
    (void)hipGetLastError();
    *dst = nullptr;
    return fail(H3Q_E_NOMEM, "device allocation of %zu bytes failed", bytes);
  }
  hipError_t e = hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(*dst);
    *dst = nullptr;
    return fail(H3Q_E_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  }
  return H3Q_OK;
}

}  // namespace

extern "C" {

const char* h3q_last_error(void) { return g_error.c_str(); }

h3q_status h3q_pack_weight(void* stream, const uint8_t* codes, const uint8_t* scales, float tensor_scale,
                           int64_t N, int64_t K, uint32_t flags, h3q_weight* out) {
  if (!codes || !scales || !out) return fail(H3Q_E_ARG, "pack: null pointer");
  if ((flags & ~static_cast<uint32_t>(H3Q_PACK_GATE_UP)) != 0) return fail(H3Q_E_ARG, "pack: unknown flags 0x%x", flags);
  if (N < 1 || N > kMaxDim || K < 16 || K > kMaxDim || K % 16 != 0)
    return fail(H3Q_E_SHAPE, "pack: need 1 <= N, K <= 2^20 and K %% 16 == 0 (N=%lld K=%lld)", (long long)N, (long long)K);
  const bool gu = (flags & H3Q_PACK_GATE_UP) != 0;
  if (gu && N % 2 != 0) return fail(H3Q_E_SHAPE, "pack: gate/up weight needs an even N (N=%lld)", (long long)N);
  if (!std::isfinite(tensor_scale) || !(tensor_scale > 0.0f))
    return fail(H3Q_E_ARG, "pack: tensor_scale must be finite and > 0");
  for (int64_t i = 0; i < N * (K / 16); ++i)
    if ((scales[i] & 0x80u) || scales[i] == 0x7Fu)
      return fail(H3Q_E_FORMAT, "pack: invalid E4M3 scale code 0x%02x at row %lld block %lld", scales[i],
                  (long long)(i / (K / 16)), (long long)(i % (K / 16)));
  int dev;
  if (h3q_status st = check_device(&dev)) return st;
  // set-up of the device for h3q_linear_ex_noalloc: its scratch address is looked up here, outside any
  // stream capture, so that a first no-allocation call under capture makes no runtime query
  uint8_t* scratch_dev = nullptr;
  if (h3q_status st = scratch_on_device(dev, &scratch_dev)) return st;

  auto w = new (std::nothrow) h3q_weight_s();
  if (!w) return fail(H3Q_E_NOMEM, "pack: host allocation failed");
  w->device = dev;
  w->N = N;
  w->K = K;
  w->K_pad = round_up(K, kGemmBK);
  w->flags = flags;
  w->ts = tensor_scale;
  w->k_tiles = static_cast<int32_t>(w->K_pad / kGemmBK);
  w->n_tiles = static_cast<int32_t>(packed_n_tiles(N, gu));

  // tile on the host: byte moves only (layout in h3q_layout.hpp)
  const int64_t tiles = static_cast<int64_t>(w->n_tiles) * w->k_tiles;
  std::vector<uint32_t> tc(static_cast<size_t>(tiles * kCodeChunksPerTile * kGemmBN), 0u);
  std::vector<uint32_t> tsc(static_cast<size_t>(tiles * kGemmBN), 0u);
  tile_weight(codes, scales, N, K, gu, tc.data(), tsc.data());
  w->codes_bytes = tc.size() * 4;
  w->scales_bytes = tsc.size() * 4;
  (void)stream;  // synchronous copies: the caller's buffers are host memory
  h3q_status st = copy_to_device(reinterpret_cast<void**>(&w->codes), tc.data(), w->codes_bytes);
  if (st == H3Q_OK) st = copy_to_device(reinterpret_cast<void**>(&w->scales), tsc.data(), w->scales_bytes);
  if (st != H3Q_OK) {
    if (w->codes) (void)hipFree(w->codes);
    delete w;
    return st;
  }
  {
    std::lock_guard<std::mutex> lk(g_handles_mu);
    g_handles.insert(w);
  }
  *out = w;
  return ok();
}

h3q_status h3q_free_weight(h3q_weight w) {
  {
    std::lock_guard<std::mutex> lk(g_handles_mu);
    if (!w || g_handles.erase(w) == 0) return fail(H3Q_E_ARG, "free: not a live weight handle");
  }
  for (auto& kv : w->adapters) free_adapter(kv.second);
  (void)hipFree(w->codes);
  (void)hipFree(w->scales);
  delete w;
  return ok();
}

h3q_status h3q_weight_info(h3q_weight w, int64_t* N, int64_t* K, uint32_t* flags) {
  if (!live(w)) return fail(H3Q_E_ARG, "weight_info: not a live weight handle");
  if (N) *N = w->N;
  if (K) *K = w->K;
  if (flags) *flags = w->flags;
  return ok();
}

h3q_status h3q_register_adapter(h3q_weight w, int32_t id, const uint16_t* A, const uint16_t* B, int32_t rank,
                                float alpha) {
  if (!live(w)) return fail(H3Q_E_ARG, "register_adapter: not a live weight handle");
  if (!A || !B) return fail(H3Q_E_ARG, "register_adapter: null A or B");
  if (id < 0) return fail(H3Q_E_ADAPTER, "register_adapter: id must be >= 0 (got %d)", id);
  if (rank < 1 || rank > kMaxRank) return fail(H3Q_E_SHAPE, "register_adapter: rank must be in [1, %d] (got %d)", kMaxRank, rank);
  if (!std::isfinite(alpha)) return fail(H3Q_E_ARG, "register_adapter: alpha must be finite");
  std::lock_guard<std::mutex> lk(w->mu);
  if (w->adapters.count(id)) return fail(H3Q_E_ADAPTER, "register_adapter: id %d already registered", id);
  int dev;
  if (h3q_status st = check_device(&dev)) return st;
  if (dev != w->device) return fail(H3Q_E_ARG, "register_adapter: weight lives on device %d, current is %d", w->device, dev);

  Adapter a;
  a.rank = rank;
  a.r_pad = static_cast<int32_t>(round_up(rank, kLoraBK));  // whole 32-deep LoRA K-tiles of the GEMM
  a.alpha = alpha;
  const int64_t K = w->K, Kp = w->K_pad, N = w->N;
  std::vector<uint16_t> Ah(static_cast<size_t>(a.r_pad * Kp), 0);
  std::vector<uint16_t> Bh(static_cast<size_t>(int64_t{w->n_tiles} * a.r_pad * kGemmBN), 0);
  tile_adapter(A, B, rank, a.r_pad, N, K, Kp, gate_up(w), Ah.data(), Bh.data());
  h3q_status st = copy_to_device(reinterpret_cast<void**>(&a.A), Ah.data(), Ah.size() * 2);
  if (st == H3Q_OK) st = copy_to_device(reinterpret_cast<void**>(&a.B), Bh.data(), Bh.size() * 2);
  if (st != H3Q_OK) {
    free_adapter(a);
    return st;
  }
  w->adapters.emplace(id, a);
  return ok();
}

h3q_status h3q_unregister_adapter(h3q_weight w, int32_t id) {
  if (!live(w)) return fail(H3Q_E_ARG, "unregister_adapter: not a live weight handle");
  std::lock_guard<std::mutex> lk(w->mu);
  auto it = w->adapters.find(id);
  if (it == w->adapters.end()) return fail(H3Q_E_ADAPTER, "unregister_adapter: unknown id %d", id);
  free_adapter(it->second);
  w->adapters.erase(it);
  return ok();
}

h3q_status h3q_list_adapters(h3q_weight w, int32_t* ids, int32_t cap, int32_t* count) {
  if (!live(w)) return fail(H3Q_E_ARG, "list_adapters: not a live weight handle");
  if (!count || (cap > 0 && !ids)) return fail(H3Q_E_ARG, "list_adapters: null pointer");
  std::lock_guard<std::mutex> lk(w->mu);
  int32_t i = 0;
  for (auto& kv : w->adapters) {
    if (i < cap) ids[i] = kv.first;
    ++i;
  }
  *count = i;
  return ok();
}

namespace {

// Arguments of the Q/K RMSNorm + rotary epilogue (h3q_linear_qk_norm_rope).
struct QkArgs {
  int64_t q_width;
  int32_t rot_dim;
  float eps;
  const float *gamma_q, *gamma_k, *cos, *sin;
  int32_t nsec;      // sections of the rotated dims (validated: 1..4, even, summing to rot_dim)
  int32_t sec[4];
};

// Producer fusion: the SwiGLU epilogue also writes the next projection's base operand
// (h3q_linear_swiglu_emit), or the call takes that operand ready-made (h3q_linear_prescaled).
struct FuseArgs {
  const float* emit_pqs;   // SwiGLU only: pqs of the next projection, fp32 [N/2]
  uint16_t* emit_out;      // SwiGLU only: bf16 [S][N/2]
  const uint16_t* xs;      // the base operand bf16 [S][K] given by the caller (x is then the LoRA input only)
};

h3q_status linear_impl(void* stream_, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                       int32_t adapter_id, float strength, uint32_t flags, uint16_t* out, const QkArgs* qk,
                       const FuseArgs* fuse = nullptr, bool noalloc = false) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!live(w)) return fail(H3Q_E_ARG, "linear: not a live weight handle");
  if (S != 0 && (!x || !out)) return fail(H3Q_E_ARG, "linear: null x or output");
  if ((flags & ~static_cast<uint32_t>(H3Q_ACT_NVFP4 | H3Q_EPI_SWIGLU)) != 0)
    return fail(H3Q_E_ARG, "linear: unknown flags 0x%x", flags);
  if (S < 0 || S > kMaxS) return fail(H3Q_E_SHAPE, "linear: S must be in [0, 2^24] (got %lld)", (long long)S);
  if (!std::isfinite(strength)) return fail(H3Q_E_ARG, "linear: strength must be finite");
  const bool swiglu = (flags & H3Q_EPI_SWIGLU) != 0;
  const bool w4a4 = (flags & H3Q_ACT_NVFP4) != 0;
  if (swiglu && !gate_up(w)) return fail(H3Q_E_ARG, "linear: SwiGLU output needs a weight packed with H3Q_PACK_GATE_UP");
  if (!aligned16(x) || (pqs && !aligned16(pqs)))
    return fail(H3Q_E_ARG, "linear: x and pqs must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(out) & 1u) != 0) return fail(H3Q_E_ARG, "linear: output must be 2-byte aligned");
  const int64_t n_out = swiglu ? w->N / 2 : w->N;
  {
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x), xe = xb + static_cast<uintptr_t>(S * w->K * 2);
    const uintptr_t ob = reinterpret_cast<uintptr_t>(out), oe = ob + static_cast<uintptr_t>(S * n_out * 2);
    if (S > 0 && xb < oe && ob < xe) return fail(H3Q_E_ARG, "linear: output overlaps x");
  }

  std::unique_lock<std::mutex> lk(w->mu);
  const Adapter* ad = nullptr;
  if (adapter_id != H3Q_ADAPTER_NONE) {
    auto it = w->adapters.find(adapter_id);
    if (it == w->adapters.end()) return fail(H3Q_E_ADAPTER, "linear: unknown adapter id %d", adapter_id);
    ad = &it->second;
  }
  const bool lora = ad != nullptr && strength != 0.0f;
  float f = 0.0f;
  if (lora) {
    const double fd = static_cast<double>(strength) * ad->alpha / (static_cast<double>(ad->rank) * w->ts);
    f = static_cast<float>(fd);
    if (!std::isfinite(f)) return fail(H3Q_E_ARG, "linear: strength*alpha/(rank*tensor_scale) overflows fp32");
  }
  if (S == 0) return ok();

  int dev = -1;
  H3Q_HIP_TRY(hipGetDevice(&dev));
  if (dev != w->device) return fail(H3Q_E_ARG, "linear: weight lives on device %d, current is %d", w->device, dev);

  // workspace: [amax/ts_a : 256 B][act operand: S x K_pad bf16][t': S x r_pad bf16]
  const bool given_xs = fuse && fuse->xs;                   // the caller's xs is the GEMM operand
  const bool direct_x = given_xs || (!w4a4 && !pqs && w->K == w->K_pad);  // no operand pass
  const size_t small = 256;
  const size_t act_bytes = direct_x ? 0 : static_cast<size_t>(round_up(S * w->K_pad * 2, 256));
  const size_t t_bytes = lora ? static_cast<size_t>(round_up(S * ad->r_pad * 2, 256)) : 0;
  uint8_t* ws = nullptr;
  if (noalloc) {  // the fixed scratch: no allocation, no synchronization
    const size_t need = small + act_bytes + t_bytes;
    if (need > H3Q_NOALLOC_SCRATCH_BYTES)
      return fail(H3Q_E_SHAPE, "linear_ex_noalloc: the call needs %zu bytes of scratch (S=%lld, K_pad=%lld, r_pad=%d); "
                  "the fixed scratch holds %zu", need, (long long)S, (long long)w->K_pad, lora ? ad->r_pad : 0,
                  static_cast<size_t>(H3Q_NOALLOC_SCRATCH_BYTES));
    if (h3q_status st = scratch_on_device(dev, &ws)) return st;
  } else if (h3q_status st = workspace(dev, stream, small + act_bytes + t_bytes, &ws)) {
    return st;
  }
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(ws);
  float* ts_a = reinterpret_cast<float*>(ws + 4);
  uint16_t* act = given_xs ? const_cast<uint16_t*>(fuse->xs)
                           : direct_x ? const_cast<uint16_t*>(x) : reinterpret_cast<uint16_t*>(ws + small);
  uint16_t* tbuf = lora ? reinterpret_cast<uint16_t*>(ws + small + act_bytes) : nullptr;

  hipError_t e = hipSuccess;
  if (w4a4) {
    ActQuantParams q{x, pqs, S, w->K, amax_bits, ts_a, nullptr, nullptr, act, w->K_pad};
    e = timed(H3Q_KERNEL_ACT_QUANT, stream, [&] { return launch_act_quant(q, stream); });
    if (e != hipSuccess) return fail(H3Q_E_HIP, "act-quant launch: %s", hipGetErrorString(e));
  }
  if (lora) {
    LoraDownParams lp{x, pqs, ad->A, S, w->K, w->K_pad, ad->r_pad, f, w4a4 ? ts_a : nullptr, tbuf,
                      (w4a4 || direct_x) ? nullptr : act};
    e = timed(H3Q_KERNEL_LORA_DOWN, stream, [&] { return launch_lora_down(lp, stream); });
    if (e != hipSuccess) return fail(H3Q_E_HIP, "lora-down launch: %s", hipGetErrorString(e));
  } else if (!w4a4 && !direct_x) {
    PrescaleParams pp{x, pqs, S, w->K, w->K_pad, act};
    e = timed(H3Q_KERNEL_PRESCALE, stream, [&] { return launch_prescale(pp, stream); });
    if (e != hipSuccess) return fail(H3Q_E_HIP, "prescale launch: %s", hipGetErrorString(e));
  }
  GemmParams g{};
  g.act = act;
  g.act_ld = direct_x ? w->K : w->K_pad;
  g.lora_t = tbuf;
  g.lora_t_ld = lora ? ad->r_pad : 0;
  g.wcodes = w->codes;
  g.wscales = w->scales;
  g.lora_b = lora ? ad->B : nullptr;
  g.S = S;
  g.k_tiles = w->k_tiles;
  g.r_tiles = lora ? ad->r_pad / kLoraBK : 0;
  g.m_tiles = static_cast<int32_t>((S + kGemmBM - 1) / kGemmBM);
  g.n_tiles = w->n_tiles;
  g.n_out = n_out;
  g.gate_up = gate_up(w) ? 1 : 0;
  g.ts = w->ts;
  g.ts_dev = w4a4 ? ts_a : nullptr;
  g.out = out;
  g.out_ld = n_out;
  if (fuse && fuse->emit_out) {
    g.emit_pqs = fuse->emit_pqs;
    g.emit_out = fuse->emit_out;
    g.emit_ld = n_out;
  }
  Epilogue epi = swiglu ? Epilogue::SwiGLU : Epilogue::Plain;
  if (qk) {
    g.qk_gamma_q = qk->gamma_q;
    g.qk_gamma_k = qk->gamma_k;
    g.rope_cos = qk->cos;
    g.rope_sin = qk->sin;
    g.q_tiles = static_cast<int32_t>(qk->q_width / kGemmBN);
    g.rope_half = qk->rot_dim / 2;
    g.qk_eps = qk->eps;
    g.rope_nsec = qk->nsec;
    g.rope_vec = 1;
    for (int j = 0, o = 0, col = 0; j < qk->nsec; ++j) {
      g.rope_sec[j] = qk->sec[j];
      const int h = qk->sec[j] / 2;
      if (h % 8 != 0) g.rope_vec = 0;
      for (int i = 0; i + 8 <= h && col < 64; i += 8, col += 8) {  // pair groups of 8 table columns
        g.rope_lo[col / 8] = o + i;
        g.rope_hi[col / 8] = o + i + h;
      }
      o += qk->sec[j];
    }
    epi = Epilogue::QkNormRope;
  }
  e = timed(H3Q_KERNEL_GEMM, stream, [&] { return launch_gemm_w4(g, epi, stream); });
  if (e != hipSuccess) return fail(H3Q_E_HIP, "gemm launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

h3q_status h3q_linear_ex(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                         int32_t adapter_id, float strength, uint32_t flags, uint16_t* out) {
  return linear_impl(stream, x, S, pqs, w, adapter_id, strength, flags, out, nullptr);
}

h3q_status h3q_linear_ex_noalloc(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                                 int32_t adapter_id, float strength, uint32_t flags, uint16_t* out) {
  return linear_impl(stream, x, S, pqs, w, adapter_id, strength, flags, out, nullptr, nullptr, true);
}

h3q_status h3q_linear_qk_norm_rope(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                                   int32_t adapter_id, float strength, uint32_t flags, int64_t q_width,
                                   int32_t rot_dim, float eps, const float* gamma_q, const float* gamma_k,
                                   const float* rope_cos, const float* rope_sin, uint16_t* y) {
  return h3q_linear_qk_norm_rope_sections(stream, x, S, pqs, w, adapter_id, strength, flags, q_width, rot_dim,
                                          &rot_dim, rot_dim > 0 ? 1 : 0, eps, gamma_q, gamma_k, rope_cos, rope_sin,
                                          y);
}

h3q_status h3q_linear_qk_norm_rope_sections(void* stream, const uint16_t* x, int64_t S, const float* pqs,
                                            h3q_weight w, int32_t adapter_id, float strength, uint32_t flags,
                                            int64_t q_width, int32_t rot_dim, const int32_t* sections,
                                            int32_t n_sections, float eps, const float* gamma_q,
                                            const float* gamma_k, const float* rope_cos, const float* rope_sin,
                                            uint16_t* y) {
  if (!live(w)) return fail(H3Q_E_ARG, "qk_norm_rope: not a live weight handle");
  if ((flags & ~static_cast<uint32_t>(H3Q_ACT_NVFP4)) != 0)
    return fail(H3Q_E_ARG, "qk_norm_rope: only H3Q_ACT_NVFP4 may be set (got flags 0x%x)", flags);
  if (gate_up(w)) return fail(H3Q_E_ARG, "qk_norm_rope: the weight is packed as gate/up");
  if (q_width <= 0 || q_width % kGemmBN != 0 || 2 * q_width > w->N || w->N % 8 != 0)
    return fail(H3Q_E_SHAPE, "qk_norm_rope: need q_width a positive multiple of %d, 2*q_width <= N, N %% 8 == 0",
                kGemmBN);
  if (rot_dim < 0 || rot_dim > 128 || rot_dim % 2 != 0)
    return fail(H3Q_E_SHAPE, "qk_norm_rope: rot_dim must be even and in [0, 128] (got %d)", rot_dim);
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(H3Q_E_ARG, "qk_norm_rope: eps must be finite and > 0");
  if (!gamma_q || !gamma_k || (rot_dim > 0 && (!rope_cos || !rope_sin)))
    return fail(H3Q_E_ARG, "qk_norm_rope: null gamma or angle table");
  if (S != 0 && !aligned16(y)) return fail(H3Q_E_ARG, "qk_norm_rope: y must be 16-byte aligned");
  QkArgs qk{q_width, rot_dim, eps, gamma_q, gamma_k, rope_cos, rope_sin, 0, {0, 0, 0, 0}};
  if (rot_dim > 0) {
    if (!sections || n_sections < 1 || n_sections > 4)
      return fail(H3Q_E_SHAPE, "qk_norm_rope: need 1 to 4 rotary sections (got %d)", n_sections);
    int32_t sum = 0;
    for (int32_t j = 0; j < n_sections; ++j) {
      if (sections[j] <= 0 || sections[j] % 2 != 0)
        return fail(H3Q_E_SHAPE, "qk_norm_rope: rotary section %d has width %d (must be even and > 0)", j, sections[j]);
      sum += sections[j];
      qk.sec[j] = sections[j];
    }
    if (sum != rot_dim) return fail(H3Q_E_SHAPE, "qk_norm_rope: rotary sections sum to %d, rot_dim is %d", sum, rot_dim);
    qk.nsec = n_sections;
  }
  return linear_impl(stream, x, S, pqs, w, adapter_id, strength, flags, y, &qk);
}

h3q_status h3q_linear_swiglu_emit(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                                  int32_t adapter_id, float strength, uint32_t flags, uint16_t* h,
                                  const float* pqs_next, uint16_t* xs_next) {
  if (!live(w)) return fail(H3Q_E_ARG, "swiglu_emit: not a live weight handle");
  if ((flags & ~static_cast<uint32_t>(H3Q_ACT_NVFP4)) != 0)
    return fail(H3Q_E_ARG, "swiglu_emit: only H3Q_ACT_NVFP4 may be set (got flags 0x%x)", flags);
  if (!gate_up(w)) return fail(H3Q_E_ARG, "swiglu_emit: needs a weight packed with H3Q_PACK_GATE_UP");
  const int64_t F = w->N / 2;
  if (F % 8 != 0) return fail(H3Q_E_SHAPE, "swiglu_emit: N/2 must be a multiple of 8 (N=%lld)", (long long)w->N);
  if (!pqs_next || !xs_next) return fail(H3Q_E_ARG, "swiglu_emit: null pqs_next or xs_next");
  if (S != 0 && (!aligned16(h) || !aligned16(xs_next) || !aligned16(pqs_next)))
    return fail(H3Q_E_ARG, "swiglu_emit: h, xs_next and pqs_next must be 16-byte aligned");
  {
    const uintptr_t hb = reinterpret_cast<uintptr_t>(h), he = hb + static_cast<uintptr_t>(S * F * 2);
    const uintptr_t sb = reinterpret_cast<uintptr_t>(xs_next), se = sb + static_cast<uintptr_t>(S * F * 2);
    if (S > 0 && hb < se && sb < he) return fail(H3Q_E_ARG, "swiglu_emit: xs_next overlaps h");
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x), xe = xb + static_cast<uintptr_t>(S * w->K * 2);
    if (S > 0 && xb < se && sb < xe) return fail(H3Q_E_ARG, "swiglu_emit: xs_next overlaps x");
  }
  const FuseArgs fa{pqs_next, xs_next, nullptr};
  return linear_impl(stream, x, S, pqs, w, adapter_id, strength, flags | H3Q_EPI_SWIGLU, h, nullptr, &fa);
}

h3q_status h3q_linear_prescaled(void* stream, const uint16_t* x, const uint16_t* xs, int64_t S, h3q_weight w,
                                int32_t adapter_id, float strength, uint16_t* y) {
  if (!live(w)) return fail(H3Q_E_ARG, "linear_prescaled: not a live weight handle");
  if (w->K % kGemmBK != 0)
    return fail(H3Q_E_SHAPE, "linear_prescaled: K must be a multiple of %d (K=%lld)", kGemmBK, (long long)w->K);
  if (S != 0 && (!xs || !aligned16(xs))) return fail(H3Q_E_ARG, "linear_prescaled: xs must be non-null and 16-byte aligned");
  {
    const uintptr_t xb = reinterpret_cast<uintptr_t>(xs), xe = xb + static_cast<uintptr_t>(S * w->K * 2);
    const uintptr_t ob = reinterpret_cast<uintptr_t>(y), oe = ob + static_cast<uintptr_t>(S * w->N * 2);
    if (S > 0 && xb < oe && ob < xe) return fail(H3Q_E_ARG, "linear_prescaled: output overlaps xs");
  }
  const FuseArgs fa{nullptr, nullptr, xs};
  return linear_impl(stream, x, S, nullptr, w, adapter_id, strength, 0u, y, nullptr, &fa);
}

h3q_status h3q_linear(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                      int32_t adapter_id, float strength, uint16_t* y) {
  return h3q_linear_ex(stream, x, S, pqs, w, adapter_id, strength, 0u, y);
}

h3q_status h3q_linear_swiglu(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                             int32_t adapter_id, float strength, uint16_t* h) {
  return h3q_linear_ex(stream, x, S, pqs, w, adapter_id, strength, H3Q_EPI_SWIGLU, h);
}

h3q_status h3q_debug_quantize_act(void* stream_, const uint16_t* x, int64_t S, int64_t K, const float* pqs,
                                  uint8_t* codes, uint8_t* scales, float* ts) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!x || !codes || !scales || !ts) return fail(H3Q_E_ARG, "quantize_act: null pointer");
  if (S < 0 || S > kMaxS || K < 16 || K > kMaxDim || K % 16 != 0)
    return fail(H3Q_E_SHAPE, "quantize_act: need 0 <= S <= 2^24, 16 <= K <= 2^20, K %% 16 == 0");
  if (!aligned16(x) || (pqs && !aligned16(pqs)) || (reinterpret_cast<uintptr_t>(codes) & 7u))
    return fail(H3Q_E_ARG, "quantize_act: x, pqs must be 16-byte and codes 8-byte aligned");
  int dev;
  if (h3q_status st = check_device(&dev)) return st;
  uint8_t* ws = nullptr;
  if (h3q_status st = workspace(dev, stream, 256, &ws)) return st;
  ActQuantParams q{x, pqs, S, K, reinterpret_cast<uint32_t*>(ws), ts, codes, scales, nullptr, K};
  hipError_t e = timed(H3Q_KERNEL_ACT_QUANT, stream, [&] { return launch_act_quant(q, stream); });
  if (e != hipSuccess) return fail(H3Q_E_HIP, "act-quant launch: %s", hipGetErrorString(e));
  return ok();
}

h3q_status h3q_quantize_nvfp4(void* stream, const uint16_t* x, int64_t S, int64_t K, const float* pqs,
                              uint8_t* codes, uint8_t* scales, float* ts) {
  return h3q_debug_quantize_act(stream, x, S, K, pqs, codes, scales, ts);
}

h3q_status h3q_debug_dequant(void* stream, h3q_weight w, uint16_t* wq) {
  if (!live(w)) return fail(H3Q_E_ARG, "debug_dequant: not a live weight handle");
  if (!wq || !aligned16(wq)) return fail(H3Q_E_ARG, "debug_dequant: output must be non-null and 16-byte aligned");
  DequantParams p{reinterpret_cast<const uint32_t*>(w->codes), reinterpret_cast<const uint32_t*>(w->scales),
                  w->n_tiles, w->k_tiles, gate_up(w), w->N, w->K, wq};
  hipError_t e = launch_debug_dequant(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(H3Q_E_HIP, "debug_dequant launch: %s", hipGetErrorString(e));
  return ok();
}

h3q_status h3q_merge_adapter(void* stream_, h3q_weight w, int32_t adapter_id, float strength, const float* pqs,
                             uint8_t* codes, uint8_t* scales, float* ts, float* merged) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!live(w)) return fail(H3Q_E_ARG, "merge_adapter: not a live weight handle");
  if (!codes || !scales || !ts) return fail(H3Q_E_ARG, "merge_adapter: null output");
  if ((reinterpret_cast<uintptr_t>(codes) & 7u) || (merged && !aligned16(merged)) || (pqs && !aligned16(pqs)))
    return fail(H3Q_E_ARG, "merge_adapter: codes must be 8-byte, pqs and merged 16-byte aligned");
  if (!std::isfinite(strength)) return fail(H3Q_E_ARG, "merge_adapter: strength must be finite");
  int dev;
  if (h3q_status st = check_device(&dev)) return st;
  if (dev != w->device) return fail(H3Q_E_ARG, "merge_adapter: weight lives on device %d, current is %d", w->device, dev);
  // the weight's lock is held until the merge has finished on the device, so that the adapter's
  // buffers cannot be unregistered (freed) while its kernels read them
  std::lock_guard<std::mutex> lk(w->mu);
  Adapter ad;
  if (adapter_id != H3Q_ADAPTER_NONE) {
    auto it = w->adapters.find(adapter_id);
    if (it == w->adapters.end()) return fail(H3Q_E_ADAPTER, "merge_adapter: unknown adapter id %d", adapter_id);
    ad = it->second;  // device buffers stay owned by the handle
  }
  const bool lora = ad.rank > 0 && strength != 0.0f;
  const int64_t N = w->N, K = w->K;
  const size_t wq_bytes = static_cast<size_t>(N * K * 2);
  const size_t m_bytes = merged ? 0 : static_cast<size_t>(N * K * 4);
  void* tmp = nullptr;
  if (dev_alloc(&tmp, 256 + wq_bytes + m_bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(H3Q_E_NOMEM, "merge_adapter: temporary allocation of %zu bytes failed", 256 + wq_bytes + m_bytes);
  }
  uint8_t* t8 = static_cast<uint8_t*>(tmp);
  uint16_t* wq = reinterpret_cast<uint16_t*>(t8 + 256);
  float* m = merged ? merged : reinterpret_cast<float*>(t8 + 256 + wq_bytes);
  DequantParams dq{reinterpret_cast<const uint32_t*>(w->codes), reinterpret_cast<const uint32_t*>(w->scales),
                   w->n_tiles, w->k_tiles, gate_up(w), N, K, wq};
  MergeParams mp{wq, ad.A, ad.B, pqs, m, static_cast<double>(w->ts),
                 lora ? static_cast<double>(strength) * ad.alpha / static_cast<double>(ad.rank) : 0.0,
                 N, K, w->K_pad, w->n_tiles, lora ? ad.r_pad : 0, gate_up(w)};
  ActQuantParams q{nullptr, nullptr, N, K, reinterpret_cast<uint32_t*>(t8), ts, codes, scales, nullptr, K, m};
  hipError_t e = launch_debug_dequant(dq, stream);
  if (e == hipSuccess) e = launch_lora_merge(mp, stream);
  if (e == hipSuccess) e = launch_act_quant(q, stream);
  const hipError_t es = hipStreamSynchronize(stream);  // the temporaries are freed below
  (void)hipFree(tmp);
  if (e != hipSuccess) return fail(H3Q_E_HIP, "merge_adapter launch: %s", hipGetErrorString(e));
  if (es != hipSuccess) return fail(H3Q_E_HIP, "merge_adapter: %s", hipGetErrorString(es));
  return ok();
}

h3q_status h3q_adaln_table(void* stream, const float* u, const float* emb, const uint16_t* A, float scale,
                           int32_t blocks, int32_t samples, int32_t emb_dim, int32_t base_rank, int32_t lora_rank,
                           float* table) {
  if (!u || !emb || !table || (lora_rank > 0 && !A)) return fail(H3Q_E_ARG, "adaln_table: null pointer");
  if (blocks < 1 || blocks > 65535 || samples < 2 || samples > 65535 * 16 || emb_dim < 1 || base_rank < 1 || base_rank > 64 ||
      lora_rank < 0 || lora_rank > 32 || base_rank + lora_rank > 64 || static_cast<int64_t>(samples) * emb_dim > (int64_t{1} << 31))
    return fail(H3Q_E_SHAPE, "adaln_table: need 1 <= blocks <= 65535, 2 <= samples <= 1048560, emb_dim >= 1, 1 <= base_rank, "
                "0 <= lora_rank <= 32, base_rank + lora_rank <= 64");
  if (!std::isfinite(scale)) return fail(H3Q_E_ARG, "adaln_table: scale must be finite");
  int dev;
  if (h3q_status st = check_device(&dev)) return st;
  AdalnTableParams p{u, emb, A, scale, blocks, samples, emb_dim, base_rank, lora_rank, table};
  hipError_t e = launch_adaln_table(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(H3Q_E_HIP, "adaln_table launch: %s", hipGetErrorString(e));
  return ok();
}

h3q_status h3q_adaln_apply(void* stream, const uint16_t* M, const float* bias, const float* table, const float* t,
                           int32_t T, int32_t blocks, int64_t rows, int32_t samples, int32_t R, float* out) {
  if (!M || !table || !t || !out) return fail(H3Q_E_ARG, "adaln_apply: null pointer");
  if (T < 1 || T > 8 || blocks < 1 || blocks > 65535 || rows < 0 || rows > (int64_t{1} << 24) || samples < 2 || R < 8 || R > 64 || R % 8 != 0)
    return fail(H3Q_E_SHAPE, "adaln_apply: need 1 <= T <= 8, blocks >= 1, 0 <= rows <= 2^24, samples >= 2, "
                "R a multiple of 8 in [8, 64]");
  if (!aligned16(M)) return fail(H3Q_E_ARG, "adaln_apply: M must be 16-byte aligned");
  int dev;
  if (h3q_status st = check_device(&dev)) return st;
  AdalnApplyParams p{M, bias, table, t, T, blocks, samples, R, rows, out};
  hipError_t e = launch_adaln_apply(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(H3Q_E_HIP, "adaln_apply launch: %s", hipGetErrorString(e));
  return ok();
}

h3q_status h3q_mfma_loop(void* stream, const uint16_t* ops_a, const uint16_t* ops_b, int32_t iters,
                         int32_t workgroups, float* sink) {
  if (!ops_a || !ops_b || !sink) return fail(H3Q_E_ARG, "mfma_loop: null pointer");
  if (!aligned16(ops_a) || !aligned16(ops_b)) return fail(H3Q_E_ARG, "mfma_loop: operands must be 16-byte aligned");
  if (iters < 1 || workgroups < 1 || workgroups > (1 << 20)) return fail(H3Q_E_ARG, "mfma_loop: bad iters or workgroups");
  int dev;
  if (h3q_status st = check_device(&dev)) return st;
  hipError_t e = launch_mfma_loop(ops_a, ops_b, iters, workgroups, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(H3Q_E_HIP, "mfma_loop launch: %s", hipGetErrorString(e));
  return ok();
}

h3q_status h3q_weight_checksum(void* stream, h3q_weight w, uint64_t* out) {
  if (!live(w)) return fail(H3Q_E_ARG, "weight_checksum: not a live weight handle");
  if (!out) return fail(H3Q_E_ARG, "weight_checksum: null output");
  H3Q_HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  std::vector<uint8_t> host(w->codes_bytes + w->scales_bytes);
  H3Q_HIP_TRY(hipMemcpy(host.data(), w->codes, w->codes_bytes, hipMemcpyDeviceToHost));
  H3Q_HIP_TRY(hipMemcpy(host.data() + w->codes_bytes, w->scales, w->scales_bytes, hipMemcpyDeviceToHost));
  uint64_t h = 1469598103934665603ull;  // FNV-1a 64
  for (uint8_t b : host) {
    h ^= b;
    h *= 1099511628211ull;
  }
  *out = h;
  return ok();
}

h3q_status h3q_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  for (auto& r : g_timing.pending) {
    (void)hipEventSynchronize(r.end);
    g_timing.pool.push_back(r.begin);
    g_timing.pool.push_back(r.end);
  }
  g_timing.pending.clear();
  for (int k = 0; k < 4; ++k) {
    g_timing.ms[k] = 0.0;
    g_timing.launches[k] = 0;
  }
  return ok();
}

h3q_status h3q_timing_get(int32_t kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind > 3 || !total_ms || !launches) return fail(H3Q_E_ARG, "timing_get: bad kind or null pointer");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  // records leave the pending list as they are counted, so a failure part-way counts none twice
  while (!g_timing.pending.empty()) {
    const TimingRec r = g_timing.pending.back();
    float ms = 0.0f;
    H3Q_HIP_TRY(hipEventSynchronize(r.end));
    H3Q_HIP_TRY(hipEventElapsedTime(&ms, r.begin, r.end));
    g_timing.pending.pop_back();
    g_timing.ms[r.kind] += ms;
    g_timing.launches[r.kind] += 1;
    g_timing.pool.push_back(r.begin);
    g_timing.pool.push_back(r.end);
  }
  *total_ms = g_timing.ms[kind];
  *launches = g_timing.launches[kind];
  g_timing.ms[kind] = 0.0;
  g_timing.launches[kind] = 0;
  return ok();
}

}  // extern "C"
