// C ABI of libfp4rl: argument validation, device check, dispatch.
// Declarations, semantics and error behaviour are documented in include/fp4rl.h.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "fp4rl.h"
#include "backward.hpp"
#include "fp8.hpp"
#include "gate_up.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

fp4rl_status fail(fp4rl_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

fp4rl_status ok() {
  g_err[0] = '\0';
  return FP4RL_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // kernels index rows and columns with int

// Test hooks of the fused LoRA hand-off (fp4rl_debug_lora_handoff): the
// consumers' poll limit and whether producers leave the ready flags down.
std::atomic<uint32_t> g_lora_spin{fp4rl::LoraFuse{}.spin};
std::atomic<uint32_t> g_lora_withhold{0u};
// Ready value of the next fused call's LoRA hand-off: unique per call in the
// process (any workspace, device or thread), never 0 (the value of a cleared
// workspace), so a flag raised late by an earlier call never matches.
static std::atomic<uint32_t> g_lora_epoch{0};
static uint32_t next_lora_epoch() {
  uint32_t e = g_lora_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  while (e == 0) e = g_lora_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  return e;
}
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other arch

fp4rl_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FP4RL_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FP4RL_ERR_HIP, "device ordinal %d out of range", dev);
  int s = g_dev_state[dev].load(std::memory_order_acquire);
  if (s == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(FP4RL_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    s = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_state[dev].store(s, std::memory_order_release);
    if (s == 2) return fail(FP4RL_ERR_ARCH, "device %d is %s, not gfx950", dev, p.gcnArchName);
  }
  if (s != 1) return fail(FP4RL_ERR_ARCH, "device %d is not gfx950", dev);
  return FP4RL_OK;
}

// Scratch of fp4rl_nvfp4_quantize_noalloc: the amax pass's per-workgroup
// partial maxima (kAmaxPartials words). Each GPU the library runs on holds
// its own copy until the process ends; every call on one GPU shares it, so
// calls that overlap on one GPU race. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in): the device address
// of each GPU's copy is looked up once, on that GPU's first call, and kept.
static __device__ __align__(256) uint32_t scratch[fp4rl::kAmaxPartials];
constexpr size_t kScratchBytes = sizeof(uint32_t) * fp4rl::kAmaxPartials;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

fp4rl_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FP4RL_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FP4RL_ERR_HIP, "device ordinal %d out of range", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with this device current
      if (e != hipSuccess || p == nullptr)
        return fail(FP4RL_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP4RL_OK;
}

fp4rl_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP4RL_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

#define FP4RL_REQUIRE(cond, status, ...) \
  do {                                   \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define FP4RL_CHECK(expr)              \
  do {                                 \
    fp4rl_status s_ = (expr);          \
    if (s_ != FP4RL_OK) return s_;     \
  } while (0)

fp4rl_status check_linear_shape(int64_t m, int64_t n, int64_t k, int64_t r) {
  FP4RL_REQUIRE(m >= 0 && n >= 0 && k >= 0 && r >= 0, FP4RL_ERR_SHAPE,
                "negative size (m=%lld n=%lld k=%lld r=%lld)", (long long)m, (long long)n, (long long)k, (long long)r);
  FP4RL_REQUIRE(k > 0 && k % 16 == 0, FP4RL_ERR_SHAPE, "k=%lld must be a positive multiple of 16", (long long)k);
  FP4RL_REQUIRE(m < kMaxDim && n < kMaxDim && k < kMaxDim, FP4RL_ERR_SHAPE, "dimension >= 2^31");
  // the kernels address activations with 32-bit byte offsets
  FP4RL_REQUIRE(m * k < ((int64_t)1 << 31), FP4RL_ERR_SHAPE, "m * k = %lld must be below 2^31", (long long)(m * k));
  // the skinny, split-K and mid-batch kernels (3..128 tokens) address x with
  // 32-bit byte offsets whose top bit marks a piece past K (a buffer load
  // that reads zero), and the prefill kernel (> 128) from a 128-token group
  FP4RL_REQUIRE(m <= 2 || m > 128 || m * k < ((int64_t)1 << 30), FP4RL_ERR_SHAPE,
                "m * k = %lld must be below 2^30 for 3 <= m <= 128", (long long)(m * k));
  FP4RL_REQUIRE(m <= 128 || k < ((int64_t)1 << 23), FP4RL_ERR_SHAPE, "k = %lld must be below 2^23 for m > 128",
                (long long)k);
  FP4RL_REQUIRE(r <= fp4rl::kMaxRank, FP4RL_ERR_SHAPE, "rank r=%lld exceeds %lld", (long long)r,
                (long long)fp4rl::kMaxRank);
  return FP4RL_OK;
}

}  // namespace

extern "C" {

const char* fp4rl_status_string(int32_t status) {
  switch (status) {
    case FP4RL_OK: return "FP4RL_OK";
    case FP4RL_ERR_NULL: return "FP4RL_ERR_NULL";
    case FP4RL_ERR_SHAPE: return "FP4RL_ERR_SHAPE";
    case FP4RL_ERR_DTYPE: return "FP4RL_ERR_DTYPE";
    case FP4RL_ERR_ALIGN: return "FP4RL_ERR_ALIGN";
    case FP4RL_ERR_WORKSPACE: return "FP4RL_ERR_WORKSPACE";
    case FP4RL_ERR_ARCH: return "FP4RL_ERR_ARCH";
    case FP4RL_ERR_HIP: return "FP4RL_ERR_HIP";
    case FP4RL_ERR_VALUE: return "FP4RL_ERR_VALUE";
    case FP4RL_ERR_TIMEOUT: return "FP4RL_ERR_TIMEOUT";
    default: return "FP4RL_UNKNOWN_STATUS";
  }
}

const char* fp4rl_last_error(void) { return g_err; }

int32_t fp4rl_abi_version(void) { return FP4RL_ABI_VERSION; }

// ---------------------------------------------------------------- quantise --

size_t fp4rl_nvfp4_quantize_workspace(int64_t n, int64_t k) {
  (void)n;
  (void)k;
  return fp4rl::quantize_workspace_bytes();
}

size_t fp4rl_nvfp4_codes_bytes(int64_t n, int64_t k, int32_t layout) {
  if (n < 0 || k < 0 || k % 16 || (layout != FP4RL_ROW_MAJOR && layout != FP4RL_TILED)) return 0;
  return (size_t)fp4rl::nvfp4_codes_bytes(n, k, layout == FP4RL_TILED);
}

size_t fp4rl_nvfp4_scales_bytes(int64_t n, int64_t k, int32_t layout) {
  if (n < 0 || k < 0 || k % 16 || (layout != FP4RL_ROW_MAJOR && layout != FP4RL_TILED)) return 0;
  return (size_t)fp4rl::nvfp4_scales_bytes(n, k, layout == FP4RL_TILED);
}

static fp4rl_status check_quantize_args(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                        const uint8_t* codes, const uint8_t* scales, const float* tensor_scale) {
  FP4RL_REQUIRE(n >= 0 && k >= 0, FP4RL_ERR_SHAPE, "negative size (n=%lld k=%lld)", (long long)n, (long long)k);
  FP4RL_REQUIRE(k % 16 == 0, FP4RL_ERR_SHAPE, "k=%lld is not a multiple of 16", (long long)k);
  FP4RL_REQUIRE(n < kMaxDim && k < kMaxDim && n * k < ((int64_t)1 << 36), FP4RL_ERR_SHAPE, "matrix too large");
  FP4RL_REQUIRE(w_dtype == FP4RL_F32 || w_dtype == FP4RL_BF16, FP4RL_ERR_DTYPE, "w_dtype=%d", (int)w_dtype);
  FP4RL_REQUIRE(layout == FP4RL_ROW_MAJOR || layout == FP4RL_TILED, FP4RL_ERR_VALUE, "layout=%d", (int)layout);
  FP4RL_REQUIRE(tensor_scale != nullptr, FP4RL_ERR_NULL, "tensor_scale is NULL");
  FP4RL_REQUIRE(aligned(tensor_scale, 4), FP4RL_ERR_ALIGN, "tensor_scale not 4-byte aligned");
  if (n > 0 && k > 0) {
    FP4RL_REQUIRE(w && codes && scales, FP4RL_ERR_NULL, "w, codes and scales must be non-NULL");
    FP4RL_REQUIRE(aligned(w, 16) && aligned(codes, 16) && aligned(scales, 16), FP4RL_ERR_ALIGN,
                  "w, codes and scales must be 16-byte aligned");
  }
  return FP4RL_OK;
}

static fp4rl_status quantize_impl(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                  uint8_t* codes, uint8_t* scales, float* tensor_scale, uint8_t* record,
                                  void* workspace, size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_CHECK(check_quantize_args(w, w_dtype, n, k, layout, codes, scales, tensor_scale));
  const bool empty = n == 0 || k == 0;
  if (!empty) {
    FP4RL_REQUIRE(workspace != nullptr, FP4RL_ERR_WORKSPACE, "workspace is NULL");
    FP4RL_REQUIRE(workspace_bytes >= fp4rl::quantize_workspace_bytes(), FP4RL_ERR_WORKSPACE,
                  "workspace %zu < %zu bytes", workspace_bytes, fp4rl::quantize_workspace_bytes());
    FP4RL_REQUIRE(aligned(w, 16) && aligned(codes, 16) && aligned(scales, 16) && aligned(workspace, 16),
                  FP4RL_ERR_ALIGN, "w, codes, scales and workspace must be 16-byte aligned");
  }
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_quantize(w, w_dtype == FP4RL_BF16, n, k, layout == FP4RL_TILED, codes, scales,
                                         tensor_scale, empty ? nullptr : record, static_cast<uint32_t*>(workspace),
                                         stream),
                  "nvfp4_quantize");
}

fp4rl_status fp4rl_nvfp4_quantize(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                  uint8_t* codes, uint8_t* scales, float* tensor_scale, void* workspace,
                                  size_t workspace_bytes, fp4rl_stream stream) {
  return quantize_impl(w, w_dtype, n, k, layout, codes, scales, tensor_scale, nullptr, workspace, workspace_bytes,
                       stream);
}

fp4rl_status fp4rl_nvfp4_quantize_noalloc(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                          uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                          fp4rl_stream stream) {
  FP4RL_CHECK(check_quantize_args(w, w_dtype, n, k, layout, codes, scales, tensor_scale));
  if (fp4rl::quantize_workspace_bytes() > kScratchBytes)  // the partials of any shape are this many words
    return fail(FP4RL_ERR_WORKSPACE, "the quantiser needs %zu bytes of scratch, above the %zu-byte array",
                fp4rl::quantize_workspace_bytes(), kScratchBytes);
  FP4RL_CHECK(check_device());
  void* ws = nullptr;
  FP4RL_CHECK(scratch_address(&ws));
  return quantize_impl(w, w_dtype, n, k, layout, codes, scales, tensor_scale, nullptr, ws, kScratchBytes, stream);
}

fp4rl_status fp4rl_nvfp4_quantize_record(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                         uint8_t* codes, uint8_t* scales, float* tensor_scale, uint8_t* round_up,
                                         void* workspace, size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_REQUIRE(n == 0 || k == 0 || round_up != nullptr, FP4RL_ERR_NULL, "round_up is NULL");
  return quantize_impl(w, w_dtype, n, k, layout, codes, scales, tensor_scale, round_up, workspace, workspace_bytes,
                       stream);
}

fp4rl_status fp4rl_nvfp4_to_tiled(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                  uint8_t* codes_tiled, uint8_t* scales_tiled, fp4rl_stream stream) {
  FP4RL_REQUIRE(n >= 0 && k >= 0 && k % 16 == 0, FP4RL_ERR_SHAPE, "bad shape n=%lld k=%lld", (long long)n,
                (long long)k);
  FP4RL_REQUIRE(n < kMaxDim && k < kMaxDim && n * k < ((int64_t)1 << 36), FP4RL_ERR_SHAPE, "matrix too large");
  if (n == 0 || k == 0) return ok();
  FP4RL_REQUIRE(codes && scales && codes_tiled && scales_tiled, FP4RL_ERR_NULL, "NULL buffer");
  FP4RL_REQUIRE(aligned(codes, 16) && aligned(scales, 16) && aligned(codes_tiled, 16) && aligned(scales_tiled, 16),
                FP4RL_ERR_ALIGN, "buffers must be 16-byte aligned");
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_to_tiled(codes, scales, n, k, codes_tiled, scales_tiled, stream), "nvfp4_to_tiled");
}

// ------------------------------------------------------------------ linear --

// Linear workspaces: [counters, kLinearCounterBytes][t K-slices, fp32][main kernel K-split partials, fp32]
// (the last two only as needed; nothing at all when neither is needed).
static size_t lora_part_bytes(int64_t m, int64_t k, int64_t r) {
  if (m <= 0 || r <= 0 || k <= 0) return 0;
  const int slices = fp4rl::lora_slices(k, fp4rl::lora_splits(m, k, r));
  return round_up((size_t)slices * (size_t)m * (size_t)r * sizeof(float), 256);
}

static size_t main_part_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  return fp4rl::linear_partial_bytes(m, n, k);
}

static size_t linear_ws_bytes(size_t tbytes, size_t pbytes) {
  return tbytes + pbytes > 0 ? fp4rl::kLinearCounterBytes + tbytes + pbytes : 0;
}

size_t fp4rl_fp4_lora_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r) {
  return linear_ws_bytes(lora_part_bytes(m, k, r), main_part_bytes(m, n, k));
}

size_t fp4rl_fp4_linear_lora_up_workspace(int64_t m, int64_t n, int64_t k) {
  return linear_ws_bytes(0, main_part_bytes(m, n, k));
}

size_t fp4rl_lora_down_workspace(int64_t m, int64_t k, int64_t r) {
  if (m <= 0 || r <= 0 || k <= 0) return 0;
  const int slices = fp4rl::lora_slices(k, fp4rl::lora_splits(m, k, r));
  return slices > 1 ? round_up((size_t)slices * (size_t)m * (size_t)r * sizeof(float), 256) : 0;
}

fp4rl_status fp4rl_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a, int64_t r,
                             float lora_scale, float* t, void* workspace, size_t workspace_bytes,
                             fp4rl_stream stream) {
  FP4RL_CHECK(check_linear_shape(m, 1, k, r));
  FP4RL_REQUIRE(std::isfinite(lora_scale), FP4RL_ERR_VALUE, "lora_scale is not finite");
  if (m == 0 || r == 0) return ok();
  FP4RL_REQUIRE(x && lora_a && t, FP4RL_ERR_NULL, "x, lora_a and t must be non-NULL");
  FP4RL_REQUIRE(aligned(x, 16) && aligned(lora_a, 16) && aligned(t, 16), FP4RL_ERR_ALIGN,
                "x, lora_a and t must be 16-byte aligned");
  const int splits = fp4rl::lora_splits(m, k, r);
  const int slices = fp4rl::lora_slices(k, splits);
  const size_t need = fp4rl_lora_down_workspace(m, k, r);
  if (need) {
    FP4RL_REQUIRE(workspace != nullptr && workspace_bytes >= need, FP4RL_ERR_WORKSPACE, "workspace %zu < %zu bytes",
                  workspace_bytes, need);
    FP4RL_REQUIRE(aligned(workspace, 16), FP4RL_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  FP4RL_CHECK(check_device());
  float* part = slices > 1 ? static_cast<float*>(workspace) : t;
  fp4rl_status s = launched(fp4rl::launch_lora_down(x, m, k, lora_a, r, lora_scale, splits, part, stream),
                            "lora_down");
  if (s != FP4RL_OK || slices == 1) return s;
  return launched(fp4rl::launch_lora_reduce(part, slices, m * r, t, stream), "lora_reduce");
}

static fp4rl_status check_linear_main(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                      const uint8_t* scales, const float* tensor_scale, const float* t,
                                      const uint16_t* lora_b, int64_t r, uint16_t* y) {
  FP4RL_REQUIRE(x && codes && scales && tensor_scale && y, FP4RL_ERR_NULL,
                "x, codes, scales, tensor_scale and y must be non-NULL");
  FP4RL_REQUIRE(aligned(x, 16) && aligned(codes, 16) && aligned(scales, 16) && aligned(y, 16), FP4RL_ERR_ALIGN,
                "x, codes, scales and y must be 16-byte aligned");
  FP4RL_REQUIRE(aligned(tensor_scale, 4), FP4RL_ERR_ALIGN, "tensor_scale not 4-byte aligned");
  if (r > 0) {
    FP4RL_REQUIRE(t && lora_b, FP4RL_ERR_NULL, "r > 0 needs t and lora_b");
    FP4RL_REQUIRE(aligned(t, 16) && aligned(lora_b, 16), FP4RL_ERR_ALIGN, "t and lora_b must be 16-byte aligned");
  }
  (void)m;
  (void)n;
  (void)k;
  return FP4RL_OK;
}

static fp4rl_status check_main_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return FP4RL_OK;
  FP4RL_REQUIRE(ws != nullptr && ws_bytes >= need, FP4RL_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  FP4RL_REQUIRE(aligned(ws, 16), FP4RL_ERR_ALIGN, "workspace must be 16-byte aligned");
  return FP4RL_OK;
}

fp4rl_status fp4rl_fp4_linear_lora_up(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                      const uint8_t* scales, const float* tensor_scale, const float* t,
                                      const uint16_t* lora_b, int64_t r, uint16_t* y, void* workspace,
                                      size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_CHECK(check_linear_shape(m, n, k, r));
  if (m == 0 || n == 0) return ok();
  FP4RL_CHECK(check_linear_main(x, m, n, k, codes, scales, tensor_scale, t, lora_b, r, y));
  const size_t pbytes = main_part_bytes(m, n, k);
  FP4RL_CHECK(check_main_ws(workspace, workspace_bytes, linear_ws_bytes(0, pbytes)));
  FP4RL_CHECK(check_device());
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* part = pbytes ? reinterpret_cast<float*>(ws + fp4rl::kLinearCounterBytes) : nullptr;
  uint32_t* counters = pbytes ? reinterpret_cast<uint32_t*>(ws) : nullptr;
  return launched(fp4rl::launch_fp4_linear(x, m, n, k, codes, scales, tensor_scale, r > 0 ? t : nullptr, 1,
                                           r > 0 ? lora_b : nullptr, r, y, part, counters, fp4rl::LoraFuse{}, stream),
                  "fp4_linear");
}

// The linear's launches on an argument-checked call (workspace sized by
// fp4rl_fp4_lora_linear_workspace, its counter words zero): the t region and
// the K-split partials are carved from the workspace, and with adapters t is
// made either by producer workgroups inside the main launch or by a separate
// down-projection launch.
static fp4rl_status run_lora_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                    const uint8_t* scales, const float* tensor_scale, const uint16_t* lora_a,
                                    const uint16_t* lora_b, int64_t r, float lora_scale, uint16_t* y, void* workspace,
                                    fp4rl_stream stream) {
  const size_t tbytes = lora_part_bytes(m, k, r), pbytes = main_part_bytes(m, n, k);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* t = tbytes ? reinterpret_cast<float*>(ws + fp4rl::kLinearCounterBytes) : nullptr;
  float* part = pbytes ? reinterpret_cast<float*>(ws + fp4rl::kLinearCounterBytes + tbytes) : nullptr;
  uint32_t* counters = pbytes ? reinterpret_cast<uint32_t*>(ws) : nullptr;
  int slices = 1;
  fp4rl::LoraFuse lf{};
  if (r > 0) {
    const int splits = fp4rl::lora_splits(m, k, r);
    slices = fp4rl::lora_slices(k, splits);
    if (fp4rl::linear_fuses_lora(m, n, k)) {
      // t is made by the first workgroups of the linear's own launch (into
      // slice 0 of the t region); counter words carry their hand-off
      lf.a = lora_a;
      lf.s = lora_scale;
      lf.kslice = (int)fp4rl::lora_slice_len(k, splits);
      lf.slices = slices;
      lf.mtiles = (int)((m + 15) / 16);
      lf.rtiles = (int)((r + 15) / 16);
      lf.producers = (int)round_up((size_t)lf.mtiles * lf.rtiles * slices, 8);
      lf.part = t;
      lf.tctr = reinterpret_cast<uint32_t*>(ws) + fp4rl::kLoraTileCtrOffset;
      lf.done = reinterpret_cast<uint32_t*>(ws) + fp4rl::kLoraDoneOffset;
      lf.lines = reinterpret_cast<uint32_t*>(ws) + fp4rl::kLoraLineOffset;
      lf.err = reinterpret_cast<uint32_t*>(ws) + fp4rl::kLinearErrOffset;
      lf.spin = g_lora_spin.load(std::memory_order_relaxed);
      lf.withhold = g_lora_withhold.load(std::memory_order_relaxed);
      lf.epoch = next_lora_epoch();
    } else {
      fp4rl_status s =
          launched(fp4rl::launch_lora_down(x, m, k, lora_a, r, lora_scale, splits, t, stream), "lora_down");
      if (s != FP4RL_OK) return s;
    }
  }
  // the main kernel's epilogue sums the K-slices of t in slice order (fused
  // producers have already summed them into slice 0)
  return launched(fp4rl::launch_fp4_linear(x, m, n, k, codes, scales, tensor_scale, r > 0 ? t : nullptr,
                                           lf.producers > 0 ? 1 : slices,
                                           r > 0 ? lora_b : nullptr, r, y, part, counters, lf, stream),
                  "fp4_linear");
}

fp4rl_status fp4rl_fp4_lora_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                   const uint8_t* scales, const float* tensor_scale, const uint16_t* lora_a,
                                   const uint16_t* lora_b, int64_t r, float lora_scale, uint16_t* y,
                                   void* workspace, size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_CHECK(check_linear_shape(m, n, k, r));
  FP4RL_REQUIRE(std::isfinite(lora_scale), FP4RL_ERR_VALUE, "lora_scale is not finite");
  FP4RL_REQUIRE((lora_a == nullptr) == (lora_b == nullptr), FP4RL_ERR_NULL,
                "lora_a and lora_b must both be NULL or both be set");
  if (lora_a == nullptr) r = 0;
  if (m == 0 || n == 0) return ok();
  const size_t tbytes = lora_part_bytes(m, k, r), pbytes = main_part_bytes(m, n, k);
  FP4RL_CHECK(check_main_ws(workspace, workspace_bytes, linear_ws_bytes(tbytes, pbytes)));
  if (r > 0) FP4RL_REQUIRE(aligned(lora_a, 16), FP4RL_ERR_ALIGN, "lora_a must be 16-byte aligned");
  const float* t = tbytes ? reinterpret_cast<const float*>(static_cast<uint8_t*>(workspace) + fp4rl::kLinearCounterBytes)
                         : nullptr;
  FP4RL_CHECK(check_linear_main(x, m, n, k, codes, scales, tensor_scale, t, lora_b, r, y));
  FP4RL_CHECK(check_device());
  return run_lora_linear(x, m, n, k, codes, scales, tensor_scale, lora_a, lora_b, r, lora_scale, y, workspace, stream);
}

fp4rl_status fp4rl_linear_workspace_check(const void* workspace, size_t workspace_bytes, fp4rl_stream stream) {
  if (workspace == nullptr || workspace_bytes == 0) return ok();  // no counter words: nothing can have failed
  FP4RL_REQUIRE(workspace_bytes >= fp4rl::kLinearCounterBytes, FP4RL_ERR_WORKSPACE,
                "workspace %zu bytes holds no counter words (%zu)", workspace_bytes, fp4rl::kLinearCounterBytes);
  FP4RL_REQUIRE(aligned(workspace, 16), FP4RL_ERR_ALIGN, "workspace must be 16-byte aligned");
  FP4RL_CHECK(check_device());
  uint32_t err = 0;
  const uint32_t* word = static_cast<const uint32_t*>(workspace) + fp4rl::kLinearErrOffset;
  hipError_t e = hipMemcpyAsync(&err, word, sizeof(err), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(FP4RL_ERR_HIP, "reading the workspace error word: %s", hipGetErrorString(e));
  if (err & fp4rl::kLinearErrLoraWait)
    return fail(FP4RL_ERR_TIMEOUT, "a fused linear on this workspace gave up waiting for its LoRA down-projection "
                                   "(error bits 0x%x); results since then are not to be trusted", err);
  return ok();
}

fp4rl_status fp4rl_linear_workspace_reset(void* workspace, size_t workspace_bytes, fp4rl_stream stream) {
  if (workspace == nullptr || workspace_bytes == 0) return ok();
  FP4RL_REQUIRE(workspace_bytes >= fp4rl::kLinearCounterBytes, FP4RL_ERR_WORKSPACE,
                "workspace %zu bytes holds no counter words (%zu)", workspace_bytes, fp4rl::kLinearCounterBytes);
  FP4RL_REQUIRE(aligned(workspace, 16), FP4RL_ERR_ALIGN, "workspace must be 16-byte aligned");
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_zero_words(workspace, fp4rl::kLinearCounters, stream), "linear_workspace_reset");
}

void fp4rl_debug_lora_handoff(uint32_t spin_limit, int32_t withhold_ready) {
  g_lora_spin.store(spin_limit == 0 ? fp4rl::LoraFuse{}.spin : spin_limit, std::memory_order_relaxed);
  g_lora_withhold.store(withhold_ready != 0 ? 1u : 0u, std::memory_order_relaxed);
}

const char* fp4rl_fp4_linear_kernel_name(int64_t m, int64_t n, int64_t k, int64_t r) {
  if (check_linear_shape(m, n, k, r) != FP4RL_OK || m == 0 || n == 0) return "";
  return fp4rl::fp4_linear_kernel_name(m, n, k, r);
}

// ---------------------------------------------------------------- backward --

static fp4rl_status check_backward_shape(int64_t m, int64_t n, int64_t k, int64_t r) {
  FP4RL_REQUIRE(m >= 0 && n >= 0 && k >= 0 && r >= 0, FP4RL_ERR_SHAPE,
                "negative size (m=%lld n=%lld k=%lld r=%lld)", (long long)m, (long long)n, (long long)k, (long long)r);
  FP4RL_REQUIRE(k > 0 && k % 16 == 0, FP4RL_ERR_SHAPE, "k=%lld must be a positive multiple of 16", (long long)k);
  FP4RL_REQUIRE(n % 8 == 0, FP4RL_ERR_SHAPE, "n=%lld must be a multiple of 8", (long long)n);
  // the GEMM kernels address one 128-row operand tile with 32-bit byte offsets
  FP4RL_REQUIRE(n < ((int64_t)1 << 22) && k < ((int64_t)1 << 22) && m < ((int64_t)1 << 22), FP4RL_ERR_SHAPE,
                "m, n and k must be below 2^22");
  FP4RL_REQUIRE(r <= fp4rl::kMaxRank, FP4RL_ERR_SHAPE, "rank r=%lld exceeds %lld", (long long)r,
                (long long)fp4rl::kMaxRank);
  return FP4RL_OK;
}

size_t fp4rl_fp4_lora_linear_backward_workspace(int64_t m, int64_t n, int64_t k, int64_t r, int32_t want_dx) {
  if (check_backward_shape(m, n, k, r) != FP4RL_OK || m == 0 || n == 0) return 0;
  return fp4rl::backward_workspace(m, n, k, r, want_dx != 0, nullptr, nullptr);
}

fp4rl_status fp4rl_fp4_lora_linear_backward(const uint16_t* dy, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                            const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                            const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                                            float lora_scale, uint16_t* dx, float* grad_a, float* grad_b,
                                            void* workspace, size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_CHECK(check_backward_shape(m, n, k, r));
  FP4RL_REQUIRE(std::isfinite(lora_scale), FP4RL_ERR_VALUE, "lora_scale is not finite");
  FP4RL_REQUIRE((lora_a == nullptr) == (lora_b == nullptr), FP4RL_ERR_NULL,
                "lora_a and lora_b must both be NULL or both be set");
  if (lora_a == nullptr) r = 0;
  FP4RL_REQUIRE(dx != nullptr || r > 0, FP4RL_ERR_NULL, "nothing to compute: dx is NULL and there are no adapters");
  if (r > 0) {
    FP4RL_REQUIRE(grad_a && grad_b, FP4RL_ERR_NULL, "r > 0 needs grad_a and grad_b");
    FP4RL_REQUIRE(aligned(lora_a, 16) && aligned(lora_b, 16) && aligned(grad_a, 16) && aligned(grad_b, 16),
                  FP4RL_ERR_ALIGN, "lora_a, lora_b, grad_a and grad_b must be 16-byte aligned");
  }
  if (dx) FP4RL_REQUIRE(aligned(dx, 16), FP4RL_ERR_ALIGN, "dx must be 16-byte aligned");
  if (m == 0 || n == 0) {
    // empty sums: every gradient is zero (dX and dA when n == 0, dA and dB when m == 0)
    if (m == 0 && n == 0) return ok();
    FP4RL_CHECK(check_device());
    hipError_t e = hipSuccess;
    if (dx && m > 0) e = fp4rl::launch_zero_words(dx, m * k / 2, stream);
    if (e == hipSuccess && r > 0) e = fp4rl::launch_zero_words(grad_a, r * k, stream);
    if (e == hipSuccess && r > 0 && n > 0) e = fp4rl::launch_zero_words(grad_b, n * r, stream);
    return launched(e, "zero_words");
  }
  FP4RL_REQUIRE(dy != nullptr && aligned(dy, 16), dy ? FP4RL_ERR_ALIGN : FP4RL_ERR_NULL,
                "dy must be non-NULL and 16-byte aligned");
  if (r > 0) FP4RL_REQUIRE(x != nullptr && aligned(x, 16), x ? FP4RL_ERR_ALIGN : FP4RL_ERR_NULL,
                           "x must be non-NULL and 16-byte aligned when r > 0");
  if (dx) {
    FP4RL_REQUIRE(codes && scales && tensor_scale, FP4RL_ERR_NULL, "dX needs codes, scales and tensor_scale");
    FP4RL_REQUIRE(aligned(codes, 16) && aligned(scales, 16) && aligned(tensor_scale, 4), FP4RL_ERR_ALIGN,
                  "codes and scales must be 16-byte aligned, tensor_scale 4-byte aligned");
  }
  const size_t need = fp4rl::backward_workspace(m, n, k, r, dx != nullptr, nullptr, nullptr);
  FP4RL_REQUIRE(workspace != nullptr && workspace_bytes >= need, FP4RL_ERR_WORKSPACE, "workspace %zu < %zu bytes",
                workspace_bytes, need);
  FP4RL_REQUIRE(aligned(workspace, 256), FP4RL_ERR_ALIGN, "workspace must be 256-byte aligned");
  FP4RL_CHECK(check_device());
  fp4rl::BackwardWs w;
  fp4rl::backward_workspace(m, n, k, r, dx != nullptr, &w, workspace);
  return launched(fp4rl::launch_lora_backward(dy, x, m, n, k, codes, scales, tensor_scale, r > 0 ? lora_a : nullptr,
                                              r > 0 ? lora_b : nullptr, r, lora_scale, dx, grad_a, grad_b, w, stream),
                  "fp4_lora_linear_backward");
}

// ----------------------------------------------------------------- gate/up --

// Above kGateUpFusedMaxTokens: [linear workspace][g: m n bf16][u: m n bf16],
// each region 256-byte aligned; the linear's counter words come first. Up to
// kGateUpFusedMaxTokens: [counter words, untouched][fused launch's t slices],
// so that one workspace serves both paths in any order.
static size_t gate_up_two_linears_ws(int64_t m, int64_t n, int64_t k, int64_t r) {
  return round_up(linear_ws_bytes(lora_part_bytes(m, k, r), main_part_bytes(m, n, k)), 256) +
         2 * round_up((size_t)m * (size_t)n * 2, 256);
}

static size_t gate_up_fused_offset() { return round_up(fp4rl::kLinearCounterBytes, 256); }

static size_t gate_up_ws_bytes(int64_t m, int64_t n, int64_t k, int64_t r) {
  if (m > fp4rl::kGateUpFusedMaxTokens) return gate_up_two_linears_ws(m, n, k, r);
  const size_t t = fp4rl::gate_up_workspace(m, k, r);
  return t ? gate_up_fused_offset() + t : 0;
}

size_t fp4rl_fp4_gate_up_silu_workspace(int64_t m, int64_t n, int64_t k, int64_t r) {
  if (check_linear_shape(m, n, k, r) != FP4RL_OK || m == 0 || n == 0 || m > fp4rl::kGateUpMaxTokens) return 0;
  return gate_up_ws_bytes(m, n, k, r);
}

fp4rl_status fp4rl_fp4_gate_up_silu(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* gate_codes,
                                    const uint8_t* gate_scales, const float* gate_tensor_scale,
                                    const uint8_t* up_codes, const uint8_t* up_scales, const float* up_tensor_scale,
                                    const uint16_t* lora_a_gate, const uint16_t* lora_b_gate,
                                    const uint16_t* lora_a_up, const uint16_t* lora_b_up, int64_t r,
                                    float lora_scale, uint16_t* h, void* workspace, size_t workspace_bytes,
                                    fp4rl_stream stream) {
  FP4RL_CHECK(check_linear_shape(m, n, k, r));
  FP4RL_REQUIRE(m <= fp4rl::kGateUpMaxTokens, FP4RL_ERR_SHAPE, "m=%lld exceeds %lld tokens", (long long)m,
                (long long)fp4rl::kGateUpMaxTokens);
  FP4RL_REQUIRE(std::isfinite(lora_scale), FP4RL_ERR_VALUE, "lora_scale is not finite");
  const bool any = lora_a_gate || lora_b_gate || lora_a_up || lora_b_up;
  const bool all = lora_a_gate && lora_b_gate && lora_a_up && lora_b_up;
  FP4RL_REQUIRE(any == all, FP4RL_ERR_NULL, "the four adapters must all be NULL or all be set");
  if (!all) r = 0;
  if (m == 0 || n == 0) return ok();
  FP4RL_REQUIRE(x && gate_codes && gate_scales && gate_tensor_scale && up_codes && up_scales && up_tensor_scale && h,
                FP4RL_ERR_NULL, "x, both weights and h must be non-NULL");
  FP4RL_REQUIRE(aligned(x, 16) && aligned(gate_codes, 16) && aligned(gate_scales, 16) && aligned(up_codes, 16) &&
                    aligned(up_scales, 16) && aligned(h, 16) && aligned(gate_tensor_scale, 4) &&
                    aligned(up_tensor_scale, 4),
                FP4RL_ERR_ALIGN, "x, codes, scales and h must be 16-byte aligned, tensor scales 4-byte aligned");
  if (r > 0)
    FP4RL_REQUIRE(aligned(lora_a_gate, 16) && aligned(lora_b_gate, 16) && aligned(lora_a_up, 16) &&
                      aligned(lora_b_up, 16),
                  FP4RL_ERR_ALIGN, "adapters must be 16-byte aligned");
  const size_t need = gate_up_ws_bytes(m, n, k, r);
  if (need) {
    FP4RL_REQUIRE(workspace != nullptr && workspace_bytes >= need, FP4RL_ERR_WORKSPACE, "workspace %zu < %zu bytes",
                  workspace_bytes, need);
    FP4RL_REQUIRE(aligned(workspace, 256), FP4RL_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  FP4RL_CHECK(check_device());
  if (m <= fp4rl::kGateUpFusedMaxTokens) {
    float* tws = need ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + gate_up_fused_offset()) : nullptr;
    return launched(fp4rl::launch_gate_up(x, m, n, k, gate_codes, gate_scales, gate_tensor_scale, up_codes, up_scales,
                                          up_tensor_scale, lora_a_gate, lora_b_gate, lora_a_up, lora_b_up, r,
                                          lora_scale, tws, h, stream),
                    "fp4_gate_up_silu");
  }
  // two linears into bf16 g and u (one workspace, used in turn), then the gated product
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t lin = round_up(linear_ws_bytes(lora_part_bytes(m, k, r), main_part_bytes(m, n, k)), 256);
  uint16_t* g = reinterpret_cast<uint16_t*>(ws + lin);
  uint16_t* u = reinterpret_cast<uint16_t*>(ws + lin + round_up((size_t)m * (size_t)n * 2, 256));
  void* lws = lin ? ws : nullptr;
  FP4RL_CHECK(run_lora_linear(x, m, n, k, gate_codes, gate_scales, gate_tensor_scale, r > 0 ? lora_a_gate : nullptr,
                              r > 0 ? lora_b_gate : nullptr, r, lora_scale, g, lws, stream));
  FP4RL_CHECK(run_lora_linear(x, m, n, k, up_codes, up_scales, up_tensor_scale, r > 0 ? lora_a_up : nullptr,
                              r > 0 ? lora_b_up : nullptr, r, lora_scale, u, lws, stream));
  return launched(fp4rl::launch_silu_mul(g, u, m * n, h, stream), "silu_mul");
}

size_t fp4rl_aqn_gate_up_silu_workspace(int64_t m, int64_t n, int64_t k, int64_t r) {
  if (check_linear_shape(m, n, k, r) != FP4RL_OK || m == 0 || n == 0 || m > fp4rl::kGateUpMaxTokens ||
      k > fp4rl::kAqnMaxD)
    return 0;
  return fp4rl::aqn_gate_up_workspace(m, k, r);
}

fp4rl_status fp4rl_aqn_gate_up_silu(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w,
                                    float sigma, uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                                    const uint8_t* gate_codes, const uint8_t* gate_scales,
                                    const float* gate_tensor_scale, const uint8_t* up_codes, const uint8_t* up_scales,
                                    const float* up_tensor_scale, const uint16_t* lora_a_gate,
                                    const uint16_t* lora_b_gate, const uint16_t* lora_a_up, const uint16_t* lora_b_up,
                                    int64_t r, float lora_scale, uint16_t* h, void* workspace,
                                    size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_CHECK(check_linear_shape(m, n, k, r));
  FP4RL_REQUIRE(m <= fp4rl::kGateUpMaxTokens, FP4RL_ERR_SHAPE, "m=%lld exceeds %lld tokens", (long long)m,
                (long long)fp4rl::kGateUpMaxTokens);
  FP4RL_REQUIRE(k <= fp4rl::kAqnMaxD, FP4RL_ERR_SHAPE, "k=%lld exceeds the norm's width %lld", (long long)k,
                (long long)fp4rl::kAqnMaxD);
  FP4RL_REQUIRE(std::isfinite(lora_scale), FP4RL_ERR_VALUE, "lora_scale is not finite");
  FP4RL_REQUIRE(std::isfinite(sigma) && sigma >= 0.0f, FP4RL_ERR_VALUE, "sigma must be finite and >= 0");
  FP4RL_REQUIRE(std::isfinite(eps) && eps >= 0.0f, FP4RL_ERR_VALUE, "eps must be finite and >= 0");
  const bool any = lora_a_gate || lora_b_gate || lora_a_up || lora_b_up;
  const bool all = lora_a_gate && lora_b_gate && lora_a_up && lora_b_up;
  FP4RL_REQUIRE(any == all, FP4RL_ERR_NULL, "the four adapters must all be NULL or all be set");
  if (!all) r = 0;
  if (m == 0 || n == 0) return ok();
  FP4RL_REQUIRE(x && norm_w && gate_codes && gate_scales && gate_tensor_scale && up_codes && up_scales &&
                    up_tensor_scale && h,
                FP4RL_ERR_NULL, "x, the norm weight, both weights and h must be non-NULL");
  FP4RL_REQUIRE(aligned(x, 16) && aligned(norm_w, 16) && aligned(gate_codes, 16) && aligned(gate_scales, 16) &&
                    aligned(up_codes, 16) && aligned(up_scales, 16) && aligned(h, 16) &&
                    aligned(gate_tensor_scale, 4) && aligned(up_tensor_scale, 4),
                FP4RL_ERR_ALIGN, "x, norm_w, codes, scales and h must be 16-byte aligned, tensor scales 4-byte aligned");
  if (r > 0)
    FP4RL_REQUIRE(aligned(lora_a_gate, 16) && aligned(lora_b_gate, 16) && aligned(lora_a_up, 16) &&
                      aligned(lora_b_up, 16),
                  FP4RL_ERR_ALIGN, "adapters must be 16-byte aligned");
  const size_t need = fp4rl::aqn_gate_up_workspace(m, k, r);
  FP4RL_REQUIRE(workspace != nullptr && workspace_bytes >= need, FP4RL_ERR_WORKSPACE, "workspace %zu < %zu bytes",
                workspace_bytes, need);
  FP4RL_REQUIRE(aligned(workspace, 256), FP4RL_ERR_ALIGN, "workspace must be 256-byte aligned");
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_aqn_gate_up(x, m, n, k, norm_w, sigma, seed, step, norm_id, eps, gate_codes,
                                            gate_scales, gate_tensor_scale, up_codes, up_scales, up_tensor_scale,
                                            lora_a_gate, lora_b_gate, lora_a_up, lora_b_up, r, lora_scale, workspace,
                                            h, stream),
                  "aqn_gate_up_silu");
}

size_t fp4rl_aqn_lora_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r) {
  if (check_linear_shape(m, n, k, r) != FP4RL_OK || m == 0 || n == 0 || m > fp4rl::kGateUpMaxTokens ||
      k > fp4rl::kAqnMaxD)
    return 0;
  return fp4rl::aqn_linear_workspace(m, k, r);
}

fp4rl_status fp4rl_aqn_lora_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w,
                                   float sigma, uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                                   const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                   const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float lora_scale,
                                   uint16_t* y, void* workspace, size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_CHECK(check_linear_shape(m, n, k, r));
  FP4RL_REQUIRE(m <= fp4rl::kGateUpMaxTokens, FP4RL_ERR_SHAPE, "m=%lld exceeds %lld tokens", (long long)m,
                (long long)fp4rl::kGateUpMaxTokens);
  FP4RL_REQUIRE(k <= fp4rl::kAqnMaxD, FP4RL_ERR_SHAPE, "k=%lld exceeds the norm's width %lld", (long long)k,
                (long long)fp4rl::kAqnMaxD);
  FP4RL_REQUIRE(std::isfinite(lora_scale), FP4RL_ERR_VALUE, "lora_scale is not finite");
  FP4RL_REQUIRE(std::isfinite(sigma) && sigma >= 0.0f, FP4RL_ERR_VALUE, "sigma must be finite and >= 0");
  FP4RL_REQUIRE(std::isfinite(eps) && eps >= 0.0f, FP4RL_ERR_VALUE, "eps must be finite and >= 0");
  FP4RL_REQUIRE((lora_a == nullptr) == (lora_b == nullptr), FP4RL_ERR_NULL,
                "lora_a and lora_b must both be NULL or both be set");
  if (lora_a == nullptr) r = 0;
  if (m == 0 || n == 0) return ok();
  FP4RL_REQUIRE(x && norm_w && codes && scales && tensor_scale && y, FP4RL_ERR_NULL,
                "x, the norm weight, the weight and y must be non-NULL");
  FP4RL_REQUIRE(aligned(x, 16) && aligned(norm_w, 16) && aligned(codes, 16) && aligned(scales, 16) &&
                    aligned(y, 16) && aligned(tensor_scale, 4),
                FP4RL_ERR_ALIGN, "x, norm_w, codes, scales and y must be 16-byte aligned, the tensor scale 4-byte aligned");
  if (r > 0)
    FP4RL_REQUIRE(aligned(lora_a, 16) && aligned(lora_b, 16), FP4RL_ERR_ALIGN, "adapters must be 16-byte aligned");
  const size_t need = fp4rl::aqn_linear_workspace(m, k, r);
  FP4RL_REQUIRE(workspace != nullptr && workspace_bytes >= need, FP4RL_ERR_WORKSPACE, "workspace %zu < %zu bytes",
                workspace_bytes, need);
  FP4RL_REQUIRE(aligned(workspace, 256), FP4RL_ERR_ALIGN, "workspace must be 256-byte aligned");
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_aqn_linear(x, m, n, k, norm_w, sigma, seed, step, norm_id, eps, codes, scales,
                                           tensor_scale, r > 0 ? lora_a : nullptr, r > 0 ? lora_b : nullptr, r,
                                           lora_scale, workspace, y, stream),
                  "aqn_lora_linear");
}

// --------------------------------------------------------------------- FP8 --

fp4rl_status fp4rl_fp8_quantize(const void* w, int32_t w_dtype, int64_t n, int64_t k, uint8_t* codes,
                                float* row_scales, fp4rl_stream stream) {
  FP4RL_REQUIRE(n >= 0 && k > 0 && k % 16 == 0, FP4RL_ERR_SHAPE, "need n >= 0 and k a positive multiple of 16 "
                "(n=%lld k=%lld)", (long long)n, (long long)k);
  FP4RL_REQUIRE(n < kMaxDim && k < ((int64_t)1 << 22), FP4RL_ERR_SHAPE, "n below 2^31 and k below 2^22 required");
  FP4RL_REQUIRE(w_dtype == FP4RL_F32 || w_dtype == FP4RL_BF16, FP4RL_ERR_DTYPE, "w_dtype=%d", (int)w_dtype);
  if (n == 0) return ok();
  FP4RL_REQUIRE(w && codes && row_scales, FP4RL_ERR_NULL, "w, codes and row_scales must be non-NULL");
  FP4RL_REQUIRE(aligned(w, 16) && aligned(codes, 16) && aligned(row_scales, 4), FP4RL_ERR_ALIGN,
                "w and codes must be 16-byte aligned, row_scales 4-byte aligned");
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_fp8_quantize(w, w_dtype == FP4RL_BF16, n, k, codes, row_scales, stream),
                  "fp8_quantize");
}

static fp4rl_status check_fp8_shape(int64_t m, int64_t n, int64_t k, int64_t r) {
  FP4RL_REQUIRE(m >= 0 && n >= 0 && r >= 0 && k > 0 && k % 16 == 0, FP4RL_ERR_SHAPE,
                "bad shape (m=%lld n=%lld k=%lld r=%lld)", (long long)m, (long long)n, (long long)k, (long long)r);
  FP4RL_REQUIRE(m < ((int64_t)1 << 22) && n < ((int64_t)1 << 22) && k < ((int64_t)1 << 22), FP4RL_ERR_SHAPE,
                "m, n and k must be below 2^22");
  // the LoRA down-projection addresses activations with 32-bit byte offsets
  FP4RL_REQUIRE(m * k < ((int64_t)1 << 30), FP4RL_ERR_SHAPE, "m * k = %lld must be below 2^30", (long long)(m * k));
  FP4RL_REQUIRE(r <= fp4rl::kMaxRank, FP4RL_ERR_SHAPE, "rank r=%lld exceeds %lld", (long long)r,
                (long long)fp4rl::kMaxRank);
  return FP4RL_OK;
}

static size_t fp8_workspace(int64_t m, int64_t n, int64_t k, int64_t r, bool a8) {
  if (check_fp8_shape(m, n, k, r) != FP4RL_OK || m == 0 || n == 0) return 0;
  return fp4rl::fp8_linear_workspace(m, n, k, r, a8, nullptr, nullptr);
}

size_t fp4rl_fp8_lora_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r) {
  return fp8_workspace(m, n, k, r, false);
}

size_t fp4rl_fp8_lora_linear_w8a8_workspace(int64_t m, int64_t n, int64_t k, int64_t r) {
  return fp8_workspace(m, n, k, r, true);
}

static fp4rl_status fp8_linear(const char* name, bool a8, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                               const uint8_t* codes, const float* row_scales, const uint16_t* lora_a,
                               const uint16_t* lora_b, int64_t r, float lora_scale, uint16_t* y, void* workspace,
                               size_t workspace_bytes, fp4rl_stream stream) {
  FP4RL_CHECK(check_fp8_shape(m, n, k, r));
  FP4RL_REQUIRE(std::isfinite(lora_scale), FP4RL_ERR_VALUE, "lora_scale is not finite");
  FP4RL_REQUIRE((lora_a == nullptr) == (lora_b == nullptr), FP4RL_ERR_NULL,
                "lora_a and lora_b must both be NULL or both be set");
  if (lora_a == nullptr) r = 0;
  if (m == 0 || n == 0) return ok();
  FP4RL_REQUIRE(x && codes && row_scales && y, FP4RL_ERR_NULL, "x, codes, row_scales and y must be non-NULL");
  FP4RL_REQUIRE(aligned(x, 16) && aligned(codes, 16) && aligned(y, 16) && aligned(row_scales, 4), FP4RL_ERR_ALIGN,
                "x, codes and y must be 16-byte aligned, row_scales 4-byte aligned");
  if (r > 0)
    FP4RL_REQUIRE(aligned(lora_a, 16) && aligned(lora_b, 16), FP4RL_ERR_ALIGN, "lora_a and lora_b must be 16-byte aligned");
  const size_t need = fp4rl::fp8_linear_workspace(m, n, k, r, a8, nullptr, nullptr);
  FP4RL_REQUIRE(workspace != nullptr && workspace_bytes >= need, FP4RL_ERR_WORKSPACE, "workspace %zu < %zu bytes",
                workspace_bytes, need);
  FP4RL_REQUIRE(aligned(workspace, 256), FP4RL_ERR_ALIGN, "workspace must be 256-byte aligned");
  FP4RL_CHECK(check_device());
  fp4rl::Fp8Ws w;
  fp4rl::fp8_linear_workspace(m, n, k, r, a8, &w, workspace);
  return launched(fp4rl::launch_fp8_linear(x, m, n, k, codes, row_scales, r > 0 ? lora_a : nullptr,
                                           r > 0 ? lora_b : nullptr, r, lora_scale, a8, y, w, stream),
                  name);
}

fp4rl_status fp4rl_fp8_lora_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                   const float* row_scales, const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                                   float lora_scale, uint16_t* y, void* workspace, size_t workspace_bytes,
                                   fp4rl_stream stream) {
  return fp8_linear("fp8_lora_linear", false, x, m, n, k, codes, row_scales, lora_a, lora_b, r, lora_scale, y,
                    workspace, workspace_bytes, stream);
}

fp4rl_status fp4rl_fp8_lora_linear_w8a8(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                        const float* row_scales, const uint16_t* lora_a, const uint16_t* lora_b,
                                        int64_t r, float lora_scale, uint16_t* y, void* workspace,
                                        size_t workspace_bytes, fp4rl_stream stream) {
  return fp8_linear("fp8_lora_linear_w8a8", true, x, m, n, k, codes, row_scales, lora_a, lora_b, r, lora_scale, y,
                    workspace, workspace_bytes, stream);
}

// --------------------------------------------------------------------- AQN --

float fp4rl_aqn_sigma(float sigma_start, float sigma_end, int32_t k, int32_t num_stages) {
  if (num_stages < 1 || k < 0 || k >= num_stages || !(sigma_start > 0.0f) || !(sigma_end > 0.0f) ||
      !std::isfinite(sigma_start) || !std::isfinite(sigma_end))
    return std::nanf("");
  if (num_stages == 1) return sigma_start;
  const double frac = (double)k / (double)(num_stages - 1);
  return (float)((double)sigma_start * std::pow((double)sigma_end / (double)sigma_start, frac));
}

fp4rl_status fp4rl_aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, const float* w, float sigma, uint64_t seed,
                               uint64_t step, uint32_t norm_id, float eps, uint16_t* y, float* w_noise_out,
                               fp4rl_stream stream) {
  FP4RL_REQUIRE(m >= 0 && d >= 0, FP4RL_ERR_SHAPE, "negative size (m=%lld d=%lld)", (long long)m, (long long)d);
  FP4RL_REQUIRE(std::isfinite(sigma) && sigma >= 0.0f, FP4RL_ERR_VALUE, "sigma must be finite and >= 0");
  FP4RL_REQUIRE(std::isfinite(eps) && eps >= 0.0f, FP4RL_ERR_VALUE, "eps must be finite and >= 0");
  if ((m == 0 && w_noise_out == nullptr) || d == 0) return ok();
  FP4RL_REQUIRE(d <= fp4rl::kAqnMaxD, FP4RL_ERR_SHAPE, "d=%lld exceeds %lld", (long long)d,
                (long long)fp4rl::kAqnMaxD);
  FP4RL_REQUIRE(m < kMaxDim * 64, FP4RL_ERR_SHAPE, "too many rows");
  FP4RL_REQUIRE(w != nullptr, FP4RL_ERR_NULL, "w is NULL");
  FP4RL_REQUIRE(aligned(w, 16), FP4RL_ERR_ALIGN, "w must be 16-byte aligned");
  if (m > 0) {
    FP4RL_REQUIRE(x && y, FP4RL_ERR_NULL, "x and y must be non-NULL");
    FP4RL_REQUIRE(aligned(x, 16) && aligned(y, 16), FP4RL_ERR_ALIGN, "x and y must be 16-byte aligned");
  }
  FP4RL_REQUIRE(w_noise_out == nullptr || aligned(w_noise_out, 16), FP4RL_ERR_ALIGN,
                "w_noise_out must be 16-byte aligned");
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_aqn_rmsnorm(x, m, d, w, sigma, seed, step, norm_id, eps, y, w_noise_out, stream),
                  "aqn_rmsnorm");
}

fp4rl_status fp4rl_philox_words(uint64_t seed, uint64_t step, uint32_t norm_id, int64_t n_blocks, uint32_t* out,
                                fp4rl_stream stream) {
  FP4RL_REQUIRE(n_blocks >= 0 && n_blocks <= ((int64_t)1 << 32), FP4RL_ERR_SHAPE, "n_blocks out of range");
  if (n_blocks == 0) return ok();
  FP4RL_REQUIRE(out != nullptr, FP4RL_ERR_NULL, "out is NULL");
  FP4RL_REQUIRE(aligned(out, 16), FP4RL_ERR_ALIGN, "out must be 16-byte aligned");
  FP4RL_CHECK(check_device());
  return launched(fp4rl::launch_philox_words(seed, step, norm_id, n_blocks, out, stream), "philox_words");
}

}  // extern "C"
