// Host-side launchers of the gfx950 kernels (internal to libfp4rl).
// Arguments are already validated by the C ABI layer; each launcher queues
// its kernels on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4rl {

// ---- NVFP4 quantiser --------------------------------------------------
constexpr int kAmaxPartials = 1024;  // workgroups of the amax pass = partial maxima
size_t quantize_workspace_bytes();
int64_t nvfp4_codes_bytes(int64_t n, int64_t k, bool tiled);
int64_t nvfp4_scales_bytes(int64_t n, int64_t k, bool tiled);
// record: NULL, or the rounding record [n][k/8] (bit e of byte j: element 8j+e rounded up in magnitude)
hipError_t launch_quantize(const void* w, bool w_bf16, int64_t n, int64_t k, bool tiled, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, uint8_t* record, uint32_t* partial,
                           hipStream_t stream);
hipError_t launch_to_tiled(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, uint8_t* codes_t,
                           uint8_t* scales_t, hipStream_t stream);

// ---- AQN ----------------------------------------------------------------
constexpr int64_t kAqnMaxD = 16384;  // noise vector lives in LDS (64 KB)
hipError_t launch_aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, const float* w, float sigma,
                              uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                              uint16_t* y, float* w_noise_out, hipStream_t stream);
hipError_t launch_philox_words(uint64_t seed, uint64_t step, uint32_t norm_id, int64_t n_blocks,
                               uint32_t* out, hipStream_t stream);

// ---- LoRA linear ----------------------------------------------------------
constexpr int64_t kMaxRank = 256;
// K-split of the LoRA down-projection: `slices` partial sums [slices][m][r].
int lora_splits(int64_t m, int64_t k, int64_t r);
// FP8 (E4M3 row-major [n][k], fp32 row scales) decode main launch over
// s = fp8_splitk_slices K ranges: with s == 1 it stores y = bf16(s_n sum +
// t B^T) (t: tks K-slices [tks][m][r], or r == 0); otherwise fp32 partials
// part[s][m][n] = s_n * (sum over K range s), left for a finishing launch.
// tok_scale (W8A8): x holds E4M3 token codes as bf16, sums times xs[m].
int fp8_splitk_slices(int64_t m, int64_t n, int64_t k);
// y[m][n] = bf16(sum_z part[z][m][n] + sum_j t[m][j] B[n][j]) (t: tks K-slices [tks][m][r], summed in order;
// t and b may be NULL with r == 0): the finishing launch of split contractions.
hipError_t launch_partials_finish(const float* part, int slices, int64_t m, int64_t n, const float* t, int tks,
                                  const uint16_t* b, int64_t r, uint16_t* y, hipStream_t stream);
hipError_t launch_fp8_splitk(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                             const float* scales, const float* t, int tks, const uint16_t* b, int64_t r, uint16_t* y,
                             float* part, const float* tok_scale, hipStream_t stream);
int lora_slices(int64_t k, int splits);
hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* a, int64_t r, float lora_scale,
                            int splits, float* part, hipStream_t stream);
hipError_t launch_lora_reduce(const float* part, int slices, int64_t count, float* t, hipStream_t stream);
const char* fp4_linear_kernel_name(int64_t m, int64_t n, int64_t k, int64_t r);
// Linear workspaces begin with kLinearCounters counter words: one per output
// tile of a K-split launch (K is split only when there are at most
// kSplitCounters tiles), then the fused LoRA hand-off words. They must be
// zero before the first call, and every launch leaves them at zero. The
// other regions (t slices, K-split partials) follow and never overlap the
// counters, whatever shapes share the workspace.
constexpr int kSplitCounters = 1024;     // words [0, 1024): K-split tile counters
constexpr int kLoraTileCounters = 128;   // words [1024, 1152): one per 16x16 tile of t (m <= 128, r <= 256)
constexpr int kLoraTileCtrOffset = 1024;
constexpr int kLoraDoneOffset = 1152;    // word 1152: finished tiles of t
constexpr int kLinearErrOffset = 1156;   // word 1156: sticky device-side error bits (kLinearErr*)
constexpr uint32_t kLinearErrLoraWait = 1u;  // a consumer gave up waiting for t (see LoraFuse::spin)
constexpr int kLoraGroups = 64;          // ready flags: one 256-byte line per group of output tiles
constexpr int kLoraLineWords = 64;
constexpr int kLoraLineOffset = 1280;    // line g: words 1280 + 64 g (flag), + 1 (count)
constexpr int kLinearCounters = kLoraLineOffset + kLoraGroups * kLoraLineWords;
constexpr size_t kLinearCounterBytes = kLinearCounters * sizeof(uint32_t);

// LoRA down-projection fused into a main-kernel launch. The first
// `producers` workgroups of the grid each compute one K-slice of one 16x16
// tile of t into part[slice]; the last producer of a tile (counted in
// tctr[tile]) adds its slices in slice order into part[0], clears tctr[tile]
// and counts the finished tile in done[0]; the producer that finishes the
// last tile clears done[0] and raises the ready flag of every group's line.
// The workgroup that writes output tile i of y (the last of its K split)
// belongs to group i % groups; it waits (a bounded wait) for its group's
// flag just before its epilogue, then counts itself on that line, and the
// group's last one clears the line. Spreading the consumers over many lines
// keeps same-address atomics few. Producers have the lowest workgroup ids
// and never wait on consumers, so they are dispatched first and always
// finish. Flags and counters are agent-scope relaxed atomics; t itself is
// written and read only with agent-coherent (sc1) accesses, after a
// vmcnt(0) wait on the writer's side and behind the flag read (a dependent
// branch and a barrier) on the reader's side, so a reader sees the data
// without acquire/release cache maintenance (an L2 invalidate per output
// workgroup, measured 13.1 -> 20.5 us for the 7B gate at one token). A
// consumer that gives up after `spin` polls sets kLinearErrLoraWait in the
// workspace's error word, which stays set (every later call on that
// workspace is then suspect) until the caller clears the counter words.
struct LoraFuse {
  const uint16_t* a = nullptr;  // A [r][K]; nullptr: no fused producers (t ready-made, or r == 0)
  float s = 0.0f;               // lora_scale
  int kslice = 0, slices = 0;   // k per slice (a multiple of 32), number of slices (<= 8)
  int mtiles = 0, rtiles = 0;   // 16x16 tiles of t
  int producers = 0;            // producer workgroups (a multiple of 8, so the grid's XCD order is kept)
  int consumers = 0;            // set by the launcher: output tiles of y (one waiting workgroup each)
  int groups = 0;               // set by the launcher: min(kLoraGroups, consumers)
  float* part = nullptr;        // t slices [slices][M][r]; t itself ends up in slice 0
  uint32_t* tctr = nullptr;     // per-tile slice counters (mtiles * rtiles <= kLoraTileCounters)
  uint32_t* done = nullptr;     // finished tiles of t
  uint32_t* lines = nullptr;    // kLoraGroups lines of kLoraLineWords words, word 0 the ready flag
  uint32_t* err = nullptr;      // the workspace's sticky error word
  uint32_t spin = 1u << 22;     // polls (each after a short sleep) before a consumer gives up
  uint32_t withhold = 0;        // test hook: the producers leave the ready flags down
  uint32_t epoch = 1;           // this call's ready value (never 0, new for every call): a flag left raised by
                                // an earlier call never satisfies this one
};

// whether the main kernel chosen for this shape runs fused LoRA producers
bool linear_fuses_lora(int64_t m, int64_t n, int64_t k);
int64_t lora_slice_len(int64_t k, int splits);
// fp32 K-split partial sums of the main kernel (0 when K is not split)
size_t linear_partial_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_fp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const float* t, int tks, const uint16_t* b, int64_t r, uint16_t* y, float* part,
                             uint32_t* counters, LoraFuse lf, hipStream_t stream);

}  // namespace fp4rl
