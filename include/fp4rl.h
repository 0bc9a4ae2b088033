/*
 * fp4rl.h — C ABI of the NVFP4 + LoRA + AQN rollout hot path for MI355X (gfx950).
 *
 * Three operations make up the quantised rollout forward that QeRL describes:
 *
 *   fp4rl_nvfp4_quantize   NVFP4 block quantiser of a frozen weight matrix
 *                          (QeRL explainer page, "NVFP4 quantization and LoRA";
 *                          TRACE article, "Engineering view of the mechanism":
 *                          small groups share one scale, each value rounds up or
 *                          down to a grid point).
 *   fp4rl_fp4_lora_linear  W4A16 linear with the LoRA update fused in,
 *                          y = x deq(Wq)^T + s (x A^T) B^T (QeRL explainer,
 *                          "NVFP4 quantization and LoRA" and "Experimental
 *                          details": NVFP4 weights with 16-bit LoRA, rollout
 *                          through a W4A16 kernel).
 *   fp4rl_aqn_rmsnorm      RMSNorm whose scale carries the adaptive quantisation
 *                          noise, W_noise = Z_noise + w (QeRL explainer, "Adaptive
 *                          Quantization Noise": the exponential scheduler and the
 *                          zero-overhead fold into the norm, with its equation).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked [host]. Array pointers must be
 *    16-byte aligned (tensor_scale: 4-byte); otherwise FP4RL_ERR_ALIGN.
 *  - Matrices are dense row-major. bf16 is passed as uint16_t bit patterns.
 *  - The caller owns every buffer, workspaces included. The library allocates
 *    and frees nothing, keeps no state across calls except a per-device
 *    "is gfx950" flag, and never synchronises: work is queued on `stream`
 *    (NULL = the legacy default stream) and the call returns at once.
 *  - Arguments are validated before anything is queued; on error nothing is
 *    written and a non-zero status is returned, with a detail string in
 *    fp4rl_last_error() (thread-local). A failed launch returns FP4RL_ERR_HIP.
 *    Device faults surface at the caller's next synchronisation, as in HIP.
 *  - Sizes are int64_t; a size of 0 is an empty no-op (OK).
 *  - Outputs must not alias inputs. Results for non-finite inputs are
 *    unspecified (the quantiser then writes a non-finite tensor scale).
 *  - Calls on different streams are independent; the library is thread-safe.
 *  - Every result is deterministic: no floating-point atomics are used, so
 *    repeated calls on the same inputs give identical bytes.
 */
#ifndef FP4RL_H
#define FP4RL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4RL_ABI_VERSION 1

/* Same object as HIP's hipStream_t. */
typedef struct ihipStream_t* fp4rl_stream;

typedef enum fp4rl_status {
  FP4RL_OK = 0,
  FP4RL_ERR_NULL = 1,      /* a required pointer is NULL */
  FP4RL_ERR_SHAPE = 2,     /* negative size, k not a multiple of 16, r > 256, d too large */
  FP4RL_ERR_DTYPE = 3,     /* unknown dtype code */
  FP4RL_ERR_ALIGN = 4,     /* pointer not aligned as stated above */
  FP4RL_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the matching *_workspace() size */
  FP4RL_ERR_ARCH = 6,      /* the current device is not gfx950 */
  FP4RL_ERR_HIP = 7,       /* a HIP runtime call failed; text in fp4rl_last_error() */
  FP4RL_ERR_VALUE = 8,     /* a scalar is out of range (negative or non-finite sigma/eps/scale) */
  FP4RL_ERR_TIMEOUT = 9    /* reported by fp4rl_linear_workspace_check: a fused launch on that workspace
                              gave up waiting for its in-launch LoRA producers */
} fp4rl_status;

typedef enum fp4rl_dtype { FP4RL_F32 = 0, FP4RL_BF16 = 1 } fp4rl_dtype;

/* [host] Static name of a status code. */
const char* fp4rl_status_string(int32_t status);
/* [host] Detail of the last failed call on this thread ("" if none). */
const char* fp4rl_last_error(void);
/* [host] FP4RL_ABI_VERSION of the built library. */
int32_t fp4rl_abi_version(void);

/* ------------------------------------------------------------------------
 * NVFP4 quantiser.
 *
 * W [n][k] (fp32 or bf16, w_dtype) -> codes, scales, tensor_scale [1] fp32.
 * k % 16 == 0; n * k < 2^36.
 *   s_t  = fp32(amax / 2688), amax = max|W| (2688 = 6 * 448);
 *   byte = E4M3 (OCP e4m3fn, nearest-even, saturating at 448, subnormals kept)
 *          of r_b = fp32(a_b / fp32(6 s_t)), a_b = max|block|; 0 if s_t == 0;
 *   code = sign(x) << 3 | k, where g_k * fp32(S_b s_t) is the E2M1 grid point
 *          {0,.5,1,1.5,2,3,4,6} nearest to |x| in exact arithmetic, ties to even k.
 * Blocks are 16 consecutive elements of a row (along k).
 * Layouts (fp4rl_nvfp4_codes_bytes / _scales_bytes give the sizes):
 *   FP4RL_ROW_MAJOR  codes [n][k/2] (element 2j = low nibble of byte j),
 *                    scales [n][k/16].
 *   FP4RL_TILED      the operand layout of the linear kernels: 16-row x 128-k
 *                    tiles, tile (rt, c) at index rt * ceil(k/128) + c, each
 *                    1024 code bytes + 128 scale bytes. Inside a tile, the
 *                    16 code bytes at offset 16 * (16 g + i) (g = 0..3,
 *                    i = 0..15) hold row 16 rt + i: their 4-byte word j
 *                    (j = 0..3) holds k = 128 c + 32 j + 8 g .. + 7, low nibble
 *                    first. The scale word at byte 4 * (16 p + i) (p = 0, 1)
 *                    holds in its byte j the scale of row 16 rt + i, block
 *                    8 c + 2 j + p. Rows >= n and k >= k of partial tiles are
 *                    zero.
 * Two HBM passes (W is read twice): a tensor-amax pass that leaves
 * per-workgroup partial maxima in the workspace (no atomics), and an encode
 * pass. Workspace: fp4rl_nvfp4_quantize_workspace(n, k) bytes, 16-byte aligned.
 * fp4rl_nvfp4_to_tiled repacks a row-major NVFP4 matrix into the tiled layout.
 * ---------------------------------------------------------------------- */
typedef enum fp4rl_layout { FP4RL_ROW_MAJOR = 0, FP4RL_TILED = 1 } fp4rl_layout;

size_t fp4rl_nvfp4_quantize_workspace(int64_t n, int64_t k);
size_t fp4rl_nvfp4_codes_bytes(int64_t n, int64_t k, int32_t layout);
size_t fp4rl_nvfp4_scales_bytes(int64_t n, int64_t k, int32_t layout);
fp4rl_status fp4rl_nvfp4_quantize(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                  uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                  void* workspace, size_t workspace_bytes, fp4rl_stream stream);
fp4rl_status fp4rl_nvfp4_to_tiled(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                  uint8_t* codes_tiled, uint8_t* scales_tiled, fp4rl_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid
 * hipMalloc): fp4rl_nvfp4_quantize with the workspace replaced by a
 * library-owned device array (the amax pass's 1024 partial maxima, 4 KB; the
 * same for every shape, so no shape is rejected for its size). Same
 * arguments otherwise, same results byte for byte, same errors. It calls no
 * allocating routine. Each GPU holds one copy of the array until the process
 * ends, looked up on that GPU's first call; calls that overlap on one GPU
 * (several streams or threads) race on it. */
fp4rl_status fp4rl_nvfp4_quantize_noalloc(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                          uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                          fp4rl_stream stream);

/* Quantise as fp4rl_nvfp4_quantize (same codes, scales and tensor scale, same
 * arguments and errors) and also write the rounding record the rollout side
 * keeps for the trainer (TRACE article, "TRACE's core idea" and "Engineering
 * view of the mechanism": each value is rounded up or down to a neighbouring
 * grid point, and the trainer replays the rollout's choices from a compact
 * record; the pages leave the format open).
 * round_up [n][k/8] bytes, row-major in both layouts, any alignment, owned by
 * the caller: bit e (LSB first) of byte j of row i is 1 when element
 * 8 j + e was rounded up in magnitude, i.e. g_k * fp32(S_b s_t) > |x| for its
 * code; 0 when rounded down or exact, and in blocks with fp32(S_b s_t) == 0.
 * With the scale bytes this fixes the grid neighbours of every value.
 * round_up == NULL with n, k > 0: FP4RL_ERR_NULL. */
fp4rl_status fp4rl_nvfp4_quantize_record(const void* w, int32_t w_dtype, int64_t n, int64_t k, int32_t layout,
                                         uint8_t* codes, uint8_t* scales, float* tensor_scale, uint8_t* round_up,
                                         void* workspace, size_t workspace_bytes, fp4rl_stream stream);

/* ------------------------------------------------------------------------
 * Fused W4A16 + LoRA linear:
 *   y[m][n] = bf16_rne( s_t * sum_k x[m][k] g(code[n][k]) S_b(n,k)
 *                       + sum_j t[m][j] B[n][j] ),   t = lora_scale * x A^T.
 * x bf16 [m][k]; codes/scales/tensor_scale of an [n][k] matrix in the
 * FP4RL_TILED layout; A bf16 [r][k]; B bf16 [n][r]; y bf16 [m][n].
 * k % 16 == 0; m * k < 2^31 (< 2^30 for 3 <= m <= 128); 0 <= r <= 256;
 * r == 0 or lora_a == lora_b ==
 * NULL means no LoRA term. Accumulation is fp32; the output is rounded once
 * to bf16.
 * For m <= 128 one launch does all of it: its first workgroups compute
 * t = lora_scale * x A^T (in K slices; the last slice of each 16x16 tile of t
 * to finish adds the slices) and the others wait for t only before their
 * epilogue. For m > 128 the LoRA down-projection (when r > 0) and then the
 * main kernel are launched. The main kernel is chosen by m (see
 * fp4rl_fp4_linear_kernel_name).
 * Workspace: fp4rl_fp4_lora_linear_workspace(m, n, k, r) bytes (0 when
 * neither split below is used), 16-byte aligned. It starts with 5376
 * counter words (21 KB: K-split tile counters, then the hand-off words of the
 * in-launch LoRA producers, spread over 64 lines of 256 bytes so that few
 * workgroups share an atomic address); then come the K-split partial sums of
 * t and, for shapes with
 * few output tiles, the main kernel's K-split partial sums of y (the last
 * workgroup of a tile to finish, found through its counter, adds them). All
 * partial sums are added in a fixed order, so results do not depend on
 * scheduling. The counter words must be zero before the first call (e.g. a
 * zero-filled workspace); every call returns them to zero and no other data
 * is ever stored there, so one workspace, sized for the largest call, serves
 * any sequence of linear calls and shapes (but not calls that run at the
 * same time).
 * ---------------------------------------------------------------------- */
size_t fp4rl_fp4_lora_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r);
fp4rl_status fp4rl_fp4_lora_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                   const uint8_t* codes, const uint8_t* scales,
                                   const float* tensor_scale, const uint16_t* lora_a,
                                   const uint16_t* lora_b, int64_t r, float lora_scale,
                                   uint16_t* y, void* workspace, size_t workspace_bytes,
                                   fp4rl_stream stream);

/* Health of a linear workspace's in-launch hand-off (QeRL explainer,
 * "NVFP4 quantization and LoRA": t = s x A^T feeds the LoRA term of the same
 * fused forward). The output workgroups of a fused launch wait for the
 * launch's own producer workgroups to finish t; the wait is bounded (about
 * 2^22 polls), so a producer that never finishes cannot hang the GPU. A
 * consumer that gives up sets an error bit in the workspace's counter words
 * and computes with whatever t holds; that call's output is wrong. Later
 * calls are not affected: each fused call raises its ready flags to a value
 * of its own (a process-wide call counter, never 0), so a flag that an
 * earlier call's producer raised after its consumers had given up never
 * releases a later call's consumers. The bit stays set until the counter
 * words are cleared, so a check reports a timeout of any call since the
 * last reset.
 * fp4rl_linear_workspace_check: synchronises `stream`, then reads the bit;
 *   FP4RL_OK, or FP4RL_ERR_TIMEOUT (detail in fp4rl_last_error()).
 *   workspace == NULL or workspace_bytes == 0: FP4RL_OK (no hand-off).
 *   workspace_bytes smaller than the counter words: FP4RL_ERR_WORKSPACE.
 * fp4rl_linear_workspace_reset: queues a fill kernel (no memset, so it may
 *   be captured in a HIP graph) that zeroes the counter words: the state of
 *   a fresh zero-filled workspace. Does not synchronise. */
fp4rl_status fp4rl_linear_workspace_check(const void* workspace, size_t workspace_bytes, fp4rl_stream stream);
fp4rl_status fp4rl_linear_workspace_reset(void* workspace, size_t workspace_bytes, fp4rl_stream stream);
/* [host] Test hook of the hand-off above, process-wide, read when a fused
 * launch is queued: consumers give up after spin_limit polls (0 restores
 * the default), and with withhold_ready != 0 the producers compute t but
 * leave the ready flags down, so every consumer gives up and every kernel
 * still ends normally. For tests of the error path only. */
void fp4rl_debug_lora_handoff(uint32_t spin_limit, int32_t withhold_ready);

/* The two halves of fp4rl_fp4_lora_linear, for callers that produce t
 * elsewhere or time the main kernel alone.
 * fp4rl_lora_down: t [m][r] fp32 = lora_scale * x A^T (fp32 accumulate). For
 *   decode-shaped m the product is split along k over many workgroups; the
 *   partial sums go to the workspace (fp4rl_lora_down_workspace bytes, 0 when
 *   no split is used) and are added in a fixed order, so t is deterministic.
 * fp4rl_fp4_linear_lora_up: y = bf16(s_t * x deq^T + t B^T); t may be NULL
 *   (with r == 0) for the base product alone. Workspace:
 *   fp4rl_fp4_linear_lora_up_workspace(m, n, k) bytes (0 for most shapes),
 *   laid out and reused as fp4rl_fp4_lora_linear's (counter words first). */
size_t fp4rl_lora_down_workspace(int64_t m, int64_t k, int64_t r);
fp4rl_status fp4rl_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a,
                             int64_t r, float lora_scale, float* t, void* workspace,
                             size_t workspace_bytes, fp4rl_stream stream);
size_t fp4rl_fp4_linear_lora_up_workspace(int64_t m, int64_t n, int64_t k);
fp4rl_status fp4rl_fp4_linear_lora_up(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                      const uint8_t* codes, const uint8_t* scales,
                                      const float* tensor_scale, const float* t,
                                      const uint16_t* lora_b, int64_t r, uint16_t* y,
                                      void* workspace, size_t workspace_bytes, fp4rl_stream stream);

/* [host] Name of the main-kernel instantiation the linear launches for this
 * shape and rank, as a demangler prints its template arguments (e.g.
 * "gemv_kernel<1, 8, 8>", "skinny_kernel<4, 2, 8>"), so profiles can be
 * matched to calls. Returns a static string; "" for invalid shapes. Touches
 * no device. Kernels by m: a VALU GEMV (one or two tokens), an MFMA skinny
 * kernel (decode batches up to 128 per launch column). */
const char* fp4rl_fp4_linear_kernel_name(int64_t m, int64_t n, int64_t k, int64_t r);

/* ------------------------------------------------------------------------
 * LoRA backward through the frozen NVFP4 base (QeRL explainer, "NVFP4
 * quantization and LoRA": the quantised base stays frozen, only the
 * low-rank adapters are trained). For y = x deq(Wq)^T + s (x A^T) B^T and
 * the incoming gradient dy = dL/dy:
 *   dx     = dy deq(Wq) + s (dy B) A      bf16 [m][k] (rounded once, nearest-even)
 *   grad_a = s (dy B)^T x                 fp32 [r][k]
 *   grad_b = s dy^T (x A^T)               fp32 [n][r]
 * There is no gradient for the base.
 * Arguments: dy bf16 [m][n]; x bf16 [m][k] (read only when r > 0);
 *   codes/scales/tensor_scale: the weight in the tiled layout, as for
 *   fp4rl_fp4_lora_linear (read only when dx is set); lora_a bf16 [r][k] and
 *   lora_b bf16 [n][r], both NULL (r ignored) or both set.
 *   dx may be NULL (adapter gradients only, e.g. for a first layer); with no
 *   adapters dx is required.
 * Shapes: k a positive multiple of 16, n a multiple of 8, m, n and k below
 *   2^22, 0 <= r <= 256. m == 0 or n == 0 writes zeros where a sum is empty.
 * Workspace: fp4rl_fp4_lora_linear_backward_workspace(m, n, k, r, dx != NULL)
 *   bytes, 256-byte aligned, caller-owned, no initial contents needed. It
 *   holds the transposed dequantised weight (2 k n bytes, with dx); with
 *   adapters also dy and x transposed (2 (n + k) m bytes), the transposed
 *   adapters, t = s x A^T and h = s dy B split into bf16 pairs, and fp32
 *   partial products.
 * Errors: FP4RL_ERR_SHAPE, _NULL, _ALIGN, _VALUE (lora_scale not finite),
 *   _WORKSPACE; nothing is launched on error. Asynchronous on `stream`. */
size_t fp4rl_fp4_lora_linear_backward_workspace(int64_t m, int64_t n, int64_t k, int64_t r, int32_t want_dx);
fp4rl_status fp4rl_fp4_lora_linear_backward(const uint16_t* dy, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                            const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                            const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                                            float lora_scale, uint16_t* dx, float* grad_a, float* grad_b,
                                            void* workspace, size_t workspace_bytes, fp4rl_stream stream);

/* ------------------------------------------------------------------------
 * Gate and up projections with the SiLU-gated product, for decode batches.
 * The Qwen2.5 models QeRL trains (QeRL explainer, experiments) gate their
 * MLP: h = SiLU(gate) * up. Each projection is an NVFP4 + LoRA linear of the
 * same x (tiled layout, own tensor scale and adapters):
 *   g = x deq(Wg)^T + s (x Ag^T) Bg^T,  u likewise,  SiLU(v) = v / (1 + exp(-v)).
 * Up to 16 tokens both projections run in one launch and h = bf16(SiLU(g) u)
 *   with g and u unrounded (fp32). From 17 tokens on they run as two linears
 *   (as fp4rl_fp4_lora_linear) into bf16 g and u in the workspace and a
 *   third launch forms h = bf16(SiLU(g) u) from those rounded values; the
 *   fused launch is the slower one there (measured, 7B gate/up 18944 x 3584,
 *   r = 32, graph replays over 4 weight copies: fused 48.4 / 74.2 / 143.8 us
 *   against 44.5 / 57.0 / 84.1 at 32 / 64 / 128 tokens; at 1 token fused
 *   28.4 us, the two linears alone 27.6 plus about 3 for the product).
 * Arguments: x bf16 [m][k], 1 <= m <= 128 (else FP4RL_ERR_SHAPE); weights
 *   [n][k] each; adapters A [r][k], B [n][r] bf16, all four NULL or all
 *   set; h bf16 [m][n]. Shapes and alignment as for fp4rl_fp4_lora_linear.
 * Workspace: fp4rl_fp4_gate_up_silu_workspace(m, n, k, r) bytes, 256-byte
 *   aligned. It begins with 21 KB of counter words, as a linear workspace:
 *   zero before the first call (e.g. a zero-filled workspace), left zero by
 *   every call. Up to 16 tokens the fp32 K-slices of t for both projections
 *   follow (0 bytes in all without adapters); from 17 tokens the rest of a
 *   linear workspace, then g and u. One workspace, sized for the largest
 *   call, serves calls of either path in any order (not at the same time). */
size_t fp4rl_fp4_gate_up_silu_workspace(int64_t m, int64_t n, int64_t k, int64_t r);
fp4rl_status fp4rl_fp4_gate_up_silu(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* gate_codes,
                                    const uint8_t* gate_scales, const float* gate_tensor_scale,
                                    const uint8_t* up_codes, const uint8_t* up_scales, const float* up_tensor_scale,
                                    const uint16_t* lora_a_gate, const uint16_t* lora_b_gate,
                                    const uint16_t* lora_a_up, const uint16_t* lora_b_up, int64_t r,
                                    float lora_scale, uint16_t* h, void* workspace, size_t workspace_bytes,
                                    fp4rl_stream stream);

/* fp4rl_aqn_gate_up_silu: the fused projections with the AQN RMSNorm of x
 * folded in (QeRL explainer, "zero overhead: folding into layer
 * normalization"): x is the raw bf16 input [m][k]; the projections see
 * xn = bf16(x r_m (w + sigma z)), r_m = 1 / sqrt(mean_k x^2 + eps), z the
 * Philox normals of (seed, step, norm_id) as in fp4rl_aqn_rmsnorm (norm_w
 * fp32 [k], k <= 16384). xn is never stored: the LoRA down-projections and
 * the projections normalise their fragments as they load them, at every
 * token count (one fused launch, g and u unrounded). Three launches (noise
 * vector, normalising LoRA down-projection, gate/up). It removes the round
 * trip of xn through memory but is not faster than fp4rl_aqn_rmsnorm
 * followed by fp4rl_fp4_gate_up_silu: every workgroup renormalises the
 * fragments it loads (measured, 7B, graph replays: 41.8 vs 31.5 us at 1
 * token, 333.3 vs 91.7 at 128).
 * Workspace: fp4rl_aqn_gate_up_silu_workspace(m, n, k, r) bytes, 256-byte
 *   aligned, no initial contents needed. */
size_t fp4rl_aqn_gate_up_silu_workspace(int64_t m, int64_t n, int64_t k, int64_t r);
fp4rl_status fp4rl_aqn_gate_up_silu(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w,
                                    float sigma, uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                                    const uint8_t* gate_codes, const uint8_t* gate_scales,
                                    const float* gate_tensor_scale, const uint8_t* up_codes, const uint8_t* up_scales,
                                    const float* up_tensor_scale, const uint16_t* lora_a_gate,
                                    const uint16_t* lora_b_gate, const uint16_t* lora_a_up, const uint16_t* lora_b_up,
                                    int64_t r, float lora_scale, uint16_t* h, void* workspace,
                                    size_t workspace_bytes, fp4rl_stream stream);

/* fp4rl_aqn_lora_linear: one NVFP4 + LoRA linear (e.g. the attention's qkv
 * projection) with the AQN RMSNorm of x folded in (QeRL explainer, "zero
 * overhead: folding into layer normalization"):
 *   y = bf16(s_t xn deq(W)^T + s (xn A^T) B^T),  xn = bf16(x r_m (w + sigma z)),
 * r_m = 1 / sqrt(mean_k x^2 + eps), z the Philox normals of (seed, step,
 * norm_id) as in fp4rl_aqn_rmsnorm; xn is never stored. Three launches
 * (noise vector; normalising LoRA down-projection and r_m; the projection,
 * whose workgroups normalise the token fragments they load). The same
 * values as fp4rl_aqn_rmsnorm followed by fp4rl_fp4_lora_linear, up to the
 * order of the fp32 sums. It removes the round trip of xn through memory
 * but is slower than those two launches (measured, 7B qkv 4608 x 3584,
 * r = 32, graph replays: 25.8 vs 14.2 us at 1 token, 35.8 vs 18.9 at 32,
 * 89.5 vs 26.5 at 128): it takes three launches, and every workgroup
 * renormalises each fragment it loads.
 * Arguments: x bf16 [m][k] raw (not normalised), 1 <= m <= 128 (else
 *   FP4RL_ERR_SHAPE); norm_w fp32 [k], k <= 16384, k % 16 == 0; the weight
 *   [n][k] (tiled codes, scales, tensor scale); A [r][k], B [n][r] bf16, both
 *   NULL or both set; y bf16 [m][n]. Alignment as for fp4rl_aqn_gate_up_silu.
 * Workspace: fp4rl_aqn_lora_linear_workspace(m, n, k, r) bytes, 256-byte
 *   aligned, no initial contents needed (noise vector, r_m, K-slices of t). */
size_t fp4rl_aqn_lora_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r);
fp4rl_status fp4rl_aqn_lora_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w,
                                   float sigma, uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                                   const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                   const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float lora_scale,
                                   uint16_t* y, void* workspace, size_t workspace_bytes, fp4rl_stream stream);

/* ------------------------------------------------------------------------
 * FP8 rollout weights (gist.science summary of adaptive importance sampling
 * for quantized RL, "Problem definition" and "Experimental results": the
 * rollout engine runs in FP8 while the trainer keeps BF16, halving the
 * rollout model's memory). The page fixes no layout; this library's reading:
 * OCP E4M3 bytes [n][k] (bias 7, max 448, no -0 codes) and one fp32 scale per
 * output row, s_n = amax_n / 448 (0 for an all-zero row).
 * fp4rl_fp8_quantize: w fp32 or bf16 [n][k] -> codes [n][k], row_scales [n];
 *   code = nearest E4M3 value to the fp32 quotient w / s_n, ties to even,
 *   saturating at 448. k a positive multiple of 16, below 2^22.
 * fp4rl_fp8_lora_linear: y = bf16(x deq(W8)^T + s (x A^T) B^T), W8A16:
 *   x bf16 [m][k], deq(W8)[n][k] = e4m3(code) s_n, lora_a bf16 [r][k] and
 *   lora_b bf16 [n][r] (both NULL or both set), y bf16 [m][n]; m, n, k below
 *   2^22. Workspace: fp4rl_fp8_lora_linear_workspace(m, n, k, r) bytes,
 *   256-byte aligned, no initial contents needed (fp32 partial products).
 * fp4rl_fp8_lora_linear_w8a8: the same product with the tokens quantised
 *   too (W8A8; the page leaves activations open, this is the reading taken):
 *   each row m of x gets s_x[m] = amax_m / 448 and E4M3 codes exactly as
 *   fp4rl_fp8_quantize gives a bf16 weight row; then
 *   y = bf16(s_x[m] s_n sum_k e4m3(x8[m,k]) e4m3(code[n,k]) + s (x A^T) B^T),
 *   the LoRA term from the bf16 x. The products e4m3 x e4m3 are exact in
 *   fp32: up to 16 and above 64 tokens they run on the FP8 matrix cores, at
 *   17..64 tokens on the bf16 ones with both codes widened to bf16 exactly
 *   (the same values, fp32 accumulation). Arguments, limits and ownership
 *   as for fp4rl_fp8_lora_linear; its workspace,
 *   fp4rl_fp8_lora_linear_w8a8_workspace(m, n, k, r) bytes, also holds the
 *   token codes and scales (no initial contents needed).
 * Errors as for the NVFP4 calls; nothing is launched on error. */
fp4rl_status fp4rl_fp8_quantize(const void* w, int32_t w_dtype, int64_t n, int64_t k, uint8_t* codes,
                                float* row_scales, fp4rl_stream stream);
size_t fp4rl_fp8_lora_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r);
fp4rl_status fp4rl_fp8_lora_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                   const float* row_scales, const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                                   float lora_scale, uint16_t* y, void* workspace, size_t workspace_bytes,
                                   fp4rl_stream stream);
size_t fp4rl_fp8_lora_linear_w8a8_workspace(int64_t m, int64_t n, int64_t k, int64_t r);
fp4rl_status fp4rl_fp8_lora_linear_w8a8(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                                        const float* row_scales, const uint16_t* lora_a, const uint16_t* lora_b,
                                        int64_t r, float lora_scale, uint16_t* y, void* workspace,
                                        size_t workspace_bytes, fp4rl_stream stream);

/* ------------------------------------------------------------------------
 * AQN.
 * fp4rl_aqn_sigma [host]: sigma_k = sigma_start (sigma_end/sigma_start)^(k/(K-1)),
 *   computed in double and returned as float; K == 1 gives sigma_start.
 *   Returns NaN for K < 1, k outside [0, K), or non-positive sigmas.
 * fp4rl_aqn_rmsnorm: with z = PhiloxNormal(seed, step, norm_id)[0:d],
 *   w_noise[i] = w[i] + sigma z[i]                     (one vector per call)
 *   y[m][i]   = bf16_rne(w_noise[i] x[m][i] / sqrt(mean_i x[m][i]^2 + eps)).
 *   x, y bf16 [m][d]; w fp32 [d]; w_noise_out fp32 [d] or NULL.
 *   1 <= d <= 16384; sigma >= 0, eps >= 0, both finite. m == 0 with w_noise_out
 *   != NULL still writes the noisy weight.
 *   PhiloxNormal: Philox4x32-10 (Salmon et al., SC'11) of counter
 *   (q, norm_id, step_lo, step_hi) and key (seed_lo, seed_hi) gives words
 *   (o0..o3); each pair (a, b) in ((o0,o1), (o2,o3)) becomes
 *   u1 = ((a>>8)+1) 2^-24, u2 = (b>>8) 2^-24, rho = sqrt(-2 ln u1), and
 *   z[4q..4q+3] = (rho cos 2pi u2, rho sin 2pi u2) of pair 0, then of pair 1.
 * fp4rl_philox_words: the raw words of blocks q = 0..n_blocks-1, [n_blocks][4].
 * ---------------------------------------------------------------------- */
float fp4rl_aqn_sigma(float sigma_start, float sigma_end, int32_t k, int32_t num_stages);
fp4rl_status fp4rl_aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, const float* w,
                               float sigma, uint64_t seed, uint64_t step, uint32_t norm_id,
                               float eps, uint16_t* y, float* w_noise_out, fp4rl_stream stream);
fp4rl_status fp4rl_philox_words(uint64_t seed, uint64_t step, uint32_t norm_id, int64_t n_blocks,
                                uint32_t* out, fp4rl_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4RL_H */
