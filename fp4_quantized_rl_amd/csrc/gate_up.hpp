// Host-side launcher of the fused gate/up projections with the SiLU-gated
// product (internal to libfp4rl); arguments are validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4rl {

constexpr int64_t kGateUpMaxTokens = 128;
// Up to this many tokens the two projections run fused in one launch; above,
// as two separate linears and the gated product (measured, 7B gate/up, graph
// replays over 4 weight copies: fused 28.4 / 29.9 us at 1 / 8 tokens against
// 27.6 / 29.7 for the two linears alone; at 32 / 64 / 128 tokens fused 48.4 /
// 74.2 / 143.8 against 44.5 / 57.0 / 84.1 for the linears and the product).
constexpr int64_t kGateUpFusedMaxTokens = 16;
// h[i] = bf16(SiLU(g[i]) * u[i]) for bf16 g, u (count elements)
hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, int64_t count, uint16_t* h, hipStream_t stream);
// token tiles of 16 per launch for m tokens (1, 2, 4 or 8)
int gate_up_token_tiles(int64_t m);
// fp32 workspace bytes: the K-slices of t_g and t_u (and their sums above 16 tokens)
size_t gate_up_workspace(int64_t m, int64_t k, int64_t r);
hipError_t launch_gate_up(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* cg, const uint8_t* sg,
                          const float* stg, const uint8_t* cu, const uint8_t* su, const float* stu,
                          const uint16_t* ag, const uint16_t* bg, const uint16_t* au, const uint16_t* bu, int64_t r,
                          float s, float* ws, uint16_t* h, hipStream_t stream);

// The AQN RMSNorm of x folded in: the noisy weight (k fp32) and r_m (m fp32)
// in the workspace, then t_g and t_u (m r fp32 each); the normalised tokens
// are never stored. k <= the norm's width limit, k % 16 == 0.
size_t aqn_gate_up_workspace(int64_t m, int64_t k, int64_t r);
hipError_t launch_aqn_gate_up(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w, float sigma,
                              uint64_t seed, uint64_t step, uint32_t norm_id, float eps, const uint8_t* cg,
                              const uint8_t* sg, const float* stg, const uint8_t* cu, const uint8_t* su,
                              const float* stu, const uint16_t* ag, const uint16_t* bg, const uint16_t* au,
                              const uint16_t* bu, int64_t r, float s, void* ws, uint16_t* h, hipStream_t stream);

// The AQN RMSNorm of x folded into one NVFP4 + LoRA linear (e.g. qkv):
// y = bf16(s_t x_n deq(W)^T + s (x_n A^T) B^T), x_n = bf16(x r_m w_noise),
// never stored. Workspace: the noisy weight (k fp32), r_m (m fp32), then the
// K-slices of t (m r fp32 each). k <= the norm's width limit, k % 16 == 0.
size_t aqn_linear_workspace(int64_t m, int64_t k, int64_t r);
hipError_t launch_aqn_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w, float sigma,
                             uint64_t seed, uint64_t step, uint32_t norm_id, float eps, const uint8_t* codes,
                             const uint8_t* scales, const float* ts, const uint16_t* a, const uint16_t* b, int64_t r,
                             float s, void* ws, uint16_t* y, hipStream_t stream);

}  // namespace fp4rl
