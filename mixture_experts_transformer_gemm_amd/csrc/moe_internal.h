// Internal declarations shared by the HIP translation units of the MoE layer.
// Not part of the public ABI (that is include/grok_moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace gmoe {

// Raises kernel `fn`'s dynamic LDS limit to `bytes` on the current device,
// once per device (the attribute belongs to the device's copy of the
// kernel); `done` is the caller's per-kernel bit set of devices 0..63.
// Thread-safe: a race sets the attribute twice, which is harmless.
inline hipError_t set_lds_limit(const void* fn, int bytes, std::atomic<unsigned long long>& done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const unsigned long long bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return err;
}

// Raw bf16 values travel as uint16_t bit patterns.
typedef uint16_t bf16_bits;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed pair of bf16 (lo in the low half), rounded to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950 (what the compiler emits for the
// __bf16 conversions), where a software rounding takes five instructions
// per pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Exact-erf GELU: z * Phi(z) (Phi the standard normal CDF, Phi(z) = erfc(-z / sqrt 2) / 2), with the
// tail Phi(-|z|) = 1 - Phi(|z|) from the rational-times-density approximation of Abramowitz and
// Stegun, 26.2.17 (after Hastings): Phi(-x) = phi(x) t (b1 + t (b2 + t (b3 + t (b4 + t b5)))),
// t = 1 / (1 + 0.2316419 x), x >= 0, absolute error below 7.5e-8; Phi(|z|) = 1 - Phi(-|z|). The
// density phi(x) = e^(-x^2 / 2) / sqrt(2 pi) is one v_exp_f32 of an FMA (1 / sqrt(2 pi) folded into
// the exponent). Branch-free: one v_rcp_f32, four FMAs for the polynomial, one v_exp_f32 (about 1 ulp
// each), where the device library's erff costs about 70 instructions with divergent range branches.
// Evaluated in fp32 against the fp64 GELU: absolute error below 3e-7 max(1, |z|), relative below
// 1e-6 for z >= 0; the far negative tail, where GELU is below 1e-7 in magnitude, is exact only
// to that absolute bound. H is rounded to bf16 after it, a relative step of 2^-9.
__device__ __forceinline__ float gelu_erf(float z) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2316419f, fabsf(z), 1.0f));
  float p = 1.330274429f;
  p = fmaf(p, t, -1.821255978f);
  p = fmaf(p, t, 1.781477937f);
  p = fmaf(p, t, -0.356563782f);
  p = fmaf(p, t, 0.319381530f);
  // phi(z) = 2^(-z^2 log2(e) / 2 - log2(sqrt(2 pi)))
  const float phi = __builtin_amdgcn_exp2f(fmaf(z * z, -0.72134752044448170f, -1.32574806473615930f));
  const float q = t * p * phi;  // Phi(-|z|)
  return z * (z >= 0.0f ? 1.0f - q : q);
}

// SiLU: z * sigmoid(z) = z / (1 + e^-z), with v_exp_f32 and v_rcp_f32 (about 1 ulp each; z -> -inf
// gives e^-z = inf and -0).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// Activation of the gate branch: ACT_GELU (Grok-1's GeGLU experts) or ACT_SILU
// (SwiGLU experts). The flag is uniform over a launch.
enum { ACT_GELU = 0, ACT_SILU = 1 };
__device__ __forceinline__ float glu_act(int act, float z) { return act == ACT_SILU ? silu(z) : gelu_erf(z); }

// Device view of the routing produced by the permutation stage.
struct RouteView {
  const int32_t* counts;   // [E] rows per expert
  const int32_t* offsets;  // [E+1] first row of each expert segment
  const int32_t* perm;     // [k*T] row -> token
  // tiled path only (else null): tiles of BM rows, experts in order
  const int32_t* tile_off;  // [E+1] first tile of each expert; tile_off[E] = tiles
  const int32_t* tile_e;    // [tiles] expert of each tile
};

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `stream` and return the launch status.

// Routing over E <= 64 experts in one kernel. Writes idx/gate [T][k + ns]:
// the k routed slots, then the ns shared experts E.. with gate 1.
// renorm: divide the k selected gates by their sum. bias (nullable, [E]):
// added to the probabilities for the choice only.
hipError_t launch_router(int act_f32, const void* x, const void* router_w, int64_t T, int d, int E, int k, int ns,
                         int renorm, const float* bias, int32_t* idx, float* gate, hipStream_t stream);

// The same for E > 64 (bf16): split-K fp64 logit GEMM into P [splits][T][E],
// then one wavefront per token for softmax and top-k. d / splits must be a
// multiple of 64.
hipError_t launch_router_many(const bf16_bits* x, const bf16_bits* router_w, int64_t T, int d, int E, int k, int ns,
                              int renorm, const float* bias, int splits, double* P, int32_t* idx, float* gate,
                              hipStream_t stream);

// Caller routing [T][k] -> idx/gate [T][k + ns] with the shared slots.
hipError_t launch_append_shared(const int32_t* ridx, const float* rgate, int64_t T, int E, int k, int ns,
                                int32_t* idx, float* gate, hipStream_t stream);

// E experts, k slots per token. cap >= 0: an expert e < E_cap keeps its
// first `cap` assignments in token order, the others get pos = -1 and no
// row; cap < 0: no cap. E <= 272, k <= 12.
// tile_off[e] = sum over q < e of ceil(counts[q] / bm) (e <= E) and
// tile_e[m] = the expert of tile m, for the tile_off[E] <= mt_ub tiles
hipError_t launch_tile_table(const int32_t* counts, int E, int bm, int32_t* tile_off, int32_t* tile_e, int64_t mt_ub,
                             hipStream_t stream);
// blk: permute_scratch_ints(T, E) ints of scratch (per-block counts)
int64_t permute_scratch_ints(int64_t T, int E);
hipError_t launch_permute(const int32_t* idx, int64_t T, int E, int k, int64_t cap, int E_cap, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* blk, hipStream_t stream);

// out[t] = sum_s gate[t][s] * (sum_{p<S} Y[p][pos[t][s]]), Y: [S][rows_cap][d] fp32
hipError_t launch_combine(int out_f32, const float* Y, int S, int64_t rows_cap, const int32_t* pos,
                          const float* gate, int64_t T, int d, int k, void* out, hipStream_t stream);

// u[t] = RMSNorm(x[t]; g, eps), computed in fp64 and rounded once to the
// activation type (bf16 RNE, or fp32).
hipError_t launch_rmsnorm(int act_f32, const void* x, const void* g, int64_t T, int d, double eps, void* u,
                          hipStream_t stream);

// Sandwich epilogue: y[t] = the gated sum of combine (fp32), then
// out[t] = x[t] + RMSNorm(y[t]; g_post, eps), one rounding to the output type.
hipError_t launch_combine_sandwich(int out_f32, const float* Y, int S, int64_t rows_cap, const int32_t* pos,
                                   const float* gate, int64_t T, int d, int k, const void* x, const void* g_post,
                                   double eps, void* out, hipStream_t stream);

// Weight-streaming path: bf16 weights with every expert segment <= max_rows
// <= 64 rows, or 8-bit weights (w8, scales) with segments processed in
// chunks of up to 128 rows. splits > 1: the gate/up reduction runs in that
// many slices whose fp32 sums go to G [splits][rows_cap][2f] (gate channels,
// then up channels), and a second kernel forms H from them.
hipError_t launch_stream_gateup(int w8, int max_rows, int splits, const bf16_bits* x, RouteView rv, const void* wg,
                                const void* wu, const float* scales, int64_t T, int64_t rows_cap, int d, int f, int E,
                                int act, bf16_bits* H, float* G, hipStream_t stream);
hipError_t launch_stream_down(int w8, int max_rows, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                              const float* scales, int64_t rows_cap, int d, int f, int E, float* Y,
                              hipStream_t stream);

// Large-M path (LDS-tiled MFMA grouped GEMM).
// bm: rows per workgroup tile (64, 128 or 256).
hipError_t launch_tiled_gateup(int w8, int bm, const bf16_bits* x, RouteView rv, const void* wg, const void* wu,
                               const float* scales, int64_t T, int64_t rows_cap, int d, int f, int E, int act,
                               bf16_bits* H, hipStream_t stream);
// splits: partial sums over equal slices of the reduction (Y holds `splits` of them).
hipError_t launch_tiled_down(int w8, int bm, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                             const float* scales, int64_t rows_cap, int d, int f, int E, float* Y,
                             hipStream_t stream);

// Large-M path with bf16 weights: the ping-pong grouped GEMM (320-row tiles;
// the tile table must be built for 320 rows).
hipError_t launch_pp_gateup(const bf16_bits* x, RouteView rv, const bf16_bits* wg, const bf16_bits* wu, int64_t T,
                            int64_t rows_cap, int d, int f, int E, int act, bf16_bits* H, hipStream_t stream);
hipError_t launch_pp_down(int splits, const bf16_bits* H, RouteView rv, const bf16_bits* wd, int64_t rows_cap, int d,
                          int f, int E, float* Y, hipStream_t stream);

// fp32 path (plain FMA kernels, fp32 accumulation).
hipError_t launch_f32_gateup(const float* x, RouteView rv, const float* wg, const float* wu, int64_t T,
                             int64_t rows_cap, int d, int f, int E, int act, float* H, hipStream_t stream);
hipError_t launch_f32_down(const float* H, RouteView rv, const float* wd, int64_t rows_cap, int d, int f, int E,
                           float* Y, hipStream_t stream);

}  // namespace gmoe
