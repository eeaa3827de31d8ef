// fp32 grouped expert GEMMs of the Grok-1 MoE layer for gfx950 (MI355X).
//
// Expert e is a gated FFN (Grok-1 field guide, "MoE 子层"; Grok-1 book ch. 10,
// section 10.4): two input projections, GELU (SiLU for SwiGLU experts) on
// the gate branch, elementwise product, and a down projection. Rows are the expert-contiguous permutation
// of the tokens, so each expert is one segment of a grouped GEMM (book
// ch. 11, section 11.3.1: sparse reorder + grouped GEMM). Used for fp32
// activations and weights, where there is no bf16 MFMA to feed: plain fp32
// FMA, fp32 accumulation.
#include "moe_device.h"

namespace gmoe {

// =====================================================================
// fp32 path: plain fp32 FMA kernels, one output per thread.
// =====================================================================
__device__ __forceinline__ int expert_of_row(const RouteView& rv, int E, int row) {
  for (int q = 0; q < E; ++q)
    if (row < rv.offsets[q + 1]) return q;
  return -1;
}

__global__ __launch_bounds__(256) void f32_gateup_kernel(const float* __restrict__ x, RouteView rv,
                                                         const float* __restrict__ wg,
                                                         const float* __restrict__ wu, int64_t T,
                                                         int64_t rows_cap, int d, int f, int E, int act,
                                                         float* __restrict__ H) {
  const int64_t total = rows_cap * f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int row = (int)(i / f);
    const int n = (int)(i - (int64_t)row * f);
    if (row >= rv.offsets[E]) continue;
    const int e = expert_of_row(rv, E, row);
    if (e < 0) continue;
    int tok = rv.perm[row];
    tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
    const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)tok * d);
    const float4* gr = reinterpret_cast<const float4*>(wg + ((int64_t)e * f + n) * d);
    const float4* ur = reinterpret_cast<const float4*>(wu + ((int64_t)e * f + n) * d);
    float a = 0.f, b = 0.f;
    for (int c = 0; c < d / 4; ++c) {
      const float4 xv = xr[c], gv = gr[c], uv = ur[c];
      a = fmaf(xv.x, gv.x, a); a = fmaf(xv.y, gv.y, a); a = fmaf(xv.z, gv.z, a); a = fmaf(xv.w, gv.w, a);
      b = fmaf(xv.x, uv.x, b); b = fmaf(xv.y, uv.y, b); b = fmaf(xv.z, uv.z, b); b = fmaf(xv.w, uv.w, b);
    }
    H[(int64_t)row * f + n] = glu_act(act, a) * b;
  }
}

__global__ __launch_bounds__(256) void f32_down_kernel(const float* __restrict__ H, RouteView rv,
                                                       const float* __restrict__ wd, int64_t rows_cap, int d,
                                                       int f, int E, float* __restrict__ Y) {
  const int64_t total = rows_cap * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int row = (int)(i / d);
    const int n = (int)(i - (int64_t)row * d);
    if (row >= rv.offsets[E]) continue;
    const int e = expert_of_row(rv, E, row);
    if (e < 0) continue;
    const float4* hr = reinterpret_cast<const float4*>(H + (int64_t)row * f);
    const float4* wr = reinterpret_cast<const float4*>(wd + ((int64_t)e * d + n) * f);
    float acc = 0.f;
    for (int c = 0; c < f / 4; ++c) {
      const float4 hv = hr[c], wv = wr[c];
      acc = fmaf(hv.x, wv.x, acc); acc = fmaf(hv.y, wv.y, acc); acc = fmaf(hv.z, wv.z, acc);
      acc = fmaf(hv.w, wv.w, acc);
    }
    Y[(int64_t)row * d + n] = acc;
  }
}

hipError_t launch_f32_gateup(const float* x, RouteView rv, const float* wg, const float* wu, int64_t T,
                             int64_t rows_cap, int d, int f, int E, int act, float* H, hipStream_t st) {
  int64_t blocks = (rows_cap * f + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(f32_gateup_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, rv, wg, wu, T, rows_cap, d,
                     f, E, act, H);
  return hipGetLastError();
}

hipError_t launch_f32_down(const float* H, RouteView rv, const float* wd, int64_t rows_cap, int d, int f, int E,
                           float* Y, hipStream_t st) {
  int64_t blocks = (rows_cap * d + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(f32_down_kernel, dim3((unsigned)blocks), dim3(256), 0, st, H, rv, wd, rows_cap, d, f, E, Y);
  return hipGetLastError();
}

}  // namespace gmoe
