// Grouped expert GEMMs of the Grok-1 MoE layer for gfx950 (MI355X).
//
// Expert e is a gated FFN (Grok-1 field guide, "MoE 子层"; Grok-1 book ch. 10,
// section 10.4): two input projections, GELU on the gate branch, elementwise
// product, and a down projection. Rows are the expert-contiguous permutation
// of the tokens, so each expert is one segment of a grouped GEMM (book
// ch. 11, section 11.3.1: sparse reorder + grouped GEMM).
//
// Both weight operands are stored output-channel-major (the reduction index
// is contiguous), so every MFMA operand fragment is one 16-byte load.
// The kernels compute C^T = W * X^T with v_mfma_f32_16x16x32_bf16: the weight
// fragment is the MFMA "A" operand (16 output channels) and the activation
// fragment the "B" operand (16 rows), so each lane owns 4 consecutive output
// channels of one row and the epilogue stores 8 or 16 contiguous bytes.
//
// Fragment layout of v_mfma_f32_16x16x32_bf16 used here: lane l supplies row
// (l mod 16) of its operand and 8 reduction values of group g = l / 16; the
// result register v of lane l is C[4g + v][l mod 16]. The 8 reduction values
// a lane supplies are taken from the same reduction indices for both
// operands, so the pairing is exact whatever order the hardware sums in.
#include "moe_device.h"

namespace gmoe {

// =====================================================================
// Small-M path. Every expert segment has at most 16*MT rows (M_e <= T).
// Block = 4 wavefronts; wavefront w owns 16 output channels over the full
// reduction, for all rows of its expert. Weights stream straight from HBM
// into registers (each weight element is used by exactly one wavefront);
// activation fragments come from L2. Experts with no rows exit at once and
// read no weights.
// =====================================================================
template <int MT, bool W8>
__global__ __launch_bounds__(256) void skinny_gateup_kernel(const bf16_bits* __restrict__ x, RouteView rv,
                                                            const void* __restrict__ wg,
                                                            const void* __restrict__ wu,
                                                            const float* __restrict__ scales, int64_t T, int d,
                                                            int f, int E, bf16_bits* __restrict__ H) {
  constexpr int U = MT <= 1 ? 4 : (MT <= 2 ? 2 : 1);  // 64-wide blocks per iteration
  const int nblk = f >> 6;
  const int e = blockIdx.x / nblk;
  const int nb = blockIdx.x - e * nblk;
  const int M = rv.counts[e];
  if (M <= 0) return;
  const int m0 = rv.offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = nb * 64 + wave * 16;
  const int nsub = (M + 15) >> 4;
  const size_t wsz = W8 ? 1 : 2;

  const bf16_bits* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int mr = mt * 16 + r16;
    if (mr >= M) mr = M - 1;
    int tok = rv.perm[m0 + mr];
    tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
    xrow[mt] = x + (int64_t)tok * d;
  }
  const int64_t wrow_idx = ((int64_t)e * f + n0 + r16) * d;
  const char* wgr = (const char*)wg + wrow_idx * wsz;
  const char* wur = (const char*)wu + wrow_idx * wsz;

  f32x4 accg[MT], accu[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int k0 = 0; k0 < d; k0 += 64 * U) {
    u32x4 gf[U][2], uf[U][2], xf[U][MT][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = k0 + 64 * u;
      if (kb < d) {
        load_wfrags<W8>(wgr, kb, g, gf[u][0], gf[u][1]);
        load_wfrags<W8>(wur, kb, g, uf[u][0], uf[u][1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < nsub) {
            xf[u][mt][0] = ld16(xrow[mt] + kb + koff<W8>(0, g));
            xf[u][mt][1] = ld16(xrow[mt] + kb + koff<W8>(1, g));
          }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + 64 * u < d) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < nsub) {
              accg[mt] = mfma16(gf[u][s], xf[u][mt][s], accg[mt]);
              accu[mt] = mfma16(uf[u][s], xf[u][mt][s], accu[mt]);
            }
      }
    }
  }

  const int nc = n0 + 4 * g;  // first of this lane's 4 output channels
  float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
  if (W8) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sg[v] = scales[(int64_t)e * f + nc + v];
      su[v] = scales[(int64_t)E * f + (int64_t)e * f + nc + v];
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    if (mt < nsub && m < M) {
      float h[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) h[v] = gelu_erf(accg[mt][v] * sg[v]) * (accu[mt][v] * su[v]);
      uint2 o;
      o.x = pack_bf16x2(h[0], h[1]);
      o.y = pack_bf16x2(h[2], h[3]);
      *reinterpret_cast<uint2*>(H + (int64_t)(m0 + m) * f + nc) = o;
    }
  }
}

template <int MT, bool W8>
__global__ __launch_bounds__(256) void skinny_down_kernel(const bf16_bits* __restrict__ H, RouteView rv,
                                                          const void* __restrict__ wd,
                                                          const float* __restrict__ scales, int64_t rows_cap,
                                                          int d, int f, int E, float* __restrict__ Y) {
  constexpr int U = MT <= 1 ? 4 : (MT <= 2 ? 2 : 1);
  const int nblk = d >> 6;
  const int e = blockIdx.x / nblk;
  const int nb = blockIdx.x - e * nblk;
  const int M = rv.counts[e];
  if (M <= 0) return;
  const int m0 = rv.offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = nb * 64 + wave * 16;
  const int nsub = (M + 15) >> 4;
  const int S = gridDim.y, sp = blockIdx.y;
  const int kspan = f / S;
  const int kbeg = sp * kspan, kend = kbeg + kspan;
  const size_t wsz = W8 ? 1 : 2;

  const bf16_bits* hrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int mr = mt * 16 + r16;
    if (mr >= M) mr = M - 1;
    hrow[mt] = H + (int64_t)(m0 + mr) * f;
  }
  const char* wr = (const char*)wd + ((int64_t)e * d + n0 + r16) * (int64_t)f * wsz;

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg; k0 < kend; k0 += 64 * U) {
    u32x4 wf[U][2], hf[U][MT][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = k0 + 64 * u;
      if (kb < kend) {
        load_wfrags<W8>(wr, kb, g, wf[u][0], wf[u][1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < nsub) {
            hf[u][mt][0] = ld16(hrow[mt] + kb + koff<W8>(0, g));
            hf[u][mt][1] = ld16(hrow[mt] + kb + koff<W8>(1, g));
          }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + 64 * u < kend) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < nsub) acc[mt] = mfma16(wf[u][s], hf[u][mt][s], acc[mt]);
      }
    }
  }

  const int nc = n0 + 4 * g;
  float sc[4] = {1.f, 1.f, 1.f, 1.f};
  if (W8) {
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = scales[2 * (int64_t)E * f + (int64_t)e * d + nc + v];
  }
  float* Ys = Y + (int64_t)sp * rows_cap * d;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    if (mt < nsub && m < M) {
      float4 o = make_float4(acc[mt][0] * sc[0], acc[mt][1] * sc[1], acc[mt][2] * sc[2], acc[mt][3] * sc[3]);
      *reinterpret_cast<float4*>(Ys + (int64_t)(m0 + m) * d + nc) = o;
    }
  }
}

template <int MT, bool W8>
static hipError_t skinny_gateup_t(const bf16_bits* x, RouteView rv, const void* wg, const void* wu,
                                  const float* scales, int64_t T, int d, int f, int E, bf16_bits* H,
                                  hipStream_t st) {
  const unsigned blocks = (unsigned)E * (unsigned)(f / 64);
  hipLaunchKernelGGL((skinny_gateup_kernel<MT, W8>), dim3(blocks), dim3(256), 0, st, x, rv, wg, wu, scales, T, d,
                     f, E, H);
  return hipGetLastError();
}

template <int MT, bool W8>
static hipError_t skinny_down_t(int splits, const bf16_bits* H, RouteView rv, const void* wd,
                                const float* scales, int64_t rows_cap, int d, int f, int E, float* Y,
                                hipStream_t st) {
  const unsigned blocks = (unsigned)E * (unsigned)(d / 64);
  hipLaunchKernelGGL((skinny_down_kernel<MT, W8>), dim3(blocks, splits), dim3(256), 0, st, H, rv, wd, scales,
                     rows_cap, d, f, E, Y);
  return hipGetLastError();
}

hipError_t launch_skinny_gateup(int w8, int mt_max, const bf16_bits* x, RouteView rv, const void* wg,
                                const void* wu, const float* scales, int64_t T, int d, int f, int E,
                                bf16_bits* H, hipStream_t st) {
#define GMOE_SG(MT)                                                                               \
  return w8 ? skinny_gateup_t<MT, true>(x, rv, wg, wu, scales, T, d, f, E, H, st)                 \
            : skinny_gateup_t<MT, false>(x, rv, wg, wu, scales, T, d, f, E, H, st)
  switch (mt_max) {
    case 1: GMOE_SG(1);
    case 2: GMOE_SG(2);
    case 4: GMOE_SG(4);
    case 8: GMOE_SG(8);
  }
#undef GMOE_SG
  return hipErrorInvalidValue;
}

hipError_t launch_skinny_down(int w8, int mt_max, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                              const float* scales, int64_t rows_cap, int d, int f, int E, float* Y,
                              hipStream_t st) {
#define GMOE_SD(MT)                                                                            \
  return w8 ? skinny_down_t<MT, true>(splits, H, rv, wd, scales, rows_cap, d, f, E, Y, st)     \
            : skinny_down_t<MT, false>(splits, H, rv, wd, scales, rows_cap, d, f, E, Y, st)
  switch (mt_max) {
    case 1: GMOE_SD(1);
    case 2: GMOE_SD(2);
    case 4: GMOE_SD(4);
    case 8: GMOE_SD(8);
  }
#undef GMOE_SD
  return hipErrorInvalidValue;
}

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
                                                         int64_t rows_cap, int d, int f, int E,
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
    H[(int64_t)row * f + n] = gelu_erf(a) * b;
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
                             int64_t rows_cap, int d, int f, int E, float* H, hipStream_t st) {
  int64_t blocks = (rows_cap * f + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(f32_gateup_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, rv, wg, wu, T, rows_cap, d,
                     f, E, H);
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
