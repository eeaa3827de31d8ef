// Router (logits -> softmax -> top-k), token permutation, gate-weighted
// combine and the sandwich RMSNorms of the MoE layer, for gfx950.
//
// Routing follows the Grok-1 code shown in the Grok-1 book ch. 10, section
// 10.3.1: softmax over all experts first, then top-k, and the gates are the
// selected probabilities with no renormalisation (renormalised on request,
// as Mixtral does; a per-expert bias can steer the choice, as in
// DeepSeek-V3's routing). The logits are accumulated in fp64 (every
// bf16*bf16 or fp32*fp32 product is exact in fp64), so the expert choice
// only depends on the summation order at the 1e-13 level.
#include "moe_internal.h"

namespace gmoe {

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}

// 8 consecutive elements -> double
__device__ __forceinline__ void load8_f64(const bf16_bits* p, double* o) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (double)__uint_as_float(w[i] << 16);
    o[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8_f64(const float* p, double* o) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// 8 consecutive elements as loaded (bf16 bits or fp32), widened later.
template <typename XT>
struct Raw8;
template <>
struct Raw8<bf16_bits> {
  uint4 v;
};
template <>
struct Raw8<float> {
  float4 a, b;
};
__device__ __forceinline__ Raw8<bf16_bits> load_raw8(const bf16_bits* p) {
  return Raw8<bf16_bits>{*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ Raw8<float> load_raw8(const float* p) {
  return Raw8<float>{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}
__device__ __forceinline__ void raw8_f64(const Raw8<bf16_bits>& r, double* o) {
  const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (double)__uint_as_float(w[i] << 16);
    o[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void raw8_f64(const Raw8<float>& r, double* o) {
  o[0] = r.a.x; o[1] = r.a.y; o[2] = r.a.z; o[3] = r.a.w;
  o[4] = r.b.x; o[5] = r.b.y; o[6] = r.b.z; o[7] = r.b.w;
}

// Softmax over the E logits of one token (lane e holds logit e; E <= 64),
// then k rounds of shuffle arg-max over (p + bias desc, index asc); lane 0
// writes the k routed slots (renormalised on request) and the ns shared ones.
__device__ __forceinline__ void wave_route_token(double my_logit, int lane, int E, int k, int ns, int renorm,
                                                 const float* __restrict__ bias, int64_t t,
                                                 int32_t* __restrict__ idx, float* __restrict__ gate) {
  const bool live = lane < E;
  const double mx = wave_max_f64(live ? my_logit : -INFINITY);
  const double ex = live ? exp(my_logit - mx) : 0.0;
  const double z = wave_sum_f64(ex);
  const double p = ex / z;
  const double key = live ? p + (bias ? (double)bias[lane] : 0.0) : -INFINITY;
  bool taken = false;
  double gsel[8];
  int isel[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    gsel[s] = 0.0;
    isel[s] = 0;
    if (s < k) {
      // arg-max over the experts not yet taken; key (p + bias desc, index asc)
      double kv = (live && !taken) ? key : -INFINITY;
      int bi = lane;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ko = __shfl_xor(kv, off, 64);
        const int io = __shfl_xor(bi, off, 64);
        if (ko > kv || (ko == kv && io < bi)) {
          kv = ko;
          bi = io;
        }
      }
      if (lane == bi) taken = true;
      gsel[s] = __shfl(p, bi, 64);  // the gate is the probability itself
      isel[s] = bi;
    }
  }
  if (lane == 0) {
    // Mixtral's renormalisation: the k gates over their sum (slot order)
    double sum = 0.0;
#pragma unroll
    for (int s = 0; s < 8; ++s) sum += gsel[s];
    const int K = k + ns;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < k) {
        idx[t * K + s] = isel[s];
        gate[t * K + s] = (float)(renorm ? gsel[s] / sum : gsel[s]);
      }
    for (int j = 0; j < ns; ++j) {
      idx[t * K + k + j] = E + j;
      gate[t * K + k + j] = 1.0f;
    }
  }
}

// One workgroup (4 wavefronts) per token, so the d-long dot products are
// spread over 256 lanes and their loads are all in flight together. Each lane
// accumulates 8 experts at a time over its 8-element chunks; the partials are
// summed across lanes (butterfly) and across the 4 wavefronts (LDS, fixed
// order). Wavefront 0 then holds logit e in lane e; softmax and the k-fold
// arg-max run across its lanes. E <= 64.
// Output rows have K = k + ns slots: the k routed ones, then the ns shared
// experts E .. E+ns-1 with gate 1. bias (nullable): added to p for the
// choice only (the aux-loss-free routing bias, book ch. 10, section 10.3.2).
template <typename XT>
__global__ __launch_bounds__(256) void router_topk_kernel(const XT* __restrict__ x, const XT* __restrict__ wr,
                                                          int64_t T, int d, int E, int k, int ns, int renorm,
                                                          const float* __restrict__ bias,
                                                          int32_t* __restrict__ idx, float* __restrict__ gate) {
  __shared__ double s_part[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = d >> 3;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const XT* xr = x + t * (int64_t)d;
    for (int e0 = 0; e0 < E; e0 += 8) {
      double acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.0;
      // U chunks per trip (c0, c0 + 256, ...; one trip covers d = 8192 bf16
      // or 4096 fp32), all their loads issued before the first FMA; the FMAs
      // then run in ascending chunk order, the order of router_topk4_kernel
      constexpr int U = sizeof(XT) == 2 ? 4 : 2;
      for (int c0 = threadIdx.x; c0 < nchunk; c0 += 256 * U) {
        Raw8<XT> rx[U], rw[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + 256 * u;
          if (c < nchunk) {
            rx[u] = load_raw8(xr + c * 8);
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (e0 + j < E) rw[u][j] = load_raw8(wr + (int64_t)(e0 + j) * d + c * 8);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (c0 + 256 * u >= nchunk) break;
          double xv[8];
          raw8_f64(rx[u], xv);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (e0 + j < E) {
              double wv[8];
              raw8_f64(rw[u][j], wv);
#pragma unroll
              for (int q = 0; q < 8; ++q) acc[j] = fma(xv[q], wv[q], acc[j]);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double s = wave_sum_f64(acc[j]);
        if (lane == 0 && e0 + j < E) s_part[wave][e0 + j] = s;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const bool live = lane < E;
      const double my_logit = live ? ((s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane])) : 0.0;
      wave_route_token(my_logit, lane, E, k, ns, renorm, bias, t, idx, gate);
    }
    __syncthreads();
  }
}

// The same routing for 4 tokens per workgroup (larger batches): each lane
// widens its router chunks once and uses them for the 4 tokens, so the
// router weights are read from L2 once per 4 tokens; the per-lane chunk
// order and the reductions are those of router_topk_kernel, so the logits
// are bit-identical. Wavefront w then routes token w of the group.
template <typename XT>
__global__ __launch_bounds__(256) void router_topk4_kernel(const XT* __restrict__ x, const XT* __restrict__ wr,
                                                           int64_t T, int d, int E, int k, int ns, int renorm,
                                                           const float* __restrict__ bias,
                                                           int32_t* __restrict__ idx, float* __restrict__ gate) {
  constexpr int TPB = 4;
  __shared__ double s_part[TPB][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = d >> 3;
  for (int64_t t0 = (int64_t)blockIdx.x * TPB; t0 < T; t0 += (int64_t)gridDim.x * TPB) {
    const int nt = (int)min((int64_t)TPB, T - t0);
    for (int e0 = 0; e0 < E; e0 += 8) {
      double acc[TPB][8];
#pragma unroll
      for (int u = 0; u < TPB; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[u][j] = 0.0;
      for (int c = threadIdx.x; c < nchunk; c += 256) {
        Raw8<XT> rx[TPB], rw[8];
#pragma unroll
        for (int u = 0; u < TPB; ++u)
          if (u < nt) rx[u] = load_raw8(x + (t0 + u) * (int64_t)d + c * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (e0 + j < E) rw[j] = load_raw8(wr + (int64_t)(e0 + j) * d + c * 8);
        double xv[TPB][8];
#pragma unroll
        for (int u = 0; u < TPB; ++u)
          if (u < nt) raw8_f64(rx[u], xv[u]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (e0 + j < E) {
            double wv[8];
            raw8_f64(rw[j], wv);
#pragma unroll
            for (int u = 0; u < TPB; ++u)
              if (u < nt) {
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[u][j] = fma(xv[u][q], wv[q], acc[u][j]);
              }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < TPB; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double sm = wave_sum_f64(acc[u][j]);
          if (lane == 0 && e0 + j < E) s_part[u][wave][e0 + j] = sm;
        }
    }
    __syncthreads();
    if (wave < nt) {
      const bool live = lane < E;
      const double my_logit =
          live ? ((s_part[wave][0][lane] + s_part[wave][1][lane]) + (s_part[wave][2][lane] + s_part[wave][3][lane]))
               : 0.0;
      wave_route_token(my_logit, lane, E, k, ns, renorm, bias, t0 + wave, idx, gate);
    }
    __syncthreads();
  }
}

hipError_t launch_router(int act_f32, const void* x, const void* router_w, int64_t T, int d, int E, int k, int ns,
                         int renorm, const float* bias, int32_t* idx, float* gate, hipStream_t stream) {
  if (T >= 256) {  // 4 tokens per workgroup
    int64_t blocks = (T + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    if (act_f32)
      hipLaunchKernelGGL(router_topk4_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const float*)x, (const float*)router_w, T, d, E, k, ns, renorm, bias, idx, gate);
    else
      hipLaunchKernelGGL(router_topk4_kernel<bf16_bits>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const bf16_bits*)x, (const bf16_bits*)router_w, T, d, E, k, ns, renorm, bias, idx, gate);
    return hipGetLastError();
  }
  int64_t blocks = T;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (act_f32)
    hipLaunchKernelGGL(router_topk_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)x, (const float*)router_w, T, d, E, k, ns, renorm, bias, idx, gate);
  else
    hipLaunchKernelGGL(router_topk_kernel<bf16_bits>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const bf16_bits*)x, (const bf16_bits*)router_w, T, d, E, k, ns, renorm, bias, idx, gate);
  return hipGetLastError();
}

// ---------------------------------------------------------------- many-expert router (E > 64)
// Fine-grained layers route over hundreds of experts (256 in DeepSeek-V3,
// book ch. 10, section 10.1 table). The logits become a [T][E] GEMM in two
// kernels: router_mfma_kernel forms split-K partial logits in fp64 (each
// bf16 product is exact in fp64); router_topk_wave_kernel (up to 8 splits,
// one wavefront per token) or router_topk_block_kernel (one workgroup per
// token) sums the partials in split order and runs softmax and top-k.

// Workgroup tile: 64 tokens x 256 experts (wavefront w: experts 64 w ..
// 64 w + 63), reduction chunks of 64 staged as bf16 in LDS (rows padded to 72
// values, so the 16 rows that a wavefront reads at once start in distinct
// banks); the next chunk is loaded into registers while this one is used.
// Products on v_mfma_f64_16x16x4f64 (A: 16 tokens x 4, B: 4 x 16 experts;
// lane l supplies row l mod 16 and reduction index l / 16 of each; result
// value v of lane l is C[l / 16 + 4 v][l mod 16], measured). Inside each block of 16
// reduction values, lane group g = l / 16 reads the 4 consecutive values
// [4 g, 4 g + 4) of its row once and feeds value q to MFMA q, so MFMA q sums
// the indices 4 g + q over g, the same ones on both operands: every product
// is exact in fp64 and only the order of the fp64 sum differs from a
// sequential one. Grid z splits the reduction (partials in P[z]).
constexpr int kRmTok = 64, kRmExp = 256, kRmK = 64, kRmLd = kRmK + 8;
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_lo_f64(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi_f64(uint32_t w) { return (double)__uint_as_float(w & 0xFFFF0000u); }

// one staged chunk for a tile whose first NTB blocks of 16 tokens hold tokens
template <int NTB>
__device__ __forceinline__ void router_mfma_chunk(const bf16_bits* sx, const bf16_bits* sw, int lane, int wave,
                                                  f64x4 (&acc)[4][4]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll 1
  for (int kb = 0; kb < kRmK; kb += 16) {
    uint2 ra[NTB], rb[4];
#pragma unroll
    for (int i = 0; i < NTB; ++i) ra[i] = *reinterpret_cast<const uint2*>(sx + (16 * i + r) * kRmLd + kb + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rb[j] = *reinterpret_cast<const uint2*>(sw + (64 * wave + 16 * j + r) * kRmLd + kb + 4 * g);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      double a[NTB], b[4];
#pragma unroll
      for (int i = 0; i < NTB; ++i) {
        const uint32_t w = (q < 2) ? ra[i].x : ra[i].y;
        a[i] = (q & 1) ? bf16_hi_f64(w) : bf16_lo_f64(w);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (q < 2) ? rb[j].x : rb[j].y;
        b[j] = (q & 1) ? bf16_hi_f64(w) : bf16_lo_f64(w);
      }
#pragma unroll
      for (int i = 0; i < NTB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(256) void router_mfma_kernel(const bf16_bits* __restrict__ x,
                                                          const bf16_bits* __restrict__ wr, int64_t T, int d, int E,
                                                          double* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) bf16_bits sx[kRmTok * kRmLd];
  __shared__ __attribute__((aligned(16))) bf16_bits sw[kRmExp * kRmLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kRmTok;
  const int e0 = blockIdx.y * kRmExp;
  const int kspan = d / (int)gridDim.z, kbeg = (int)blockIdx.z * kspan, kend = kbeg + kspan;
  const int64_t rows = T - t0;
  const int ntb = rows >= 64 ? 4 : (int)((rows + 15) / 16);
  f64x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  // 16-byte pieces: x 64 rows x 8 (2 per thread), weights 256 rows x 8 (8 per thread)
  uint4 vx[2], vw[8];
  auto load = [&](int kc) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int lin = tid + 256 * q, rr = lin >> 3, c = (lin & 7) * 8;
      const int64_t tok = t0 + rr;
      vx[q] = tok < T ? *reinterpret_cast<const uint4*>(x + tok * d + kc + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int lin = tid + 256 * q, rr = lin >> 3, c = (lin & 7) * 8;
      const int e = e0 + rr;
      vw[q] = e < E ? *reinterpret_cast<const uint4*>(wr + (int64_t)e * d + kc + c) : make_uint4(0, 0, 0, 0);
    }
  };
  load(kbeg);
  for (int kc = kbeg; kc < kend; kc += kRmK) {
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int lin = tid + 256 * q;
      *reinterpret_cast<uint4*>(sx + (lin >> 3) * kRmLd + (lin & 7) * 8) = vx[q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int lin = tid + 256 * q;
      *reinterpret_cast<uint4*>(sw + (lin >> 3) * kRmLd + (lin & 7) * 8) = vw[q];
    }
    __syncthreads();
    if (kc + kRmK < kend) load(kc + kRmK);
    switch (ntb) {
      case 4: router_mfma_chunk<4>(sx, sw, lane, wave, acc); break;
      case 3: router_mfma_chunk<3>(sx, sw, lane, wave, acc); break;
      case 2: router_mfma_chunk<2>(sx, sw, lane, wave, acc); break;
      default: router_mfma_chunk<1>(sx, sw, lane, wave, acc); break;
    }
  }
  double* Ps = P + (int64_t)blockIdx.z * T * E;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 64 * wave + 16 * j + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t tok = t0 + 16 * i + g + 4 * v;
        if (tok < T && e < E) Ps[tok * E + e] = acc[i][j][v];
      }
    }
}

// Softmax and the k rounds of arg-max over (p + b desc, index asc) for one
// token in one wavefront: lane l holds the logits of experts l, l + 64,
// l + 128, l + 192 (-inf past E). No workgroup barriers. E <= 256.
__device__ __forceinline__ void wave_route_many(const double (&lg)[4], int lane, int E, int k, int ns, int renorm,
                                                const float* __restrict__ bias, int64_t t,
                                                int32_t* __restrict__ idx, float* __restrict__ gate) {
  double p[4], key[4];
  bool live[4], taken[4];
  double m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    live[j] = lane + 64 * j < E;
    taken[j] = false;
    m = fmax(m, lg[j]);
  }
  m = wave_max_f64(m);
  double z = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = live[j] ? exp(lg[j] - m) : 0.0;
    z += p[j];
  }
  z = wave_sum_f64(z);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] /= z;
    key[j] = live[j] ? p[j] + (bias ? (double)bias[lane + 64 * j] : 0.0) : -INFINITY;
  }
  double gsel[8];
  int isel[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    gsel[r] = 0.0;
    isel[r] = 0;
    if (r < k) {
      // this lane's best untaken expert (ascending index breaks ties), then across lanes
      double kv = -INFINITY, pv = 0.0;
      int bi = 1 << 30;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (live[j] && !taken[j] && key[j] > kv) {
          kv = key[j];
          pv = p[j];
          bi = lane + 64 * j;
        }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ko = __shfl_xor(kv, off, 64);
        const double po = __shfl_xor(pv, off, 64);
        const int io = __shfl_xor(bi, off, 64);
        if (ko > kv || (ko == kv && io < bi)) {
          kv = ko;
          pv = po;
          bi = io;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (bi == lane + 64 * j) taken[j] = true;
      gsel[r] = pv;
      isel[r] = bi < E ? bi : -1;  // -1 (dropped) only when no key compares, i.e. NaN logits
    }
  }
  if (lane == 0) {
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < 8; ++r) sum += gsel[r];
    const int K = k + ns;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < k) {
        idx[t * K + r] = isel[r];
        gate[t * K + r] = (float)(renorm ? gsel[r] / sum : gsel[r]);
      }
    for (int jj = 0; jj < ns; ++jj) {
      idx[t * K + k + jj] = E + jj;
      gate[t * K + k + jj] = 1.0f;
    }
  }
}

// Few split partials (S <= 8): one wavefront per token, lane l summing the
// partials of its four experts in split order, then wave_route_many.
__global__ __launch_bounds__(256) void router_topk_wave_kernel(const double* __restrict__ P, int S, int64_t T, int E,
                                                               int k, int ns, int renorm,
                                                               const float* __restrict__ bias,
                                                               int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < T; t += (int64_t)gridDim.x * 4) {
    const double* pt = P + t * E;
    const int64_t stride = T * E;
    double v[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int s = 0; s < 8; ++s) v[j][s] = (s < S && lane + 64 * j < E) ? pt[s * stride + lane + 64 * j] : 0.0;
    double lg[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lg[j] = 0.0;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s < S) lg[j] += v[j][s];
      if (lane + 64 * j >= E) lg[j] = -INFINITY;
    }
    wave_route_many(lg, lane, E, k, ns, renorm, bias, t, idx, gate);
  }
}

// More partials: one workgroup of 1024 threads per token. Thread (g, e)
// (g = tid / 256) sums the partials [g S / 4, (g + 1) S / 4) of logit e in
// split order, eight loads at a time; the four quarter sums are added in
// fixed order and wavefront 0 routes the token.
__global__ __launch_bounds__(1024) void router_topk_block_kernel(const double* __restrict__ P, int S, int64_t T, int E,
                                                                 int k, int ns, int renorm,
                                                                 const float* __restrict__ bias,
                                                                 int32_t* __restrict__ idx, float* __restrict__ gate) {
  __shared__ double s_part[4][256];
  const int tid = threadIdx.x, lane = tid & 63, g = tid >> 8, e = tid & 255;
  const int s0 = g * S / 4, s1 = (g + 1) * S / 4;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    if (e < E) {
      const double* pe = P + t * E + e;
      const int64_t stride = T * E;
      double sum = 0.0;
      int s = s0;
      for (; s + 8 <= s1; s += 8) {
        double v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = pe[(int64_t)(s + q) * stride];
#pragma unroll
        for (int q = 0; q < 8; ++q) sum += v[q];
      }
      for (; s < s1; ++s) sum += pe[(int64_t)s * stride];
      s_part[g][e] = sum;
    }
    __syncthreads();
    if (tid < 64) {
      double lg[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ej = lane + 64 * j;
        lg[j] = ej < E ? (s_part[0][ej] + s_part[1][ej]) + (s_part[2][ej] + s_part[3][ej]) : -INFINITY;
      }
      wave_route_many(lg, lane, E, k, ns, renorm, bias, t, idx, gate);
    }
    __syncthreads();
  }
}

hipError_t launch_router_many(const bf16_bits* x, const bf16_bits* router_w, int64_t T, int d, int E, int k, int ns,
                              int renorm, const float* bias, int splits, double* P, int32_t* idx, float* gate,
                              hipStream_t stream) {
  const dim3 grid((unsigned)((T + kRmTok - 1) / kRmTok), (unsigned)((E + kRmExp - 1) / kRmExp), (unsigned)splits);
  hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(256), 0, stream, x, router_w, T, d, E, P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (splits <= 8) {
    int64_t blocks = (T + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(router_topk_wave_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, P, splits, T, E, k, ns,
                       renorm, bias, idx, gate);
    return hipGetLastError();
  }
  int64_t blocks = T < 16384 ? T : 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(router_topk_block_kernel, dim3((unsigned)blocks), dim3(1024), 0, stream, P, splits, T, E, k, ns,
                     renorm, bias, idx, gate);
  return hipGetLastError();
}

// Caller-given routing [T][k] plus the ns shared slots -> [T][k + ns]. A
// caller index outside [0, E) becomes -1 (dropped by the permutation).
__global__ __launch_bounds__(256) void append_shared_kernel(const int32_t* __restrict__ ridx,
                                                            const float* __restrict__ rgate, int64_t T, int E, int k,
                                                            int ns, int32_t* __restrict__ idx,
                                                            float* __restrict__ gate) {
  const int K = k + ns;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < T * K; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / K;
    const int s = (int)(i - t * K);
    int e = E + (s - k);
    if (s < k) {
      e = ridx[t * k + s];
      if (e < 0 || e >= E) e = -1;  // outside the routed experts: dropped, never a shared expert
    }
    idx[i] = e;
    gate[i] = s < k ? rgate[t * k + s] : 1.0f;
  }
}

hipError_t launch_append_shared(const int32_t* ridx, const float* rgate, int64_t T, int E, int k, int ns,
                                int32_t* idx, float* gate, hipStream_t stream) {
  int64_t blocks = (T * (k + ns) + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(append_shared_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ridx, rgate, T, E, k, ns,
                     idx, gate);
  return hipGetLastError();
}

// ---------------------------------------------------------------- permutation
// A stable counting sort of the (token, slot) assignments by expert, in three
// launches over B blocks, each owning a contiguous chunk of tokens:
//   count:   block b counts the assignments of each expert in its chunk (LDS
//            integer atomics: order-independent) into blk[b][e];
//   scan:    one workgroup turns blk[.][e] into exclusive prefixes over the
//            blocks (the rank of block b's first assignment of expert e),
//            caps the totals and scans them into the segment offsets;
//   scatter: block b walks its chunk in sub-chunks of 256 tokens in token
//            order; per wavefront and expert a 64-bit LDS mask of the lanes
//            (tokens) that list it gives each assignment its rank inside its
//            wavefront (earlier lanes), the masks of earlier wavefronts and
//            the running base of the block its rank among all assignments
//            of its expert.
// Segment e thus holds its tokens in ascending order. A token that lists an
// expert twice is counted once (both slots then point at the same row);
// indices outside [0, E) are dropped (pos = -1). With a capacity (cap >= 0;
// book ch. 10, section 10.3.2, the capacity factor box) an assignment to a
// capped expert (e < E_cap: the routed ones) of rank >= cap in token order is
// dropped too: pos = -1, no row, and the segment holds the first cap.
constexpr int kPermMaxE = 272;     // routed + shared experts
constexpr int kPermMaxK = 12;      // slots per token
constexpr int kPermTB = 256;       // tokens per sub-chunk: one per thread
constexpr int kPermMaxBlocks = 256;

// tokens per block: whole sub-chunks, at most kPermMaxBlocks blocks
static int64_t permute_chunk(int64_t T) {
  const int64_t sub = (T + kPermTB - 1) / kPermTB;
  return (sub + kPermMaxBlocks - 1) / kPermMaxBlocks * kPermTB;
}

int64_t permute_scratch_ints(int64_t T, int E) {
  const int64_t chunk = permute_chunk(T);
  const int64_t B = T > 0 ? (T + chunk - 1) / chunk : 1;
  return B * (int64_t)E;
}

// the slots of token t: expert or -1 (outside [0, E)); dup[s]: slot s repeats
// an expert of an earlier slot of the same token
__device__ __forceinline__ void token_slots(const int32_t* __restrict__ idx, int64_t t, int E, int k,
                                            int (&es)[kPermMaxK], bool (&dup)[kPermMaxK]) {
#pragma unroll
  for (int s = 0; s < kPermMaxK; ++s) {
    es[s] = -1;
    dup[s] = false;
    if (s < k) {
      const int e = idx[t * k + s];
      es[s] = (e >= 0 && e < E) ? e : -1;
#pragma unroll
      for (int q = 0; q < s; ++q) dup[s] = dup[s] || (es[s] >= 0 && es[q] == es[s]);
    }
  }
}

__global__ __launch_bounds__(kPermTB) void permute_count_kernel(const int32_t* __restrict__ idx, int64_t T, int E,
                                                                int k, int64_t chunk, int32_t* __restrict__ blk) {
  __shared__ int s_cnt[kPermMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermTB) s_cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * chunk, t1 = min(T, t0 + chunk);
  for (int64_t t = t0 + tid; t < t1; t += kPermTB) {
    int es[kPermMaxK];
    bool dup[kPermMaxK];
    token_slots(idx, t, E, k, es, dup);
#pragma unroll
    for (int s = 0; s < kPermMaxK; ++s)
      if (es[s] >= 0 && !dup[s]) atomicAdd(&s_cnt[es[s]], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermTB) blk[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

// one workgroup of 1024 threads: thread e < E prefixes blk[.][e] over the
// blocks (8 loads in flight), wave 0 scans the capped totals
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ blk, int B, int E, int64_t cap,
                                                            int E_cap, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int s_tot[kPermMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < E) {
    int run = 0;
    for (int b0 = 0; b0 < B; b0 += 8) {
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = b0 + j < B ? blk[(int64_t)(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b0 + j < B) blk[(int64_t)(b0 + j) * E + tid] = run;
        run += c[j];
      }
    }
    s_tot[tid] = run;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the capped totals: lane l owns experts kPer*l .. kPer*l + kPer - 1
    constexpr int kPer = (kPermMaxE + 63) / 64;
    int c[kPer], local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane * kPer + j;
      c[j] = 0;
      if (e < E) c[j] = (cap >= 0 && e < E_cap && (int64_t)s_tot[e] > cap) ? (int)cap : s_tot[e];
      local += c[j];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    int acc = incl - local;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane * kPer + j;
      if (e < E) {
        offsets[e] = acc;
        counts[e] = c[j];
      }
      acc += c[j];
    }
    if (lane == 63) offsets[E] = incl;
  }
}

__global__ __launch_bounds__(kPermTB) void permute_scatter_kernel(const int32_t* __restrict__ idx, int64_t T, int E,
                                                                  int k, int64_t chunk,
                                                                  const int32_t* __restrict__ blk,
                                                                  const int32_t* __restrict__ counts,
                                                                  const int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ perm,
                                                                  int32_t* __restrict__ pos) {
  constexpr int kWaves = kPermTB / 64;
  __shared__ int s_base[kPermMaxE];  // assignments of expert e before the current sub-chunk
  __shared__ int s_off[kPermMaxE];   // first row of segment e
  __shared__ int s_lim[kPermMaxE];   // rows segment e keeps
  // lanes of wavefront w whose token lists expert e (a token listing e twice
  // sets its bit once)
  __shared__ unsigned long long s_mask[kWaves][kPermMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kPermTB) {
    s_base[e] = blk[(int64_t)blockIdx.x * E + e];
    s_off[e] = offsets[e];
    s_lim[e] = counts[e];
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t c0 = (int64_t)blockIdx.x * chunk, c1 = min(T, c0 + chunk);
  for (int64_t t0 = c0; t0 < c1; t0 += kPermTB) {
    const int64_t t = t0 + tid;
    int my_e[kPermMaxK];
    bool dup[kPermMaxK];
    if (t < c1) {
      token_slots(idx, t, E, k, my_e, dup);
    } else {
#pragma unroll
      for (int s = 0; s < kPermMaxK; ++s) {
        my_e[s] = -1;
        dup[s] = false;
      }
    }
    for (int e = lane; e < E; e += 64) s_mask[wave][e] = 0ull;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kPermMaxK; ++s)
      if (my_e[s] >= 0) atomicOr(&s_mask[wave][my_e[s]], 1ull << lane);
    __syncthreads();
    // rank = earlier sub-chunks and blocks + earlier wavefronts of this
    // sub-chunk + earlier lanes of this wavefront
    if (t < c1) {
#pragma unroll
      for (int s = 0; s < kPermMaxK; ++s) {
        if (s >= k) break;
        const int e = my_e[s];
        int row = -1;
        if (e >= 0) {
          int rank = s_base[e] + __popcll(s_mask[wave][e] & lt_mask);
          for (int w = 0; w < wave; ++w) rank += __popcll(s_mask[w][e]);
          if (rank < s_lim[e]) {
            row = s_off[e] + rank;
            if (!dup[s]) perm[row] = (int32_t)t;
          }
        }
        pos[t * k + s] = row;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPermTB) {
      int tot = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += __popcll(s_mask[w][e]);
      s_base[e] += tot;
    }
    __syncthreads();
  }
}

// The same permutation for at most kSmallN = 96 assignments (decode-sized
// batches), in one wavefront: lane l holds assignments l and l + 64 of the
// token-major list (a = t k + s). An assignment that repeats an expert of
// its own token is a duplicate: it is not counted and shares the row of the
// first one. The rank of assignment a of expert e is the number of counted
// assignments of e by earlier tokens, read off the whole list with one scalar
// lane read per assignment; counts come from LDS atomics (order-free).
constexpr int kSmallN = 96;
__global__ __launch_bounds__(64) void permute_small_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                           int64_t cap, int E_cap, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  __shared__ int s_cnt[kPermMaxE];
  __shared__ int s_off[kPermMaxE];
  __shared__ int s_lim[kPermMaxE];
  __shared__ int s_idx[kSmallN];
  const int lane = threadIdx.x;
  const int n = T * k;
  for (int e = lane; e < kPermMaxE; e += 64) s_cnt[e] = 0;
  int raw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int a = lane + 64 * j;
    raw[j] = a < n ? idx[a] : -1;
    if (a < n) s_idx[a] = raw[j];
  }
  __syncthreads();
  int own[2], cnt[2];  // own: this assignment's expert (-1: none); cnt: the same unless a duplicate (-2)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int a = lane + 64 * j;
    own[j] = -1;
    cnt[j] = -1;
    const int e = raw[j];
    if (a < n && e >= 0 && e < E) {
      const int t = a / k, s = a - t * k;
      own[j] = e;
      cnt[j] = e;
      for (int q = 0; q < s; ++q)
        if (s_idx[t * k + q] == e) cnt[j] = -2;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (cnt[j] >= 0) atomicAdd(&s_cnt[cnt[j]], 1);
  __syncthreads();
  {
    // exclusive scan of the capped counts: lane l owns experts kPer*l .. kPer*l + kPer - 1
    constexpr int kPer = (kPermMaxE + 63) / 64;
    int c[kPer], local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane * kPer + j;
      c[j] = 0;
      if (e < E) c[j] = (cap >= 0 && e < E_cap && (int64_t)s_cnt[e] > cap) ? (int)cap : s_cnt[e];
      local += c[j];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    int acc = incl - local;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane * kPer + j;
      if (e < E) {
        offsets[e] = acc;
        counts[e] = c[j];
        s_off[e] = acc;
        s_lim[e] = c[j];
      }
      acc += c[j];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  // ranks: counted assignments of the same expert by earlier tokens
  int rank[2] = {0, 0};
  const int tk0 = (lane / k) * k, tk1 = ((lane + 64) / k) * k;  // first assignment of this lane's tokens
  for (int b = 0; b < n; ++b) {
    const int eb = __builtin_amdgcn_readlane(b < 64 ? cnt[0] : cnt[1], b & 63);
    if (eb == own[0] && b < tk0) ++rank[0];
    if (eb == own[1] && b < tk1) ++rank[1];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int a = lane + 64 * j;
    if (a < n) {
      int row = -1;
      const int e = own[j];
      if (e >= 0 && rank[j] < s_lim[e]) {
        row = s_off[e] + rank[j];
        if (cnt[j] >= 0) perm[row] = (int32_t)(a / k);
      }
      pos[a] = row;
    }
  }
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int E, int k, int64_t cap, int E_cap, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* pos, int32_t* blk, hipStream_t stream) {
  if (E > kPermMaxE || k > kPermMaxK) return hipErrorInvalidValue;
  if (T * k <= kSmallN) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(64), 0, stream, idx, (int)T, E, k, cap, E_cap, counts,
                       offsets, perm, pos);
    return hipGetLastError();
  }
  const int64_t chunk = permute_chunk(T);
  const int B = (int)((T + chunk - 1) / chunk);
  hipLaunchKernelGGL(permute_count_kernel, dim3(B), dim3(kPermTB), 0, stream, idx, T, E, k, chunk, blk);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, blk, B, E, cap, E_cap, counts, offsets);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(B), dim3(kPermTB), 0, stream, idx, T, E, k, chunk, blk, counts,
                     offsets, perm, pos);
  return hipGetLastError();
}

// ---------------------------------------------------------------- tile table
// The tiled GEMMs walk tiles of bm rows over the expert segments in order.
// One workgroup: wavefront 0 scans the per-expert tile counts into tile_off,
// then every thread fills tile_e for a stride of tiles by binary search.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ counts, int E, int bm,
                                                          int32_t* __restrict__ tile_off, int32_t* __restrict__ tile_e,
                                                          int64_t mt_ub) {
  __shared__ int s_off[kPermMaxE + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    constexpr int kPer = (kPermMaxE + 63) / 64;
    int c[kPer], local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane * kPer + j;
      c[j] = e < E ? (counts[e] + bm - 1) / bm : 0;
      local += c[j];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    int acc = incl - local;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane * kPer + j;
      if (e < E) {
        s_off[e] = acc;
        tile_off[e] = acc;
      }
      acc += c[j];
    }
    if (lane == 63) {
      s_off[E] = incl;
      tile_off[E] = incl;
    }
  }
  __syncthreads();
  const int total = (int)min((int64_t)s_off[E], mt_ub);
  for (int m = tid; m < total; m += 1024) {
    int lo = 0, hi = E - 1;  // the last e with s_off[e] <= m
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= m) lo = mid;
      else hi = mid - 1;
    }
    tile_e[m] = lo;
  }
}

hipError_t launch_tile_table(const int32_t* counts, int E, int bm, int32_t* tile_off, int32_t* tile_e, int64_t mt_ub,
                             hipStream_t stream) {
  if (E > kPermMaxE || bm <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream, counts, E, bm, tile_off, tile_e, mt_ub);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// out[t][n] = sum over slots s (slot order) of gate[t][s] * y_s[n], where y_s
// is the down-projection row of assignment (t, s) summed over the split-K
// partials in ascending split order. fp32 arithmetic, one RNE rounding to the
// output type. Each thread owns 4 consecutive outputs. Dropped assignments
// (pos = -1) contribute nothing.
__device__ __forceinline__ float4 gated_sum4(const float* __restrict__ Y, int S, int64_t split_stride,
                                             const int32_t* __restrict__ pos, const float* __restrict__ gate,
                                             int64_t t, int d, int k, int c) {
  // every slot's row and first partial are loaded before any is added (k <= 12)
  int row[kPermMaxK];
  float g[kPermMaxK];
  float4 y[kPermMaxK];
#pragma unroll
  for (int s = 0; s < kPermMaxK; ++s) {
    row[s] = -1;
    if (s < k) {
      row[s] = pos[t * k + s];
      g[s] = gate[t * k + s];
    }
  }
#pragma unroll
  for (int s = 0; s < kPermMaxK; ++s)
    if (s < k && row[s] >= 0) y[s] = *reinterpret_cast<const float4*>(Y + (int64_t)row[s] * d + c);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < kPermMaxK; ++s) {
    if (s >= k || row[s] < 0) continue;
    float4 v = y[s];
    const float* yr = Y + (int64_t)row[s] * d + c;
    for (int p = 1; p < S; ++p) {
      const float4 q = *reinterpret_cast<const float4*>(yr + p * split_stride);
      v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
    }
    acc.x += g[s] * v.x;
    acc.y += g[s] * v.y;
    acc.z += g[s] * v.z;
    acc.w += g[s] * v.w;
  }
  return acc;
}

template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y, int S, int64_t rows_cap,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ gate, int64_t T, int d, int k,
                                                      void* __restrict__ out) {
  const int nq = d >> 2;
  const int64_t total = T * (int64_t)nq;
  const int64_t split_stride = rows_cap * (int64_t)d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / nq;
    const int c = (int)(i - t * nq) * 4;
    const float4 acc = gated_sum4(Y, S, split_stride, pos, gate, t, d, k, c);
    if (OUT_F32) {
      *reinterpret_cast<float4*>((float*)out + t * d + c) = acc;
    } else {
      uint2 o;
      o.x = pack_bf16x2(acc.x, acc.y);
      o.y = pack_bf16x2(acc.z, acc.w);
      *reinterpret_cast<uint2*>((bf16_bits*)out + t * d + c) = o;
    }
  }
}

hipError_t launch_combine(int out_f32, const float* Y, int S, int64_t rows_cap, const int32_t* pos,
                          const float* gate, int64_t T, int d, int k, void* out, hipStream_t stream) {
  const int64_t total = T * (int64_t)(d / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (out_f32)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, Y, S, rows_cap, pos,
                       gate, T, d, k, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, Y, S, rows_cap, pos,
                       gate, T, d, k, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- sandwich norms
// The MoE sub-layer of Grok-1 carries an RMSNorm on each side (field guide,
// the data-flow section: normalise, run the MoE, add the gated sum back to
// the trunk; book ch. 10, section 10.3.1: the post-norm bounds the output
// scale that un-normalised gates leave free):
//   u   = RMSNorm(x; g_pre)     stored in the activation type, fed to router and experts
//   out = x + RMSNorm(y; g_post)  y = the gated expert sum
// RMSNorm(v; g)[i] = g[i] * v[i] / sqrt(mean(v^2) + eps).

// fp64 -> bf16, round to nearest even, for values in bf16's normal range
// (smaller magnitudes flush to a signed zero; RMSNorm outputs stay far above).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(b >> 63) << 15;
  uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if ((mag >> 52) <= 896) return sign;                 // |v| < 2^-126 (or zero)
  mag += 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1);  // round at the 7th mantissa bit, ties to even
  mag >>= 45;                                          // [11-bit exponent | 7-bit mantissa]
  return sign | (uint32_t)(mag - (896u << 7));         // exponent bias 1023 -> 127
}

__device__ __forceinline__ double block_sum_f64(double v, double* s_part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  if (lane == 0) s_part[wave] = v;
  __syncthreads();
  const double tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  __syncthreads();  // s_part is reused by the next row
  return tot;
}

// One workgroup (4 wavefronts) per token row: sum of squares in fp64 (each
// bf16 or fp32 square is exact in fp64), r = 1 / sqrt(ms + eps) in fp64, then
// u = (x * r) * g rounded once to the activation type.
template <typename XT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const XT* __restrict__ x, const XT* __restrict__ g, int64_t T,
                                                      int d, double eps, XT* __restrict__ u) {
  __shared__ double s_part[4];
  const int nchunk = d >> 3;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const XT* xr = x + t * (int64_t)d;
    double ss = 0.0;
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      double v[8];
      load8_f64(xr + c * 8, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) ss = fma(v[q], v[q], ss);
    }
    const double r = 1.0 / sqrt(block_sum_f64(ss, s_part) / (double)d + eps);
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      double v[8], gv[8];
      load8_f64(xr + c * 8, v);
      load8_f64(g + c * 8, gv);
      if constexpr (sizeof(XT) == 2) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = f64_to_bf16_rne((v[2 * q] * r) * gv[2 * q]) | (f64_to_bf16_rne((v[2 * q + 1] * r) * gv[2 * q + 1]) << 16);
        *reinterpret_cast<uint4*>(u + t * (int64_t)d + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = (float)((v[q] * r) * gv[q]);
        float4* ur = reinterpret_cast<float4*>(u + t * (int64_t)d + c * 8);
        ur[0] = make_float4(o[0], o[1], o[2], o[3]);
        ur[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
}

hipError_t launch_rmsnorm(int act_f32, const void* x, const void* g, int64_t T, int d, double eps, void* u,
                          hipStream_t stream) {
  int64_t blocks = T < 16384 ? T : 16384;
  if (blocks < 1) blocks = 1;
  if (act_f32)
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, (const float*)x,
                       (const float*)g, T, d, eps, (float*)u);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_bits>, dim3((unsigned)blocks), dim3(256), 0, stream, (const bf16_bits*)x,
                       (const bf16_bits*)g, T, d, eps, (bf16_bits*)u);
  return hipGetLastError();
}

__device__ __forceinline__ float4 load4_f32(const bf16_bits* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                     bf16_to_f32(v.y >> 16));
}
__device__ __forceinline__ float4 load4_f32(const float* p) { return *reinterpret_cast<const float4*>(p); }

// One workgroup per token row. Pass 1 forms the gated sum y (the same fp32
// arithmetic as combine_kernel) and its sum of squares in fp64; pass 2 forms y
// again and writes x + g_post * (y * r), rounded once to the output type.
template <typename XT>
__global__ __launch_bounds__(256) void combine_sandwich_kernel(const float* __restrict__ Y, int S, int64_t rows_cap,
                                                               const int32_t* __restrict__ pos,
                                                               const float* __restrict__ gate, int64_t T, int d,
                                                               int k, const XT* __restrict__ x,
                                                               const XT* __restrict__ g_post, double eps,
                                                               XT* __restrict__ out) {
  __shared__ double s_part[4];
  const int nq = d >> 2;
  const int64_t split_stride = rows_cap * (int64_t)d;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    double ss = 0.0;
    for (int q = threadIdx.x; q < nq; q += 256) {
      const float4 y = gated_sum4(Y, S, split_stride, pos, gate, t, d, k, 4 * q);
      ss += ((double)y.x * y.x + (double)y.y * y.y) + ((double)y.z * y.z + (double)y.w * y.w);
    }
    const float r = (float)(1.0 / sqrt(block_sum_f64(ss, s_part) / (double)d + eps));
    for (int q = threadIdx.x; q < nq; q += 256) {
      const int c = 4 * q;
      const float4 y = gated_sum4(Y, S, split_stride, pos, gate, t, d, k, c);
      const float4 xv = load4_f32(x + t * (int64_t)d + c);
      const float4 gv = load4_f32(g_post + c);
      const float4 o = make_float4(xv.x + gv.x * (y.x * r), xv.y + gv.y * (y.y * r), xv.z + gv.z * (y.z * r),
                                   xv.w + gv.w * (y.w * r));
      if constexpr (sizeof(XT) == 2) {
        *reinterpret_cast<uint2*>(out + t * (int64_t)d + c) = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
      } else {
        *reinterpret_cast<float4*>(out + t * (int64_t)d + c) = o;
      }
    }
  }
}

hipError_t launch_combine_sandwich(int out_f32, const float* Y, int S, int64_t rows_cap, const int32_t* pos,
                                   const float* gate, int64_t T, int d, int k, const void* x, const void* g_post,
                                   double eps, void* out, hipStream_t stream) {
  int64_t blocks = T < 16384 ? T : 16384;
  if (blocks < 1) blocks = 1;
  if (out_f32)
    hipLaunchKernelGGL(combine_sandwich_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, Y, S, rows_cap,
                       pos, gate, T, d, k, (const float*)x, (const float*)g_post, eps, (float*)out);
  else
    hipLaunchKernelGGL(combine_sandwich_kernel<bf16_bits>, dim3((unsigned)blocks), dim3(256), 0, stream, Y, S,
                       rows_cap, pos, gate, T, d, k, (const bf16_bits*)x, (const bf16_bits*)g_post, eps,
                       (bf16_bits*)out);
  return hipGetLastError();
}

}  // namespace gmoe
