// Router (logits -> softmax -> top-k), token permutation and gate-weighted
// combine of the Grok-1 MoE layer, for gfx950.
//
// Routing follows the Grok-1 code shown in the Grok-1 book ch. 10, section
// 10.3.1: softmax over all experts first, then top-k, and the gates are the
// selected probabilities with no renormalisation. The logits are accumulated
// in fp64 (every bf16*bf16 or fp32*fp32 product is exact in fp64), so the
// expert choice only depends on the summation order at the 1e-13 level.
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

// One workgroup (4 wavefronts) per token, so the d-long dot products are
// spread over 256 lanes and their loads are all in flight together. Each lane
// accumulates 8 experts at a time over its 8-element chunks; the partials are
// summed across lanes (butterfly) and across the 4 wavefronts (LDS, fixed
// order). Wavefront 0 then holds logit e in lane e; softmax and the k-fold
// arg-max run across its lanes.
template <typename XT>
__global__ __launch_bounds__(256) void router_topk_kernel(const XT* __restrict__ x, const XT* __restrict__ wr,
                                                          int64_t T, int d, int E, int k, int renorm,
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
      for (int c = threadIdx.x; c < nchunk; c += 256) {
        double xv[8];
        load8_f64(xr + c * 8, xv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (e0 + j < E) {
            double wv[8];
            load8_f64(wr + (int64_t)(e0 + j) * d + c * 8, wv);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[j] = fma(xv[q], wv[q], acc[j]);
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
      const double mx = wave_max_f64(live ? my_logit : -INFINITY);
      const double ex = live ? exp(my_logit - mx) : 0.0;
      const double z = wave_sum_f64(ex);
      const double p = ex / z;
      bool taken = false;
      double gsel[8];
      int isel[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        gsel[s] = 0.0;
        isel[s] = 0;
        if (s < k) {
          // arg-max of p over the experts not yet taken; key (p desc, index asc)
          double pv = (live && !taken) ? p : -1.0;
          int bi = lane;
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) {
            const double po = __shfl_xor(pv, off, 64);
            const int io = __shfl_xor(bi, off, 64);
            if (po > pv || (po == pv && io < bi)) {
              pv = po;
              bi = io;
            }
          }
          if (lane == bi) taken = true;
          gsel[s] = pv;
          isel[s] = bi;
        }
      }
      if (lane == 0) {
        // Mixtral's renormalisation: the k gates over their sum (slot order)
        double sum = 0.0;
#pragma unroll
        for (int s = 0; s < 8; ++s) sum += gsel[s];
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (s < k) {
            idx[t * k + s] = isel[s];
            gate[t * k + s] = (float)(renorm ? gsel[s] / sum : gsel[s]);
          }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_router(int act_f32, const void* x, const void* router_w, int64_t T, int d, int E, int k,
                         int renorm, int32_t* idx, float* gate, hipStream_t stream) {
  int64_t blocks = T;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (act_f32)
    hipLaunchKernelGGL(router_topk_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)x, (const float*)router_w, T, d, E, k, renorm, idx, gate);
  else
    hipLaunchKernelGGL(router_topk_kernel<bf16_bits>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const bf16_bits*)x, (const bf16_bits*)router_w, T, d, E, k, renorm, idx, gate);
  return hipGetLastError();
}

// ---------------------------------------------------------------- permutation
// One workgroup of 1024 threads (16 wavefronts). Pass 1 counts the tokens of
// each expert (integer LDS atomics: order-independent), one scan gives the
// segment offsets, and pass 2 walks the tokens in chunks of 1024 in token
// order; wave ballots give each token its rank inside its wavefront, and a
// prefix over the wavefronts gives its rank inside the chunk. The result is a
// stable counting sort: segment e holds its tokens in ascending order.
// A token that lists an expert twice is counted once (both slots then point
// at the same row); indices outside [0, E) are dropped (pos = -1).
// With a capacity (cap >= 0; book ch. 10, section 10.3.2, the capacity
// factor box) an expert's assignments of rank >= cap in token order are
// dropped too: pos = -1, no row, and the segment holds the first cap.
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ idx, int64_t T, int E, int k,
                                                       int64_t cap, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ pos) {
  __shared__ int s_cnt[64];
  __shared__ int s_base[64];  // assignments of expert e in the chunks already walked
  __shared__ int s_off[64];   // first row of segment e
  __shared__ int s_lim[64];   // rows segment e keeps
  __shared__ int s_wave[16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) s_cnt[tid] = 0;
  __syncthreads();
  for (int64_t t = tid; t < T; t += 1024) {
    int es[8];
    for (int s = 0; s < k; ++s) {
      int e = idx[t * k + s];
      bool ok = e >= 0 && e < E;
      for (int q = 0; q < s; ++q) ok = ok && es[q] != e;
      es[s] = e;
      if (ok) atomicAdd(&s_cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      const int c = (cap >= 0 && (int64_t)s_cnt[e] > cap) ? (int)cap : s_cnt[e];
      offsets[e] = acc;
      counts[e] = c;
      s_off[e] = acc;
      s_lim[e] = c;
      s_base[e] = 0;
      acc += c;
    }
    offsets[E] = acc;
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t t0 = 0; t0 < T; t0 += 1024) {
    const int64_t t = t0 + tid;
    int my_e[8], my_rank[8];
    for (int s = 0; s < 8; ++s) {
      my_e[s] = -1;
      my_rank[s] = 0;
    }
    if (t < T)
      for (int s = 0; s < k; ++s) {
        int e = idx[t * k + s];
        my_e[s] = (e >= 0 && e < E) ? e : -1;
      }
    for (int e = 0; e < E; ++e) {
      bool sel = false;
      for (int s = 0; s < k; ++s) sel = sel || (my_e[s] == e);
      const uint64_t m = __ballot(sel);
      if (lane == 0) s_wave[wave][e] = __popcll(m);
      const int r = __popcll(m & lt_mask);
      for (int s = 0; s < k; ++s)
        if (my_e[s] == e) my_rank[s] = r;
    }
    __syncthreads();
    if (t < T) {
      for (int s = 0; s < k; ++s) {
        const int e = my_e[s];
        int row = -1;
        if (e >= 0) {
          int pre = 0;
          for (int w = 0; w < wave; ++w) pre += s_wave[w][e];
          const int rank = s_base[e] + pre + my_rank[s];
          if (rank < s_lim[e]) {
            row = s_off[e] + rank;
            perm[row] = (int32_t)t;
          }
        }
        pos[t * k + s] = row;
      }
    }
    __syncthreads();
    if (tid < E) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += s_wave[w][tid];
      s_base[tid] += tot;
    }
    __syncthreads();
  }
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int E, int k, int64_t cap, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, stream, idx, T, E, k, cap, counts, offsets, perm,
                     pos);
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
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < k; ++s) {
    const int row = pos[t * k + s];
    if (row < 0) continue;
    const float g = gate[t * k + s];
    const float* yr = Y + (int64_t)row * d + c;
    float4 y = *reinterpret_cast<const float4*>(yr);
    for (int p = 1; p < S; ++p) {
      const float4 q = *reinterpret_cast<const float4*>(yr + p * split_stride);
      y.x += q.x; y.y += q.y; y.z += q.z; y.w += q.w;
    }
    acc.x += g * y.x;
    acc.y += g * y.y;
    acc.z += g * y.z;
    acc.w += g * y.w;
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
