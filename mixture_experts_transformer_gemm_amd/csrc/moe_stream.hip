// Weight-streaming grouped GEMMs for decode-sized batches (every expert
// segment has at most 64 rows), gfx950.
//
// In decode the layer is bound by reading the hit experts' weights from HBM
// once (Grok-1 book ch. 1, section 1.2.1: generation moves the active weights
// per token and is bandwidth-bound). Measured on MI355X, reads that fetch at
// least one whole 128-byte line of each row per load instruction, with the
// nontemporal hint, sustain about 7 TB/s, while 64-byte pieces of 16 rows per
// instruction stay near 6 TB/s. So weight rows are streamed with
// global_load_lds_dwordx4 in the 8-rows-x-128-bytes shape (lane i fetches 16
// bytes of row i / 8) into an LDS ring of 6-8 stages and re-read from LDS in
// the MFMA fragment layout.
//
// Workgroup = 8 wavefronts, each streaming its own 16 weight rows. The
// segment's activation rows (token rows of x through the permutation, or H
// rows) of each stage are loaded once per workgroup, one 8-row instruction
// per wavefront for as many wavefronts as the segment needs, and shared by
// all 8 wavefronts. Each wavefront waits for its own loads of a stage
// (vmcnt), then one workgroup barrier makes the stage complete and frees the
// slot read in the previous stage. MFMAs run only for the 16-row tiles that
// hold rows of the segment; experts without rows exit at once and read no
// weights.
//
// Gate/up pass: a wavefront owns 8 gate channels and the same 8 up channels
// (16 weight rows, one 16x16x32 MFMA tile per 16 activation rows); lanes
// holding gate results take the matching up results from lane + 32 and form
// GELU(gate) * up. Down pass: a wavefront owns 16 output channels, split over
// the reduction into `gridDim.y` partial sums (fixed order, reduced by the
// combine stage).
//
// Fragment layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l mod 16)
// and 8 reduction values of group l / 16; result register v of lane l is
// C[4 (l / 16) + v][l mod 16] (weight row, activation row).
#include "moe_device.h"

#include <type_traits>

namespace gmoe {

namespace {

constexpr int kSB = 64;      // reduction values per stage
constexpr int kRowB = 128;   // LDS bytes per row and stage

// 16 bytes per lane straight into LDS with the nontemporal cache policy:
// each weight byte is read exactly once, and on MI355X the streaming reads
// reach about 7 TB/s only with this hint.
__device__ __forceinline__ void dma16s(const void* src, char* lds_base) { dma16_policy<2>(src, lds_base); }

}  // namespace

// Segments of up to 16*MT rows (MT = 1, 2, 4).
constexpr int kBW = 8;               // wavefronts per workgroup
constexpr int kBWRows = 16 * kBW;    // weight rows per workgroup stage

template <int MT>
struct BsCfg {
  static constexpr int XR = 16 * MT;                    // activation rows per stage
  static constexpr int kStageB = (kBWRows + XR) * kRowB;
  static constexpr int NS = 147456 / kStageB < 8 ? 147456 / kStageB : 8;
  static constexpr int kLdsBytes = NS * kStageB;
};

// s_waitcnt vmcnt(p * Q) for a run-time p in [0, 6]
template <int Q>
__device__ __forceinline__ void wait_stages(int p) {
  switch (p) {
    case 6: GMOE_WAIT_VM(6 * Q); break;
    case 5: GMOE_WAIT_VM(5 * Q); break;
    case 4: GMOE_WAIT_VM(4 * Q); break;
    case 3: GMOE_WAIT_VM(3 * Q); break;
    case 2: GMOE_WAIT_VM(2 * Q); break;
    case 1: GMOE_WAIT_VM(1 * Q); break;
    default: GMOE_WAIT_VM(0); break;
  }
  __asm__ __volatile__("" ::: "memory");  // no LDS access moves above the wait
}

template <bool GATEUP, int MT>
__global__ __launch_bounds__(kBW * 64) void stream_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                          const bf16_bits* __restrict__ w0,
                                                          const bf16_bits* __restrict__ w1, int64_t T, int K,
                                                          int N, int E, int64_t rows_cap, void* __restrict__ out) {
  using C = BsCfg<MT>;
  constexpr int NS = C::NS;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kChW = GATEUP ? 8 : 16;  // output channels per wavefront
  const int nblk = N / (kBW * kChW);
  const int e = blockIdx.x / nblk;
  const int nb = blockIdx.x - e * nblk;
  const int M = rv.counts[e];
  if (M <= 0) return;
  const int m0 = rv.offsets[e];
  const int c0 = nb * kBW * kChW + wave * kChW;
  const int S = gridDim.y, sp = blockIdx.y;
  const int kspan = K / S, kbeg = sp * kspan;
  const int nk = kspan / kSB;
  const int rows = min(M, C::XR);
  const int na = (rows + 7) >> 3;   // activation load instructions per stage
  const int mv = (rows + 15) >> 4;  // 16-row MFMA tiles with rows

  // this lane's sources: two weight instructions (rows 8q + lane / 8 of the
  // wavefront's 16) and, for wavefronts below na, one activation instruction
  const char* wsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int R = 16 * wave + r;  // ring row
    const int c = rslot(R, lane & 7);
    const bf16_bits* row;
    if (GATEUP)
      row = (r < 8 ? w0 : w1) + ((int64_t)e * N + c0 + (r & 7)) * K;
    else
      row = w0 + ((int64_t)e * N + c0 + r) * K;
    wsrc[q] = (const char*)(row + kbeg) + c * 16;
  }
  const char* asrc = nullptr;
  if (wave < na) {
    int xr = 8 * wave + (lane >> 3);
    const int c = rslot(kBWRows + xr, lane & 7);
    if (xr >= M) xr = M - 1;
    const bf16_bits* row;
    if (GATEUP) {
      int tok = rv.perm[m0 + xr];
      tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
      row = A + (int64_t)tok * K;
    } else {
      row = A + (int64_t)(m0 + xr) * K;
    }
    asrc = (const char*)(row + kbeg) + c * 16;
  }
  // workgroups start their walk over the reduction at different stages, so
  // that concurrent workgroups spread over the HBM channels
  const int rot = (int)(((unsigned)blockIdx.x * 37u + (unsigned)sp * 11u) % (unsigned)nk);

  const int r16 = lane & 15, g = lane >> 4;
  f32x4 acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto run = [&](auto act_tag) {
    constexpr bool HAS_ACT = decltype(act_tag)::value;
    constexpr int Q = HAS_ACT ? 3 : 2;  // this wavefront's load instructions per stage
    auto issue = [&](int stage, int slot) {
      int ks = stage + rot;
      if (ks >= nk) ks -= nk;
      char* dst = lds + slot * C::kStageB;
      dma16s(wsrc[0] + (size_t)ks * kRowB, dst + (16 * wave) * kRowB);
      dma16s(wsrc[1] + (size_t)ks * kRowB, dst + (16 * wave + 8) * kRowB);
      if (HAS_ACT) dma16s(asrc + (size_t)ks * kRowB, dst + (kBWRows + 8 * wave) * kRowB);
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nk) issue(s, s);
    for (int kt = 0; kt < nk; ++kt) {
      // this wavefront's loads of stage kt have landed ...
      wait_stages<Q>(min(nk - 1 - kt, NS - 2));
      // ... and everyone's: stage kt is complete in LDS, and slot (kt-1) mod
      // NS, read in the previous stage, is free
      lds_barrier();
      if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
      const char* b = lds + (kt % NS) * C::kStageB;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 4 * s + g;
        const int wr = 16 * wave + r16;
        const u32x4 wa = *reinterpret_cast<const u32x4*>(b + wr * kRowB + rslot(wr, c) * 16);
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          if (j < mv) {
            const int xr = kBWRows + 16 * j + r16;
            const u32x4 xa = *reinterpret_cast<const u32x4*>(b + xr * kRowB + rslot(xr, c) * 16);
            acc[j] = mfma16(wa, xa, acc[j]);
          }
        }
      }
    }
  };
  if (wave < na)
    run(std::integral_constant<bool, true>{});
  else
    run(std::integral_constant<bool, false>{});

#pragma unroll
  for (int j = 0; j < MT; ++j) {
    if (j < mv) {
      const int m = 16 * j + r16;  // activation row of this lane's results
      if (GATEUP) {
        // lanes with g < 2 hold gate channels 4g..4g+3, lane + 32 the same up channels
        float up[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) up[v] = __shfl(acc[j][v], lane + 32, 64);
        if (g < 2 && m < M) {
          float h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = gelu_erf(acc[j][v]) * up[v];
          uint2 o;
          o.x = pack_bf16x2(h[0], h[1]);
          o.y = pack_bf16x2(h[2], h[3]);
          *reinterpret_cast<uint2*>((bf16_bits*)out + (int64_t)(m0 + m) * N + c0 + 4 * g) = o;
        }
      } else if (m < M) {
        float* Ys = (float*)out + (int64_t)sp * rows_cap * N;
        *reinterpret_cast<float4*>(Ys + (int64_t)(m0 + m) * N + c0 + 4 * g) =
            make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      }
    }
  }
}

template <bool GATEUP, int MT>
static hipError_t stream_launch(dim3 grid, hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0,
                                 const void* w1, int64_t T, int K, int N, int E, int64_t rows_cap, void* out) {
  constexpr int lds = BsCfg<MT>::kLdsBytes;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&stream_kernel<GATEUP, MT>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((stream_kernel<GATEUP, MT>), grid, dim3(kBW * 64), lds, st, A, rv, (const bf16_bits*)w0,
                     (const bf16_bits*)w1, T, K, N, E, rows_cap, out);
  return hipGetLastError();
}

hipError_t launch_stream_gateup(int max_rows, const bf16_bits* x, RouteView rv, const void* wg, const void* wu,
                                int64_t T, int d, int f, int E, bf16_bits* H, hipStream_t st) {
  const dim3 grid((unsigned)E * (unsigned)(f / (kBW * 8)));
  if (max_rows <= 16) return stream_launch<true, 1>(grid, st, x, rv, wg, wu, T, d, f, E, 0, H);
  if (max_rows <= 32) return stream_launch<true, 2>(grid, st, x, rv, wg, wu, T, d, f, E, 0, H);
  return stream_launch<true, 4>(grid, st, x, rv, wg, wu, T, d, f, E, 0, H);
}

hipError_t launch_stream_down(int max_rows, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                              int64_t rows_cap, int d, int f, int E, float* Y, hipStream_t st) {
  const dim3 grid((unsigned)E * (unsigned)(d / (kBW * 16)), (unsigned)splits);
  if (max_rows <= 16) return stream_launch<false, 1>(grid, st, H, rv, wd, wd, 0, f, d, E, rows_cap, Y);
  if (max_rows <= 32) return stream_launch<false, 2>(grid, st, H, rv, wd, wd, 0, f, d, E, rows_cap, Y);
  return stream_launch<false, 4>(grid, st, H, rv, wd, wd, 0, f, d, E, rows_cap, Y);
}

}  // namespace gmoe
