// Weight-streaming grouped GEMMs for decode-sized batches (every expert
// segment has at most 16 rows), gfx950.
//
// In decode the layer is bound by reading the hit experts' weights from HBM
// once (Grok-1 book ch. 1, section 1.2.1: generation moves the active weights
// per token and is bandwidth-bound). Measured on MI355X, reads that fetch at
// least one whole 128-byte line of each row per load instruction sustain
// about 7 TB/s, while 64-byte pieces of 16 rows per instruction stay near
// 6 TB/s. So each wavefront streams its weight rows with
// global_load_lds_dwordx4 in the 8-rows-x-128-bytes shape (lane i fetches
// 16 bytes of row i / 8) into a wavefront-private LDS ring, and re-reads them
// from LDS in the MFMA fragment layout. The ring is private to the
// wavefront, so no workgroup barrier is needed: each wavefront waits only
// for its own loads (vmcnt).
//
// Gate/up pass: a wavefront owns 8 gate channels and the same 8 up channels
// (16 weight rows, one 16x16x32 MFMA tile); lanes holding gate results take
// the matching up results from lane + 32 and form GELU(gate) * up.
// Down pass: a wavefront owns 16 output channels, split over the reduction
// into `gridDim.y` partial sums (fixed order, reduced by the combine stage).
// Activation rows (token rows of x through the permutation, or H rows) are
// loaded into the same ring with the same instruction shape.
//
// Fragment layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l mod 16)
// and 8 reduction values of group l / 16; result register v of lane l is
// C[4 (l / 16) + v][l mod 16] (weight row, activation row).
#include "moe_device.h"

namespace gmoe {

namespace {

constexpr int kSB = 64;      // reduction values per stage
constexpr int kRowB = 128;   // LDS bytes per row and stage
constexpr int kWR = 16;      // weight rows per wavefront
constexpr int kNS = 6;       // ring stages per wavefront

// slot of 16-byte chunk c of ring row r (conflict-free for the fragment reads)
__device__ __forceinline__ int rslot(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// 16 bytes per lane straight into LDS (lane i writes lds_base + 16 i) with
// the nontemporal cache policy: each weight byte is read exactly once, and
// on MI355X the streaming reads reach about 7 TB/s only with this hint.
__device__ __forceinline__ void dma16s(const void* src, char* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, /*nt*/ 2);
#endif
}

#define GMOE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

}  // namespace

template <bool GATEUP, int XR>
__global__ __launch_bounds__(256) void stream_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                     const bf16_bits* __restrict__ w0,
                                                     const bf16_bits* __restrict__ w1, int64_t T, int K, int N,
                                                     int E, int64_t rows_cap, void* __restrict__ out) {
  constexpr int RS = kWR + XR;      // ring rows per stage
  constexpr int Q = RS / 8;         // load instructions per stage
  constexpr int kStageB = RS * kRowB;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kChW = GATEUP ? 8 : 16;  // output channels per wavefront
  const int nblk = N / (4 * kChW);
  const int e = blockIdx.x / nblk;
  const int nb = blockIdx.x - e * nblk;
  const int M = rv.counts[e];
  if (M <= 0) return;
  const int m0 = rv.offsets[e];
  const int c0 = nb * 4 * kChW + wave * kChW;  // first channel of this wavefront
  const int S = gridDim.y, sp = blockIdx.y;
  const int kspan = K / S, kbeg = sp * kspan;
  const int nk = kspan / kSB;
  char* ring = lds + wave * (kNS * kStageB);

  // source row of each load instruction q for this lane (stage 0 of the split)
  const char* src[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int c = rslot(r, lane & 7);  // chunk that belongs in slot lane & 7
    const bf16_bits* row;
    if (r < kWR) {
      if (GATEUP)
        row = (r < 8 ? w0 : w1) + ((int64_t)e * N + c0 + (r & 7)) * K;
      else
        row = w0 + ((int64_t)e * N + c0 + r) * K;
    } else {
      int xr = r - kWR;
      if (xr >= M) xr = M - 1;
      if (GATEUP) {
        int tok = rv.perm[m0 + xr];
        tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
        row = A + (int64_t)tok * K;
      } else {
        row = A + (int64_t)(m0 + xr) * K;
      }
    }
    src[q] = (const char*)(row + kbeg) + c * 16;
  }
  // Each wavefront starts its walk over the reduction at its own stage: down
  // weight rows are 64 KB apart, and wavefronts all reading the same offset of
  // neighbouring rows would hit the same HBM channels. The order of the
  // partial sums is fixed per wavefront, so results stay deterministic.
  const int rot = (int)(((unsigned)(blockIdx.x * 4 + wave) * 37u) % (unsigned)nk);
  auto issue = [&](int stage, int slot) {
    int ks = stage + rot;
    if (ks >= nk) ks -= nk;
    char* dst = ring + slot * kStageB;
#pragma unroll
    for (int q = 0; q < Q; ++q) dma16s(src[q] + (size_t)ks * kRowB, dst + q * 1024);
  };

  const int r16 = lane & 15, g = lane >> 4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // prologue: stages 0..kNS-2 in flight (no load past the last stage: every
  // weight byte is fetched once)
#pragma unroll
  for (int s = 0; s < kNS - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed in the ring: the loads of the stages after it
    // (min(nk - 1 - kt, kNS - 2) of them) may still be in flight
    switch (min(nk - 1 - kt, kNS - 2)) {
      case 4: GMOE_WAIT_VM(4 * Q); break;
      case 3: GMOE_WAIT_VM(3 * Q); break;
      case 2: GMOE_WAIT_VM(2 * Q); break;
      case 1: GMOE_WAIT_VM(1 * Q); break;
      default: GMOE_WAIT_VM(0); break;
    }
    __asm__ __volatile__("" ::: "memory");  // no LDS access moves above the wait
    // the slot of stage kt-1 was fully read (its MFMAs consumed it): refill it
    if (kt + kNS - 1 < nk) issue(kt + kNS - 1, (kt + kNS - 1) % kNS);
    const char* b = ring + (kt % kNS) * kStageB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * s + g;
      const int wr = r16;
      const int xr = kWR + (XR == 8 ? (r16 & 7) : r16);
      const u32x4 wa = *reinterpret_cast<const u32x4*>(b + wr * kRowB + rslot(wr, c) * 16);
      const u32x4 xa = *reinterpret_cast<const u32x4*>(b + xr * kRowB + rslot(xr, c) * 16);
      acc = mfma16(wa, xa, acc);
    }
  }
  GMOE_WAIT_VM(0);  // no load may still be writing the ring when the wavefront exits

  const int m = r16;  // activation row of this lane's results
  if (GATEUP) {
    // lanes with g < 2 hold gate channels 4g..4g+3, lane + 32 the same up channels
    float up[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) up[v] = __shfl(acc[v], lane + 32, 64);
    if (g < 2 && m < M) {
      float h[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) h[v] = gelu_erf(acc[v]) * up[v];
      uint2 o;
      o.x = pack_bf16x2(h[0], h[1]);
      o.y = pack_bf16x2(h[2], h[3]);
      *reinterpret_cast<uint2*>((bf16_bits*)out + (int64_t)(m0 + m) * N + c0 + 4 * g) = o;
    }
  } else {
    if (m < M) {
      float* Ys = (float*)out + (int64_t)sp * rows_cap * N;
      *reinterpret_cast<float4*>(Ys + (int64_t)(m0 + m) * N + c0 + 4 * g) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

template <bool GATEUP, int XR>
static hipError_t stream_launch(dim3 grid, hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0,
                                const void* w1, int64_t T, int K, int N, int E, int64_t rows_cap, void* out) {
  constexpr int lds = 4 * kNS * (kWR + XR) * kRowB;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&stream_kernel<GATEUP, XR>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((stream_kernel<GATEUP, XR>), grid, dim3(256), lds, st, A, rv, (const bf16_bits*)w0,
                     (const bf16_bits*)w1, T, K, N, E, rows_cap, out);
  return hipGetLastError();
}

hipError_t launch_stream_gateup(int max_rows, const bf16_bits* x, RouteView rv, const void* wg, const void* wu,
                                int64_t T, int d, int f, int E, bf16_bits* H, hipStream_t st) {
  const dim3 grid((unsigned)E * (unsigned)(f / 32));
  if (max_rows <= 8) return stream_launch<true, 8>(grid, st, x, rv, wg, wu, T, d, f, E, 0, H);
  return stream_launch<true, 16>(grid, st, x, rv, wg, wu, T, d, f, E, 0, H);
}

hipError_t launch_stream_down(int max_rows, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                              int64_t rows_cap, int d, int f, int E, float* Y, hipStream_t st) {
  const dim3 grid((unsigned)E * (unsigned)(d / 64), (unsigned)splits);
  if (max_rows <= 8) return stream_launch<false, 8>(grid, st, H, rv, wd, wd, 0, f, d, E, rows_cap, Y);
  return stream_launch<false, 16>(grid, st, H, rv, wd, wd, 0, f, d, E, rows_cap, Y);
}

}  // namespace gmoe
