// Weight-streaming grouped GEMMs for small batches, gfx950: bf16 weights
// with every expert segment of at most 64 rows, and 8-bit weights with
// segments processed in chunks of up to 128 rows.
//
// In decode the layer is bound by reading the hit experts' weights from HBM
// once (Grok-1 book ch. 1, section 1.2.1: generation moves the active weights
// per token and is bandwidth-bound). Measured on MI355X, reads that fetch at
// least one whole 128-byte line of each row per load instruction, with the
// nontemporal hint, sustain about 7 TB/s, while 64-byte pieces of 16 rows per
// instruction stay near 6 TB/s. So weight rows are streamed with
// global_load_lds_dwordx4 in the 8-rows-x-128-bytes shape (lane i fetches 16
// bytes of row i / 8) into an LDS ring of 3-8 stages and re-read from LDS in
// the MFMA fragment layout. A stage holds 128 bytes of each weight row: 64
// reduction values of bf16 weights, 128 of 8-bit weights (Grok-1 book ch. 1,
// section 1.2, the INT8 box: int8 values with a scale per group, dequantised
// at compute time; here one fp32 scale per output channel, applied in the
// epilogue).
//
// Workgroup = 8 wavefronts, each streaming its own 16 weight rows (32 for
// 8-bit weights: each activation fragment read from LDS then feeds two
// MFMAs, and 8-bit rows are half as long, so a workgroup keeps a long
// stream). The
// segment's activation rows (token rows of x through the permutation, or H
// rows) of each stage are loaded once per workgroup, spread over the
// wavefronts for as many load instructions as the rows need, and shared by
// all 8 wavefronts. Each wavefront waits for its own loads of a stage
// (vmcnt), then one workgroup barrier makes the stage complete and frees the
// slot read in the previous stage. MFMAs run only for the 16-row tiles that
// hold rows of the segment; experts without rows exit at once and read no
// weights.
//
// Gate/up pass: a wavefront owns 8 gate channels and the same 8 up channels
// (16 weight rows, one 16x16x32 MFMA tile per 16 activation rows); lanes
// holding gate results take the matching up results from lane + 32 and form
// act(gate) * up (GELU, or SiLU for SwiGLU experts); with gridDim.y > 1
// (fine-grained layers at small batches) each slice of the reduction writes
// its fp32 gate and up sums instead, and glu_splits_kernel forms H. Down
// pass: a wavefront owns 16 output channels, split over the reduction into
// `gridDim.y` partial sums (fixed order, reduced by the combine stage).
//
// Fragment layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l mod 16)
// and 8 reduction values of group l / 16; result register v of lane l is
// C[4 (l / 16) + v][l mod 16] (weight row, activation row). With 8-bit
// weights a lane's 16-byte weight read holds 16 reduction values of two MFMA
// steps (widened to bf16, exact); the activation fragment of each step is
// read from the same reduction indices, so every product pairs equal
// indices.
#include "moe_device.h"

#include <type_traits>
#include <utility>

namespace gmoe {

namespace {

constexpr int kRowB = 128;   // LDS bytes per row and stage

// 16 bytes per lane straight into LDS with the nontemporal cache policy:
// each weight byte is read exactly once, and on MI355X the streaming reads
// reach about 7 TB/s only with this hint. Activation rows, which every
// channel block of an expert reads again, keep the default policy: with the
// hint they were refetched from beyond L2 (FETCH_SIZE of the 8-bit down
// pass at 256 tokens 1.5x its weight bytes), and without it the 8-bit layer
// at 256 tokens measured 1.31 ms instead of 1.40 ms.
__device__ __forceinline__ void dma16s(const void* src, char* lds_base) { dma16_policy<2>(src, lds_base); }

}  // namespace

// Segments processed in chunks of up to 16*MT rows (MT = 1, 2, 4, 8; chunk
// z of a segment along grid z). W8: 8-bit weights.
constexpr int kBW = 8;               // wavefronts per workgroup

// A stage holds kRowB bytes of every weight row: 64 reduction values of bf16
// weights, 128 of 8-bit weights; activation rows (bf16) hold the same
// reduction values: 128 or 256 bytes.
// WT: 16-row weight tiles per wavefront (each activation fragment read from
// LDS then feeds WT MFMAs).
template <int MT, bool W8, int WT = 1>
struct BsCfg {
  static constexpr int kBWRows = 16 * WT * kBW;          // weight rows per workgroup stage
  static constexpr int XR = 16 * MT;                     // activation rows per chunk
  static constexpr int KS = W8 ? 128 : 64;               // reduction values per stage
  static constexpr int AROWB = KS * 2;                   // activation bytes per row and stage
  static constexpr int ARPI = 1024 / AROWB;              // activation rows per load instruction
  static constexpr int NI = XR / ARPI;                   // activation load instructions per stage (max)
  static constexpr int kQA = (NI + kBW - 1) / kBW;       // of which one wavefront issues at most
  static constexpr int kActOff = kBWRows * kRowB;        // activation rows follow the weight rows
  // ring space: all 160 KB (one workgroup per CU either way; with 8-bit
  // weights and 65-80 rows a stage is 52 KB, so 3 stages fit instead of 2:
  // 2% off both 8-bit passes at 256 tokens, neutral elsewhere)
  static constexpr int kLdsBytes = 163840;
  // Ring of a workgroup whose chunk needs MV 16-row tiles: its stages hold
  // only those activation rows, so fewer rows leave room for more stages
  // (as many as fit in the ring space, at most 8).
  template <int MV>
  struct Ring {
    static constexpr int kStageB = kActOff + 16 * MV * AROWB;
    static constexpr int NS = kLdsBytes / kStageB < 8 ? kLdsBytes / kStageB : 8;
  };
};

// slot of 16-byte chunk c of a 256-byte activation row r (16 chunks; the 16
// rows read at one chunk land in 16 distinct bank groups)
__device__ __forceinline__ int aslot256(int r, int c) { return c ^ (r & 15); }

// f(integral_constant<int, u>) for u = 0 .. N-1, unrolled
template <class F, int... U>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

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

template <bool GATEUP, int MT, bool W8, int WT>
__global__ __launch_bounds__(kBW * 64) void stream_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                          const void* __restrict__ w0, const void* __restrict__ w1,
                                                          const float* __restrict__ scales, int64_t T, int K,
                                                          int N, int E, int64_t rows_cap, int act,
                                                          void* __restrict__ out) {
  using C = BsCfg<MT, W8, WT>;
  constexpr int kBWRows = C::kBWRows;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kChW = (GATEUP ? 8 : 16) * WT;  // output channels per wavefront
  // workgroups per expert; the last one may reach past N (the down pass with
  // d % 128 != 0): its wavefronts past N read clamped weight rows, store nothing
  const int nblk = (N + kBW * kChW - 1) / (kBW * kChW);
  // Down pass with E % 8 == 0 (E <= 64) and every expert holding rows:
  // workgroup x runs on XCD x mod 8, and the order below keeps all of expert
  // e's workgroups on XCD e mod 8, so its H rows are fetched into one L2
  // instead of eight (measured 2-3% faster on the down pass; the gate/up
  // pass, whose x rows are few, measured slower with it). With an expert
  // empty its XCD would idle (one token: 2 of 8 experts, the down pass 2.7x
  // slower), so then every expert's workgroups stay spread over all XCDs.
  bool by_xcd = !GATEUP && (E & 7) == 0 && E <= 64;
  if (by_xcd)
    for (int i = 0; i < E; ++i) by_xcd = by_xcd && rv.counts[i] > 0;
  int e, nb;
  if (by_xcd) {
    const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
    e = xcd + 8 * (i / nblk);
    nb = i - (i / nblk) * nblk;
  } else {
    e = blockIdx.x / nblk;
    nb = blockIdx.x - e * nblk;
  }
  const int M = rv.counts[e];
  const int mbase = (int)blockIdx.z * C::XR;  // first row of this chunk within the segment
  if (mbase >= M) return;
  const int m0 = rv.offsets[e] + mbase;
  const int c0 = nb * kBW * kChW + wave * kChW;
  const int S = gridDim.y, sp = blockIdx.y;
  const int kspan = K / S, kbeg = sp * kspan;
  const int nk = kspan / C::KS;
  const int rows = min(M - mbase, C::XR);
  const int na = (rows + C::ARPI - 1) / C::ARPI;  // activation load instructions per stage
  const int mv = (rows + 15) >> 4;                // 16-row MFMA tiles with rows
  constexpr size_t wsz = W8 ? 1 : 2;

  // this lane's sources: 2 WT weight instructions (rows 8q + lane / 8 of the
  // wavefront's 16 WT; gate/up: tile w holds gate channels 8w.. in rows
  // 16w..16w+7 and the same up channels in rows 16w+8..16w+15) and the
  // activation instructions wave, wave + 8, ... < na
  const char* wsrc[2 * WT];
#pragma unroll
  for (int q = 0; q < 2 * WT; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int R = 16 * WT * wave + r;  // ring row
    const int c = rslot(R, lane & 7);
    const char* row;
    if (GATEUP)
      row = (const char*)((r & 8) == 0 ? w0 : w1) + ((int64_t)e * N + min(c0 + 8 * (r >> 4) + (r & 7), N - 1)) * K * wsz;
    else
      row = (const char*)w0 + ((int64_t)e * N + min(c0 + r, N - 1)) * K * wsz;
    wsrc[q] = row + kbeg * wsz + c * 16;
  }
  const char* asrc[C::kQA];
#pragma unroll
  for (int a = 0; a < C::kQA; ++a) {
    const int inst = wave + kBW * a;
    const int ar = C::ARPI * (inst < C::NI ? inst : 0) + lane / (C::AROWB / 16);  // activation row
    const int ch = lane % (C::AROWB / 16);
    const int c = W8 ? aslot256(ar, ch) : rslot(kBWRows + ar, ch);
    const int xr = ar < rows ? ar : rows - 1;
    const bf16_bits* row;
    if (GATEUP) {
      int tok = rv.perm[m0 + xr];
      tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
      row = A + (int64_t)tok * K;
    } else {
      row = A + (int64_t)(m0 + xr) * K;
    }
    asrc[a] = (const char*)(row + kbeg) + c * 16;
  }
  // instructions this wavefront issues per stage (0 .. kQA)
  const int naw = na > wave ? (na - wave + kBW - 1) / kBW : 0;
  // workgroups start their walk over the reduction at different stages, so
  // that concurrent workgroups spread over the HBM channels
  const int rot = (int)(((unsigned)blockIdx.x * 37u + (unsigned)sp * 11u + (unsigned)blockIdx.z * 5u) % (unsigned)nk);

  const int r16 = lane & 15, g = lane >> 4;
  f32x4 acc[WT][MT];
#pragma unroll
  for (int w = 0; w < WT; ++w)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[w][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA step on tiles 0..MV-1: weight fragments wa[WT], activation chunk cx
  auto tiles = [&](const char* b, const u32x4* wa, int cx, auto mv_tag) __attribute__((always_inline)) {
    constexpr int MV = decltype(mv_tag)::value;
    u32x4 xa[MV];
#pragma unroll
    for (int j = 0; j < MV; ++j) {
      const int xr = 16 * j + r16;
      const int slot = W8 ? aslot256(xr, cx) : rslot(kBWRows + xr, cx);
      xa[j] = *reinterpret_cast<const u32x4*>(b + C::kActOff + xr * C::AROWB + slot * 16);
    }
#pragma unroll
    for (int w = 0; w < WT; ++w)
#pragma unroll
      for (int j = 0; j < MV; ++j) acc[w][j] = mfma16(wa[w], xa[j], acc[w][j]);
  };

  auto run = [&](auto naw_tag, auto mv_tag) __attribute__((always_inline)) {
    constexpr int NAW = decltype(naw_tag)::value;
    constexpr int Q = 2 * WT + NAW;  // this wavefront's load instructions per stage
    constexpr int MVT = decltype(mv_tag)::value;
    using Rg = typename C::template Ring<MVT>;
    constexpr int NS = Rg::NS;
    auto issue = [&](int stage, int slot) __attribute__((always_inline)) {
      int ks = stage + rot;
      if (ks >= nk) ks -= nk;
      char* dst = lds + slot * Rg::kStageB;
#pragma unroll
      for (int q = 0; q < 2 * WT; ++q) dma16s(wsrc[q] + (size_t)ks * kRowB, dst + (16 * WT * wave + 8 * q) * kRowB);
#pragma unroll
      for (int a = 0; a < NAW; ++a)
        dma16_policy<0>(asrc[a] + (size_t)ks * C::AROWB, dst + C::kActOff + (wave + kBW * a) * 1024);
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
      const char* b = lds + (kt % NS) * Rg::kStageB;
      if (!W8) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int c = 4 * s + g;  // reduction values [32s + 8g, +8)
          u32x4 wa[WT];
#pragma unroll
          for (int w = 0; w < WT; ++w) {
            const int wr = 16 * WT * wave + 16 * w + r16;
            wa[w] = *reinterpret_cast<const u32x4*>(b + wr * kRowB + rslot(wr, c) * 16);
          }
          tiles(b, wa, c, mv_tag);
        }
      } else {
        // 8-bit weights: lane group g of half h reads values [64h + 16g, +16):
        // the low 8 feed step (h, 0), the high 8 step (h, 1); the activation
        // chunk of step (h, s) holds values [64h + 16g + 8s, +8)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = 4 * h + g;
          u32x4 lo[WT], hi[WT];
#pragma unroll
          for (int w = 0; w < WT; ++w) {
            const int wr = 16 * WT * wave + 16 * w + r16;
            const u32x4 q = *reinterpret_cast<const u32x4*>(b + wr * kRowB + rslot(wr, c) * 16);
            i8x16_to_frags(q, lo[w], hi[w]);
          }
          tiles(b, lo, 8 * h + 2 * g, mv_tag);
          tiles(b, hi, 8 * h + 2 * g + 1, mv_tag);
        }
      }
    }
  };
  // MV: tiles that get MFMAs. 8-bit weights: exactly the 16-row tiles that
  // hold rows (the stage is bound by its MFMA and LDS work, both linear in
  // MV: at 256 Grok-1 tokens 5 of 8 experts hold 65-71 rows, 80 rows of work
  // instead of 96). bf16: the chunk's rows rounded up to MT/4 (chunks of 64
  // rows or more), MT/2 or MT tiles. Rows past the segment's end repeat its
  // last row.
  constexpr int kHalf = MT > 1 ? MT / 2 : 1;
  constexpr int kQuarter = MT >= 4 ? MT / 4 : kHalf;
  auto run_naw = [&](auto naw_tag) __attribute__((always_inline)) {
    if constexpr (W8) {
      static_for<MT>([&](auto u_tag) __attribute__((always_inline)) {
        if (mv == decltype(u_tag)::value + 1) run(naw_tag, std::integral_constant<int, decltype(u_tag)::value + 1>{});
      });
    } else if (kQuarter < kHalf && mv <= kQuarter)
      run(naw_tag, std::integral_constant<int, kQuarter>{});
    else if (mv <= kHalf)
      run(naw_tag, std::integral_constant<int, kHalf>{});
    else if (MT == 8 && mv <= 6)  // 128-row chunks also stop at 96 rows
      run(naw_tag, std::integral_constant<int, (MT == 8 ? 6 : MT)>{});
    else
      run(naw_tag, std::integral_constant<int, MT>{});
  };
  static_assert(C::kQA <= 4, "up to 4 activation loads per wavefront and stage");
  if (naw >= 4 && C::kQA >= 4)
    run_naw(std::integral_constant<int, (C::kQA >= 4 ? 4 : 0)>{});
  else if (naw == 3 && C::kQA >= 3)
    run_naw(std::integral_constant<int, (C::kQA >= 3 ? 3 : 0)>{});
  else if (naw == 2 && C::kQA >= 2)
    run_naw(std::integral_constant<int, (C::kQA >= 2 ? 2 : 0)>{});
  else if (naw == 1)
    run_naw(std::integral_constant<int, 1>{});
  else
    run_naw(std::integral_constant<int, 0>{});

#pragma unroll
  for (int w = 0; w < WT; ++w) {
    // weight tile w: gate/up channels cw..cw+7, or down channels cw..cw+15
    const int cw = c0 + (GATEUP ? 8 : 16) * w;
    if (cw >= N) continue;  // past the last channel (N is a multiple of 16)
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      if (j < mv) {
        const int m = 16 * j + r16;  // activation row (within the chunk) of this lane's results
        if (GATEUP && S > 1) {
          // split sp's sums: lanes with g < 2 hold gate channels cw + 4g.., the
          // others the same up channels; G row = [gate 0..N) [up 0..N)
          if (m < rows) {
            const int up = g >> 1, ch = cw + 4 * (g & 1);
            float y[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
              y[v] = acc[w][j][v] * (W8 ? scales[(int64_t)up * E * N + (int64_t)e * N + ch + v] : 1.f);
            float* Gs = (float*)out + ((int64_t)sp * rows_cap + m0 + m) * (2 * (int64_t)N) + (int64_t)up * N;
            *reinterpret_cast<float4*>(Gs + ch) = make_float4(y[0], y[1], y[2], y[3]);
          }
        } else if (GATEUP) {
          // lanes with g < 2 hold gate channels 4g..4g+3, lane + 32 the same up channels
          float up[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) up[v] = __shfl(acc[w][j][v], lane + 32, 64);
          if (g < 2 && m < rows) {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              float gt = acc[w][j][v], u = up[v];
              if (W8) {
                gt *= scales[(int64_t)e * N + cw + 4 * g + v];
                u *= scales[(int64_t)E * N + (int64_t)e * N + cw + 4 * g + v];
              }
              h[v] = glu_act(act, gt) * u;
            }
            uint2 o;
            o.x = pack_bf16x2(h[0], h[1]);
            o.y = pack_bf16x2(h[2], h[3]);
            *reinterpret_cast<uint2*>((bf16_bits*)out + (int64_t)(m0 + m) * N + cw + 4 * g) = o;
          }
        } else if (m < rows) {
          float y[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            y[v] = acc[w][j][v] * (W8 ? scales[2 * (int64_t)E * K + (int64_t)e * N + cw + 4 * g + v] : 1.f);
          float* Ys = (float*)out + (int64_t)sp * rows_cap * N;
          *reinterpret_cast<float4*>(Ys + (int64_t)(m0 + m) * N + cw + 4 * g) = make_float4(y[0], y[1], y[2], y[3]);
        }
      }
    }
  }
}

template <bool GATEUP, int MT, bool W8, int WT>
static hipError_t stream_launch(unsigned gz, unsigned gy, hipStream_t st, const bf16_bits* A, RouteView rv,
                                const void* w0, const void* w1, const float* scales, int64_t T, int K, int N, int E,
                                int64_t rows_cap, int act, void* out) {
  constexpr int lds = BsCfg<MT, W8, WT>::kLdsBytes;
  static std::atomic<unsigned long long> lds_set{0};
  const hipError_t attr =
      set_lds_limit(reinterpret_cast<const void*>(&stream_kernel<GATEUP, MT, W8, WT>), lds, lds_set);
  if (attr != hipSuccess) return attr;
  // one workgroup per (expert, 8 wavefronts x channels per wavefront)
  constexpr int kWgCh = kBW * (GATEUP ? 8 : 16) * WT;
  const unsigned gx = (unsigned)E * (unsigned)((N + kWgCh - 1) / kWgCh);
  hipLaunchKernelGGL((stream_kernel<GATEUP, MT, W8, WT>), dim3(gx, gy, gz), dim3(kBW * 64), lds, st, A, rv, w0, w1,
                     scales, T, K, N, E, rows_cap, act, out);
  return hipGetLastError();
}

// Weight tiles per wavefront: 2 for 8-bit weights, 1 for bf16. Chunks of
// more than 32 rows are bound by the activation fragment reads, which then
// feed two MFMAs each; at small chunks the longer per-workgroup stream
// measured 10-19% faster (8-bit rows are half as long as bf16 ones, so one
// tile per wavefront leaves twice the workgroups, each with half the work).
// The down projection's split count assumes this (256 output channels per
// 8-bit workgroup).
template <int MT, bool W8, bool GATEUP>
constexpr int stream_wt() {
  return W8 ? 2 : 1;
}

// rows of one expert <= max_rows; chunks of 16*MT rows along grid z
template <bool GATEUP, bool W8>
static hipError_t stream_dispatch(int max_rows, unsigned gy, hipStream_t st, const bf16_bits* A, RouteView rv,
                                  const void* w0, const void* w1, const float* scales, int64_t T, int K, int N, int E,
                                  int64_t rows_cap, int act, void* out) {
  auto chunks = [&](int xr) { return (unsigned)((max_rows + xr - 1) / xr); };
  if (max_rows <= 16)
    return stream_launch<GATEUP, 1, W8, stream_wt<1, W8, GATEUP>()>(1, gy, st, A, rv, w0, w1, scales, T, K, N, E,
                                                                    rows_cap, act, out);
  if (max_rows <= 32)
    return stream_launch<GATEUP, 2, W8, stream_wt<2, W8, GATEUP>()>(1, gy, st, A, rv, w0, w1, scales, T, K, N, E,
                                                                    rows_cap, act, out);
  if (max_rows <= 64 || !W8)
    return stream_launch<GATEUP, 4, W8, stream_wt<4, W8, GATEUP>()>(chunks(64), gy, st, A, rv, w0, w1, scales, T, K,
                                                                    N, E, rows_cap, act, out);
  return stream_launch<GATEUP, 8, W8, stream_wt<8, W8, GATEUP>()>(chunks(128), gy, st, A, rv, w0, w1, scales, T, K, N,
                                                                  E, rows_cap, act, out);
}

// H[r][c] = act(sum_s G[s][r][c]) * (sum_s G[s][r][f + c]) in fp32 (slices
// added in ascending order), rounded to bf16, for the rows the permutation
// filled (offsets[E]); four channels per thread.
__global__ __launch_bounds__(256) void glu_splits_kernel(const float* __restrict__ G, int S, int64_t rows_cap,
                                                         const int32_t* __restrict__ offsets, int E, int f, int act,
                                                         bf16_bits* __restrict__ H) {
  const int64_t rows = offsets[E];
  const int64_t q = f / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * q; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / q;
    const int c = (int)(i - r * q) * 4;
    float gs[4] = {0.f, 0.f, 0.f, 0.f}, us[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const float* row = G + ((int64_t)s * rows_cap + r) * (2 * (int64_t)f);
      const float4 a = *reinterpret_cast<const float4*>(row + c);
      const float4 b = *reinterpret_cast<const float4*>(row + f + c);
      gs[0] += a.x; gs[1] += a.y; gs[2] += a.z; gs[3] += a.w;
      us[0] += b.x; us[1] += b.y; us[2] += b.z; us[3] += b.w;
    }
    float h[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) h[v] = glu_act(act, gs[v]) * us[v];
    uint2 o;
    o.x = pack_bf16x2(h[0], h[1]);
    o.y = pack_bf16x2(h[2], h[3]);
    *reinterpret_cast<uint2*>(H + r * f + c) = o;
  }
}

hipError_t launch_stream_gateup(int w8, int max_rows, int splits, const bf16_bits* x, RouteView rv, const void* wg,
                                const void* wu, const float* scales, int64_t T, int64_t rows_cap, int d, int f, int E,
                                int act, bf16_bits* H, float* G, hipStream_t st) {
  if (splits <= 1)
    return w8 ? stream_dispatch<true, true>(max_rows, 1u, st, x, rv, wg, wu, scales, T, d, f, E, 0, act, H)
              : stream_dispatch<true, false>(max_rows, 1u, st, x, rv, wg, wu, scales, T, d, f, E, 0, act, H);
  const unsigned gy = (unsigned)splits;
  const hipError_t err =
      w8 ? stream_dispatch<true, true>(max_rows, gy, st, x, rv, wg, wu, scales, T, d, f, E, rows_cap, act, G)
         : stream_dispatch<true, false>(max_rows, gy, st, x, rv, wg, wu, scales, T, d, f, E, rows_cap, act, G);
  if (err != hipSuccess) return err;
  int64_t blocks = (rows_cap * (f / 4) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(glu_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, st, G, splits, rows_cap, rv.offsets, E,
                     f, act, H);
  return hipGetLastError();
}

hipError_t launch_stream_down(int w8, int max_rows, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                              const float* scales, int64_t rows_cap, int d, int f, int E, float* Y,
                              hipStream_t st) {
  return w8 ? stream_dispatch<false, true>(max_rows, (unsigned)splits, st, H, rv, wd, wd, scales, 0, f, d, E,
                                           rows_cap, 0, Y)
            : stream_dispatch<false, false>(max_rows, (unsigned)splits, st, H, rv, wd, wd, scales, 0, f, d, E,
                                            rows_cap, 0, Y);
}

}  // namespace gmoe
