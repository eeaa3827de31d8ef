// Weight-streaming grouped GEMMs for 8-bit expert weights and small or
// medium expert segments (processed in chunks of up to 16*MT rows), gfx950.
//
// With 8-bit weights (Grok-1 book ch. 1, section 1.2, the INT8 box: int8
// values with a scale per group, dequantised at compute time) a weight byte
// carries half the reduction values a bf16 byte does, so each stage's
// activation rows are as large as its weight rows. Weights are used by one
// wavefront only, so they bypass LDS: every wavefront loads its own 32
// weight rows straight into registers (16 rows x 64 bytes per load
// instruction, in a register ring of NS stages), while the segment's
// activation rows of each stage go once per workgroup into an LDS ring
// (global_load_lds) shared by all 8 wavefronts. LDS thus holds only
// activations, NS stages deep.
//
// MFMA v_mfma_f32_16x16x32_bf16 with the weights as the "A" operand: lane l
// supplies row (l mod 16) and 8 reduction values of group g = l / 16; result
// register v of lane l is C[4g + v][l mod 16] (weight row, activation row).
// A lane's 16-byte weight load holds the 16 reduction values [16g, 16g+16)
// of the 64-value stage: widened to bf16 (exact), the low 8 feed step 0 and
// the high 8 step 1, and the activation fragment of step s for group g is
// read from the same indices [16g + 8s, +8). Each MFMA pairs equal reduction
// indices; only the order of the sum within a stage differs.
//
// Gate/up pass: a wavefront owns 16 gate channels (A tile 0) and the same 16
// up channels (A tile 1), so each lane holds matching gate and up results
// and forms GELU(gate * s_gate) * (up * s_up) in registers. Down pass: a
// wavefront owns 32 output channels, split over the reduction into
// gridDim.y partial sums (reduced in fixed order by the combine stage).
#include "moe_device.h"

#include <type_traits>

namespace gmoe {

namespace {

constexpr int kW8Waves = 8;     // wavefronts per workgroup
constexpr int kW8Stage = 64;    // reduction values per stage
constexpr int kActRowB = 128;   // LDS bytes per activation row and stage

template <int MT>
struct S8Cfg {
  static constexpr int XR = 16 * MT;           // activation rows per chunk
  static constexpr int NS = 8;                 // stages in flight + 1
  static constexpr int kStageB = XR * kActRowB;
  static constexpr int kLdsBytes = NS * kStageB;
  static constexpr int NI = 2 * MT;            // activation load instructions per stage (8 rows each)
};

// calls f(integral_constant<int, I>) for I = B .. N-1 in order
template <int B, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < N) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, N>(f);
  }
}

}  // namespace

template <bool GATEUP, int MT>
__global__ __launch_bounds__(kW8Waves * 64) void stream8_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                               const int8_t* __restrict__ w0,
                                                               const int8_t* __restrict__ w1,
                                                               const float* __restrict__ scales, int64_t T, int K,
                                                               int N, int E, int Ftot, int64_t rows_cap,
                                                               void* __restrict__ out) {
  using C = S8Cfg<MT>;
  constexpr int NS = C::NS;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  constexpr int kChW = GATEUP ? 16 : 32;  // output channels per wavefront
  const int nblk = N / (kW8Waves * kChW);
  const int e = blockIdx.x / nblk;
  const int nb = blockIdx.x - e * nblk;
  const int M = rv.counts[e];
  const int mbase = (int)blockIdx.z * C::XR;  // first row of this chunk within the segment
  if (mbase >= M) return;
  const int m0 = rv.offsets[e] + mbase;
  const int rows = min(M - mbase, C::XR);
  const int mv = (rows + 15) >> 4;  // 16-row MFMA tiles with rows
  const int c0 = nb * kW8Waves * kChW + wave * kChW;
  const int S = gridDim.y, sp = blockIdx.y;
  const int kspan = K / S, kbeg = sp * kspan;
  const int nk = kspan / kW8Stage;

  // this lane's weight rows: A tile t, row r16, reduction values 16g.. of each stage
  const int8_t* wrow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int ch = GATEUP ? c0 + r16 : c0 + 16 * t + r16;
    const int8_t* base = (GATEUP && t == 1) ? w1 : w0;
    wrow[t] = base + ((int64_t)e * N + ch) * K + kbeg + 16 * g;
  }
  // activation load instructions of this wavefront: wave, wave + 8, ... < NI
  constexpr int kQA = (C::NI + kW8Waves - 1) / kW8Waves;
  const char* asrc[kQA];
#pragma unroll
  for (int a = 0; a < kQA; ++a) {
    const int inst = wave + kW8Waves * a;
    const int R = 8 * (inst < C::NI ? inst : 0) + (lane >> 3);  // ring row
    const int c = rslot(R, lane & 7);
    const int xr = R < rows ? R : rows - 1;
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
  const int na = (C::NI - wave + kW8Waves - 1) / kW8Waves;  // instructions this wavefront issues (0..kQA)

  f32x4 acc[2][MT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 wq[NS][2];

  // MV: 16-row tiles that get MFMAs (the segment's rows, rounded up to MT/2
  // or MT tiles; rows past the segment's end repeat its last row)
  // MV: 16-row tiles that get MFMAs (the segment's rows, rounded up to MT/2
  // or MT tiles; rows past the segment's end repeat its last row)
  auto run = [&](auto na_tag, auto mv_tag) {
    constexpr int NA = decltype(na_tag)::value;
    constexpr int MV = decltype(mv_tag)::value;
    constexpr int Q = NA + 2;  // this wavefront's load instructions per stage
    auto issue = [&](int stage, auto slot_tag) {
      constexpr int slot = decltype(slot_tag)::value;
      char* dst = lds + slot * C::kStageB;
#pragma unroll
      for (int a = 0; a < NA; ++a)
        dma16_policy<0>(asrc[a] + (size_t)stage * kActRowB, dst + (wave + kW8Waves * a) * 1024);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        wq[slot][t] = __builtin_nontemporal_load((const u32x4*)(wrow[t] + (size_t)stage * kW8Stage));
    };
    auto wait_stages = [&](int p) {  // at most p later stages of loads in flight
      switch (p) {
        case 6: GMOE_WAIT_VM(6 * Q); break;
        case 5: GMOE_WAIT_VM(5 * Q); break;
        case 4: GMOE_WAIT_VM(4 * Q); break;
        case 3: GMOE_WAIT_VM(3 * Q); break;
        case 2: GMOE_WAIT_VM(2 * Q); break;
        case 1: GMOE_WAIT_VM(1 * Q); break;
        default: GMOE_WAIT_VM(0); break;
      }
      __asm__ __volatile__("" ::: "memory");
    };
    static_assert(NS - 2 <= 6, "wait_stages covers up to 6 stages in flight");
    // prologue: stages 0..NS-2 (each stage s in ring / register slot s)
    static_for<0, NS - 1>([&](auto i_tag) {
      if (decltype(i_tag)::value < nk) issue(decltype(i_tag)::value, i_tag);
    });
    for (int kt0 = 0; kt0 < nk; kt0 += NS) {
      // stage kt = kt0 + u lives in slot u
      static_for<0, NS>([&](auto u_tag) {
        constexpr int u = decltype(u_tag)::value;
        const int kt = kt0 + u;
        if (kt >= nk) return;
        wait_stages(min(nk - 1 - kt, NS - 2));
        // every wavefront's loads of stage kt have landed, and the ring slot
        // read in the previous stage is free
        lds_barrier();
        if (kt + NS - 1 < nk) issue(kt + NS - 1, std::integral_constant<int, (u + NS - 1) % NS>{});
        const char* b = lds + u * C::kStageB;
        u32x4 lo[2], hi[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) i8x16_to_frags(wq[u][t], lo[t], hi[t]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          u32x4 xa[MV];
#pragma unroll
          for (int j = 0; j < MV; ++j) {
            const int xr = 16 * j + r16;
            xa[j] = *reinterpret_cast<const u32x4*>(b + xr * kActRowB + rslot(xr, 2 * g + s) * 16);
          }
#pragma unroll
          for (int j = 0; j < MV; ++j) {
            acc[0][j] = mfma16(s ? hi[0] : lo[0], xa[j], acc[0][j]);
            acc[1][j] = mfma16(s ? hi[1] : lo[1], xa[j], acc[1][j]);
          }
        }
      });
    }
    GMOE_WAIT_VM(0);
  };
  constexpr int kHalf = MT > 1 ? MT / 2 : 1;
  auto run_na = [&](auto na_tag) {
    if (mv <= kHalf)
      run(na_tag, std::integral_constant<int, kHalf>{});
    else
      run(na_tag, std::integral_constant<int, MT>{});
  };
  if (na >= 2)
    run_na(std::integral_constant<int, (kQA >= 2 ? 2 : kQA)>{});
  else if (na == 1)
    run_na(std::integral_constant<int, 1>{});
  else
    run_na(std::integral_constant<int, 0>{});

#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = 16 * j + r16;  // activation row (within the chunk) of this lane's results
    if (j < mv && m < rows) {
      if (GATEUP) {
        const float* sg = scales + (int64_t)e * N + c0 + 4 * g;
        const float* su = scales + (int64_t)E * N + (int64_t)e * N + c0 + 4 * g;
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = gelu_erf(acc[0][j][v] * sg[v]) * (acc[1][j][v] * su[v]);
        uint2 o;
        o.x = pack_bf16x2(h[0], h[1]);
        o.y = pack_bf16x2(h[2], h[3]);
        *reinterpret_cast<uint2*>((bf16_bits*)out + (int64_t)(m0 + m) * N + c0 + 4 * g) = o;
      } else {
        float* Ys = (float*)out + (int64_t)sp * rows_cap * N;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int ch = c0 + 16 * t + 4 * g;
          const float* sd = scales + 2 * (int64_t)E * Ftot + (int64_t)e * N + ch;
          *reinterpret_cast<float4*>(Ys + (int64_t)(m0 + m) * N + ch) =
              make_float4(acc[t][j][0] * sd[0], acc[t][j][1] * sd[1], acc[t][j][2] * sd[2], acc[t][j][3] * sd[3]);
        }
      }
    }
  }
}

template <bool GATEUP, int MT>
static hipError_t stream8_launch(dim3 grid, hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0,
                                 const void* w1, const float* scales, int64_t T, int K, int N, int E, int Ftot,
                                 int64_t rows_cap, void* out) {
  constexpr int lds = S8Cfg<MT>::kLdsBytes;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&stream8_kernel<GATEUP, MT>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((stream8_kernel<GATEUP, MT>), grid, dim3(kW8Waves * 64), lds, st, A, rv, (const int8_t*)w0,
                     (const int8_t*)w1, scales, T, K, N, E, Ftot, rows_cap, out);
  return hipGetLastError();
}

// rows of one expert <= max_rows; chunks of 16*MT rows along grid z
template <bool GATEUP>
static hipError_t stream8_dispatch(int max_rows, unsigned gx, unsigned gy, hipStream_t st, const bf16_bits* A,
                                   RouteView rv, const void* w0, const void* w1, const float* scales, int64_t T,
                                   int K, int N, int E, int Ftot, int64_t rows_cap, void* out) {
  auto chunks = [&](int xr) { return (unsigned)((max_rows + xr - 1) / xr); };
  if (max_rows <= 16)
    return stream8_launch<GATEUP, 1>(dim3(gx, gy, chunks(16)), st, A, rv, w0, w1, scales, T, K, N, E, Ftot, rows_cap,
                                     out);
  if (max_rows <= 32)
    return stream8_launch<GATEUP, 2>(dim3(gx, gy, chunks(32)), st, A, rv, w0, w1, scales, T, K, N, E, Ftot, rows_cap,
                                     out);
  if (max_rows <= 64)
    return stream8_launch<GATEUP, 4>(dim3(gx, gy, chunks(64)), st, A, rv, w0, w1, scales, T, K, N, E, Ftot, rows_cap,
                                     out);
  return stream8_launch<GATEUP, 8>(dim3(gx, gy, chunks(128)), st, A, rv, w0, w1, scales, T, K, N, E, Ftot, rows_cap,
                                   out);
}

hipError_t launch_stream8_gateup(int max_rows, const bf16_bits* x, RouteView rv, const void* wg, const void* wu,
                                 const float* scales, int64_t T, int d, int f, int E, bf16_bits* H,
                                 hipStream_t st) {
  return stream8_dispatch<true>(max_rows, (unsigned)E * (unsigned)(f / (kW8Waves * 16)), 1u, st, x, rv, wg, wu,
                                scales, T, d, f, E, f, 0, H);
}

hipError_t launch_stream8_down(int max_rows, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                               const float* scales, int64_t rows_cap, int d, int f, int E, float* Y,
                               hipStream_t st) {
  return stream8_dispatch<false>(max_rows, (unsigned)E * (unsigned)(d / (kW8Waves * 32)), (unsigned)splits, st, H, rv,
                                 wd, wd, scales, rows_cap, f, d, E, f, rows_cap, Y);
}

}  // namespace gmoe
