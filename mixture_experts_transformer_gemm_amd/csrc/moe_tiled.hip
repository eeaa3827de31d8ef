// LDS-tiled grouped GEMMs of the Grok-1 MoE layer for gfx950 (MI355X), used
// when experts hold more rows than the weight-streaming path handles.
//
// Each expert is one segment of a grouped GEMM over the expert-contiguous row
// permutation (Grok-1 book ch. 11, section 11.3.1: sparse reorder + grouped
// GEMM). Gate/up pass: H = GELU(X Wg^T) * (X Wu^T) -> bf16 (field guide,
// "MoE 子层": two input projections, GELU on one, elementwise product).
// Down pass: Y = H Wd^T -> fp32.
//
// Workgroup tile: BM rows x 256 weight rows, 4 wavefronts. For the gate/up
// pass the 256 weight rows are 128 gate channels and the same 128 up
// channels, so GELU(gate) * up is formed in registers. Products use
// v_mfma_f32_32x32x16_bf16 with the weight fragment as the "A" operand (32
// channels) and the activation fragment as "B" (32 rows): lane l supplies row
// (l mod 32) and the 8 reduction values of group l / 32; result register v of
// lane l is C[8 (v / 4) + 4 (l / 32) + (v mod 4)][l mod 32], so each lane
// owns runs of 4 consecutive channels of one row.
//
// Two feeds of LDS:
//  * bf16 weights (dma_kernel): global_load_lds_dwordx4 writes each stage of
//    32 reduction values straight into LDS (lane i of a wavefront lands at
//    LDS base + 16 i), four LDS stages, loads issued three stages ahead, an
//    explicit vmcnt wait and one barrier per stage. No staging registers.
//  * 8-bit weights (staged_kernel): 64-wide stages pass through registers so
//    the int8 values can be widened to bf16 (exact) on the way into LDS; two
//    LDS stages, loads issued a stage ahead of their LDS write.
//
// Tile order: the tiles that exist (sum over experts of ceil(rows / BM),
// times the channel tiles) are split into 8 contiguous ranges, one per XCD
// (workgroup i runs on XCD i mod 8); each range walks groups of 8 row tiles
// with the row tile fastest, so the workgroups resident on one XCD share
// weight tiles through its L2.
#include "moe_device.h"

#include <type_traits>

namespace gmoe {

constexpr int TBN = 256;

#ifndef GMOE_DMA_SB
#define GMOE_DMA_SB 64
#endif
#ifndef GMOE_PHASED
#define GMOE_PHASED 1
#endif
#ifndef GMOE_ISSUE_STEP
#define GMOE_ISSUE_STEP 0
#endif
#ifndef GMOE_PERSIST
#define GMOE_PERSIST 0
#endif
#ifndef GMOE_GROUPM
#define GMOE_GROUPM 8
#endif
constexpr int kGroupM = GMOE_GROUPM;

template <int BM, int NW = 4>
struct TileCfg {
  static constexpr int WM = (NW == 8 || BM >= 128) ? 2 : 1;  // wavefronts along rows
  static constexpr int WN = NW / WM;                         // wavefronts along weight rows
  static constexpr int RW = BM / WM;            // rows per wavefront
  static constexpr int CW = TBN / WN;           // weight rows per wavefront
  static constexpr int TJ = RW / 32;            // MFMA tiles along rows
  static constexpr int TI = CW / 32;            // MFMA tiles along weight rows
};

struct Tile {
  int e, m0, M, n0;
};

// accumulator tiles of one wavefront
template <int BM, int NW>
using AccT = f32x16[TileCfg<BM, NW>::TI][TileCfg<BM, NW>::TJ];

// Balanced per-XCD ranges over the tiles that exist; false when this
// workgroup has no tile.
template <int BM, bool GATEUP>
__device__ __forceinline__ bool select_tile(const RouteView& rv, int E, int N, Tile& t, int slot) {
  constexpr int kTileCh = GATEUP ? TBN / 2 : TBN;  // output channels per tile
  const int nN = N / kTileCh;
  int mtiles = 0;
  for (int q = 0; q < E; ++q) mtiles += (rv.counts[q] + BM - 1) / BM;
  const int total = mtiles * nN;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  if (slot >= per_xcd) return false;
  const int L = xcd * per_xcd + slot;
  if (L >= total) return false;
  const int group = L / (kGroupM * nN);
  const int first_m = group * kGroupM;
  const int gsz = min(kGroupM, mtiles - first_m);
  const int within = L - group * kGroupM * nN;
  const int mt = first_m + within % gsz;
  const int nt = within / gsz;
  t.e = find_tile<BM>(rv, E, mt, t.m0, t.M);
  t.n0 = nt * kTileCh;
  return t.e >= 0;
}

// Row pointer of tile row r (clamped into the segment): the token's row of x
// for the gate/up pass (gather through perm), the H row for the down pass.
template <bool GATEUP>
__device__ __forceinline__ const bf16_bits* act_row(const bf16_bits* A, const RouteView& rv, const Tile& t,
                                                    int64_t T, int K, int r) {
  if (r >= t.M) r = t.M - 1;
  if (GATEUP) {
    int tok = rv.perm[t.m0 + r];
    tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
    return A + (int64_t)tok * K;
  }
  return A + (int64_t)(t.m0 + r) * K;
}

// Weight row r (0..255) of the tile: gate channels then up channels for the
// gate/up pass, 256 down channels otherwise.
template <bool GATEUP>
__device__ __forceinline__ const char* weight_row(const void* w0, const void* w1, const Tile& t, int N, int K,
                                                  size_t wsz, int r) {
  const char* base = (const char*)((GATEUP && r >= TBN / 2) ? w1 : w0);
  const int ch = t.n0 + (GATEUP ? (r & (TBN / 2 - 1)) : r);
  return base + ((int64_t)t.e * N + ch) * (int64_t)K * wsz;
}

// Scales each accumulator by its channel's 8-bit-weight scale (W8), forms
// GELU(gate) * up (gate/up pass, bf16 H) or stores the fp32 down product.
template <int BM, bool GATEUP, bool W8, int NW = 4>
__device__ __forceinline__ void epilogue(AccT<BM, NW>& acc, const Tile& t,
                                         const float* __restrict__ scales, int N, int E, int Ftot,
                                         void* __restrict__ out) {
  using C = TileCfg<BM, NW>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hg = lane >> 5;
  const int wn = wave % C::WN, wm = wave / C::WN;
  if (GATEUP) {
#pragma unroll
    for (int i = 0; i < C::TI / 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nc = t.n0 + wn * (C::CW / 2) + i * 32 + 8 * q + 4 * hg;
        float s0[4] = {1.f, 1.f, 1.f, 1.f}, s1[4] = {1.f, 1.f, 1.f, 1.f};
        if (W8) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            s0[v] = scales[(int64_t)t.e * N + nc + v];
            s1[v] = scales[(int64_t)E * N + (int64_t)t.e * N + nc + v];
          }
        }
#pragma unroll
        for (int j = 0; j < C::TJ; ++j) {
          const int m = wm * C::RW + j * 32 + r32;
          if (m < t.M) {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
              h[v] = gelu_erf(acc[i][j][4 * q + v] * s0[v]) * (acc[i + C::TI / 2][j][4 * q + v] * s1[v]);
            uint2 o;
            o.x = pack_bf16x2(h[0], h[1]);
            o.y = pack_bf16x2(h[2], h[3]);
            *reinterpret_cast<uint2*>((bf16_bits*)out + (int64_t)(t.m0 + m) * N + nc) = o;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::TI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nc = t.n0 + wn * C::CW + i * 32 + 8 * q + 4 * hg;
        float s0[4] = {1.f, 1.f, 1.f, 1.f};
        if (W8) {
#pragma unroll
          for (int v = 0; v < 4; ++v) s0[v] = scales[2 * (int64_t)E * Ftot + (int64_t)t.e * N + nc + v];
        }
#pragma unroll
        for (int j = 0; j < C::TJ; ++j) {
          const int m = wm * C::RW + j * 32 + r32;
          if (m < t.M) {
            const float4 o = make_float4(acc[i][j][4 * q] * s0[0], acc[i][j][4 * q + 1] * s0[1],
                                         acc[i][j][4 * q + 2] * s0[2], acc[i][j][4 * q + 3] * s0[3]);
            *reinterpret_cast<float4*>((float*)out + (int64_t)(t.m0 + m) * N + nc) = o;
          }
        }
      }
    }
  }
}

// LDS row of the wavefront's weight MFMA tile i (relative to the weight rows)
template <int BM, bool GATEUP, int NW = 4>
__device__ __forceinline__ int wtile_row(int wn, int i) {
  using C = TileCfg<BM, NW>;
  if (GATEUP) return (i < C::TI / 2 ? 0 : TBN / 2) + wn * (C::CW / 2) + (i % (C::TI / 2)) * 32;
  return wn * C::CW + i * 32;
}

template <int BM, int NW = 4>
__device__ __forceinline__ void zero_acc(AccT<BM, NW>& acc) {
#pragma unroll
  for (int i = 0; i < TileCfg<BM, NW>::TI; ++i)
#pragma unroll
    for (int j = 0; j < TileCfg<BM, NW>::TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
}

// =====================================================================
// bf16 weights: LDS filled by global_load_lds_dwordx4.
//
// A stage holds SB reduction values of every tile row: SB = 32 gives 64-byte
// LDS rows (4 chunks of 16 bytes), SB = 64 gives 128-byte rows (8 chunks),
// i.e. whole 128-byte lines of each global row per stage. NS LDS stages;
// the loads of stage k+NS-1 are issued at the start of stage k. One
// wavefront load instruction fills 1 KB of LDS: lane i writes row
// (1024 / row bytes) t + i / chunks, slot i mod chunks, so it fetches the
// chunk that belongs in that slot.
//
// Slots (measured on gfx950, where a conflict-free 1 KB ds_read_b128 takes 4
// clocks): 64-byte rows put chunk c of row R at c ^ ((R >> 2) & 3); 128-byte
// rows at c ^ (R & 7) ^ ((R >> 3) & 1). Both keep the fragment reads (lane
// l: row l mod 32, chunk c + l / 32) free of bank conflicts.
// =====================================================================
template <int BM, int NW, int SB, int NS>
struct DmaCfg {
  static constexpr int RT = BM + TBN;          // LDS rows per stage (activations, then weights)
  static constexpr int ROWB = SB * 2;          // bytes per LDS row
  static constexpr int CH = ROWB / 16;         // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;      // rows per load instruction
  static constexpr int Q = RT / (RPI * NW);    // load instructions per wavefront per stage
  static constexpr int STEPS = SB / 16;        // MFMA steps per stage
  static constexpr int kStageBytes = RT * ROWB;
  static constexpr int kLdsBytes = NS * kStageBytes;
};

template <int SB>
__device__ __forceinline__ int dslot(int R, int c) {
  if (SB == 32) return c ^ ((R >> 2) & 3);
  return c ^ (R & 7) ^ ((R >> 3) & 1);
}

// 16 bytes per lane from global memory straight into LDS: lane i of the
// wavefront writes lds_base + 16 i (lds_base must be wavefront-uniform).
// The builtin only exists in the device compilation pass.
__device__ __forceinline__ void dma16(const void* src, char* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
#endif
}

// s_waitcnt with vmcnt(n) and lgkmcnt(0) (expcnt left at its maximum)
#define GMOE_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (((n) >> 4) << 14))

template <int BM, bool GATEUP, int NW, int SB, int NS>
__global__ __launch_bounds__(NW * 64, 1) void dma_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                     const void* __restrict__ w0, const void* __restrict__ w1,
                                                     int64_t T, int K, int N, int E, int Ftot,
                                                     void* __restrict__ out) {
  using C = TileCfg<BM, NW>;
  using D = DmaCfg<BM, NW, SB, NS>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  // Persistent form: the grid holds as many workgroups as fit on the chip
  // at once, and each walks the tiles of its XCD's range in steps of the
  // XCD's workgroup count, so the workgroups of one XCD move through their
  // tiles together and share operand stages in its L2.
  const int slot_step = GMOE_PERSIST ? (int)(gridDim.x >> 3) : 0;
  for (int slot = blockIdx.x >> 3;; slot += slot_step) {
  Tile t;
  if (!select_tile<BM, GATEUP>(rv, E, N, t, slot)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hg = lane >> 5;
  const int wn = wave % C::WN, wm = wave / C::WN;

  // source of each of this lane's Q load instructions (stage 0)
  const char* src[D::Q];
#pragma unroll
  for (int q = 0; q < D::Q; ++q) {
    const int R = D::RPI * (q * NW + wave) + lane / D::CH;
    const int c = dslot<SB>(R, lane % D::CH);
    const char* row = R < BM ? (const char*)act_row<GATEUP>(A, rv, t, T, K, R)
                             : weight_row<GATEUP>(w0, w1, t, N, K, 2, R - BM);
    src[q] = row + c * 16;
  }
  auto issue = [&](int stage, int buf) {
    char* dst = lds + buf * D::kStageBytes;
#pragma unroll
    for (int q = 0; q < D::Q; ++q) dma16(src[q] + (size_t)stage * D::ROWB, dst + (q * NW + wave) * 1024);
  };

  f32x16 acc[C::TI][C::TJ];
  zero_acc<BM, NW>(acc);
  u32x4 fw[2][C::TI], fx[2][C::TJ];
  const int nk = K / SB;

  // The stage loop, for a wavefront whose first TJV row subtiles (of 32 rows)
  // hold rows of the segment: the others are past its end and get neither
  // fragment reads nor MFMAs (a nearly empty last tile of an expert costs its
  // loads, not a tile of MFMAs). Every instance has the same loads and
  // barriers, so the wavefronts of a workgroup stay in step.
  auto stage_loop = [&](auto tjv_tag) {
    constexpr int TJV = decltype(tjv_tag)::value;
    auto frags = [&](int buf, int s, u32x4* wa, u32x4* xa) {
      if constexpr (TJV > 0) {
        const char* b = lds + buf * D::kStageBytes;
        const int c = 2 * s + hg;
#pragma unroll
        for (int i = 0; i < C::TI; ++i) {
          const int R = BM + wtile_row<BM, GATEUP, NW>(wn, i) + r32;
          wa[i] = *reinterpret_cast<const u32x4*>(b + R * D::ROWB + dslot<SB>(R, c) * 16);
        }
#pragma unroll
        for (int j = 0; j < TJV; ++j) {
          const int R = wm * C::RW + j * 32 + r32;
          xa[j] = *reinterpret_cast<const u32x4*>(b + R * D::ROWB + dslot<SB>(R, c) * 16);
        }
      }
    };
    auto mfma_step = [&](int b) {
#pragma unroll
      for (int i = 0; i < C::TI; ++i)
#pragma unroll
        for (int j = 0; j < TJV; ++j) acc[i][j] = mfma32(fw[b][i], fx[b][j], acc[i][j]);
    };
    constexpr int kMf = C::TI * TJV;               // MFMAs per step
    constexpr int kRd = TJV > 0 ? C::TI + TJV : 0;  // fragment reads per step

    // prologue: stages 0..NS-2 in flight (indices past the end re-read the
    // last stage, in bounds, into buffers nobody reads)
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(min(s, nk - 1), s);
    GMOE_WAIT_VM_LGKM0((NS - 2) * D::Q);  // stage 0 has landed
    lds_barrier();
    frags(0, 0, fw[0], fx[0]);
#if GMOE_PHASED
    // Each step is one phase: the fragment reads of the next step, then the
    // MFMAs of this step (which use the fragments read one phase earlier).
    // Scheduling fences keep the phases apart, so no MFMA waits on a read
    // issued in its own phase.
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt % NS;
#pragma unroll
      for (int s = 0; s + 1 < D::STEPS; ++s) {
        frags(buf, s + 1, fw[(s + 1) & 1], fx[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(s & 1);
        // buffer (kt+NS-1) mod NS was last read in stage kt-1, released by its barrier
        if (s == GMOE_ISSUE_STEP) issue(min(kt + NS - 1, nk - 1), (kt + NS - 1) % NS);
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage kt+1 has landed (at most NS-2 later stages in flight) and every
      // read of this buffer is complete
      GMOE_WAIT_VM_LGKM0((NS - 2) * D::Q);
      lds_barrier();
      frags((kt + 1) % NS, 0, fw[0], fx[0]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step((D::STEPS - 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#else
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt % NS;
      // buffer (kt+NS-1) mod NS was last read in stage kt-1, released by its barrier
      issue(min(kt + NS - 1, nk - 1), (kt + NS - 1) % NS);
#pragma unroll
      for (int s = 0; s + 1 < D::STEPS; ++s) {
        frags(buf, s + 1, fw[(s + 1) & 1], fx[(s + 1) & 1]);
        mfma_step(s & 1);
      }
      // order in the region above: the next step's fragment reads each paired
      // with an MFMA, the stage loads spread over the remaining MFMAs
      constexpr int kM = kMf * (D::STEPS - 1), kR = kRd * (D::STEPS - 1);
      constexpr int kRP = kR < kM ? kR : kM;
      constexpr int kGP = D::Q < kM - kRP ? D::Q : kM - kRP;
#pragma unroll
      for (int q = 0; q < kRP; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < kGP; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if constexpr (kM > kRP + kGP) __builtin_amdgcn_sched_group_barrier(0x008, kM - kRP - kGP, 0);
      if constexpr (kR > kRP) __builtin_amdgcn_sched_group_barrier(0x100, kR - kRP, 0);
      if constexpr (D::Q > kGP) __builtin_amdgcn_sched_group_barrier(0x020, D::Q - kGP, 0);
      // the MFMAs above stay above the wait, so the MFMA pipe is busy while
      // the last fragment reads of the stage complete
      __builtin_amdgcn_sched_barrier(0);
      // stage kt+1 has landed (at most NS-2 later stages in flight) and every
      // read of this buffer is complete
      GMOE_WAIT_VM_LGKM0((NS - 2) * D::Q);
      lds_barrier();
      frags((kt + 1) % NS, 0, fw[0], fx[0]);
      mfma_step((D::STEPS - 1) & 1);
      if constexpr (kRd > 0) __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
      if constexpr (kMf > 0) __builtin_amdgcn_sched_group_barrier(0x008, kMf, 0);
    }
#endif
  };
  const int valid_rows = t.M - wm * C::RW;
  const int tjv = valid_rows <= 0 ? 0 : min(C::TJ, (valid_rows + 31) / 32);
  if (tjv >= C::TJ) {
    stage_loop(std::integral_constant<int, C::TJ>{});
  } else if (tjv == 0) {
    stage_loop(std::integral_constant<int, 0>{});
  } else if (tjv == 1) {
    stage_loop(std::integral_constant<int, 1>{});
  } else if constexpr (C::TJ > 2) {
    if (tjv == 2)
      stage_loop(std::integral_constant<int, 2>{});
    else
      stage_loop(std::integral_constant<int, (C::TJ > 3 ? 3 : 2)>{});
  }
  // drain the (duplicate) loads still in flight before the workgroup exits
  GMOE_WAIT_VM_LGKM0(0);
  epilogue<BM, GATEUP, false, NW>(acc, t, nullptr, N, E, Ftot, out);
  if (!GMOE_PERSIST) return;
  // every wavefront is done with the LDS stages before the next tile's loads
  lds_barrier();
  }
}

// =====================================================================
// 8-bit weights: 64-wide stages through registers (int8 -> bf16 on the way
// into LDS). LDS rows hold 64 bf16 = 8 chunks of 16 bytes; chunk c of row r
// sits at slot c ^ (r mod 8) ^ (bit 3 of r), so the rows read by 8 or by 16
// consecutive lanes hit distinct bank groups.
// =====================================================================
constexpr int SBK = 64;

__device__ __forceinline__ int swz(int r, int c) { return (r * 8 + (c ^ (r & 7) ^ ((r >> 3) & 1))) * 8; }

template <int BM>
struct StagedCfg {
  static constexpr int AL = BM / 32;                // 16-byte activation chunks per thread per stage
  static constexpr int WL = 4;                      // 16-byte int8 weight chunks per thread per stage
  static constexpr int kStage = (BM + TBN) * SBK;   // bf16 elements per LDS stage
  static constexpr int kLdsBytes = 2 * kStage * 2;
};

template <int BM, bool GATEUP>
__global__ __launch_bounds__(256, 1) void staged_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                        const void* __restrict__ w0, const void* __restrict__ w1,
                                                        const float* __restrict__ scales, int64_t T, int K, int N,
                                                        int E, int Ftot, void* __restrict__ out) {
  using C = TileCfg<BM>;
  using S = StagedCfg<BM>;
  extern __shared__ __attribute__((aligned(16))) bf16_bits smem[];
  Tile t;
  if (!select_tile<BM, GATEUP>(rv, E, N, t, blockIdx.x >> 3)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, hg = lane >> 5;
  const int wn = wave % C::WN, wm = wave / C::WN;

  // activation rows: chunk lc of rows lr + 32p; weight rows: 16-byte chunk qc
  // of rows qr + 64p
  const int lc = tid & 7, lr = tid >> 3;
  const int qc = tid & 3, qr = tid >> 2;
  const bf16_bits* arow[S::AL];
#pragma unroll
  for (int p = 0; p < S::AL; ++p) arow[p] = act_row<GATEUP>(A, rv, t, T, K, lr + 32 * p);
  const char* wrow[S::WL];
#pragma unroll
  for (int p = 0; p < S::WL; ++p) wrow[p] = weight_row<GATEUP>(w0, w1, t, N, K, 1, qr + 64 * p);

  u32x4 ra[S::AL], rw[S::WL];
  auto gload = [&](int kb) {
#pragma unroll
    for (int p = 0; p < S::AL; ++p) ra[p] = ld16(arow[p] + kb + lc * 8);
#pragma unroll
    for (int p = 0; p < S::WL; ++p) rw[p] = ld16(wrow[p] + kb + qc * 16);
  };
  auto lstore = [&](int stage) {
    bf16_bits* sa = smem + stage * S::kStage;
    bf16_bits* sw = sa + BM * SBK;
#pragma unroll
    for (int p = 0; p < S::AL; ++p) *reinterpret_cast<u32x4*>(&sa[swz(lr + 32 * p, lc)]) = ra[p];
#pragma unroll
    for (int p = 0; p < S::WL; ++p) {
      u32x4 lo, hi;
      i8x16_to_frags(rw[p], lo, hi);
      const int r = qr + 64 * p;
      *reinterpret_cast<u32x4*>(&sw[swz(r, 2 * qc)]) = lo;
      *reinterpret_cast<u32x4*>(&sw[swz(r, 2 * qc + 1)]) = hi;
    }
  };
  auto read_frags = [&](int stage, int s, u32x4* wa, u32x4* xa) {
    const bf16_bits* sa = smem + stage * S::kStage;
    const bf16_bits* sw = sa + BM * SBK;
    const int c = 2 * s + hg;
#pragma unroll
    for (int i = 0; i < C::TI; ++i)
      wa[i] = *reinterpret_cast<const u32x4*>(&sw[swz(wtile_row<BM, GATEUP>(wn, i) + r32, c)]);
#pragma unroll
    for (int j = 0; j < C::TJ; ++j)
      xa[j] = *reinterpret_cast<const u32x4*>(&sa[swz(wm * C::RW + j * 32 + r32, c)]);
  };

  f32x16 acc[C::TI][C::TJ];
  zero_acc<BM>(acc);
  u32x4 fw[2][C::TI], fx[2][C::TJ];
  const int nk = K / SBK;
  gload(0);
  lstore(0);
  gload(min(1, nk - 1) * SBK);
  __syncthreads();
  read_frags(0, 0, fw[0], fx[0]);
  // one basic block per stage: past the end the prefetch re-reads the last
  // stage (in bounds) and the store goes to the buffer nobody reads
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    lstore(cur ^ 1);
    // keep the new loads behind the stores, so the stores wait for the loads
    // issued a stage ago and not for these
    __builtin_amdgcn_sched_barrier(0);
    gload(min(kt + 2, nk - 1) * SBK);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) read_frags(cur, s + 1, fw[(s + 1) & 1], fx[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < C::TI; ++i)
#pragma unroll
        for (int j = 0; j < C::TJ; ++j) acc[i][j] = mfma32(fw[s & 1][i], fx[s & 1][j], acc[i][j]);
    }
    __syncthreads();
    read_frags(cur ^ 1, 0, fw[0], fx[0]);
  }
  epilogue<BM, GATEUP, true>(acc, t, scales, N, E, Ftot, out);
}

// =====================================================================
// launch
// =====================================================================
// Grid: an upper bound of the tile count, rounded up to a multiple of 8
// (sum over experts of ceil(rows_e / BM) <= rows / BM + E).
static unsigned tiled_blocks(int bm, int64_t rows_cap, int E, int nN) {
  const int64_t mt_ub = rows_cap / bm + E;
  return (unsigned)(((mt_ub * nN) + 7) / 8 * 8);
}

template <int BM, bool GATEUP>
static hipError_t launch_staged(hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0, const void* w1,
                                const float* scales, int64_t T, int64_t rows_cap, int K, int N, int E, int Ftot,
                                void* out) {
  constexpr int lds = StagedCfg<BM>::kLdsBytes;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&staged_kernel<BM, GATEUP>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const dim3 grid(tiled_blocks(BM, rows_cap, E, N / (GATEUP ? TBN / 2 : TBN)));
  hipLaunchKernelGGL((staged_kernel<BM, GATEUP>), grid, dim3(256), lds, st, A, rv, w0, w1, scales, T, K, N, E,
                     Ftot, out);
  return hipGetLastError();
}

// Pipeline shape per tile height: 256-row tiles run 8 wavefronts (two per
// SIMD, so one's MFMAs cover the other's waits).
template <int BM>
struct DmaChoice {
#ifndef GMOE_NW256
#define GMOE_NW256 8
#endif
#ifndef GMOE_DMA_NS256
#define GMOE_DMA_NS256 2
#endif
  static constexpr int NW = BM == 256 ? GMOE_NW256 : 4;
  static constexpr int SB = BM == 256 ? GMOE_DMA_SB : 64;
  static constexpr int NS = BM == 256 ? GMOE_DMA_NS256 : 3;
};

template <int BM, bool GATEUP>
static hipError_t launch_dma(hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0, const void* w1,
                             int64_t T, int64_t rows_cap, int K, int N, int E, int Ftot, void* out) {
  using P = DmaChoice<BM>;
  constexpr int lds = DmaCfg<BM, P::NW, P::SB, P::NS>::kLdsBytes;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&dma_kernel<BM, GATEUP, P::NW, P::SB, P::NS>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  unsigned blocks = tiled_blocks(BM, rows_cap, E, N / (GATEUP ? TBN / 2 : TBN));
  if (GMOE_PERSIST) {
    static const unsigned resident = [] {
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
      return (unsigned)(cus + 7) / 8 * 8;  // one workgroup per CU (LDS-bound)
    }();
    blocks = blocks < resident ? blocks : resident;
  }
  const dim3 grid(blocks);
  hipLaunchKernelGGL((dma_kernel<BM, GATEUP, P::NW, P::SB, P::NS>), grid, dim3(P::NW * 64), lds, st, A, rv, w0, w1,
                     T, K, N, E, Ftot, out);
  return hipGetLastError();
}

template <int BM, bool GATEUP>
static hipError_t tiled_launch(bool w8, hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0,
                               const void* w1, const float* scales, int64_t T, int64_t rows_cap, int K, int N, int E,
                               int Ftot, void* out) {
  return w8 ? launch_staged<BM, GATEUP>(st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, out)
            : launch_dma<BM, GATEUP>(st, A, rv, w0, w1, T, rows_cap, K, N, E, Ftot, out);
}

template <bool GATEUP>
static hipError_t tiled_dispatch(bool w8, int bm, hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0,
                                 const void* w1, const float* scales, int64_t T, int64_t rows_cap, int K, int N,
                                 int E, int Ftot, void* out) {
  switch (bm) {
    case 64: return tiled_launch<64, GATEUP>(w8, st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, out);
    case 128: return tiled_launch<128, GATEUP>(w8, st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, out);
    case 256: return tiled_launch<256, GATEUP>(w8, st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, out);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tiled_gateup(int w8, int bm, const bf16_bits* x, RouteView rv, const void* wg, const void* wu,
                               const float* scales, int64_t T, int64_t rows_cap, int d, int f, int E,
                               bf16_bits* H, hipStream_t st) {
  return tiled_dispatch<true>(w8 != 0, bm, st, x, rv, wg, wu, scales, T, rows_cap, d, f, E, f, H);
}

hipError_t launch_tiled_down(int w8, int bm, const bf16_bits* H, RouteView rv, const void* wd, const float* scales,
                             int64_t rows_cap, int d, int f, int E, float* Y, hipStream_t st) {
  return tiled_dispatch<false>(w8 != 0, bm, st, H, rv, wd, wd, scales, rows_cap, rows_cap, f, d, E, f, Y);
}

}  // namespace gmoe
