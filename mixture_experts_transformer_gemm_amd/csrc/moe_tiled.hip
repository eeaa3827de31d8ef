// LDS-tiled grouped GEMMs of the Grok-1 MoE layer for gfx950 (MI355X), used
// when experts hold more rows than the weight-streaming path handles.
//
// Each expert is one segment of a grouped GEMM over the expert-contiguous row
// permutation (Grok-1 book ch. 11, section 11.3.1: sparse reorder + grouped
// GEMM). Gate/up pass: H = GELU(X Wg^T) * (X Wu^T) -> bf16 (field guide,
// "MoE 子层": two input projections, GELU on one, elementwise product).
// Down pass: Y = H Wd^T -> fp32.
//
// Workgroup tile: BM rows x 256 weight rows (BM = 64 or 128 with 4
// wavefronts, 256 with 8). For the gate/up pass the 256 weight rows
// are 128 gate channels and the same 128 up channels, so act(gate) * up is
// formed in registers. With two wavefront rows, row subtile q (32 rows) goes
// to wavefront row q mod 2, so a partly filled tile keeps both busy.
// Products use v_mfma_f32_32x32x16_bf16 with the weight fragment as the "A"
// operand (32 channels) and the activation fragment as "B" (32 rows): lane l
// supplies row (l mod 32) and the 8 reduction values of group l / 32; result
// register v of lane l is C[8 (v / 4) + 4 (l / 32) + (v mod 4)][l mod 32], so
// each lane owns runs of 4 consecutive channels of one row.
//
// Both operands reach LDS by global_load_lds_dwordx4 (no staging registers):
// stages of 64 reduction values, as many stages as fit in 144 KB (2 for the
// 256-row tile), loads issued NS - 1 stages ahead, one vmcnt wait and one
// barrier per stage. 8-bit weights stay int8 in LDS and are widened to bf16
// after the fragment read (exact); their per-channel scales are applied in
// the epilogue. The down pass can split its reduction over grid y (partial
// sums in Y, added in the combine).
//
// Tile order: the tiles that exist (sum over experts of ceil(rows / BM),
// times the channel tiles) are split into 8 contiguous ranges, one per XCD
// (workgroup i runs on XCD i mod 8); each range walks groups of kGroupM row
// tiles with the row tile fastest, so the workgroups resident on one XCD
// share weight tiles through its L2.
#include "moe_device.h"

#include <type_traits>

namespace gmoe {

constexpr int TBN = 256;

constexpr int kGroupM = 4;  // row tiles per tile group (see select_tile)

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
  const int nN = (N + kTileCh - 1) / kTileCh;       // the last may reach past N
  const int mtiles = rv.tile_off[E];
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
  t.e = rv.tile_e[mt];
  const int mloc = (mt - rv.tile_off[t.e]) * BM;
  t.m0 = rv.offsets[t.e] + mloc;
  t.M = min(BM, rv.counts[t.e] - mloc);
  t.n0 = nt * kTileCh;
  return true;
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

// Scales each accumulator by its channel's 8-bit-weight scale (W8), forms
// GELU(gate) * up (gate/up pass, bf16 H) or stores the fp32 down product.
template <int BM, bool GATEUP, bool W8, int NW = 4>
__device__ __forceinline__ void epilogue(AccT<BM, NW>& acc, const Tile& t,
                                         const float* __restrict__ scales, int N, int E, int Ftot, int act,
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
          const int m = (j * C::WM + wm) * 32 + r32;
          if (m < t.M) {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
              h[v] = glu_act(act, acc[i][j][4 * q + v] * s0[v]) * (acc[i + C::TI / 2][j][4 * q + v] * s1[v]);
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
        if (nc >= N) continue;  // past the last output channel (N is a multiple of 64)
        float s0[4] = {1.f, 1.f, 1.f, 1.f};
        if (W8) {
#pragma unroll
          for (int v = 0; v < 4; ++v) s0[v] = scales[2 * (int64_t)E * Ftot + (int64_t)t.e * N + nc + v];
        }
#pragma unroll
        for (int j = 0; j < C::TJ; ++j) {
          const int m = (j * C::WM + wm) * 32 + r32;
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
// LDS filled by global_load_lds_dwordx4 (both weight types).
//
// A stage holds SB = 64 reduction values of every tile row: activation rows
// of 128 bytes (bf16), weight rows of 128 bytes (bf16) or 64 bytes (8-bit,
// kept as int8 in LDS and widened to bf16 after the fragment read, which is
// exact). NS LDS stages; the loads of stage k+NS-1 are issued during stage
// k. One wavefront load instruction fills 1 KB of LDS: lane i writes row
// (1024 / row bytes) t + i / chunks, slot i mod chunks, so it fetches the
// chunk that belongs in that slot.
//
// Slots (measured on gfx950, where a conflict-free 1 KB ds_read_b128 takes 4
// clocks): 64-byte rows put chunk c of row R at c ^ ((R >> 2) & 3); 128-byte
// rows at c ^ (R & 7) ^ ((R >> 3) & 1). Both keep the fragment reads (lane
// l: row l mod 32, chunk c + l / 32) free of bank conflicts.
//
// 8-bit weights: one 16-byte read gives a lane the 16 reduction values of
// two MFMA steps. Lane half h (= l / 32) of the 32-value block d reads
// values [32d + 16h, 32d + 16h + 16); the low 8 feed step 2d and the high 8
// step 2d + 1, and the activation fragment of step 2d + e for lane half h is
// read from the same reduction indices, [32d + 16h + 8e, +8). Each MFMA thus
// pairs equal indices; only the order of the sum over the block differs.
// =====================================================================
template <int BM, int NW, int NS, bool W8>
struct DmaCfg {
  static constexpr int SB = 64;                       // reduction values per stage
  static constexpr int AROWB = SB * 2;                // activation bytes per LDS row
  static constexpr int WROWB = W8 ? SB : SB * 2;      // weight bytes per LDS row
  static constexpr int ACH = AROWB / 16, WCH = WROWB / 16;
  static constexpr int ARPI = 1024 / AROWB, WRPI = 1024 / WROWB;  // rows per load instruction
  static constexpr int QA = BM / (ARPI * NW);         // activation loads per wavefront per stage
  static constexpr int QW = TBN / (WRPI * NW);        // weight loads per wavefront per stage
  static constexpr int Q = QA + QW;
  static constexpr int STEPS = SB / 16;               // MFMA steps per stage
  static constexpr int kActBytes = BM * AROWB;
  static constexpr int kStageBytes = kActBytes + TBN * WROWB;
  static constexpr int kLdsBytes = NS * kStageBytes;
  static_assert(QA * ARPI * NW == BM && QW * WRPI * NW == TBN, "load shape");
};

template <int ROWB>
__device__ __forceinline__ int dslot(int R, int c) {
  if (ROWB == 64) return c ^ ((R >> 2) & 3);
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


template <int BM, bool GATEUP, int NW, int NS, bool W8>
__global__ __launch_bounds__(NW * 64, 1) void dma_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                     const void* __restrict__ w0, const void* __restrict__ w1,
                                                     const float* __restrict__ scales, int64_t T, int K, int N,
                                                     int E, int Ftot, int64_t rows_cap, int act,
                                                     void* __restrict__ out) {
  using C = TileCfg<BM, NW>;
  using D = DmaCfg<BM, NW, NS, W8>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  Tile t;
  if (!select_tile<BM, GATEUP>(rv, E, N, t, blockIdx.x >> 3)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hg = lane >> 5;
  const int wn = wave % C::WN, wm = wave / C::WN;
  // split-K (down pass only): this workgroup reduces [kbeg, kbeg + K / S)
  // into partial sum sp
  const int S = gridDim.y, sp = blockIdx.y;
  const int kbeg = sp * (K / S);
  if (!GATEUP) out = (float*)out + (int64_t)sp * rows_cap * N;

  // source of each of this lane's load instructions (stage 0): QA activation
  // instructions, then QW weight instructions. Activation instruction q holds
  // tile rows [q ARPI NW, (q + 1) ARPI NW); those wholly past the segment's
  // end are not issued (qav of them are). Sources inside one tile are a
  // workgroup-uniform base plus a 32-bit per-lane offset (weight rows and the
  // down pass's contiguous H rows); gathered token rows keep full pointers.
  const int qav = min(D::QA, (t.M + D::ARPI * NW - 1) / (D::ARPI * NW));
  constexpr int wsz = W8 ? 1 : 2;
  const char* abase = (const char*)(A + (int64_t)t.m0 * K + kbeg);  // down pass
  const char* agather[GATEUP ? D::QA : 1];
  uint32_t aoff[GATEUP ? 1 : D::QA];
#pragma unroll
  for (int q = 0; q < D::QA; ++q) {
    const int R = D::ARPI * (q * NW + wave) + lane / D::ACH;
    const int c = dslot<D::AROWB>(R, lane % D::ACH);
    if constexpr (GATEUP)
      agather[q] = (const char*)(act_row<GATEUP>(A, rv, t, T, K, R) + kbeg) + c * 16;
    else
      aoff[q] = (uint32_t)(min(R, t.M - 1) * (K * 2) + c * 16);
  }
  // weight rows: gate channels [n0, n0 + 128) then up channels for the
  // gate/up pass (instruction q reads up rows when q ARPI NW >= 128, the same
  // for every lane), 256 down channels otherwise
  const int64_t wrow0 = ((int64_t)t.e * N + t.n0) * K + kbeg;
  const char* wbase0 = (const char*)w0 + wrow0 * wsz;
  const char* wbase1 = (const char*)w1 + wrow0 * wsz;
  uint32_t woff[D::QW];
#pragma unroll
  for (int q = 0; q < D::QW; ++q) {
    const int R = D::WRPI * (q * NW + wave) + lane / D::WCH;
    const int c = dslot<D::WROWB>(R, lane % D::WCH);
    // down pass: rows past the last output channel read the last one (their
    // sums are not stored)
    const int wr = GATEUP ? (R & (TBN / 2 - 1)) : min(R & (TBN - 1), N - 1 - t.n0);
    woff[q] = (uint32_t)(wr * (K * wsz) + c * 16);
  }
  auto issue_act = [&](int stage, int buf) {
    char* dst = lds + buf * D::kStageBytes;
#pragma unroll
    for (int q = 0; q < D::QA; ++q) {
      if (q < qav) {
        if constexpr (GATEUP)
          dma16(agather[q] + (size_t)stage * D::AROWB, dst + (q * NW + wave) * 1024);
        else
          dma16(abase + (size_t)stage * D::AROWB + aoff[q], dst + (q * NW + wave) * 1024);
      }
    }
  };
  auto issue_w = [&](int stage, int buf) {
    char* dst = lds + buf * D::kStageBytes;
#pragma unroll
    for (int q = 0; q < D::QW; ++q) {
      const bool up = GATEUP && q * D::WRPI * NW >= TBN / 2;
      dma16((up ? wbase1 : wbase0) + (size_t)stage * D::WROWB + woff[q], dst + D::kActBytes + (q * NW + wave) * 1024);
    }
  };
  // stage k has landed when at most NS-2 later stages of this wavefront's
  // loads (qav + QW instructions each) are in flight; lgkmcnt(0) as well
  auto wait_stage = [&]() {
    switch (qav) {
      case 1: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 1)); break;
      case 2: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 2)); break;
      case 3: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 3)); break;
      case 4: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 4)); break;
      case 5: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 5)); break;
      case 6: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 6)); break;
      case 7: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 7)); break;
      default: GMOE_WAIT_VM_LGKM0((NS - 2) * (D::QW + 8)); break;
    }
  };
  static_assert(D::QA <= 8 && (NS - 2) * (D::QW + D::QA) <= 63, "wait_stage covers up to 8 activation loads");

  f32x16 acc[C::TI][C::TJ];
  zero_acc<BM, NW>(acc);
  u32x4 fw[2][C::TI], fx[2][C::TJ];
  u32x4 fhi[C::TI];  // 8-bit weights: the widened fragment of the next (odd) step
  const int nk = K / S / D::SB;

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
        if (!W8) {
          const int c = 2 * s + hg;
#pragma unroll
          for (int i = 0; i < C::TI; ++i) {
            const int R = wtile_row<BM, GATEUP, NW>(wn, i) + r32;
            wa[i] = *reinterpret_cast<const u32x4*>(b + D::kActBytes + R * D::WROWB + dslot<D::WROWB>(R, c) * 16);
          }
        } else if ((s & 1) == 0) {
          const int c = s + hg;  // block d = s / 2, chunk 2d + h
#pragma unroll
          for (int i = 0; i < C::TI; ++i) {
            const int R = wtile_row<BM, GATEUP, NW>(wn, i) + r32;
            const u32x4 q =
                *reinterpret_cast<const u32x4*>(b + D::kActBytes + R * D::WROWB + dslot<D::WROWB>(R, c) * 16);
            i8x16_to_frags(q, wa[i], fhi[i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < C::TI; ++i) wa[i] = fhi[i];
        }
        const int cx = W8 ? (2 * (s & ~1) + 2 * hg + (s & 1)) : (2 * s + hg);
#pragma unroll
        for (int j = 0; j < TJV; ++j) {
          const int R = (j * C::WM + wm) * 32 + r32;
          xa[j] = *reinterpret_cast<const u32x4*>(b + R * D::AROWB + dslot<D::AROWB>(R, cx) * 16);
        }
      }
    };
    auto mfma_step = [&](int b) {
#pragma unroll
      for (int i = 0; i < C::TI; ++i)
#pragma unroll
        for (int j = 0; j < TJV; ++j) acc[i][j] = mfma32(fw[b][i], fx[b][j], acc[i][j]);
    };

    // prologue: stages 0..NS-2 in flight (indices past the end re-read the
    // last stage, in bounds, into buffers nobody reads)
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      issue_act(min(s, nk - 1), s);
      issue_w(min(s, nk - 1), s);
    }
    wait_stage();  // stage 0 has landed
    lds_barrier();
    // Activation loads of a stage are issued right after the barrier that
    // frees their buffer (outside the MFMA phases: whether each is issued
    // depends on the segment), the weight loads inside the first phase.
    issue_act(min(NS - 1, nk - 1), (NS - 1) % NS);
    frags(0, 0, fw[0], fx[0]);
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
        if (s == 0) issue_w(min(kt + NS - 1, nk - 1), (kt + NS - 1) % NS);
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage kt+1 has landed (at most NS-2 later stages in flight) and every
      // read of this buffer is complete
      wait_stage();
      lds_barrier();
      issue_act(min(kt + NS, nk - 1), (kt + NS) % NS);
      frags((kt + 1) % NS, 0, fw[0], fx[0]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step((D::STEPS - 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // row subtiles j * WM + wm (j < TJ) belong to wavefront row wm, so a
  // partly filled tile spreads its rows over both wavefront rows
  const int nsub = (t.M + 31) / 32;
  const int tjv = nsub <= wm ? 0 : min(C::TJ, (nsub - wm + C::WM - 1) / C::WM);
  if (tjv >= C::TJ) {
    stage_loop(std::integral_constant<int, C::TJ>{});
  } else if (tjv == 0) {
    stage_loop(std::integral_constant<int, 0>{});
  } else if (tjv == 1) {
    stage_loop(std::integral_constant<int, 1>{});
  } else if constexpr (C::TJ > 2) {
    if (tjv == 2) {
      stage_loop(std::integral_constant<int, 2>{});
    } else if constexpr (C::TJ > 3) {
      if (tjv == 3)
        stage_loop(std::integral_constant<int, 3>{});
      else if constexpr (C::TJ > 4)
        stage_loop(std::integral_constant<int, 4>{});  // tjv == 4 < TJ == 5
    }
  }
  // drain the (duplicate) loads still in flight before the workgroup exits
  GMOE_WAIT_VM_LGKM0(0);
  epilogue<BM, GATEUP, W8, NW>(acc, t, scales, N, E, Ftot, act, out);
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

// Pipeline shape per tile height: 256-row tiles run 8 wavefronts
// (two per SIMD, so one's MFMAs cover the other's waits); as many LDS stages
// as fit in 144 KB, at most 6, except for 8-bit weights, whose smaller
// stages measured faster less deep: 2 stages for 256-row tiles (3.5% faster
// than 3 at 8,192 tokens), 3 for 128-row tiles (4% faster than 4).
template <int BM, bool W8>
struct DmaChoice {
  static constexpr int NW = BM >= 256 ? 8 : 4;
  static constexpr int kStage = DmaCfg<BM, NW, 2, W8>::kStageBytes;
  static constexpr int kFit = 147456 / kStage < 6 ? 147456 / kStage : 6;
  static constexpr int NS = !W8 ? kFit : (BM >= 256 ? 2 : (BM == 128 && kFit > 3 ? 3 : kFit));
};

template <int BM, bool GATEUP, bool W8>
static hipError_t launch_dma(hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0, const void* w1,
                             const float* scales, int64_t T, int64_t rows_cap, int K, int N, int E, int Ftot,
                             int splits, int act, void* out) {
  using P = DmaChoice<BM, W8>;
  constexpr int lds = DmaCfg<BM, P::NW, P::NS, W8>::kLdsBytes;
  static std::atomic<unsigned long long> lds_set{0};
  const hipError_t attr =
      set_lds_limit(reinterpret_cast<const void*>(&dma_kernel<BM, GATEUP, P::NW, P::NS, W8>), lds, lds_set);
  if (attr != hipSuccess) return attr;
  constexpr int kTileCh = GATEUP ? TBN / 2 : TBN;
  const dim3 grid(tiled_blocks(BM, rows_cap, E, (N + kTileCh - 1) / kTileCh), (unsigned)splits);
  hipLaunchKernelGGL((dma_kernel<BM, GATEUP, P::NW, P::NS, W8>), grid, dim3(P::NW * 64), lds, st, A, rv, w0, w1,
                     scales, T, K, N, E, Ftot, rows_cap, act, out);
  return hipGetLastError();
}

template <int BM, bool GATEUP>
static hipError_t tiled_launch(bool w8, hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0,
                               const void* w1, const float* scales, int64_t T, int64_t rows_cap, int K, int N, int E,
                               int Ftot, int splits, int act, void* out) {
  return w8 ? launch_dma<BM, GATEUP, true>(st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, splits, act, out)
            : launch_dma<BM, GATEUP, false>(st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, splits, act, out);
}

template <bool GATEUP>
static hipError_t tiled_dispatch(bool w8, int bm, hipStream_t st, const bf16_bits* A, RouteView rv, const void* w0,
                                 const void* w1, const float* scales, int64_t T, int64_t rows_cap, int K, int N,
                                 int E, int Ftot, int splits, int act, void* out) {
  switch (bm) {
    case 64: return tiled_launch<64, GATEUP>(w8, st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, splits, act, out);
    case 128:
      return tiled_launch<128, GATEUP>(w8, st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, splits, act, out);
    case 256:
      return tiled_launch<256, GATEUP>(w8, st, A, rv, w0, w1, scales, T, rows_cap, K, N, E, Ftot, splits, act, out);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tiled_gateup(int w8, int bm, const bf16_bits* x, RouteView rv, const void* wg, const void* wu,
                               const float* scales, int64_t T, int64_t rows_cap, int d, int f, int E, int act,
                               bf16_bits* H, hipStream_t st) {
  return tiled_dispatch<true>(w8 != 0, bm, st, x, rv, wg, wu, scales, T, rows_cap, d, f, E, f, 1, act, H);
}

hipError_t launch_tiled_down(int w8, int bm, int splits, const bf16_bits* H, RouteView rv, const void* wd,
                             const float* scales, int64_t rows_cap, int d, int f, int E, float* Y, hipStream_t st) {
  return tiled_dispatch<false>(w8 != 0, bm, st, H, rv, wd, wd, scales, rows_cap, rows_cap, f, d, E, f, splits, 0, Y);
}

}  // namespace gmoe
