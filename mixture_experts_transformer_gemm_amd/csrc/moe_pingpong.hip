// Ping-pong grouped GEMM of the MoE layer for gfx950 (MI355X): the gate/up
// and down projections with bf16 weights once experts hold about 200 rows or
// more (the Grok-1 and Mixtral prefill, the skewed layer, and the
// fine-grained layer's prefill, where 8192 tokens give about 256 rows per
// expert; book ch. 10, section 10.1 table). Each expert is one segment of a
// grouped GEMM over the expert-contiguous permutation (book ch. 11, section
// 11.3.1: sparse reorder, then grouped GEMM): the gate/up pass forms H =
// act(X Wg^T) * (X Wu^T) in bf16, the down pass Y = H Wd^T as fp32 partial
// sums.
//
// Workgroup tile: 320 rows x 256 weight rows, 8 wavefronts, two per SIMD
// (wavefronts w and w + 4 share a SIMD on gfx950). 320-row tiles leave an
// expert of 257-320 rows one tile instead of a full and a nearly empty
// 256-row tile, each of which would stream the whole weight tile.
// Products use v_mfma_f32_16x16x32_bf16 (20 row tiles of 16 split evenly over
// the 4 SIMDs; 320 rows are 10 tiles of 32, which 4 SIMDs cannot share
// evenly): lane l supplies row (l mod 16) and reduction values 8 (l / 16) ..
// 8 (l / 16) + 7 of the 32 an MFMA takes; result register v of lane l is
// C[4 (l / 16) + v][l mod 16] (weight row, activation row). Wavefront (s, g),
// s = SIMD, g = group, holds 8 weight tiles of 16 rows x 5 row tiles of 16
// (rows 16 (s + 4 j) .. + 15, j = 0..4) in 160 fp32 accumulator registers.
//
// The reduction runs in slices of 64 values; every load instruction
// (global_load_lds_dwordx4) fills one 1 KB LDS block of 8 rows x 128 bytes,
// so the 8 lanes of a row fetch one whole 128-byte line.
// LDS holds two activation slices (40 KB each) and two weight slices (32 KB
// each), 144 KB. The two wavefront groups take turns between workgroup
// barriers: one group issues MFMAs on fragments already in registers while
// the other reads the next fragments from LDS and issues loads, so each
// SIMD's matrix core is fed by one wavefront while its partner waits on
// memory. A slice is read in four phases (half 0 by group 0, half 0 by group
// 1, half 1 by group 0, half 1 by group 1). Activations of slice sl + 1 are
// loaded in the first two phases of slice sl, into the buffer of slice sl - 1
// (both groups read every activation row, so that buffer is free only once
// slice sl - 1 is done); each group loads its own weight rows of slice sl + 2
// right after its last read of slice sl (the groups read disjoint weight
// rows). Before the barrier that ends a slice, every wavefront waits for its
// loads of the next slice. Weights get about six phases to arrive;
// activations, shared by all channel tiles of an expert and mostly served by
// L2, about three.
#include "moe_device.h"

#include <type_traits>

namespace gmoe {

namespace {

constexpr int kPM = 320;                    // rows per tile
constexpr int kPN = 256;                    // weight rows per tile
constexpr int kPK = 64;                     // reduction values per slice
constexpr int kPRow = kPK * 2;              // LDS bytes per row and slice: one 128-byte line
constexpr int kPSliceA = kPM * kPRow;       // activation half of a slice: 40 KB
constexpr int kPSliceW = kPN * kPRow;       // weight half: 32 KB
constexpr int kPWOff = 2 * kPSliceA;        // two activation buffers, then two weight buffers
constexpr int kPLds = kPWOff + 2 * kPSliceW;  // 144 KB
constexpr int kPGroup = 4;                  // row tiles per tile group
constexpr int kPABlk = kPM / 8 / 8;         // activation blocks per wavefront and slice: 5

struct PTile {
  int e, m0, M, n0;
};

// This workgroup's tile, or false when it has none. The tiles that exist are
// numbered expert by expert; within an expert, groups of kPGroup row tiles
// are walked channel tile by channel tile with the row tiles fastest; the
// numbering is split into 8 contiguous ranges, one per XCD (workgroup i runs
// on XCD i mod 8). Output channels per tile: 128 (gate/up: 128 gate + the
// same 128 up weight rows) or 256 (down).
//
// An XCD runs 32 tiles at once (one per CU), so a group of 4 row tiles moves
// through its channel tiles 8 at a time, each round 4 activation slices and
// 8 weight slices shared through the XCD's L2. A group that holds all 7 row
// tiles of a Grok-1 prefill expert runs 7 x 4.6 tiles per round instead:
// rounds straddle channel tiles, whose weights are then fetched again a
// tile's time later (FETCH_SIZE of the gate/up launch 63 GB against 32 GB
// with groups of 4, and 2-3% slower).
template <bool GATEUP>
__device__ __forceinline__ bool pp_select(const RouteView& rv, int E, int N, PTile& t) {
  constexpr int kCh = GATEUP ? kPN / 2 : kPN;
  const int nN = (N + kCh - 1) / kCh;
  const int mtiles = rv.tile_off[E];
  const int total = mtiles * nN;
  const int per_xcd = (total + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return false;
  const int L = (blockIdx.x & 7) * per_xcd + slot;
  if (L >= total) return false;
  const int e = rv.tile_e[L / nN];
  const int mt0 = rv.tile_off[e];
  const int mte = rv.tile_off[e + 1] - mt0;
  const int within = L - mt0 * nN;
  const int gfull = mte / kPGroup;
  int nt, mrow;
  if (within < gfull * kPGroup * nN) {
    const int gi = within / (kPGroup * nN), rem = within - gi * kPGroup * nN;
    nt = rem / kPGroup;
    mrow = gi * kPGroup + (rem - nt * kPGroup);
  } else {
    const int gl = mte - gfull * kPGroup, rem = within - gfull * kPGroup * nN;
    nt = rem / gl;
    mrow = gfull * kPGroup + (rem - nt * gl);
  }
  const int mloc = mrow * kPM;
  t.e = e;
  t.m0 = rv.offsets[e] + mloc;
  t.M = min(kPM, rv.counts[e] - mloc);
  t.n0 = nt * kCh;
  return true;
}

}  // namespace

// A: x (gate/up, rows gathered through perm) or H (down, contiguous rows);
// w0, w1: gate and up weights (gate/up) or the down weights (both); K: the
// reduction length (d or f), N: output channels of the weight matrices (f or
// d); out: H (bf16) or Y (fp32, gridDim.y partial sums over equal slices of
// the reduction).
template <bool GATEUP>
__global__ __launch_bounds__(512, 1) void pp_kernel(const bf16_bits* __restrict__ A, RouteView rv,
                                                     const bf16_bits* __restrict__ w0,
                                                     const bf16_bits* __restrict__ w1, int64_t T, int K, int N,
                                                     int E, int64_t rows_cap, int act, void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  PTile t;
  if (!pp_select<GATEUP>(rv, E, N, t)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = wave & 3, g = wave >> 2;
  const int r16 = lane & 15, kg = lane >> 4;
  const int S = gridDim.y, sp = blockIdx.y;
  const int kspan = K / S, kbeg = sp * kspan;
  const int nsl = kspan / kPK;  // slices

  // Load instructions: lane l of a load writes row 8 I + l / 8 of block I at
  // slot l mod 8, so it reads the chunk stored there (the 8 lanes of a row
  // fetch one whole 128-byte line). Wavefront w loads activation blocks 5 w ..
  // 5 w + 4 and 4 of the 16 blocks of weight rows its group reads (gate/up:
  // gate rows 64 g .. 64 g + 63, blocks 8 g .., and the same up rows, blocks
  // 16 + 8 g ..; down: rows 128 g .. 128 g + 127, blocks 16 g ..).
  int wblk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    wblk[q] = GATEUP ? (q < 2 ? 8 * g : 16 + 8 * g) + 2 * s + (q & 1) : 16 * g + 4 * s + q;
  // Sources: gathered token rows (gate/up) keep full pointers; the down
  // pass's contiguous H rows and the weight rows are a workgroup-uniform base
  // plus a 32-bit per-lane offset (at most 320 or 128 rows of the tile).
  const char* agather[GATEUP ? kPABlk : 1];
  uint32_t aoff[GATEUP ? 1 : kPABlk];
  const char* abase = (const char*)(A + (int64_t)t.m0 * K + kbeg);  // down pass
#pragma unroll
  for (int q = 0; q < kPABlk; ++q) {
    const int R = 8 * (kPABlk * wave + q) + (lane >> 3);
    const int c = rslot(R, lane & 7);
    const int r = R < t.M ? R : t.M - 1;  // rows past the segment's end repeat its last row
    if constexpr (GATEUP) {
      int tok = rv.perm[t.m0 + r];
      tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
      agather[q] = (const char*)(A + (int64_t)tok * K + kbeg) + c * 16;
    } else {
      aoff[q] = (uint32_t)(r * (K * 2) + c * 16);
    }
  }
  const int64_t wrow0 = ((int64_t)t.e * N + t.n0) * K + kbeg;
  const char* wbase0 = (const char*)(w0 + wrow0);
  const char* wbase1 = (const char*)(w1 + wrow0);
  uint32_t woff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int R = 8 * wblk[q] + (lane >> 3);
    const int c = rslot(R, lane & 7);
    // down pass: rows past the last output channel read the last one (not stored)
    const int wr = GATEUP ? (R & (kPN / 2 - 1)) : min(R, N - 1 - t.n0);
    woff[q] = (uint32_t)(wr * (K * 2) + c * 16);
  }
  // activation slice sl lives in buffer sl mod 2, weight slice sl in buffer sl mod 2
  auto issue_a = [&](int sl) {
    char* dst = lds + (sl & 1) * kPSliceA + kPABlk * wave * 1024;
#pragma unroll
    for (int q = 0; q < kPABlk; ++q) {
      if constexpr (GATEUP)
        dma16_policy<0>(agather[q] + (size_t)sl * kPRow, dst + q * 1024);
      else
        dma16_policy<0>(abase + (size_t)sl * kPRow + aoff[q], dst + q * 1024);
    }
  };
  auto issue_w = [&](int sl) {
    char* dst = lds + kPWOff + (sl & 1) * kPSliceW;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // gate/up: blocks 16 .. 31 hold up rows (q >= 2 for every lane)
      const char* base = (GATEUP && q >= 2) ? wbase1 : wbase0;
      dma16_policy<0>(base + (size_t)sl * kPRow + woff[q], dst + wblk[q] * 1024);
    }
  };

  // fragments of half h (32 reduction values, chunks 4 h .. 4 h + 3) of one
  // slice: 8 weight tiles, JV row tiles
  u32x4 fw[8], fx[5];
  auto read_frags = [&](int sl, int h, auto jv_tag) {
    constexpr int JV = decltype(jv_tag)::value;
    const char* ba = lds + (sl & 1) * kPSliceA;
    const char* bw = lds + kPWOff + (sl & 1) * kPSliceW;
    const int c = 4 * h + kg;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int R = (GATEUP ? (i < 4 ? 0 : kPN / 2) + 64 * g + 16 * (i & 3) : 128 * g + 16 * i) + r16;
      fw[i] = *reinterpret_cast<const u32x4*>(bw + R * kPRow + rslot(R, c) * 16);
    }
#pragma unroll
    for (int j = 0; j < JV; ++j) {
      const int R = 16 * (s + 4 * j) + r16;
      fx[j] = *reinterpret_cast<const u32x4*>(ba + R * kPRow + rslot(R, c) * 16);
    }
  };
  f32x4 acc[8][5];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 5; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // row tiles per wavefront that hold rows of the segment, as many as SIMD 0
  // has (a phase lasts as long as its busiest SIMD, so the others lose
  // nothing by running as many): 5, or 4 for every tile of at most 256 rows
  // (a third instance of the loop, for shorter tiles, makes the compiler
  // spill registers; the extra row tiles hold clamped rows that are never
  // stored). Row tiles past those get no fragment reads and no MFMAs.
  const int jv = ((t.M + 15) / 16 + 3) / 4;
  auto mfmas = [&](auto jv_tag) {
    constexpr int JV = decltype(jv_tag)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < JV; ++j) acc[i][j] = mfma16(fw[i], fx[j], acc[i][j]);
  };
  // a workgroup barrier that no instruction crosses in either direction
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Phases of slice sl (group 0 one phase ahead of group 1): 4 sl + 1: group
  // 0 reads half 0 and loads its activation blocks of slice sl + 1; 4 sl + 2:
  // group 1 does the same; 4 sl + 3: group 0 reads half 1, waits for its
  // reads (lgkmcnt) and loads its weight rows of slice sl + 2; 4 sl + 4:
  // group 1 likewise, and before the barrier that ends it every wavefront
  // waits (vmcnt) for its loads of slice sl + 1, allowing the 4 weight loads
  // of slice sl + 2 to be in flight (a wavefront's loads land in issue order).
  auto run = [&](auto jv_tag) {
    issue_a(0);
    issue_w(0);
    if (nsl > 1) {
      issue_w(1);
      GMOE_WAIT_VM(4);
    } else {
      GMOE_WAIT_VM(0);
    }
    phase_end();
    if (g == 0) {
      for (int sl = 0; sl < nsl; ++sl) {
        const bool more_a = sl + 1 < nsl, more_w = sl + 2 < nsl;
        read_frags(sl, 0, jv_tag);
        if (more_a) issue_a(sl + 1);
        phase_end();
        mfmas(jv_tag);
        phase_end();
        read_frags(sl, 1, jv_tag);
        if (more_w) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's reads of its weight rows are done
          issue_w(sl + 2);
        }
        phase_end();
        mfmas(jv_tag);
        __builtin_amdgcn_sched_barrier(0);
        if (more_w)
          GMOE_WAIT_VM(4);
        else
          GMOE_WAIT_VM(0);
        phase_end();
      }
      phase_end();  // group 1's last compute phase
    } else {
      phase_end();  // group 0's first memory phase
      for (int sl = 0; sl < nsl; ++sl) {
        const bool more_a = sl + 1 < nsl, more_w = sl + 2 < nsl;
        read_frags(sl, 0, jv_tag);
        if (more_a) issue_a(sl + 1);
        phase_end();
        mfmas(jv_tag);
        phase_end();
        read_frags(sl, 1, jv_tag);
        if (more_w) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
          issue_w(sl + 2);
          GMOE_WAIT_VM_LGKM0(4);
        } else {
          GMOE_WAIT_VM_LGKM0(0);
        }
        phase_end();
        mfmas(jv_tag);
        phase_end();
      }
    }
  };
  if (jv == 5)
    run(std::integral_constant<int, 5>{});
  else
    run(std::integral_constant<int, 4>{});

  // epilogue: this lane's rows 16 (s + 4 j) + r16 of the tile, channels
  // 4 kg .. 4 kg + 3 of each 16-row weight tile
  if (GATEUP) {
    // The 320 x 128 H tile goes through LDS (256-byte rows; 16-byte chunk c
    // of row R at slot c ^ (R mod 16)), so that every row leaves as whole
    // 128-byte lines.
    bf16_bits* H = (bf16_bits*)out;
    __syncthreads();  // every wavefront is past its last fragment read
    auto stage_h = [&](auto silu_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const int m = 16 * (s + 4 * j) + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float z = acc[i][j][v];
            h[v] = (decltype(silu_tag)::value ? silu(z) : gelu_erf(z)) * acc[i + 4][j][v];
          }
          uint2 o;
          o.x = pack_bf16x2(h[0], h[1]);
          o.y = pack_bf16x2(h[2], h[3]);
          const int c = 8 * g + 2 * i + (kg >> 1);  // 16-byte chunk (8 channels) of the 128
          *reinterpret_cast<uint2*>(lds + m * 256 + ((c ^ (m & 15)) * 16) + 8 * (kg & 1)) = o;
        }
      }
    };
    if (act == ACT_SILU)
      stage_h(std::true_type{});
    else
      stage_h(std::false_type{});
    __syncthreads();
    // wavefront w stores rows 40 w .. 40 w + 39, four rows per instruction
#pragma unroll
    for (int it = 0; it < 10; ++it) {
      const int R = 40 * wave + 4 * it + (lane >> 4);
      const int c = lane & 15;
      if (R < t.M) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + R * 256 + ((c ^ (R & 15)) * 16));
        *reinterpret_cast<u32x4*>(H + (int64_t)(t.m0 + R) * N + t.n0 + 8 * c) = v;
      }
    }
  } else {
    // The 320 x 256 fp32 tile goes through LDS in five passes of 64 rows (1 KB
    // rows; 16-byte chunk c of row R at slot c ^ (R mod 16)): pass j holds
    // every wavefront's row tile j, and each row then leaves as one 1 KB
    // store (16 bytes per lane).
    float* Y = (float*)out + (int64_t)sp * rows_cap * N;
    const int nleft = N - t.n0;  // output channels of the tile inside N (a multiple of 64)
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      __syncthreads();  // the LDS is free (loop done, or the previous pass stored)
      const int m = 16 * s + r16;  // row within this pass
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = 32 * g + 4 * i + kg;  // 16-byte chunk: channels 4 c .. 4 c + 3
        *reinterpret_cast<f32x4*>(lds + m * 1024 + ((c ^ (m & 15)) * 16)) = acc[i][j];
      }
      __syncthreads();
      // wavefront w stores rows 8 w .. 8 w + 7 of the pass, one row per instruction
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int R = 8 * wave + it;
        const int row = 64 * j + R;
        if (row < t.M && 4 * lane < nleft) {
          const float4 v = *reinterpret_cast<const float4*>(lds + R * 1024 + ((lane ^ (R & 15)) * 16));
          *reinterpret_cast<float4*>(Y + (int64_t)(t.m0 + row) * N + t.n0 + 4 * lane) = v;
        }
      }
    }
  }
}

namespace {

template <bool GATEUP>
hipError_t pp_launch(hipStream_t st, const bf16_bits* A, RouteView rv, const bf16_bits* w0, const bf16_bits* w1,
                      int64_t T, int64_t rows_cap, int K, int N, int E, int splits, int act, void* out) {
  constexpr int lds = kPLds;
  static std::atomic<unsigned long long> lds_set{0};
  const hipError_t attr = set_lds_limit(reinterpret_cast<const void*>(&pp_kernel<GATEUP>), lds, lds_set);
  if (attr != hipSuccess) return attr;
  // grid: an upper bound of the tiles (sum over experts of ceil(rows_e / 320)
  // <= rows / 320 + E), times the channel tiles, rounded up to a multiple of 8
  constexpr int kCh = GATEUP ? kPN / 2 : kPN;
  const int nN = (N + kCh - 1) / kCh;
  const int64_t tiles = (rows_cap / kPM + E) * nN;
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8), (unsigned)splits);
  hipLaunchKernelGGL((pp_kernel<GATEUP>), grid, dim3(512), lds, st, A, rv, w0, w1, T, K, N, E, rows_cap, act,
                     out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pp_gateup(const bf16_bits* x, RouteView rv, const bf16_bits* wg, const bf16_bits* wu, int64_t T,
                             int64_t rows_cap, int d, int f, int E, int act, bf16_bits* H, hipStream_t st) {
  return pp_launch<true>(st, x, rv, wg, wu, T, rows_cap, d, f, E, 1, act, H);
}

hipError_t launch_pp_down(int splits, const bf16_bits* H, RouteView rv, const bf16_bits* wd, int64_t rows_cap,
                           int d, int f, int E, float* Y, hipStream_t st) {
  return pp_launch<false>(st, H, rv, wd, wd, rows_cap, rows_cap, f, d, E, splits, 0, Y);
}

}  // namespace gmoe
