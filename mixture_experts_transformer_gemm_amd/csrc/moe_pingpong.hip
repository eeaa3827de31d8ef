// Ping-pong grouped GEMM of the Grok-1 MoE layer for gfx950 (MI355X): the
// large-batch (prefill) gate/up and down projections with bf16 weights.
//
// Each expert is one segment of a grouped GEMM over the expert-contiguous row
// permutation (Grok-1 book ch. 11, section 11.3.1: sparse reorder + grouped
// GEMM). Gate/up pass: H = act(X Wg^T) * (X Wu^T) -> bf16 (field guide, "MoE
// 子层": two input projections, GELU on one, elementwise product). Down pass:
// Y = H Wd^T -> fp32 partial sums.
//
// Workgroup tile: 256 rows x 256 weight rows, 8 wavefronts, two per SIMD
// (256 x 256 fp32 accumulators fill half of each SIMD's register file). The
// reduction runs in slices of 64 values; both operands of a slice reach LDS
// by global_load_lds_dwordx4, each load instruction fetching 8 whole 128-byte
// lines (8 rows x 64 values: fetching half lines, a slice of 32 values,
// measured slower, since the other half of every line is evicted from the
// vector L1 before the next slice asks for it). LDS holds three activation
// slices and two weight slices (160 KB): the activation rows, gathered token
// rows that mostly miss L2, are loaded two slices ahead, the weights one.
//
// The two wavefronts of a SIMD take turns (a ping-pong): wavefronts 0-3
// (group 0) and 4-7 (group 1) run the same loop one phase apart, and between
// two workgroup barriers one group only issues MFMAs on fragments it already
// holds in registers while the other group reads the next fragments from LDS
// and issues global loads. Each SIMD's matrix core is thus fed by one
// wavefront while its partner waits on memory (measured with the operands
// held in registers, this barrier pattern keeps the matrix cores 99% busy).
// A slice is read in four memory phases (half 0 and half 1 of its
// reduction values, by group 0 and then group 1), and every memory phase
// issues 4 load instructions per wavefront (the loads measured 3-7% faster
// spread evenly than issued 8 or 16 at a time by one group): both groups
// load activation rows, and each group loads the weight rows it reads
// itself, right after its last read of the previous occupant of their
// buffer. The barrier that ends a slice's last phase follows every
// wavefront's wait (vmcnt) for its own loads of the next slice.
//
// Wavefront (s, g), s = SIMD (wavefront mod 4; wavefronts w and w + 4 share a
// SIMD on gfx950), g = group: rows 32 s .. 32 s + 31 and 128 + 32 s .. 128 +
// 32 s + 31 of the tile (so a partly filled tile spreads its rows over all
// four SIMDs); weight rows: the gate/up pass pairs gate channels 64 g .. 64 g
// + 63 with the same up channels (LDS rows 0-127 gate, 128-255 up), the down
// pass takes output channels 128 g .. 128 g + 127. Products use
// v_mfma_f32_32x32x16_bf16 with the weight fragment as "A" and the activation
// fragment as "B": lane l supplies row (l mod 32) and 8 reduction values of
// half l / 32; result register v of lane l is C[8 (v / 4) + 4 (l / 32) +
// (v mod 4)][l mod 32] (channel, row).
//
// Tile order: the tiles that exist are numbered expert by expert; within an
// expert, groups of 8 row tiles are walked channel tile by channel tile with
// the row tiles fastest; the numbering is split into 8 contiguous ranges, one
// per XCD (workgroup i runs on XCD i mod 8), so the 32 workgroups resident on
// an XCD share 8 row tiles of activations and 4 weight tiles through its L2.
//
// What bounds it (Grok-1 prefill, measured): with no global loads in the loop
// the gate/up pass runs at 64% of the bf16 peak and the down pass at 75%; the
// loads alone (almost no MFMAs) take about as long as the MFMAs alone, and the
// two overlap only in part. The waits for loads are a few percent of the
// loop: the limit is the rate at which the memory system delivers the 64 KB
// of a slice (L2 hit rate 0.78 in the gate/up pass, 0.75 in the down pass),
// and with random bf16 operands the chip holds about 1.6 GHz under this load
// (MFMA busy 0.69 / 0.74 of the CU-busy cycles).
#include "moe_device.h"

#include <type_traits>

namespace gmoe {

namespace {

constexpr int kPM = 256;          // rows per tile
constexpr int kPN = 256;          // weight rows per tile
constexpr int kPK = 64;           // reduction values per slice
constexpr int kPRow = kPK * 2;    // LDS bytes per row and slice: one 128-byte line
constexpr int kPSliceA = kPM * kPRow;  // activation half of a slice: 32 KB
constexpr int kPSliceW = kPN * kPRow;  // weight half: 32 KB
// Row tiles per tile group: 32 workgroups resident on one XCD then hold 8
// row tiles x 4 channel tiles of one expert (measured at the Grok-1 prefill,
// gate/up launch: 11.08-11.18 ms with groups of 8, 11.38 with 4, 11.54 with
// 6, 11.88 with 3, 12.04 with 2, 11.30-11.37 with 10, 12 or 16; Mixtral
// prefill and the skewed layer also best or level at 8)
constexpr int kPGroup = 8;
// LDS: three activation buffers, then two weight buffers (160 KB)
constexpr int kPWOff = 3 * kPSliceA;
constexpr int kPLds = kPWOff + 2 * kPSliceW;

struct PTile {
  int e, m0, M, n0;
};

// slot of 16-byte chunk c of LDS row R (8 chunks): conflict-free for fragment
// reads of 32 rows at two chunks and for the 1 KB load writes (8 rows)
__device__ __forceinline__ int pslot(int R, int c) { return c ^ (R & 7) ^ ((R >> 3) & 1); }

// This workgroup's tile, or false when it has none. Output channels per tile:
// 128 (gate/up: 128 gate + the same 128 up weight rows) or 256 (down).
template <bool GATEUP>
__device__ __forceinline__ bool pp_select(const RouteView& rv, int E, int N, PTile& t) {
  constexpr int kCh = GATEUP ? kPN / 2 : kPN;
  const int nN = (N + kCh - 1) / kCh;  // the last channel tile may reach past N
  const int mtiles = rv.tile_off[E];
  const int total = mtiles * nN;
  const int per_xcd = (total + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return false;
  const int L = (blockIdx.x & 7) * per_xcd + slot;
  if (L >= total) return false;
  // expert e's tiles are [tile_off[e] nN, tile_off[e+1] nN), so L / nN is one
  // of e's row tiles
  const int e = rv.tile_e[L / nN];
  const int mt0 = rv.tile_off[e];
  const int mte = rv.tile_off[e + 1] - mt0;
  // within the expert: groups of kPGroup row tiles, each walked channel tile
  // by channel tile with its row tiles fastest (the last group may be smaller)
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
  const int r32 = lane & 31, hg = lane >> 5;
  const int S = gridDim.y, sp = blockIdx.y;
  const int kspan = K / S, kbeg = sp * kspan;
  const int nsl = kspan / kPK;  // slices

  // Load instructions: each fills one 1 KB LDS block of 8 rows (lane l writes
  // row 8 I + l / 8 of block I at slot l mod 8, so it reads the chunk stored
  // there; the 8 lanes of a row fetch one whole 128-byte line). Each
  // wavefront issues 4 activation blocks (8 s + 4 g + q: the two groups split
  // the 32 blocks of a slice) and the 4 blocks of weight rows it reads itself
  // among the 16 of its group (gate/up: gate rows 64 g .. 64 g + 63, blocks
  // 8 g .., and the same up rows, blocks 16 + 8 g ..; down: rows 128 g ..
  // 128 g + 127, blocks 16 g ..).
  int wblk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    wblk[q] = GATEUP ? (q < 2 ? 8 * g : 16 + 8 * g) + 2 * s + (q & 1) : 16 * g + 4 * s + q;
  const char* asrc[4];
  const char* wsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    {
      const int R = 8 * (8 * s + 4 * g + q) + (lane >> 3);
      const int c = pslot(R, lane & 7);
      const int r = R < t.M ? R : t.M - 1;  // rows past the segment's end repeat its last row
      const bf16_bits* row;
      if (GATEUP) {
        int tok = rv.perm[t.m0 + r];
        tok = tok < 0 ? 0 : (tok >= T ? (int)(T - 1) : tok);
        row = A + (int64_t)tok * K;
      } else {
        row = A + (int64_t)(t.m0 + r) * K;
      }
      asrc[q] = (const char*)(row + kbeg) + c * 16;
    }
    {
      const int R = 8 * wblk[q] + (lane >> 3);
      const int c = pslot(R, lane & 7);
      const bf16_bits* row;
      if (GATEUP)
        row = (R < kPN / 2 ? w0 : w1) + ((int64_t)t.e * N + t.n0 + (R & (kPN / 2 - 1))) * K;
      else  // rows past the last output channel read the last one (not stored)
        row = w0 + ((int64_t)t.e * N + min(t.n0 + R, N - 1)) * K;
      wsrc[q] = (const char*)(row + kbeg) + c * 16;
    }
  }
  // activation slice sl lives in buffer sl mod 3, weight slice sl in buffer sl mod 2
  auto issue_a = [&](int sl) {
    char* dst = lds + (sl % 3) * kPSliceA + (8 * s + 4 * g) * 1024;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_policy<0>(asrc[q] + (size_t)sl * kPRow, dst + q * 1024);
  };
  auto issue_w = [&](int sl) {
    char* dst = lds + kPWOff + (sl & 1) * kPSliceW;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_policy<0>(wsrc[q] + (size_t)sl * kPRow, dst + wblk[q] * 1024);
  };

  // fragments of half h (32 reduction values) of one slice: 4 weight tiles
  // x 2 steps, 2 row tiles x 2 steps
  u32x4 fw[2][4], fx[2][2];
  auto read_frags = [&](int sl, int h) {
    const char* ba = lds + (sl % 3) * kPSliceA;
    const char* bw = lds + kPWOff + (sl & 1) * kPSliceW;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int c = 4 * h + 2 * st + hg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int R = (GATEUP ? (i < 2 ? 0 : kPN / 2) + 64 * g + 32 * (i & 1) : 128 * g + 32 * i) + r32;
        fw[st][i] = *reinterpret_cast<const u32x4*>(bw + R * kPRow + pslot(R, c) * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int R = 32 * (s + 4 * j) + r32;
        fx[st][j] = *reinterpret_cast<const u32x4*>(ba + R * kPRow + pslot(R, c) * 16);
      }
    }
  };
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // row tiles of this wavefront that hold rows of the segment (0, 1 or 2):
  // the others get no MFMAs (loads and barriers are the same for all)
  const int jv = (32 * s < t.M ? 1 : 0) + (128 + 32 * s < t.M ? 1 : 0);
  auto mfmas = [&](auto jv_tag) {
    constexpr int JV = decltype(jv_tag)::value;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JV; ++j) acc[i][j] = mfma32(fw[st][i], fx[st][j], acc[i][j]);
  };
  // a workgroup barrier that no instruction crosses in either direction
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Phases: slice sl is read in four memory phases, half 0 then half 1 of
  // its reduction values by group 0 (phases 4 sl, 4 sl + 2) and by group 1
  // one phase later. Every memory phase issues 4 loads per wavefront: the
  // activation blocks of slice sl + 2 in each group's first phase of slice sl
  // (its activation buffer, slice sl - 1's, is free from phase 4 sl on), and
  // each group's own weight rows of slice sl + 2 at the end of its last read
  // of slice sl (they take slice sl's weight buffer, whose other rows the
  // other group still reads). Before the barrier that ends phase 4 sl + 3,
  // every wavefront waits for its loads of slice sl + 1: a wavefront's loads
  // land in issue order, so group 0 allows the 8 it issued for slice sl + 2
  // to be in flight, group 1 the 4.
  auto run = [&](auto jv_tag) {
    issue_a(0);
    issue_w(0);
    if (nsl > 1) {
      issue_a(1);
      issue_w(1);
      GMOE_WAIT_VM(8);
    } else {
      GMOE_WAIT_VM(0);
    }
    phase_end();
    if (g == 0) {
      for (int sl = 0; sl < nsl; ++sl) {
        const bool more = sl + 2 < nsl;
        read_frags(sl, 0);
        if (more) issue_a(sl + 2);
        phase_end();
        mfmas(jv_tag);
        phase_end();
        read_frags(sl, 1);
        if (more) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's reads of its weight rows are done
          issue_w(sl + 2);
        }
        phase_end();
        mfmas(jv_tag);
        __builtin_amdgcn_sched_barrier(0);
        if (more)
          GMOE_WAIT_VM(8);
        else
          GMOE_WAIT_VM(0);
        phase_end();
      }
      phase_end();  // group 1's last compute phase
    } else {
      phase_end();  // group 0's first memory phase
      for (int sl = 0; sl < nsl; ++sl) {
        const bool more = sl + 2 < nsl;
        read_frags(sl, 0);
        if (more) issue_a(sl + 2);
        phase_end();
        mfmas(jv_tag);
        phase_end();
        read_frags(sl, 1);
        if (more)
          GMOE_WAIT_VM_LGKM0(4);
        else
          GMOE_WAIT_VM_LGKM0(0);
        if (more) issue_w(sl + 2);
        phase_end();
        mfmas(jv_tag);
        phase_end();
      }
    }
  };
  if (jv == 2)
    run(std::integral_constant<int, 2>{});
  else if (jv == 1)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});

  // epilogue: this lane's rows 32 (s + 4 j) + r32 of the tile
  if (GATEUP) {
    // The 256 x 128 H tile goes through LDS (256-byte rows; 16-byte chunk c
    // of row R at slot c ^ (R mod 16)), so that every row leaves as whole
    // 128-byte lines, 16 bytes per lane, instead of 8-byte pieces from four
    // wavefronts.
    bf16_bits* H = (bf16_bits*)out;
    __syncthreads();  // every wavefront is past its last fragment read
    // the activation is uniform over the launch: one branch around the whole tile
    auto stage_h = [&](auto silu_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = 32 * (s + 4 * j) + r32;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float z = acc[i][j][4 * q + v];
              h[v] = (decltype(silu_tag)::value ? silu(z) : gelu_erf(z)) * acc[i + 2][j][4 * q + v];
            }
            uint2 o;
            o.x = pack_bf16x2(h[0], h[1]);
            o.y = pack_bf16x2(h[2], h[3]);
            const int c = 8 * g + 4 * i + q;  // 16-byte chunk of the 128 channels
            *reinterpret_cast<uint2*>(lds + m * 256 + ((c ^ (m & 15)) * 16) + 8 * hg) = o;
          }
      }
    };
    if (act == ACT_SILU)
      stage_h(std::true_type{});
    else
      stage_h(std::false_type{});
    __syncthreads();
    // wavefront w stores rows 32 w .. 32 w + 31, four rows per instruction
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int R = 32 * wave + 4 * it + (lane >> 4);
      const int c = lane & 15;
      if (R < t.M) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + R * 256 + ((c ^ (R & 15)) * 16));
        *reinterpret_cast<u32x4*>(H + (int64_t)(t.m0 + R) * N + t.n0 + 8 * c) = v;
      }
    }
  } else {
    // The 256 x 256 fp32 tile goes through LDS in two passes of 128 rows
    // (1 KB rows; 16-byte chunk c of row R at slot c ^ (R mod 16)): pass p
    // holds every wavefront's row tile j = p, and each row then leaves as one
    // 1 KB store (16 bytes per lane) instead of 32-byte pieces of 32 rows
    // per instruction (those took a fifth of the down pass).
    float* Y = (float*)out + (int64_t)sp * rows_cap * N;
    const int nleft = N - t.n0;  // output channels of the tile inside N (a multiple of 64)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __syncthreads();  // the LDS is free (loop done, or the previous pass stored)
      const int m = 32 * s + r32;  // row within this pass
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 32 * g + 8 * i + 2 * q + hg;  // 16-byte chunk: channels 4 c .. 4 c + 3
          *reinterpret_cast<float4*>(lds + m * 1024 + ((c ^ (m & 15)) * 16)) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      __syncthreads();
      // wavefront w stores rows 16 w .. 16 w + 15 of the pass, one row per instruction
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int R = 16 * wave + it;
        const int row = 128 * j + R;
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
  // grid: an upper bound of the tiles (sum over experts of ceil(rows_e / 256)
  // <= rows / 256 + E), times the channel tiles, rounded up to a multiple of 8
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

hipError_t launch_pp_down(int splits, const bf16_bits* H, RouteView rv, const bf16_bits* wd, int64_t rows_cap, int d,
                          int f, int E, float* Y, hipStream_t st) {
  return pp_launch<false>(st, H, rv, wd, wd, rows_cap, rows_cap, f, d, E, splits, 0, Y);
}

}  // namespace gmoe
