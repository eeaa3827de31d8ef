// C ABI of the MoE layer: argument validation, workspace layout, kernel
// sequence. No kernel code lives here. See grok_moe.h for the contract.
#include "grok_moe.h"
#include "moe_internal.h"

#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

using namespace gmoe;

// Workspace of grok_moe_forward_static: one copy per device, held until the
// process ends. Host code never uses this name as an address (on the host it
// is only a stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) unsigned char scratch[GROK_MOE_STATIC_WORKSPACE_BYTES];

namespace {

enum Path { PATH_F32 = 0, PATH_TILED = 2, PATH_STREAM = 3 };

constexpr int64_t kMaxT = int64_t(1) << 20;
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int kStream8MaxT = 256;
constexpr int kStreamMaxT = 64;
constexpr int kMaxE = 256;       // routed experts
constexpr int kMaxShared = 4;    // shared experts
constexpr int kFusedRouterE = 64;  // the one-kernel router's limit

struct Plan {
  int path = 0;
  int mt_max = 1;  // small-M path: rows per expert tile / 16
  int splits = 1;  // split-K factor of the down projection
  int gsplits = 1; // split-K factor of the streaming gate/up projection
  int bm = 256;    // tiled path: rows per workgroup tile
  int rsplits = 0; // split-K factor of the many-expert router GEMM (0: fused router)
  int pp = 0;      // tiled path: the ping-pong kernel (bf16 weights, 320-row tiles)
  int64_t rows_cap = 0;
  size_t off_idx = 0, off_gate = 0, off_counts = 0, off_offsets = 0, off_perm = 0, off_pos = 0, off_pblk = 0;
  size_t off_tiles = 0;
  int64_t mt_ub = 0;  // tiled path: tiles of bm rows, at most rows_cap / bm + Et
  size_t off_logits = 0, off_U = 0, off_H = 0, off_Y = 0, off_G = 0, total = 0;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int check_shape(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t ns, int32_t act, int32_t wdt) {
  if (T < 0 || d <= 0 || f <= 0 || E < 1 || k < 1 || k > E || ns < 0) return GROK_MOE_EINVAL;
  const bool combo_ok = (act == GROK_MOE_BF16 && (wdt == GROK_MOE_BF16 || wdt == GROK_MOE_I8)) ||
                        (act == GROK_MOE_F32 && wdt == GROK_MOE_F32);
  if (!combo_ok) return GROK_MOE_EINVAL;
  if (E > kMaxE || k > 8 || ns > kMaxShared || T > kMaxT || d > kMaxDim || f > kMaxDim) return GROK_MOE_EUNSUPPORTED;
  if (act == GROK_MOE_F32 && E > kFusedRouterE) return GROK_MOE_EUNSUPPORTED;
  if (act == GROK_MOE_F32) {
    if (d % 8 || f % 4) return GROK_MOE_EUNSUPPORTED;
  } else {
    if (d % 64 || f % 128) return GROK_MOE_EUNSUPPORTED;
  }
  return GROK_MOE_OK;
}

// E routed experts, k routed slots, ns shared experts: the kernels see
// Et = E + ns experts and K = k + ns slots per token.
Plan make_plan(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t ns, int32_t act, int32_t wdt) {
  Plan p;
  const int Et = E + ns, K = k + ns;
  p.rows_cap = T * K;
  if (act == GROK_MOE_F32) {
    p.path = PATH_F32;
  } else if ((wdt == GROK_MOE_BF16 && T <= kStreamMaxT) || (wdt == GROK_MOE_I8 && T <= kStream8MaxT && d % 128 == 0)) {
    // (8-bit weights stream in stages of 128 reduction values, so d % 128;
    // other widths take the tiled path, whose stages are 64 values)
    p.path = PATH_STREAM;
    p.mt_max = (int)T;  // rows of one expert <= T
    // enough workgroups for the down projection, about 3 per CU (measured
    // at decode: 768 workgroups stream the down weights 3-5% faster than
    // 1536 or 384 with bf16 weights, and 19% faster than 384 with 8-bit
    // ones); a workgroup covers 128 output channels (bf16) or 256 (8-bit
    // weights, two weight tiles per wavefront), and each split keeps whole
    // stages (64 bf16 or 128 8-bit reduction values)
    const int64_t ks = wdt == GROK_MOE_I8 ? 128 : 64;
    const int64_t ch_per_wg = wdt == GROK_MOE_I8 ? 256 : 128;
    int s = 1;
    while (s < 8 && (int64_t)Et * ((d + ch_per_wg - 1) / ch_per_wg) * s < 512 && (f / (2 * s)) % ks == 0) s *= 2;
    p.splits = s;
    // Fine-grained layers (64 or more routed experts, bf16 weights): each
    // expert has few gate/up workgroups (f / 64) and the count that runs
    // depends on how many experts the batch hits, E (1 - (1 - k/E)^T) on
    // average, so with only a few rounds of 256 CUs the last, partly empty
    // one costs a large share. Below 8 rounds two splits of the reduction
    // (fp32 partial sums, then a kernel forming act(gate) * up) even it out;
    // beyond, the doubled per-workgroup cost wins. Measured at the
    // DeepSeek-V3 decode shape (7168 x 2048, 256 + 1 experts, top-8): 1
    // token -6%, 8 tokens -0.9%; 16, 32, 64 tokens +0.6, +2.5, +3.3%.
    if (wdt == GROK_MOE_BF16 && E >= 64 && (d / 2) % 64 == 0) {
      const double hit = E * (1.0 - pow(1.0 - (double)k / E, (double)T)) + ns;
      if (hit * (double)(f / 64) < 2048.0) p.gsplits = 2;
    }
  } else {
    p.path = PATH_TILED;
    // about K*T/Et rows per expert. Taller tiles reuse each weight tile over
    // more rows and run the 8-wavefront kernel; measured on the Grok-1 and
    // 256-expert shapes, 256-row tiles win from about 100 rows per expert
    // on even when half of an expert's last tile is empty
    const int64_t r = p.rows_cap / Et;
    p.bm = r <= 32 ? 64 : (r <= 96 ? 128 : 256);
    // from about 200 rows per expert on, bf16 weights run the ping-pong
    // kernel with 320-row tiles (measured against the tiled kernel with 256-
    // or 320-row tiles and against a ping-pong kernel with 256-row tiles: the
    // Grok-1 layer at 800 tokens 2.71 against 2.85 ms, at 1,200 tokens 3.09
    // against 3.52, at 8,192 tokens 15.7 against 16.7, at 32,768 tokens 58.1
    // against 66.6; the DeepSeek-V3-shaped prefill, about 287 rows per
    // expert, 7.7 against 8.9 ms; level at 700 tokens, 0.17 ms slower at 600)
    if (wdt == GROK_MOE_BF16 && r > 192) {
      p.bm = 320;
      p.pp = 1;
    }
    // 8-bit weights: 128-row tiles up to about 384 rows per expert (their
    // LDS stages are smaller, so the 4-wavefront tile keeps more in flight)
    if (wdt == GROK_MOE_I8 && r <= 384) p.bm = 128;
    // split the down projection's reduction while its tiles alone would
    // leave CUs idle: (row tiles upper bound) x (d / 256) tiles per split
    const int64_t dtiles = (d + 255) / 256;  // down channel tiles (the last may be partial)
    const int64_t tiles = (p.rows_cap / p.bm + Et) * dtiles;
    int s = 1;
    while (s < 8 && tiles * s < 1024 && (f / (2 * s)) % 64 == 0) s *= 2;
    // The down tiles run one workgroup per CU (256 CUs). When the tiles
    // expected at balanced routing leave the last round at most half full,
    // two splits even it out for the cost of one more partial sum in Y
    // (measured at 8,192 tokens, 1,344 tiles = 5.25 rounds: down 6.8 ->
    // 6.5 ms; at 16,384 tokens, 9.75 rounds, splitting is 3% slower)
    const int64_t exp_tiles =
        ((int64_t)E * ((T * k / E + p.bm - 1) / p.bm) + (int64_t)ns * ((T + p.bm - 1) / p.bm)) * dtiles;
    const int64_t last = exp_tiles % 256;
    // (the ping-pong kernel at 8,192 tokens, 1,344 tiles: 15.7 ms with two
    // splits against 16.1 ms with one)
    if (s == 1 && last > 0 && last <= 128 && (f / 2) % 64 == 0) s = 2;
    p.splits = s;
  }
  if (E > kFusedRouterE) {
    // many-expert router: its (64 tokens x 256 experts) tiles split the
    // reduction into whole 64-wide chunks until about 512 workgroups (two
    // per CU) run, keeping at least 2 chunks per split so that the top-k
    // kernel sums few partials
    const int64_t rtiles = ((T + 63) / 64) * ((E + 255) / 256);
    const int nchunk = (int)(d / 64);
    int s = 1;
    for (int c = 2; c <= nchunk / 2; ++c)
      if (nchunk % c == 0 && rtiles * c <= 512) s = c;
    p.rsplits = s;
  }
  const size_t hsz = act == GROK_MOE_F32 ? 4 : 2;
  size_t o = 0;
  p.off_idx = o;     o = align256(o + sizeof(int32_t) * (size_t)(T * K));
  p.off_gate = o;    o = align256(o + sizeof(float) * (size_t)(T * K));
  p.off_counts = o;  o = align256(o + sizeof(int32_t) * (size_t)Et);
  p.off_offsets = o; o = align256(o + sizeof(int32_t) * (size_t)(Et + 1));
  p.off_perm = o;    o = align256(o + sizeof(int32_t) * (size_t)(T * K));
  p.off_pos = o;     o = align256(o + sizeof(int32_t) * (size_t)(T * K));
  p.off_pblk = o;    o = align256(o + sizeof(int32_t) * (size_t)permute_scratch_ints(T, Et));
  if (p.path == PATH_TILED) p.mt_ub = p.rows_cap / p.bm + Et;
  p.off_tiles = o;   o = align256(o + sizeof(int32_t) * (size_t)(Et + 1 + p.mt_ub));  // tile_off, tile_e
  p.off_logits = o;  o = align256(o + sizeof(double) * (size_t)p.rsplits * (size_t)T * (size_t)E);
  p.off_U = o;       o = align256(o + (act == GROK_MOE_F32 ? 4 : 2) * (size_t)T * (size_t)d);  // sandwich pre-norm
  p.off_H = o;       o = align256(o + hsz * (size_t)p.rows_cap * (size_t)f);
  p.off_Y = o;       o = align256(o + sizeof(float) * (size_t)p.splits * (size_t)p.rows_cap * (size_t)d);
  p.off_G = o;
  if (p.gsplits > 1) o = align256(o + sizeof(float) * (size_t)p.gsplits * (size_t)p.rows_cap * 2 * (size_t)f);
  p.total = o;
  return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int validate(const grok_moe_args* a) {
  if (!a) return GROK_MOE_EINVAL;
  int rc = check_shape(a->T, a->d, a->f, a->E, a->k, a->n_shared, a->act_dtype, a->w_dtype);
  if (rc != GROK_MOE_OK || a->T == 0) return rc;
  if (!a->x || !a->out || !a->w_gate || !a->w_up || !a->w_down) return GROK_MOE_EINVAL;
  if (a->route_idx) {
    if (!a->route_gate) return GROK_MOE_EINVAL;
  } else if (!a->router_w) {
    return GROK_MOE_EINVAL;
  }
  if (a->w_dtype == GROK_MOE_I8 && !a->scales) return GROK_MOE_EINVAL;
  if (a->activation != GROK_MOE_ACT_GELU && a->activation != GROK_MOE_ACT_SILU) return GROK_MOE_EINVAL;
  if (!(a->capacity_factor >= 0.0) || !isfinite(a->capacity_factor)) return GROK_MOE_EINVAL;
  if ((a->norm_pre == nullptr) != (a->norm_post == nullptr)) return GROK_MOE_EINVAL;
  if (a->norm_pre && (!(a->norm_eps >= 0.0) || !isfinite(a->norm_eps))) return GROK_MOE_EINVAL;
  const void* ptrs[] = {a->x, a->router_w, a->w_gate, a->w_up, a->w_down, a->scales, a->out,
                        a->route_idx, a->route_gate, a->norm_pre, a->norm_post, a->router_bias};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GROK_MOE_EALIGN;
  return GROK_MOE_OK;
}

#define GMOE_TRY(expr)                        \
  do {                                        \
    if ((expr) != hipSuccess) return GROK_MOE_EHIP; \
  } while (0)

int record(const grok_moe_debug* dbg, int i, hipStream_t st) {
  if (dbg && dbg->events[i]) return hipEventRecord((hipEvent_t)dbg->events[i], st) == hipSuccess;
  return 1;
}

// Rows each expert keeps under capacity factor c: floor(c * k * T / E), or -1
// (no cap) for c == 0; at most k*T.
int64_t capacity_rows(double c, int64_t T, int E, int k) {
  if (!(c > 0.0)) return -1;
  const double v = floor(c * (double)(k * T) / (double)E);
  return v >= (double)(k * T) ? k * T : (int64_t)v;
}

int copy_out(void* dst, const void* src, size_t bytes, hipStream_t st) {
  if (!dst || bytes == 0) return 1;
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) == hipSuccess;
}

}  // namespace

extern "C" {

size_t grok_moe_workspace_bytes(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t act_dtype,
                                int32_t w_dtype) {
  if (check_shape(T, d, f, E, k, 0, act_dtype, w_dtype) != GROK_MOE_OK) return 0;
  return make_plan(T, d, f, E, k, 0, act_dtype, w_dtype).total;
}

size_t grok_moe_workspace_bytes_ex(const grok_moe_args* a) {
  if (!a || check_shape(a->T, a->d, a->f, a->E, a->k, a->n_shared, a->act_dtype, a->w_dtype) != GROK_MOE_OK) return 0;
  return make_plan(a->T, a->d, a->f, a->E, a->k, a->n_shared, a->act_dtype, a->w_dtype).total;
}

int32_t grok_moe_tile_rows(const grok_moe_args* a) {
  if (!a || check_shape(a->T, a->d, a->f, a->E, a->k, a->n_shared, a->act_dtype, a->w_dtype) != GROK_MOE_OK) return 0;
  const Plan p = make_plan(a->T, a->d, a->f, a->E, a->k, a->n_shared, a->act_dtype, a->w_dtype);
  if (p.path == PATH_TILED) return p.bm;
  if (p.path == PATH_STREAM) {
    // the streaming kernels' chunk: 16, 32, 64 rows, or 128 with 8-bit weights
    const int64_t r = p.mt_max;
    return r <= 16 ? 16 : (r <= 32 ? 32 : ((r <= 64 || a->w_dtype != GROK_MOE_I8) ? 64 : 128));
  }
  return 0;
}

int grok_moe_forward_ex(const grok_moe_args* a, void* ws, size_t ws_bytes, const grok_moe_debug* dbg,
                        void* stream) {
  int rc = validate(a);
  if (rc != GROK_MOE_OK) return rc;
  if (a->T == 0) return GROK_MOE_OK;
  const Plan p = make_plan(a->T, a->d, a->f, a->E, a->k, a->n_shared, a->act_dtype, a->w_dtype);
  if (!ws || ws_bytes < p.total) return GROK_MOE_EWORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return GROK_MOE_EALIGN;

  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  int32_t* idx = (int32_t*)(w + p.off_idx);
  float* gate = (float*)(w + p.off_gate);
  int32_t* counts = (int32_t*)(w + p.off_counts);
  int32_t* offsets = (int32_t*)(w + p.off_offsets);
  int32_t* perm = (int32_t*)(w + p.off_perm);
  int32_t* pos = (int32_t*)(w + p.off_pos);
  int32_t* pblk = (int32_t*)(w + p.off_pblk);
  double* logits = (double*)(w + p.off_logits);
  void* U = w + p.off_U;
  void* H = w + p.off_H;
  float* Y = (float*)(w + p.off_Y);
  const int64_t T = a->T;
  // E routed experts and k routed slots; with the ns shared experts the
  // kernels after the router see Et experts and K slots per token
  const int d = (int)a->d, f = (int)a->f, Er = a->E, kr = a->k, ns = a->n_shared;
  const int E = Er + ns, k = kr + ns;
  const int act_f32 = a->act_dtype == GROK_MOE_F32;
  const int w8 = a->w_dtype == GROK_MOE_I8;
  const int sandwich = a->norm_pre != nullptr;
  const int act = a->activation;

  // stage 0: the sandwich pre-norm (the MoE input A is then u), router
  if (!record(dbg, 0, st)) return GROK_MOE_EHIP;
  const void* A = a->x;
  if (sandwich) {
    GMOE_TRY(launch_rmsnorm(act_f32, a->x, a->norm_pre, T, d, a->norm_eps, U, st));
    A = U;
  }
  const int32_t* ridx = idx;
  const float* rgate = gate;
  if (a->route_idx) {
    if (ns == 0) {
      ridx = a->route_idx;
      rgate = a->route_gate;
    } else {
      GMOE_TRY(launch_append_shared(a->route_idx, a->route_gate, T, Er, kr, ns, idx, gate, st));
    }
  } else if (p.rsplits == 0) {
    GMOE_TRY(launch_router(act_f32, A, a->router_w, T, d, Er, kr, ns, a->renormalize != 0, a->router_bias, idx, gate,
                           st));
  } else {
    GMOE_TRY(launch_router_many((const bf16_bits*)A, (const bf16_bits*)a->router_w, T, d, Er, kr, ns,
                                a->renormalize != 0, a->router_bias, p.rsplits, logits, idx, gate, st));
  }
  // stage 1: permutation (with the capacity cap on the routed experts)
  if (!record(dbg, 1, st)) return GROK_MOE_EHIP;
  GMOE_TRY(launch_permute(ridx, T, E, k, capacity_rows(a->capacity_factor, T, Er, kr), Er, counts, offsets, perm, pos,
                          pblk, st));
  RouteView rv{counts, offsets, perm, nullptr, nullptr};
  if (p.path == PATH_TILED) {
    int32_t* tile_off = (int32_t*)(w + p.off_tiles);
    int32_t* tile_e = tile_off + (E + 1);
    GMOE_TRY(launch_tile_table(counts, E, p.bm, tile_off, tile_e, p.mt_ub, st));
    rv.tile_off = tile_off;
    rv.tile_e = tile_e;
  }

  // stage 2: gate/up projections + GELU * up
  if (!record(dbg, 2, st)) return GROK_MOE_EHIP;
  if (p.path == PATH_F32) {
    GMOE_TRY(launch_f32_gateup((const float*)A, rv, (const float*)a->w_gate, (const float*)a->w_up, T,
                               p.rows_cap, d, f, E, act, (float*)H, st));
  } else if (p.path == PATH_STREAM) {
    GMOE_TRY(launch_stream_gateup(w8, p.mt_max, p.gsplits, (const bf16_bits*)A, rv, a->w_gate, a->w_up, a->scales, T,
                                  p.rows_cap, d, f, E, act, (bf16_bits*)H, (float*)(w + p.off_G), st));
  } else {
    if (p.pp)
      GMOE_TRY(launch_pp_gateup((const bf16_bits*)A, rv, (const bf16_bits*)a->w_gate, (const bf16_bits*)a->w_up, T,
                                p.rows_cap, d, f, E, act, (bf16_bits*)H, st));
    else
      GMOE_TRY(launch_tiled_gateup(w8, p.bm, (const bf16_bits*)A, rv, a->w_gate, a->w_up, a->scales, T, p.rows_cap,
                                   d, f, E, act, (bf16_bits*)H, st));
  }
  // stage 3: down projection
  if (!record(dbg, 3, st)) return GROK_MOE_EHIP;
  if (p.path == PATH_F32) {
    GMOE_TRY(launch_f32_down((const float*)H, rv, (const float*)a->w_down, p.rows_cap, d, f, E, Y, st));
  } else if (p.path == PATH_STREAM) {
    GMOE_TRY(launch_stream_down(w8, p.mt_max, p.splits, (const bf16_bits*)H, rv, a->w_down, a->scales, p.rows_cap, d,
                                f, E, Y, st));
  } else {
    if (p.pp)
      GMOE_TRY(launch_pp_down(p.splits, (const bf16_bits*)H, rv, (const bf16_bits*)a->w_down, p.rows_cap, d, f, E, Y,
                              st));
    else
      GMOE_TRY(launch_tiled_down(w8, p.bm, p.splits, (const bf16_bits*)H, rv, a->w_down, a->scales, p.rows_cap, d, f,
                                 E, Y, st));
  }
  // stage 4: gate-weighted combine
  if (!record(dbg, 4, st)) return GROK_MOE_EHIP;
  if (sandwich) {
    GMOE_TRY(launch_combine_sandwich(act_f32, Y, p.splits, p.rows_cap, pos, rgate, T, d, k, a->x, a->norm_post,
                                     a->norm_eps, a->out, st));
  } else {
    GMOE_TRY(launch_combine(act_f32, Y, p.splits, p.rows_cap, pos, rgate, T, d, k, a->out, st));
  }
  if (!record(dbg, 5, st)) return GROK_MOE_EHIP;

  if (dbg) {
    const size_t tk = (size_t)(T * k);
    if (!copy_out(dbg->idx, ridx, 4 * tk, st) || !copy_out(dbg->gate, rgate, 4 * tk, st) ||
        !copy_out(dbg->counts, counts, 4 * (size_t)E, st) || !copy_out(dbg->offsets, offsets, 4 * (size_t)(E + 1), st) ||
        !copy_out(dbg->perm, perm, 4 * tk, st) || !copy_out(dbg->pos, pos, 4 * tk, st) ||
        (sandwich && !copy_out(dbg->u, U, (act_f32 ? 4 : 2) * (size_t)T * (size_t)d, st)))
      return GROK_MOE_EHIP;
  }
  return GROK_MOE_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call per device (with that device current) and kept.
static int static_workspace(void** out) {
  static std::mutex mu;
  static std::atomic<void*> ptr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GROK_MOE_EHIP;
  if (dev < 0 || dev >= 64) return GROK_MOE_EUNSUPPORTED;
  void* p = ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GROK_MOE_EHIP;
      ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GROK_MOE_OK;
}

int grok_moe_forward_static(const grok_moe_args* a, const grok_moe_debug* dbg, void* stream) {
  const int rc = validate(a);
  if (rc != GROK_MOE_OK || a->T == 0) return rc;
  const size_t need = make_plan(a->T, a->d, a->f, a->E, a->k, a->n_shared, a->act_dtype, a->w_dtype).total;
  if (need > GROK_MOE_STATIC_WORKSPACE_BYTES) return GROK_MOE_EWORKSPACE;
  void* ws = nullptr;
  const int st = static_workspace(&ws);
  if (st != GROK_MOE_OK) return st;
  return grok_moe_forward_ex(a, ws, GROK_MOE_STATIC_WORKSPACE_BYTES, dbg, stream);
}

static int forward_alloc(const grok_moe_args* a, void* stream) {
  int rc = validate(a);
  if (rc != GROK_MOE_OK) return rc;
  if (a->T == 0) return GROK_MOE_OK;
  const size_t bytes = grok_moe_workspace_bytes_ex(a);
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, bytes, st) != hipSuccess) return GROK_MOE_EHIP;
  rc = grok_moe_forward_ex(a, ws, bytes, nullptr, stream);
  if (hipFreeAsync(ws, st) != hipSuccess && rc == GROK_MOE_OK) rc = GROK_MOE_EHIP;
  return rc;
}

int grok_moe_forward(const void* x, const void* router_w, const void* w_gate, const void* w_up,
                     const void* w_down, void* out, int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                     void* stream) {
  grok_moe_args a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.router_w = router_w; a.w_gate = w_gate; a.w_up = w_up; a.w_down = w_down; a.out = out;
  a.T = T; a.d = d; a.f = f; a.E = E; a.k = k;
  a.act_dtype = GROK_MOE_BF16; a.w_dtype = GROK_MOE_BF16;
  return forward_alloc(&a, stream);
}

int grok_moe_forward_w8(const void* x, const void* router_w, const int8_t* w_gate, const int8_t* w_up,
                        const int8_t* w_down, const float* scales, void* out, int64_t T, int64_t d, int64_t f,
                        int32_t E, int32_t k, void* stream) {
  grok_moe_args a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.router_w = router_w; a.w_gate = w_gate; a.w_up = w_up; a.w_down = w_down; a.scales = scales;
  a.out = out; a.T = T; a.d = d; a.f = f; a.E = E; a.k = k;
  a.act_dtype = GROK_MOE_BF16; a.w_dtype = GROK_MOE_I8;
  return forward_alloc(&a, stream);
}

int grok_moe_forward_f32(const float* x, const float* router_w, const float* w_gate, const float* w_up,
                         const float* w_down, float* out, int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                         void* stream) {
  grok_moe_args a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.router_w = router_w; a.w_gate = w_gate; a.w_up = w_up; a.w_down = w_down; a.out = out;
  a.T = T; a.d = d; a.f = f; a.E = E; a.k = k;
  a.act_dtype = GROK_MOE_F32; a.w_dtype = GROK_MOE_F32;
  return forward_alloc(&a, stream);
}

const char* grok_moe_status_string(int status) {
  switch (status) {
    case GROK_MOE_OK: return "ok";
    case GROK_MOE_EINVAL: return "invalid argument (null pointer, negative size, k > E or bad dtype)";
    case GROK_MOE_EUNSUPPORTED:
      return "unsupported shape (E <= 256 (64 for fp32), k <= 8, n_shared <= 4, d % 64 == 0, f % 128 == 0 for "
             "bf16/int8, d % 8 == 0, f % 4 == 0 for fp32)";
    case GROK_MOE_EALIGN: return "misaligned pointer (16-byte tensors, 256-byte workspace)";
    case GROK_MOE_EWORKSPACE:
      return "workspace missing or too small (grok_moe_forward_static: the shape needs more than its static "
             "workspace)";
    case GROK_MOE_EHIP: return "HIP runtime call failed";
  }
  return "unknown status";
}

}  // extern "C"
