/*
 * grok_moe.h - C ABI of the MI355X (gfx950) Grok-1 mixture-of-experts
 * feed-forward layer.
 *
 * The operation (Grok-1 field guide, "MoE 子层" section; Grok-1 book ch. 10,
 * section 10.3.1 for the routing code and section 10.4 for the GeGLU expert):
 *
 *   logits[t][e] = sum_i x[t][i] * router_w[e][i]          (no bias)
 *   p[t]         = softmax(logits[t]) over all E experts
 *   (idx, gate)  = the k largest p[t][e], largest first, lower index on
 *                  exact ties; the gates are those p values, NOT renormalised
 *   for each selected expert e of token t:
 *     a[j] = sum_i x[t][i] w_gate[e][j][i],  b[j] = sum_i x[t][i] w_up[e][j][i]
 *     h[j] = GELU(a[j]) * b[j],  GELU(z) = z * Phi(z)   (exact erf, no tanh)
 *     y[i] = sum_j h[j] w_down[e][i][j]
 *   out[t] = sum over the k slots (in slot order) of gate * y
 *
 * The experts run sparsely: tokens are permuted into expert-contiguous rows
 * and each expert runs as one segment of a grouped GEMM (the sparse reorder
 * plus grouped GEMM that book ch. 11, section 11.3.1 names as what
 * deployment needs instead of running all experts densely).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *    keeps no pointer after the call returns.
 *  - Layouts are row-major and contiguous:
 *      x, out    [T][d]
 *      router_w  [E][d]         row e = the d router weights of expert e
 *      w_gate    [E][f][d]      row j of expert e = the d input weights of
 *      w_up      [E][f][d]        its channel j (output-channel-major)
 *      w_down    [E][d][f]      row i of expert e = the f weights of output i
 *      scales    fp32, [gate: E*f | up: E*f | down: E*d]; 8-bit weights only;
 *                the weight is q * scale of its output channel
 *    The weight layouts are the transposes of the [in][out] matrices the pages
 *    write (router [d][E], input projections [E][d][f], down projection
 *    [E][f][d]): every weight row holds one output channel's reduction values
 *    contiguously, which is what the matrix-core operands take (8 consecutive
 *    reduction values per lane) and what lets the decode kernels stream each
 *    weight row as whole 128-byte lines. A caller holding [in][out] matrices
 *    transposes them once, at load time.
 *  - Asynchronous: a return of GROK_MOE_OK means the work is enqueued on
 *    `stream` (a hipStream_t; NULL is the default stream). Nothing is
 *    synchronised and nothing is copied to the host; device faults surface at
 *    the caller's next synchronisation. Buffers must stay valid until the
 *    stream work completes.
 *  - Arguments are validated before anything is enqueued: a failing call
 *    enqueues nothing and writes nothing.
 *  - `out` must not alias any input. T = 0 is a no-op that returns OK.
 *  - Supported shapes (GROK_MOE_EUNSUPPORTED otherwise): 1 <= k <= min(E, 8),
 *    E <= 256 routed experts (E <= 64 with fp32 activations), at most 4
 *    shared experts; bf16 and 8-bit weights need d % 64 == 0 and
 *    f % 128 == 0; fp32 needs d % 8 == 0 and f % 4 == 0; T <= 2^20.
 *  - Pointers must be 16-byte aligned (GROK_MOE_EALIGN otherwise).
 *  - Thread-safe: the only global state is each kernel's LDS limit, set
 *    once per device on first use. Concurrent calls on different streams
 *    need separate workspaces (the plain forms allocate their own).
 */
#ifndef GROK_MOE_H
#define GROK_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GROK_MOE_OK = 0,
  GROK_MOE_EINVAL = -1,        /* null pointer, negative size, k > E, bad dtype */
  GROK_MOE_EUNSUPPORTED = -2,  /* a shape outside the supported set above */
  GROK_MOE_EALIGN = -3,        /* a pointer that is not 16-byte aligned */
  GROK_MOE_EWORKSPACE = -4,    /* workspace smaller than grok_moe_workspace_bytes() */
  GROK_MOE_EHIP = -5           /* a HIP runtime call (allocation or launch) failed */
} grok_moe_status;

/* element types */
enum { GROK_MOE_BF16 = 0, GROK_MOE_F32 = 1, GROK_MOE_I8 = 2 };

/* activation of the gate branch: GELU with the exact Gaussian CDF (Grok-1's
 * GeGLU experts) or SiLU, z * sigmoid(z) (the SwiGLU experts of Mixtral and
 * others; book ch. 10, section 10.4, the expert-structure table and the
 * GeGLU vs SwiGLU box) */
enum { GROK_MOE_ACT_GELU = 0, GROK_MOE_ACT_SILU = 1 };

/* Full argument set of one layer call. act_dtype is the type of x, router_w
 * and out (GROK_MOE_BF16 or GROK_MOE_F32); w_dtype the type of the expert
 * weights (GROK_MOE_BF16 with bf16 activations, GROK_MOE_I8 with bf16
 * activations and `scales`, or GROK_MOE_F32 with fp32 activations).
 * route_idx / route_gate: optional DEVICE arrays [T][k] (int32 expert
 * indices, fp32 gates). When route_idx is non-NULL the router is skipped and
 * this routing is used instead (router_w may then be NULL); each row must
 * hold k distinct indices in [0, E) (an index outside that range is dropped
 * and contributes nothing).
 *
 * Variants (a zero-filled tail after route_gate is the Grok-1 layer):
 *  activation       GROK_MOE_ACT_GELU or GROK_MOE_ACT_SILU.
 *  renormalize      non-zero: the router's k gates are divided by their sum
 *                   (Mixtral; book ch. 10, section 10.3.1, the Mixtral code).
 *                   Gates given in route_gate are used as they are.
 *  capacity_factor  > 0: each expert runs at most floor(c * k * T / E) of the
 *                   k*T assignments, those of its lowest token indices; the
 *                   rest are dropped and contribute nothing (book ch. 10,
 *                   section 10.3.2, the capacity factor box). 0: no cap.
 *                   Negative or NaN: GROK_MOE_EINVAL.
 *  norm_pre,        both NULL, or both [d] arrays of the activation type:
 *  norm_post        the sandwich sub-layer (field guide, the data-flow
 *                   section; book ch. 10, section 10.3.1 on the post-norm):
 *                     u   = RMSNorm(x; norm_pre), stored in the activation type
 *                     out = x + RMSNorm(MoE(u); norm_post)
 *                   with RMSNorm(v; g)[i] = g[i] v[i] / sqrt(mean(v^2) + eps);
 *                   the router and the experts see u. Dropped assignments
 *                   leave a token's MoE sum at zero, so out = x for a token
 *                   whose every assignment overflowed.
 *  norm_eps         eps of both norms (>= 0, finite).
 *  n_shared         shared experts (0..4; DeepSeek-style fine-grained layers,
 *                   book ch. 10, section 10.1 table and the shared-expert
 *                   box): w_gate, w_up, w_down and scales then hold
 *                   E + n_shared experts, the shared ones last, and every
 *                   token also runs each of them with gate 1 (after the
 *                   routed gates, never capped). The debug idx/gate/pos
 *                   arrays then have k + n_shared columns, the shared slots
 *                   last; counts/offsets cover E + n_shared experts.
 *  router_bias      NULL, or E fp32 values: a per-expert bias of the
 *                   aux-loss-free routing (book ch. 10, section 10.3.2),
 *                   added to the softmax probabilities for the choice of
 *                   the top k only; the gates remain the probabilities. */
typedef struct grok_moe_args {
  const void* x;
  const void* router_w;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* scales;
  void* out;
  int64_t T, d, f;
  int32_t E, k;
  int32_t act_dtype, w_dtype;
  const int32_t* route_idx;
  const float* route_gate;
  int32_t activation;
  int32_t renormalize;
  double capacity_factor;
  const void* norm_pre;
  const void* norm_post;
  double norm_eps;
  int32_t n_shared;
  const float* router_bias;
} grok_moe_args;

/* Optional outputs for tests and profiling (every field may be NULL).
 * Device arrays receive copies of the intermediate results:
 *   idx [T][k] int32, gate [T][k] fp32  - the routing
 *   counts [E], offsets [E+1] int32     - rows per expert and their exclusive scan
 *   perm [k*T] int32                    - row -> token (segment e in ascending token order)
 *   pos [T][k] int32                    - (token, slot) -> row, -1 if dropped
 *   u [T][d] activation type            - the pre-norm output (sandwich only)
 * events: hipEvent_t handles; when events[i] is non-NULL it is recorded on the
 * stream before stage i (0 router, with the pre-norm when there is one, 1
 * permutation, 2 gate/up GEMM, 3 down GEMM, 4 combine) and events[5] after the
 * last stage. */
typedef struct grok_moe_debug {
  int32_t* idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
  void* events[6];
  void* u;
} grok_moe_debug;

/* Bytes of device workspace grok_moe_forward_ex needs for this shape without
 * shared experts, or 0 for an invalid or unsupported shape. */
size_t grok_moe_workspace_bytes(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t act_dtype,
                                int32_t w_dtype);

/* The same for a full argument set (counts shared experts); only the shape,
 * type and n_shared fields are read. 0 for an invalid or unsupported shape. */
size_t grok_moe_workspace_bytes_ex(const grok_moe_args* a);

/* Rows per tile of the grouped GEMMs that grok_moe_forward_ex runs for the
 * sizes, dtypes and variant knobs of `a` (its pointers are not read): each
 * expert's rows run as ceil(rows / tile_rows) tiles, and every tile reads that
 * expert's weights for the tile's output channels, so an expert's GEMM time
 * follows its tile count rather than its rows. 16, 32, 64 or 128 on the
 * streaming (small-batch) path, 64, 128, 256 or 320 on the tiled path. Returns
 * 0 for a shape grok_moe_forward_ex rejects, and for fp32 activations, whose
 * kernels have no row tiles. Host only; enqueues nothing. */
int32_t grok_moe_tile_rows(const grok_moe_args* a);

/* The layer with caller-owned workspace (ws: device memory, 256-byte aligned,
 * at least grok_moe_workspace_bytes(); its contents on entry do not matter and
 * are clobbered). dbg may be NULL. Allocates nothing. */
int grok_moe_forward_ex(const grok_moe_args* a, void* ws, size_t ws_bytes, const grok_moe_debug* dbg,
                        void* stream);

/* bf16 activations, bf16 router and bf16 expert weights. Takes its workspace
 * from hipMallocAsync/hipFreeAsync on `stream` (stream-ordered). */
int grok_moe_forward(const void* x, const void* router_w, const void* w_gate, const void* w_up,
                     const void* w_down, void* out, int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                     void* stream);

/* bf16 activations and router; 8-bit expert weights (int8 q in [-127, 127])
 * with one fp32 scale per output channel (book ch. 1, section 1.2, INT8 box:
 * int8 values plus a scale per group, dequantised at compute time). */
int grok_moe_forward_w8(const void* x, const void* router_w, const int8_t* w_gate, const int8_t* w_up,
                        const int8_t* w_down, const float* scales, void* out, int64_t T, int64_t d, int64_t f,
                        int32_t E, int32_t k, void* stream);

/* fp32 activations, router and expert weights (fp32 accumulation). */
int grok_moe_forward_f32(const float* x, const float* router_w, const float* w_gate, const float* w_up,
                         const float* w_down, float* out, int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                         void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer of
 * grok_moe_forward_ex with the same kernels, its workspace taken from a
 * static device array of GROK_MOE_STATIC_WORKSPACE_BYTES bytes that the
 * library holds on each device it runs on until the process ends. Calls no
 * allocating routine. Returns GROK_MOE_EWORKSPACE (enqueuing nothing) when
 * this shape needs more workspace than that (grok_moe_workspace_bytes_ex());
 * 64 MiB holds, for example, the Grok-1 layer (d = 6144, f = 32768, E = 8,
 * k = 2, bf16 or 8-bit weights) up to T = 128 tokens. The array belongs to the current
 * device, which must be the stream's. Every call on a device shares that
 * device's array: calls that overlap in time on one device (on different
 * streams, or from different host threads without ordering) race and give
 * wrong results; calls ordered on one stream are safe. dbg may be NULL. */
#define GROK_MOE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int grok_moe_forward_static(const grok_moe_args* a, const grok_moe_debug* dbg, void* stream);

/* Static text for a status code (never NULL). */
const char* grok_moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GROK_MOE_H */
