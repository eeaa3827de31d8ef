/*
 * Host-side sanitizer run (AddressSanitizer + UndefinedBehaviorSanitizer) of
 * the CPU oracle and the seeded input generator: every entry point once on
 * small inputs, the layer variants included. Built and run by
 * tests/test_sanitizers_cpu.py; exits non-zero on a failed call.
 */
#include "../oracle/moe_oracle.c"
#include "../synthetic/philox_gen.c"

#include <stdio.h>
#include <stdlib.h>

#define CHECK(x)                                              \
  do {                                                        \
    int rc_ = (x);                                            \
    if (rc_ != 0) {                                           \
      fprintf(stderr, "%s failed: %d\n", #x, rc_);            \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  const int64_t T = 13, d = 64, f = 96;
  const int E = 8, k = 2, E2 = 40, k2 = 5, ns = 1;
  uint16_t* x = malloc(sizeof(uint16_t) * T * d);
  uint16_t* wr = malloc(sizeof(uint16_t) * E2 * d);
  uint16_t* wg = malloc(sizeof(uint16_t) * (E2 + ns) * f * d);
  uint16_t* wu = malloc(sizeof(uint16_t) * (E2 + ns) * f * d);
  uint16_t* wd = malloc(sizeof(uint16_t) * (E2 + ns) * d * f);
  int8_t* qg = malloc((size_t)E * f * d);
  int8_t* qu = malloc((size_t)E * f * d);
  int8_t* qd = malloc((size_t)E * d * f);
  float* sc = malloc(sizeof(float) * (2 * E * f + E * d));
  uint16_t* npre = malloc(sizeof(uint16_t) * d);
  uint16_t* npost = malloc(sizeof(uint16_t) * d);
  float* bias = malloc(sizeof(float) * E2);
  syn_normal_bf16(x, T * d, 0, 0, 1.0, 2);
  syn_normal_bf16(wr, E2 * d, 0, 1, 0.125, 2);
  syn_normal_bf16(wg, (E2 + ns) * f * d, 0, 2, 0.125, 2);
  syn_normal_bf16(wu, (E2 + ns) * f * d, 0, 3, 0.125, 2);
  syn_normal_bf16(wd, (E2 + ns) * d * f, 0, 4, 0.1, 2);
  syn_uniform_i8(qg, E * f * d, 0, 2, 2);
  syn_uniform_i8(qu, E * f * d, 0, 3, 2);
  syn_uniform_i8(qd, E * d * f, 0, 4, 2);
  syn_normal_bf16(npre, d, 0, 5, 0.1, 1);
  syn_normal_bf16(npost, d, 0, 6, 0.1, 1);
  syn_normal_f32(bias, E2, 0, 8, 1e-3, 1);
  for (int i = 0; i < 2 * E * f + E * d; ++i) sc[i] = 1e-3f;
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, rnd[4];
  syn_philox4x32_10(ctr, key, rnd);

  double probs[13 * 40], gate[13 * 8], out[13 * 64], out2[13 * 64], y[64], u64[13 * 64];
  int32_t idx[13 * 8], counts[64], offsets[65], perm[13 * 8], pos[13 * 8];
  CHECK(oracle_route(x, ORC_BF16, wr, ORC_BF16, T, d, E, k, probs, idx, gate, 2));
  CHECK(oracle_permute(idx, T, E, k, counts, offsets, perm, pos));
  CHECK(oracle_permute_cap(idx, T, E, k, 2, E, counts, offsets, perm, pos));
  CHECK(oracle_route_v(x, ORC_BF16, wr, ORC_BF16, T, d, E2, k2, 1, bias, probs, idx, gate, 2));
  CHECK(oracle_expert(x, ORC_BF16, 3, wg, wu, wd, ORC_BF16, NULL, d, f, E, 5, y));
  CHECK(oracle_expert(x, ORC_BF16, 4, qg, qu, qd, ORC_I8, sc, d, f, E, 6, y));
  CHECK(oracle_forward(x, ORC_BF16, wr, ORC_BF16, wg, wu, wd, ORC_BF16, NULL, T, d, f, E, k, out, idx, gate, 2));
  const int64_t toks[3] = {12, 0, 5};
  CHECK(oracle_forward_given_routing(x, ORC_BF16, wg, wu, wd, ORC_BF16, NULL, idx, gate, T, d, f, E, k, toks, 3,
                                     out2, 2));
  CHECK(oracle_dense_onehot(x, ORC_BF16, wr, ORC_BF16, qg, qu, qd, ORC_I8, sc, T, d, f, E, k, out, 2));
  CHECK(oracle_rmsnorm(x, ORC_BF16, T, d, npre, ORC_BF16, 1e-5, u64));

  orc_layer L = {x, ORC_BF16, wr, ORC_BF16, wg, wu, wd, ORC_BF16, NULL, T, d, f, E, k, 1, 1, 0.75,
                 npre, npost, ORC_BF16, 1e-5, 0, NULL};
  uint16_t ub[13 * 64];
  CHECK(oracle_layer(&L, NULL, T, out, idx, gate, pos, ub, 2));
  orc_layer L2 = {x, ORC_BF16, wr, ORC_BF16, wg, wu, wd, ORC_BF16, NULL, T, d, f, E2, k2, 1, 1, 0.6,
                  NULL, NULL, ORC_BF16, 0.0, ns, bias};
  double gate2[13 * 8];
  int32_t idx2[13 * 8], pos2[13 * 8];
  CHECK(oracle_layer(&L2, toks, 3, out2, idx2, gate2, pos2, NULL, 2));
  orc_layer L3 = {x, ORC_BF16, wr, ORC_BF16, qg, qu, qd, ORC_I8, sc, T, d, f, E, k, 0, 0, 0.0,
                  npre, npost, ORC_BF16, 1e-5, 0, NULL};
  CHECK(oracle_layer(&L3, NULL, T, out, idx, gate, pos, ub, 2));
  if (oracle_bf16_rne(1.0) != 0x3F80 || oracle_capacity(1.0, 2048, 8, 2) != 512) return 1;
  if (!(oracle_silu(1.0) > 0.73 && oracle_gelu(1.0) > 0.84)) return 1;
  free(x); free(wr); free(wg); free(wu); free(wd); free(qg); free(qu); free(qd); free(sc);
  free(npre); free(npost); free(bias);
  printf("sanitized run ok\n");
  return 0;
}
