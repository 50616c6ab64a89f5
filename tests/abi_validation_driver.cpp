// Host-only driver of the C ABI's validation, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  The kernel
// launchers are replaced by stubs that count their calls, so the driver
// runs without a GPU and checks that no invalid call reaches a launch.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "sketchssm.h"
#include "../ssm_decode_amd/csrc/sk_params.hpp"

static int g_launches = 0;
static int g_scratch_calls = 0;

namespace sk {
int launch_m2(int, int, int, int, int, int, const Params& p, hipStream_t) {
  ++g_launches;
  // read every host-side field the dispatch filled, so that the sanitizers
  // see a use of uninitialised or out-of-range values
  volatile int sink = p.B + p.H + p.G + p.HPG + p.W + p.R + p.ndense + (p.ndense ? p.dense_list[p.ndense - 1] : 0);
  (void)sink;
  return 0;
}
int launch_gdn(int a, int b, int c, int d, int e, int f, const Params& p, hipStream_t s) {
  return launch_m2(a, b, c, d, e, f, p, s);
}
int launch_kda(int a, int b, int c, int d, int e, int f, const Params& p, hipStream_t s) {
  return launch_m2(a, b, c, d, e, f, p, s);
}
int noalloc_scratch(void** out) {
  ++g_scratch_calls;
  *out = reinterpret_cast<void*>(0x40000);
  return 0;
}
}  // namespace sk

static int g_fail = 0;
#define EXPECT(cond)                                                         \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

static void* const FAKE = reinterpret_cast<void*>(0x10000);

static sketchssm_buffers bufs() {
  sketchssm_buffers b;
  memset(&b, 0, sizeof b);
  b.S = static_cast<float*>(FAKE);
  b.U = FAKE;
  b.Pt = static_cast<const float*>(FAKE);
  b.C = static_cast<const float*>(FAKE);
  b.rank_offsets = static_cast<const int32_t*>(FAKE);
  b.ring_k = b.ring_v = b.ring_gate = FAKE;
  b.ring_beta = static_cast<float*>(FAKE);
  b.count = static_cast<int32_t*>(FAKE);
  b.A = static_cast<const float*>(FAKE);
  b.err = static_cast<int32_t*>(FAKE);
  b.work = b.Cstate = b.Scopy = FAKE;
  return b;
}

static sketchssm_step step() {
  sketchssm_step s;
  s.q = s.k = s.v = s.gate = FAKE;
  s.beta = static_cast<const float*>(FAKE);
  s.o = FAKE;
  return s;
}

static sketchssm_layer layer(const std::vector<int32_t>& off, int family, int batch, int heads, int groups,
                             int dk, int dv, int W) {
  sketchssm_layer L;
  memset(&L, 0, sizeof L);
  L.family = family;
  L.batch = batch;
  L.heads = heads;
  L.qk_groups = groups;
  L.dk = dk;
  L.dv = dv;
  L.window = W;
  L.act_dtype = L.sketch_dtype = SKSSM_BF16;
  L.rank_offsets_host = off.data();
  return L;
}

static int all_calls(const sketchssm_layer* L, const sketchssm_buffers* B, const sketchssm_step* S) {
  const int32_t seq = 0;
  int bad = 0;
  bad += sketchssm_read(L, B, S, nullptr) != 0;
  bad += sketchssm_read_noalloc(L, B, S, nullptr) != 0;
  bad += sketchssm_flush(L, B, S, SKSSM_FLUSH_DUE, nullptr) != 0;
  bad += sketchssm_flush_seqs(L, B, S, &seq, 1, nullptr) != 0;
  bad += sketchssm_full_step(L, B, S, nullptr) != 0;
  bad += sketchssm_replay_step(L, B, S, nullptr) != 0;
  return bad;
}

int main() {
  std::vector<int32_t> off(129);
  for (int h = 0; h <= 128; ++h) off[h] = 8 * h;
  sketchssm_buffers B = bufs();
  sketchssm_step S = step();

  // a valid layer reaches one launch per call
  sketchssm_layer L = layer(off, SKSSM_MAMBA2, 320, 128, 8, 128, 64, 16);
  g_launches = 0;
  EXPECT(all_calls(&L, &B, &S) == 0);
  EXPECT(g_launches == 6);
  EXPECT(g_scratch_calls == 1);
  EXPECT(sketchssm_workspace_bytes(&L) > 0);

  // invalid layers: nothing launched
  const int before = g_launches;
  struct { int fam, batch, heads, groups, dk, dv, W, act, sk; } badl[] = {
      {3, 2, 128, 8, 128, 64, 16, 1, 1},   {0, 2, 128, 8, 32, 32, 16, 1, 1},
      {0, 2, 128, 8, 128, 64, 0, 1, 1},    {0, 2, 128, 8, 128, 64, 33, 1, 1},
      {0, 2, 128, 7, 128, 64, 16, 1, 1},   {1, 2, 128, 8, 128, 64, 16, 1, 1},
      {0, -1, 128, 8, 128, 64, 16, 1, 1},  {0, 2, 128, 8, 128, 64, 16, 0, 1},
      {0, 2, 128, 8, 128, 64, 16, 2, 2},   {0, 2, 128, 4, 128, 64, 16, 1, 1},
  };
  for (const auto& c : badl) {
    sketchssm_layer Lb = layer(off, c.fam, c.batch, c.heads, c.groups, c.dk, c.dv, c.W);
    Lb.act_dtype = c.act;
    Lb.sketch_dtype = c.sk;
    EXPECT(all_calls(&Lb, &B, &S) == 6);
    EXPECT(sketchssm_workspace_bytes(&Lb) < 0);
  }
  // invalid rank tables
  std::vector<int32_t> o1 = off; o1[0] = 1;
  std::vector<int32_t> o2 = off; o2[5] = o2[4] - 1;
  std::vector<int32_t> o3 = off; for (int h = 1; h <= 128; ++h) o3[h] = 17 * h;
  for (const auto* o : {&o1, &o2, &o3}) {
    sketchssm_layer Lb = layer(*o, SKSSM_MAMBA2, 2, 128, 8, 128, 64, 16);
    EXPECT(all_calls(&Lb, &B, &S) == 6);
  }
  // null and misaligned pointers, one field at a time
  for (int f = 0; f < 15; ++f) {
    for (int mis = 0; mis < 2; ++mis) {
      sketchssm_buffers Bb = bufs();
      void* const v = mis ? reinterpret_cast<void*>(0x10004) : nullptr;
      switch (f) {
        case 0: Bb.S = static_cast<float*>(v); break;
        case 1: Bb.U = v; break;
        case 2: Bb.Pt = static_cast<const float*>(v); break;
        case 3: Bb.C = static_cast<const float*>(v); break;
        case 4: Bb.rank_offsets = static_cast<const int32_t*>(v); break;
        case 5: Bb.ring_k = v; break;
        case 6: Bb.ring_v = v; break;
        case 7: Bb.ring_gate = v; break;
        case 8: Bb.ring_beta = static_cast<float*>(v); break;
        case 9: Bb.count = static_cast<int32_t*>(v); break;
        case 10: Bb.A = static_cast<const float*>(v); break;
        case 11: Bb.err = static_cast<int32_t*>(v); break;
        case 12: Bb.work = v; break;
        case 13: Bb.Cstate = v; break;
        default: Bb.Scopy = v; break;
      }
      sketchssm_layer Lg = layer(off, SKSSM_GDN, 2, 128, 128, 128, 128, 16);
      (void)all_calls(&L, &Bb, &S);
      (void)all_calls(&Lg, &Bb, &S);
    }
  }
  EXPECT(sketchssm_read(nullptr, &B, &S, nullptr) == SKSSM_EINVAL);
  EXPECT(sketchssm_read(&L, nullptr, &S, nullptr) == SKSSM_EINVAL);
  EXPECT(sketchssm_read(&L, &B, nullptr, nullptr) == SKSSM_EINVAL);
  EXPECT(sketchssm_flush(&L, &B, nullptr, 7, nullptr) == SKSSM_EFLAG);
  EXPECT(sketchssm_flush_seqs(&L, &B, nullptr, nullptr, 3, nullptr) == SKSSM_EINVAL);
  EXPECT(sketchssm_flush_seqs(&L, &B, nullptr, nullptr, 321, nullptr) == SKSSM_EDIM);
  // the no-alloc read refuses layers beyond its array
  std::vector<int32_t> o16(129);
  for (int h = 0; h <= 128; ++h) o16[h] = 16 * h;
  sketchssm_layer Lbig = layer(o16, SKSSM_MAMBA2, 4096, 128, 8, 128, 64, 32);
  const int nl = g_launches;
  EXPECT(sketchssm_read_noalloc(&Lbig, &B, &S, nullptr) == SKSSM_ESCRATCH);
  EXPECT(g_launches == nl);
  // dense-fallback heads (rank 0) and every head dense
  std::vector<int32_t> od(129);
  for (int h = 0; h < 128; ++h) od[h + 1] = od[h] + (h % 32 == 0 ? 0 : 8);
  sketchssm_layer Ld = layer(od, SKSSM_MAMBA2, 3, 128, 8, 128, 64, 16);
  EXPECT(all_calls(&Ld, &B, &S) == 0);
  std::vector<int32_t> oz(129, 0);
  sketchssm_layer Lz = layer(oz, SKSSM_GDN, 3, 128, 128, 128, 128, 16);
  EXPECT(all_calls(&Lz, &B, &S) == 6);                    // 128 dense heads: more than 64
  // the state-dependent map's ridge
  sketchssm_layer Lm = L;
  Lm.coef_map = SKSSM_COEF_STATE;
  Lm.coef_ridge = 0.f;
  EXPECT(sketchssm_read(&Lm, &B, &S, nullptr) == SKSSM_EINVAL);
  Lm.coef_ridge = 1e-4f;
  EXPECT(sketchssm_read(&Lm, &B, &S, nullptr) == 0);
  EXPECT(g_launches > before);
  EXPECT(sketchssm_version() > 0);

  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("abi validation driver: all checks passed (%d launches reached)\n", g_launches);
  return 0;
}
