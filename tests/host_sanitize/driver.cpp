// Drives the C ABI's host code over many shapes, forced plans and bad
// arguments, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitize.py).  Device pointers are fake aligned
// addresses: the host code never dereferences them and the launchers are
// stand-ins (stubs.cpp).  Exits non-zero on an unexpected status; the
// sanitizers abort on any memory error or undefined behaviour.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "exl3.h"

namespace exl3 {
exl3_status linear_in_scratch(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                              void *scratch, size_t scratch_bytes, void *stream, bool launch);
}
extern long g_launches;

static uint16_t *fake(uintptr_t a) { return reinterpret_cast<uint16_t *>(a); }
static int g_fail = 0;

#define EXPECT(cond)                                                                               \
  do {                                                                                             \
    if (!(cond)) {                                                                                 \
      std::fprintf(stderr, "line %d: expected %s (last error: %s)\n", __LINE__, #cond, exl3_last_error()); \
      ++g_fail;                                                                                    \
    }                                                                                              \
  } while (0)

static exl3_weight view(int K, const std::vector<int32_t> &shards, int bits, int cb) {
  exl3_weight w{};
  w.trellis = fake(1 << 20);
  w.suh = fake(2 << 20);
  w.svh = fake(3 << 20);
  w.K = K;
  int N = 0;
  for (int s : shards) N += s;
  w.N = N;
  w.bits = bits;
  w.codebook = cb;
  w.n_shards = (int)shards.size();
  w.shard_n = shards.data();
  w.bias = nullptr;
  return w;
}

static exl3_plan force(int parts, int mode, int bm, int decoder, int groups = -1, int unit = -1, int wg = -1) {
  exl3_plan f{};
  f.parts = parts;
  f.groups = groups;
  f.mode = mode;
  f.bm = bm;
  f.decoder = decoder;
  f.unit = unit;
  f.wg_cols = wg;
  return f;
}

int main() {
  const uintptr_t big = uintptr_t(1) << 40;
  struct Shape {
    int K;
    std::vector<int32_t> shards;
    int bits, cb;
  };
  std::vector<Shape> shapes = {
      {1024, {1024}, 4, 0},           {4096, {2048}, 4, 1},       {2048, {4096}, 4, 1},
      {5120, {12288}, 6, 2},          {17408, {5120}, 6, 2},      {5120, {17408, 17408}, 5, 2},
      {4096, {154880}, 6, 2},         {128, {128}, 1, 0},         {16384, {128}, 8, 1},
      {128, {1 << 20}, 3, 2},         {1 << 16, {256, 384}, 7, 0}, {4096, std::vector<int32_t>(16, 256), 2, 1},
      {5120, {32768}, 4, 2},          {5120, {32640}, 4, 2},      {1 << 20, {128}, 5, 1},
  };
  const int Ms[] = {0, 1, 7, 16, 17, 33, 64, 65, 128, 300, 512, 2047, 2048, 4096, 70000, 1 << 20};
  for (auto &s : shapes) {
    exl3_weight w = view(s.K, s.shards, s.bits, s.cb);
    for (int M : Ms) {
      exl3_plan pl{};
      EXPECT(exl3_plan_query(&w, M, &pl) == EXL3_OK);
      const size_t ws = exl3_workspace_bytes(&w, M);
      EXPECT(ws == pl.workspace);
      EXPECT(exl3_linear(&w, fake(4 << 20), M, fake(big), EXL3_BF16, ws ? fake(big + (uintptr_t(1) << 39)) : nullptr,
                         ws, nullptr) == EXL3_OK);
      // the no-allocation schedule planner, with a 64 MiB scratch
      EXPECT(exl3::linear_in_scratch(&w, fake(4 << 20), M, fake(big), EXL3_F16, fake(5 << 20), 64u << 20, nullptr,
                                     true) == EXL3_OK);
      // forced schedules of the same tree: every mode, tile and decoder
      for (int mode : {EXL3_MODE_FUSED, EXL3_MODE_SLABS})
        for (int bm : {16, 32, 64, 128, 256, 512})
          for (int dec : {EXL3_DECODER_ALU, EXL3_DECODER_TABLE, EXL3_DECODER_DENSE}) {
            exl3_plan f = force(pl.parts, mode, bm, dec, pl.groups);
            const size_t need = exl3_workspace_bytes_ex(&w, M, &f);
            exl3_plan q{};
            const exl3_status st = exl3_plan_query_ex(&w, M, &f, &q);
            if (st == EXL3_OK) {
              EXPECT(q.workspace == need);
              if (need < (size_t(1) << 36))
                EXPECT(exl3_linear_ex(&w, fake(4 << 20), M, fake(big), EXL3_BF16,
                                      need ? fake(big + (uintptr_t(1) << 39)) : nullptr, need, nullptr, &f) == EXL3_OK);
            } else {
              EXPECT(need == 0);
            }
          }
      // a one-slab-per-part schedule and 64-column workgroups
      exl3_plan f1 = force(pl.parts, EXL3_MODE_SLABS, 16, EXL3_DECODER_ALU, pl.groups, 1, 64);
      exl3_plan q1{};
      (void)exl3_plan_query_ex(&w, M, &f1, &q1);
      // the GEMM stage and output stage hooks
      const size_t zb = size_t(pl.parts) * size_t((M + 3) / 4) * 4 * size_t(w.N) * 4;
      (void)exl3_debug_parts(&w, fake(4 << 20), M, reinterpret_cast<float *>(fake(big)), zb, nullptr, nullptr);
      (void)exl3_debug_epilogue(reinterpret_cast<float *>(fake(big)), pl.parts, pl.groups, M, &w, fake(big), 1,
                                nullptr);
    }
    // tuned schedules: set, used, cleared; tuning itself needs events (refused here)
    exl3_plan pl{};
    EXPECT(exl3_plan_query(&w, 16, &pl) == EXL3_OK);
    EXPECT(exl3_tune_set(&w, 16, &pl) == EXL3_OK);
    EXPECT(exl3_tune(&w, 1, fake(4 << 20), 16, fake(big), EXL3_BF16, fake(big), size_t(1) << 34, 2, nullptr,
                     nullptr) != EXL3_OK);
    (void)exl3_tune_workspace_bytes(&w, 16);
    exl3_tune_clear();
  }
  // bad arguments: every one refused with a message, nothing launched
  const long before = g_launches;
  std::vector<int32_t> one{128}, odd{100}, many(17, 128);
  exl3_weight w = view(128, one, 4, 1);
  EXPECT(exl3_linear(&w, fake(4 << 20), -1, fake(big), 1, nullptr, 0, nullptr) == EXL3_ERR_INVALID_ARG);
  EXPECT(exl3_linear(&w, fake(4 << 20), 4, fake(big), 9, nullptr, 0, nullptr) == EXL3_ERR_INVALID_ARG);
  EXPECT(exl3_linear(&w, fake((4 << 20) + 2), 4, fake(big), 1, nullptr, 0, nullptr) == EXL3_ERR_INVALID_ARG);
  exl3_weight wo = view(128, odd, 4, 1);
  EXPECT(exl3_linear(&wo, fake(4 << 20), 4, fake(big), 1, nullptr, 0, nullptr) == EXL3_ERR_INVALID_ARG);
  exl3_weight wm = view(128, many, 4, 1);
  EXPECT(exl3_linear(&wm, fake(4 << 20), 4, fake(big), 1, nullptr, 0, nullptr) == EXL3_ERR_INVALID_ARG);
  exl3_weight wb = view(128, one, 9, 1);
  EXPECT(exl3_plan_query(&wb, 4, nullptr) == EXL3_ERR_INVALID_ARG);
  exl3_plan bad = force(3, EXL3_MODE_FUSED, 512, EXL3_DECODER_ALU, 1);
  exl3_weight wk = view(4096, one, 4, 1);
  EXPECT(exl3_linear_ex(&wk, fake(4 << 20), 600, fake(big), 1, fake(big), size_t(1) << 30, nullptr, &bad) != EXL3_OK);
  EXPECT(exl3_input_transform(fake(4 << 20), 1, 4, 100, fake(2 << 20), 1, fake(big), nullptr) == EXL3_ERR_INVALID_ARG);
  EXPECT(exl3_moe_align(reinterpret_cast<int32_t *>(fake(4 << 20)), 5, 2, 5000, 16,
                        reinterpret_cast<int32_t *>(fake(big)), reinterpret_cast<int32_t *>(fake(big)),
                        reinterpret_cast<int32_t *>(fake(big)), nullptr) == EXL3_ERR_INVALID_ARG);
  EXPECT(g_launches == before);
  // routed experts: row counts and plans for several token counts
  std::vector<int32_t> expert{2048};
  exl3_weight we = view(4096, expert, 4, 1);
  for (int T : {0, 1, 16, 64, 4096})
    for (int block : {16, 32, 64}) {
      const int rows = exl3_moe_rows_max(T, 8, 64, block);
      EXPECT(rows >= 0 && rows % block == 0);
      const size_t need = exl3_moe_workspace_bytes(&we, rows, block);
      for (int dec : {EXL3_DECODER_AUTO, EXL3_DECODER_ALU, EXL3_DECODER_TABLE}) {
        const exl3_status st = exl3_moe_linear_ex(&we, 64, fake(4 << 20), rows,
                                                  reinterpret_cast<int32_t *>(fake(8 << 20)), block, fake(big), 1,
                                                  fake(big), need, nullptr, dec);
        if (dec == EXL3_DECODER_TABLE && block != 16) EXPECT(st == EXL3_ERR_UNSUPPORTED);
        else EXPECT(st == EXL3_OK || st == EXL3_ERR_UNSUPPORTED);
      }
    }
  EXPECT(exl3_moe_linear_ex(&we, 64, fake(4 << 20), 64, reinterpret_cast<int32_t *>(fake(8 << 20)), 16, fake(big),
                            1, fake(big), size_t(1) << 30, nullptr, 5) == EXL3_ERR_INVALID_ARG);
  std::printf("host checks done: %d failures, %ld launches\n", g_fail, g_launches);
  return g_fail ? 1 : 0;
}
