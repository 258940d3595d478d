// Host side of the C ABI declared in include/exl3.h: argument validation,
// the shape-only K-part rule, the schedule choice, and kernel launches.
//
// Every check runs before any HIP call, so a rejected call touches no device
// state (the cuda-exl3 README, "Loading into a dim vLLM has padded", asks
// for errors that say which check failed and by how much; the TensorFold PR
// refuses what it cannot read, "What it adds").
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/exl3.h"
#include "exl3_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

exl3_status fail(exl3_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_last_error[0] = '\0'; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int32_t MAX_M = 1 << 20;
constexpr int32_t MAX_KN = 1 << 24;

exl3_status check_ptr(const void *p, const char *name) {
  if (p == nullptr) return fail(EXL3_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(EXL3_ERR_INVALID_ARG, "%s=%p is not 16-byte aligned", name, p);
  return EXL3_OK;
}

exl3_status validate_weight(const exl3_weight *w, bool need_trellis, bool need_suh) {
  if (w == nullptr) return fail(EXL3_ERR_INVALID_ARG, "weight view is NULL");
  if (w->bits < 1 || w->bits > 8) return fail(EXL3_ERR_INVALID_ARG, "bits=%d, must be 1..8", w->bits);
  if (w->codebook < EXL3_CB_3INST || w->codebook > EXL3_CB_MUL1)
    return fail(EXL3_ERR_INVALID_ARG, "codebook=%d, must be 0 (3inst), 1 (mcg) or 2 (mul1)", w->codebook);
  if (w->K <= 0 || w->K % 128 != 0)
    return fail(EXL3_ERR_INVALID_ARG, "K=%d must be a positive multiple of 128 (off by %d)", w->K,
                w->K > 0 ? w->K % 128 : w->K);
  if (w->N <= 0 || w->N % 128 != 0)
    return fail(EXL3_ERR_INVALID_ARG, "N=%d must be a positive multiple of 128 (off by %d)", w->N,
                w->N > 0 ? w->N % 128 : w->N);
  if (w->K > MAX_KN || w->N > MAX_KN)
    return fail(EXL3_ERR_UNSUPPORTED, "K=%d or N=%d exceeds the supported %d", w->K, w->N, MAX_KN);
  if (w->n_shards < 1 || w->n_shards > EXL3_MAX_SHARDS)
    return fail(EXL3_ERR_INVALID_ARG, "n_shards=%d, must be 1..%d", w->n_shards, EXL3_MAX_SHARDS);
  if (w->shard_n == nullptr) return fail(EXL3_ERR_INVALID_ARG, "shard_n (host array) is NULL");
  int64_t total = 0;
  for (int s = 0; s < w->n_shards; ++s) {
    const int32_t n = w->shard_n[s];
    if (n <= 0 || n % 128 != 0)
      return fail(EXL3_ERR_INVALID_ARG, "shard %d width %d must be a positive multiple of 128 (off by %d)", s, n,
                  n > 0 ? n % 128 : n);
    total += n;
  }
  if (total != w->N)
    return fail(EXL3_ERR_INVALID_ARG, "shard widths sum to %lld but N=%d (off by %lld)", (long long)total, w->N,
                (long long)(total - w->N));
  exl3_status st;
  if (need_trellis && (st = check_ptr(w->trellis, "trellis")) != EXL3_OK) return st;
  if (need_suh && (st = check_ptr(w->suh, "suh")) != EXL3_OK) return st;
  if (w->bias != nullptr && (st = check_ptr(w->bias, "bias")) != EXL3_OK) return st;
  if ((st = check_ptr(w->svh, "svh")) != EXL3_OK) return st;
  return EXL3_OK;
}

// Column blocks from which a layer keeps K whole (choose_groups).
constexpr int32_t WIDE_ONE_PART = 256;
// Weights from which a layer takes the large-layer part rule.
constexpr double SMALL_LAYER_WEIGHTS = 33554432.0;  // 2^25

// K groups: a function of (K, N, bits) only.  On a small layer (under 2^25
// weights) enough (column block, group) pairs to occupy the GPU at decode
// sizes (about 1024; large layers take about 512, below), groups of at least
// four 128-k blocks (or four groups of two blocks, for short K), and the fp32
// partial traffic at 16 rows kept near the trellis bytes it helps to stream
// (the cuda-exl3 README caps split-k accumulator traffic at ~30% of the
// weight bytes and discounts it when it stays in cache, "Two further
// departures" and "Where the time goes"; on this GPU the partials of a
// decode-size call stay in the 256 MB cache, so the cap is looser).  Shorter
// groups help one-row calls little and cost batched ones partial traffic: at
// K=4096, N=2048 eight groups against sixteen are 9% slower at one row and
// 26% faster at 512 (when every group was one part).  A small layer (fewer
// than 512 block x group pairs, whose groups split into parts) keeps at most
// 128 pairs: its one-row calls run four part quads per group anyway, and at
// K = N = 4096 (32 blocks) 4 groups of 4 parts against 8 of 4 took 64 rows
// from 19.6 to 18.3 us and one row from 12.2 to 10.7 us (4-bit mcg, calls
// back to back; after a rotation in a graph the 64-row calls tie), while
// at K = 4096, N = 2048 (16 blocks) the 8 groups stay (4 were faster at 1 and
// 16 rows but slower at 512: 33.4 against 30.5 us).  G divides the number of
// 128-k blocks so every group has the same length.
int32_t choose_groups(int32_t K, int32_t N, int32_t bits) {
  const int32_t kb = K / 128;
  const int32_t nblk = N / 128;
  // A layer of at least WIDE_ONE_PART column blocks gives every CU a block
  // at one row without splitting K.  Splitting it anyway still pays at a
  // few rows (gate_up 5120 x 34816: 16 rows 43 us in 4 parts, 61 us in one;
  // 128 rows 147 / 179 us) but takes the register fold from batched calls,
  // whose one-part GEMM runs 256-column tiles with twice the products per
  // barrier (2048 rows 971 -> 844 us, 4096 rows 1709 -> 1471 us).
  if (nblk >= WIDE_ONE_PART) return 1;
  const int32_t cap_len = std::max(1, std::max(kb / 4, std::min(kb / 2, 4)));
  const int32_t cap_traffic = std::max(1, (int32_t)(1.2 * (double)K * bits / 1024.0));
  const int32_t cap = std::max(1, std::min(cap_len, cap_traffic));
  if ((double)K * (double)N >= SMALL_LAYER_WEIGHTS) {
    // A large layer takes about two workgroups per CU at one row (512
    // pairs): the divisor of the block count nearest 512 / nblk in ratio.
    // Fewer groups than a four-per-CU target cost the one-row call nothing
    // and halve the partial traffic of batched calls: q_proj 5120 x 12288
    // over its nine row counts 425 us in 10 groups, 374 us in 5 (256 rows
    // 91 -> 66 us); down_proj 17408 x 5120 keeps 17 (536 us; 8 groups 541).
    const double want = 512.0 / nblk;
    int32_t best = 1;
    double best_d = 1e30;
    for (int32_t g = 1; g <= cap; ++g)
      if (kb % g == 0) {
        const double d = std::fabs(std::log((double)g / want));
        if (d < best_d) {
          best_d = d;
          best = g;
        }
      }
    return best;
  }
  int32_t want = (1024 + nblk - 1) / nblk;
  int32_t gmax = std::max(1, std::min(want, cap));
  if ((int64_t)nblk * gmax < 512) gmax = std::max(1, std::min(gmax, 128 / nblk));
  for (int32_t g = gmax; g >= 1; --g)
    if (kb % g == 0) return g;
  return 1;
}

// Parts per group: also a function of the shape only.  A small layer (fewer
// than 512 column-block x group pairs, too few workgroups to give every SIMD
// of the GPU work at one row) splits each group into 4 (or 2) equal parts, so
// a one-row call runs one workgroup of four- (two-) part quads per group;
// larger layers keep one part per group.
int32_t choose_q(int32_t K, int32_t N, int32_t groups) {
  const int32_t kb = K / 128;
  const int32_t nblk = N / 128;
  if ((double)K * (double)N >= SMALL_LAYER_WEIGHTS || (int64_t)nblk * groups >= 512 || nblk >= WIDE_ONE_PART) return 1;
  const int32_t len = kb / groups;
  return len % 4 == 0 ? 4 : len % 2 == 0 ? 2 : 1;
}

// Compute units of the current device (queried once per device; calls from
// several threads may race to fill an entry, all with the same value).
hipError_t device_cus(int *out) {
  static std::atomic<int> cache[64];  // zero: not yet queried
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

// The CU count for planning; 256 (an MI355X) when no device is visible.
int device_cus_or_default() {
  int n = 0;
  return device_cus(&n) == hipSuccess ? n : 256;
}

struct Plan {
  int32_t parts;     // P
  int32_t groups;    // G
  int32_t mode;
  int32_t bm;
  int32_t decoder;
  int32_t unit;      // parts per workgroup unit
  int32_t quads;     // small tiles: one part per quad of waves
  bool half;         // small tiles: 64-column workgroups
  bool multi;        // the workgroup folds unit > 1 parts in registers
  bool finisher;     // slab mode: the last workgroup of a tile does the output
  int32_t chunk;     // rows per launch
  int32_t launches;  // kernels per exl3_linear call
  size_t slab_off;   // workspace byte offsets of the slabs and the dense W_q
  size_t dense_off;
  size_t workspace;
};

// The table decoder pays a fixed cost per CU (filling a 65,536-entry table)
// that the layer's weights have to amortize.  Up to 16 rows the ALU tiles
// with the finishing workgroup (one launch) beat it below 2^26 weights
// (measured by the schedule tuner on q_proj 5120 x 12288: 22.9 -> 20.3 us at
// one row, 24.1 -> 22.9 at 16), above 16 rows from 2^25.
constexpr double TABLE_MIN_WEIGHTS = 33554432.0;         // 2^25
constexpr double TABLE_MIN_WEIGHTS_SMALL_M = 67108864.0;  // 2^26, M <= 16
constexpr int32_t TABLE_MAX_M = 64;
// Grouped (MoE) calls take the table decoder from this many (16-row block,
// column block) units: with fewer the fused units leave CUs idle where the
// ALU tiles split K.  Measured on the expert pair's shapes, 64 experts,
// top-8: one token on 4096 x 2048 (128 units) 39.5 us ALU / 40.9 us table,
// on 2048 x 4096 (256 units) 38.6 / 25.3 us; 16 tokens 216 / 89 us.
constexpr int64_t MOE_TABLE_MIN_UNITS = 256;
// The table kernel addresses the trellis with 32-bit byte offsets.
constexpr double TABLE_MAX_TRELLIS_BYTES = 2147483648.0;  // 2 GiB
// Partial slabs beyond this go through the fused fold (or row chunks).
constexpr double SLAB_CAP_BYTES = 192.0 * 1024 * 1024;
// Row tiles a tile-kernel launch can hold (the grid's third dimension).
constexpr int32_t MAX_GRID_Z = 65535;
// Slab bytes the finishing workgroup's 32-bit buffer offsets reach.
constexpr double FINISHER_MAX_SLAB_BYTES = 2147483648.0;  // 2 GiB
// Tiles the finisher's counters can hold (one 32-bit counter each).
constexpr int64_t MAX_COUNTERS = EXL3_WORKSPACE_COUNTER_BYTES / 4;
// Dense path (dequantize once, then a plain MFMA GEMM): batches and layers
// large enough for the K*N*2 bytes of fp16 fragments to pay off.  Measured:
// gate_up 5120 x 34816 at 2048 rows 986 -> 937 us, at 4096 rows
// 1847 -> 1661 us; at 512 rows it loses on every layer shape (lm_head
// 761 -> 1081 us: its fp16 fragments are 1.27 GB against 476 MB of trellis).
constexpr int32_t DENSE_MIN_M = 2048;
constexpr double DENSE_MIN_WEIGHTS = 33554432.0;

size_t slab_bytes(int32_t n_slabs, int32_t rows, int32_t N) {
  return (size_t)n_slabs * (size_t)((rows + 3) / 4) * 4 * (size_t)N * sizeof(float);
}

// Column tiles of the dense decoder's 256 x 256 kernel: each shard's
// column blocks in pairs (an odd shard ends in a one-block tile).
int32_t dense_col_tiles(const exl3_weight *w) {
  int32_t t = 0;
  for (int s = 0; s < w->n_shards; ++s) t += (w->shard_n[s] / 128 + 1) / 2;
  return t;
}

// The first column block of 256 x 256 column tile t.
int32_t dense_tile_first_block(const exl3_weight *w, int32_t t) {
  int32_t start = 0;
  for (int s = 0; s < w->n_shards; ++s) {
    const int32_t blocks = w->shard_n[s] / 128;
    const int32_t tiles = (blocks + 1) / 2;
    if (t < tiles) return start + 2 * t;
    t -= tiles;
    start += blocks;
  }
  return start;
}

// Column tiles of the dense GEMM's 256 x 256 launch over `rows` rows and
// `units` units; the column blocks after them run as 256 x 128 tiles in a
// second launch.  One workgroup of 256 x 256 tiles fills a CU and they all
// take about as long, so the kernel runs in rounds of `cus` workgroups, and
// a last round of few workgroups leaves most CUs idle for most of a round
// (gate_up 5120 x 2 x 17408: 816 tiles at 1536 rows and 952 at 1792 took
// 551 and 581 us, 1088 at 2048 rows 711 us).  When the last round's tiles,
// as twice as many 256 x 128 tiles of half the work, fit one round, they run
// that way after whole rounds of the wide tiles.  Measured on gate_up: 727
// -> 704 us at 2048 rows, 1376 -> 1370 us at 4096; less than the rounds
// suggest, since a partial round runs faster than a full one (its few
// workgroups share the clock and the memory with no others).
int32_t dense_bulk_tiles(const exl3_weight *w, int32_t rows, int32_t units, int cus) {
  const int64_t ct = dense_col_tiles(w);
  const int64_t per_tile = (int64_t)((rows + 255) / 256) * units;  // workgroups per column tile
  const int64_t r = ct * per_tile % cus;
  if (r == 0) return (int32_t)ct;
  const int64_t c = (r + per_tile - 1) / per_tile;  // column tiles of the last round
  if (c >= ct || 2 * c * per_tile > cus) return (int32_t)ct;
  return (int32_t)(ct - c);
}

// slab_cap: the partial slabs a plan may keep at once (row chunks beyond it).
exl3_status make_plan(const exl3_weight *w, int32_t M, const exl3_plan *force, Plan *out,
                      double slab_cap = SLAB_CAP_BYTES) {
  Plan pl;
  const int32_t KB = w->K / 128;
  const int32_t nblk = w->N / 128;
  pl.groups = choose_groups(w->K, w->N, w->bits);
  pl.parts = pl.groups * choose_q(w->K, w->N, pl.groups);
  if (force && force->parts > 0) {
    if (force->parts > KB)
      return fail(EXL3_ERR_INVALID_ARG, "forced parts=%d exceeds the %d blocks of 128 in K", force->parts, KB);
    pl.parts = force->parts;
    pl.groups = force->parts;
    if (force->groups > 0) {
      if (force->parts % force->groups != 0)
        return fail(EXL3_ERR_INVALID_ARG, "forced groups=%d do not divide parts=%d (remainder %d)", force->groups,
                    force->parts, force->parts % force->groups);
      pl.groups = force->groups;
    }
  } else if (force && force->groups > 0) {
    return fail(EXL3_ERR_INVALID_ARG, "forced groups=%d needs forced parts", force->groups);
  }
  const int32_t Q = pl.parts / pl.groups;
  if (Q > 1 && KB % pl.parts != 0)
    return fail(EXL3_ERR_UNSUPPORTED, "%d parts in groups of %d need equal parts: %d blocks of 128 leave %d",
                pl.parts, Q, KB, KB % pl.parts);
  // Rows per tile: the smallest tile that holds M rows, up to 512 (the
  // measured best at every layer shape and batch of the plan sweep).
  pl.bm = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : M <= 128 ? 128 : M <= 256 ? 256 : 512;
  const bool bm_forced = force && force->bm > 0;
  const double weights = (double)w->K * (double)w->N;
  const bool table_fits = weights * w->bits / 8.0 <= TABLE_MAX_TRELLIS_BYTES;
  pl.decoder = (M <= TABLE_MAX_M && weights >= (M <= 16 ? TABLE_MIN_WEIGHTS_SMALL_M : TABLE_MIN_WEIGHTS) &&
                table_fits) ? EXL3_DECODER_TABLE
                : (M >= DENSE_MIN_M && weights >= DENSE_MIN_WEIGHTS) ? EXL3_DECODER_DENSE
                                                                    : EXL3_DECODER_ALU;
  if (bm_forced) pl.decoder = EXL3_DECODER_ALU;
  if (force && force->decoder >= 0) {
    if (force->decoder != EXL3_DECODER_ALU && force->decoder != EXL3_DECODER_TABLE &&
        force->decoder != EXL3_DECODER_DENSE)
      return fail(EXL3_ERR_INVALID_ARG, "forced decoder=%d, must be 0 (alu), 1 (table) or 2 (dense)",
                  force->decoder);
    if (force->decoder == EXL3_DECODER_TABLE && M > TABLE_MAX_M)
      return fail(EXL3_ERR_UNSUPPORTED, "the table decoder takes at most %d rows; M=%d (over by %d)", TABLE_MAX_M,
                  M, M - TABLE_MAX_M);
    if (force->decoder == EXL3_DECODER_TABLE && !table_fits)
      return fail(EXL3_ERR_UNSUPPORTED, "the table decoder reads at most %.0f trellis bytes; this weight has %.0f",
                  TABLE_MAX_TRELLIS_BYTES, weights * w->bits / 8.0);
    pl.decoder = force->decoder;
  }
  if (bm_forced) {
    if (force->bm != 16 && force->bm != 32 && force->bm != 64 && force->bm != 128 && force->bm != 256 &&
        force->bm != 512)
      return fail(EXL3_ERR_INVALID_ARG, "forced bm=%d, must be 16, 32, 64, 128, 256 or 512", force->bm);
    pl.bm = force->bm;
  }
  if (pl.decoder == EXL3_DECODER_TABLE) pl.bm = M <= 16 ? 16 : M <= 32 ? 32 : 64;
  if (pl.decoder == EXL3_DECODER_DENSE) pl.bm = 256;  // the dense kernel's tile
  // Mode.  One group: a workgroup folds all parts (one level).  One part per
  // group: separate fp32 partials (one workgroup per part: P times the
  // workgroups) while their traffic is small next to the GEMM's; beyond
  // 192 MiB one workgroup folds all parts of its tile.  Several parts per
  // group in several groups: always partials, one slab per group (the fused
  // fold is one level), in row chunks that keep the slabs within 192 MiB.
  // One part per group from 512 rows also folds in registers when the
  // 256-row tiles of the fused plan cover three quarters of the CUs: the
  // schedule tuner's choice on q_proj 5120 x 12288 at 512 rows (5 groups,
  // 116 -> 108 us); down_proj's 40 blocks stay with the partials.
  const size_t full_slabs = slab_bytes(pl.groups, M, w->N);
  const bool fused_fills = M >= 512 && (int64_t)nblk * ((M + 255) / 256) * 4 >= 3 * (int64_t)device_cus_or_default();
  if (pl.parts == 1 || pl.groups == 1) pl.mode = EXL3_MODE_FUSED;
  else if (Q > 1) pl.mode = EXL3_MODE_SLABS;
  else pl.mode = (double)full_slabs <= slab_cap && !fused_fills ? EXL3_MODE_SLABS : EXL3_MODE_FUSED;
  if (force && force->mode != EXL3_MODE_AUTO && force->mode >= 0) {
    if (force->mode != EXL3_MODE_FUSED && force->mode != EXL3_MODE_SLABS)
      return fail(EXL3_ERR_INVALID_ARG, "forced mode=%d, must be 0 (fused) or 1 (slabs)", force->mode);
    if (force->mode == EXL3_MODE_FUSED && pl.groups > 1 && Q > 1)
      return fail(EXL3_ERR_UNSUPPORTED, "mode=fused folds one level; %d groups of %d parts need mode=slabs",
                  pl.groups, Q);
    pl.mode = force->mode;
  }
  if (pl.parts == 1) pl.mode = EXL3_MODE_FUSED;  // one part: nothing to sum
  // Workgroup unit: all parts (fused), else one group per slab; the
  // part-sums hook (and a forced unit of 1) writes one slab per part.
  pl.unit = pl.mode == EXL3_MODE_FUSED ? pl.parts : Q;
  if (force && force->unit > 0 && pl.mode == EXL3_MODE_SLABS) {
    if (force->unit != 1 && force->unit != Q)
      return fail(EXL3_ERR_INVALID_ARG, "forced unit=%d, must be 1 or the %d parts of a group", force->unit, Q);
    pl.unit = force->unit;
  }
  // 512-row tiles hold one accumulator set: a unit of one part only
  if (pl.bm == 512 && pl.unit > 1) {
    if (bm_forced)
      return fail(EXL3_ERR_UNSUPPORTED, "bm=512 runs one K part per workgroup; units of %d parts need bm<=256",
                  pl.unit);
    pl.bm = 256;
  }
  // 512-row tiles run one workgroup per CU: with fewer tiles than CUs,
  // 256-row tiles (twice the workgroups) finish first
  if (!bm_forced && pl.bm == 512) {
    const int64_t tiles =
        (int64_t)nblk * (pl.mode == EXL3_MODE_SLABS ? pl.parts / pl.unit : 1) * ((M + 511) / 512);
    if (tiles < device_cus_or_default()) pl.bm = 256;
  }
  // Small tiles: a unit of 2 or 4 equal parts runs as that many quads of
  // waves, one part each; other units fold in registers.
  pl.quads = 1;
  pl.multi = pl.unit > 1;
  if (pl.decoder == EXL3_DECODER_ALU && pl.bm <= 64 && (pl.unit == 2 || pl.unit == 4) && KB % pl.parts == 0) {
    pl.quads = pl.unit;
    pl.multi = false;
  }
  const int32_t n_slabs = pl.parts / pl.unit;
  pl.chunk = M;
  // the tile kernels put row tiles on the grid's third dimension (at most
  // 65535 a launch): a million rows in 16-row tiles run in two launches
  if (pl.decoder == EXL3_DECODER_ALU && (int64_t)M > (int64_t)MAX_GRID_Z * pl.bm) pl.chunk = MAX_GRID_Z * pl.bm;
  if (pl.mode == EXL3_MODE_SLABS && (double)slab_bytes(n_slabs, pl.chunk, w->N) > slab_cap) {
    const double per_tile = (double)slab_bytes(n_slabs, pl.bm, w->N);
    pl.chunk = (int32_t)std::max<double>(pl.bm, std::floor(slab_cap / per_tile) * pl.bm);
    pl.chunk = std::min(pl.chunk, std::min(M, MAX_GRID_Z * pl.bm));
  }
  // (The table kernel keeps the second kernel: a finishing team inside it
  // measured slower, 21 -> 25 us on q_proj at one row.)
  // The finishing workgroup addresses the slabs with 32-bit buffer offsets:
  // a (forced) plan with 2 GiB of slabs or more sums them in the second
  // kernel instead, which uses 64-bit addresses.
  pl.finisher = pl.mode == EXL3_MODE_SLABS && pl.decoder == EXL3_DECODER_ALU && pl.bm <= 64 &&
                (int64_t)nblk * ((pl.chunk + pl.bm - 1) / pl.bm) <= MAX_COUNTERS &&
                (double)slab_bytes(n_slabs, pl.chunk, w->N) < FINISHER_MAX_SLAB_BYTES;
  // Small tiles in slab mode with fewer workgroups than CUs: split each
  // 128-column block between two workgroups of half the waves (the same
  // per-wave work on twice the CUs; the finishing workgroup or the output
  // kernel sums both halves' slabs).
  pl.half = pl.mode == EXL3_MODE_SLABS && pl.decoder == EXL3_DECODER_ALU && pl.bm <= 64 && !pl.multi &&
            (int64_t)nblk * n_slabs * ((pl.chunk + pl.bm - 1) / pl.bm) < device_cus_or_default();
  // 33-64 rows that would need half-width workgroups to fill the CUs run
  // as two 32-row tiles of full width instead: as many workgroups, each of
  // twice the waves (the schedule tuner's choice on all 24 layers of the
  // K = N = 4096 bit-width sweep at 64 rows, 3-7% faster)
  if (pl.half && !bm_forced && pl.bm == 64 && M > 32 && !(force && force->wg_cols > 0)) {
    pl.bm = 32;
    pl.half = (int64_t)nblk * n_slabs * ((pl.chunk + pl.bm - 1) / pl.bm) < device_cus_or_default();
    pl.finisher = pl.mode == EXL3_MODE_SLABS && pl.decoder == EXL3_DECODER_ALU &&
                  (int64_t)nblk * ((pl.chunk + pl.bm - 1) / pl.bm) <= MAX_COUNTERS &&
                  (double)slab_bytes(n_slabs, pl.chunk, w->N) < FINISHER_MAX_SLAB_BYTES;
  }
  if (force && force->wg_cols > 0) {
    if (force->wg_cols != 64 && force->wg_cols != 128)
      return fail(EXL3_ERR_INVALID_ARG, "forced wg_cols=%d, must be 64 or 128", force->wg_cols);
    if (force->wg_cols == 64 &&
        !(pl.mode == EXL3_MODE_SLABS && pl.decoder == EXL3_DECODER_ALU && pl.bm <= 64 && !pl.multi))
      return fail(EXL3_ERR_UNSUPPORTED,
                  "64-column workgroups need slab mode, the ALU decoder, at most 64 rows per tile and no register "
                  "fold (mode=%d decoder=%d bm=%d unit=%d)", pl.mode, pl.decoder, pl.bm, pl.unit);
    pl.half = force->wg_cols == 64;
  }
  pl.launches = pl.mode == EXL3_MODE_SLABS && !pl.finisher ? 2 : 1;
  if (pl.chunk < M && M > 0) pl.launches *= (M + pl.chunk - 1) / pl.chunk;
  if (pl.decoder == EXL3_DECODER_DENSE) {
    pl.launches += 1;  // the dequantization
    if (!pl.multi && M > 0) {  // a 256 x 128 launch after the 256 x 256 one (dense_bulk_tiles)
      const int cus = device_cus_or_default();
      const int32_t units = pl.mode == EXL3_MODE_SLABS ? pl.parts / pl.unit : 1;
      for (int32_t r0 = 0; r0 < M; r0 += pl.chunk)
        if (dense_bulk_tiles(w, std::min(M, r0 + pl.chunk) - r0, units, cus) < dense_col_tiles(w)) pl.launches += 1;
    }
  }
  // counters, then slabs [n_slabs][ceil(chunk/4)][N][4] fp32, then (dense)
  // W_q as B fragments, K*N fp16
  pl.slab_off = EXL3_WORKSPACE_COUNTER_BYTES;
  pl.dense_off = pl.slab_off + (pl.mode == EXL3_MODE_SLABS ? slab_bytes(n_slabs, pl.chunk, w->N) : 0);
  pl.dense_off = (pl.dense_off + 255) & ~(size_t)255;
  pl.workspace = pl.decoder == EXL3_DECODER_DENSE ? pl.dense_off + (size_t)w->K * (size_t)w->N * 2
                 : pl.mode == EXL3_MODE_SLABS     ? pl.slab_off + slab_bytes(n_slabs, pl.chunk, w->N)
                                                  : 0;
  *out = pl;
  return EXL3_OK;
}

exl3_status run_linear(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                       uint32_t *counters, float *slabs, uint16_t *dense, const Plan &pl, hipStream_t s,
                       bool with_output, const int32_t *block_expert = nullptr, int64_t expert_trellis = 0,
                       int32_t n_experts = 0, const void *x_in = nullptr, bool x_in_bf16 = false,
                       int dense_which = 3);

exl3_status launch_error(hipError_t e, const char *what) {
  return fail(EXL3_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

// Both input transforms: every argument checked before the launch.
exl3_status input_transform_checked(const void *x, int32_t x_dtype, bool swiglu, int32_t M, int32_t K,
                                    const uint16_t *suh, int32_t n_shards, uint16_t *x_rot, void *stream) {
  clear_error();
  if (x_dtype != EXL3_F16 && x_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "x_dtype=%d, must be 0 (fp16) or 1 (bf16)", x_dtype);
  if (M < 0) return fail(EXL3_ERR_INVALID_ARG, "M=%d is negative", M);
  if (M > MAX_M) return fail(EXL3_ERR_UNSUPPORTED, "M=%d exceeds the supported %d", M, MAX_M);
  if (K <= 0 || K % 128 != 0)
    return fail(EXL3_ERR_INVALID_ARG, "K=%d must be a positive multiple of 128 (off by %d)", K, K > 0 ? K % 128 : K);
  if (K > MAX_KN) return fail(EXL3_ERR_UNSUPPORTED, "K=%d exceeds the supported %d", K, MAX_KN);
  if (n_shards < 1 || n_shards > EXL3_MAX_SHARDS)
    return fail(EXL3_ERR_INVALID_ARG, "n_shards=%d, must be 1..%d", n_shards, EXL3_MAX_SHARDS);
  exl3_status st;
  if ((st = check_ptr(suh, "suh")) != EXL3_OK) return st;
  if (M == 0) return EXL3_OK;
  if ((st = check_ptr(x, swiglu ? "gate_up" : "x")) != EXL3_OK) return st;
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_input_transform(x, x_dtype == EXL3_BF16, swiglu, M, K, suh, n_shards, x_rot,
                                                    (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "input transform launch");
}

// ------------------------------------------------------- tuned schedules
//
// The schedule autotuner (cuda-exl3 README, "Where the time goes": the best
// tile tier depends on the shape, so the kernel times the tiers once per
// shape and caches the winner, skipped under graph capture, with the cost
// model as the fallback).  Every candidate here is a schedule of the same
// shape-fixed part tree, so no choice changes a result bit.  Key: the shape
// and the M bucket (the next power of two >= M).

struct TuneKey {
  int32_t K, N, bits, codebook, n_shards, mb;
  int32_t shard_n[EXL3_MAX_SHARDS];
  bool operator<(const TuneKey &o) const { return std::memcmp(this, &o, sizeof(TuneKey)) < 0; }
};

std::mutex g_tune_mu;
std::map<TuneKey, exl3_plan> g_tuned;

int32_t m_bucket(int32_t M) {
  int32_t b = 1;
  while (b < M && b < (1 << 30)) b <<= 1;
  return b;
}

TuneKey tune_key(const exl3_weight *w, int32_t M) {
  TuneKey k;
  std::memset(&k, 0, sizeof k);
  k.K = w->K;
  k.N = w->N;
  k.bits = w->bits;
  k.codebook = w->codebook;
  k.n_shards = w->n_shards;
  k.mb = m_bucket(M);
  for (int s = 0; s < w->n_shards && s < EXL3_MAX_SHARDS; ++s) k.shard_n[s] = w->shard_n[s];
  return k;
}

// The plan a call runs: the forced one; else the tuned one for the shape and
// M bucket if it is valid at this M; else the planner's.
exl3_status plan_for(const exl3_weight *w, int32_t M, const exl3_plan *force, Plan *out) {
  if (force) return make_plan(w, M, force, out);
  exl3_plan tuned;
  bool have = false;
  {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    auto it = g_tuned.find(tune_key(w, M));
    if (it != g_tuned.end()) {
      tuned = it->second;
      have = true;
    }
  }
  if (have && make_plan(w, M, &tuned, out) == EXL3_OK) return EXL3_OK;
  return make_plan(w, M, nullptr, out);
}

bool same_schedule(const Plan &a, const Plan &b) {
  return a.parts == b.parts && a.groups == b.groups && a.mode == b.mode && a.bm == b.bm && a.decoder == b.decoder &&
         a.unit == b.unit && a.quads == b.quads && a.half == b.half && a.multi == b.multi &&
         a.finisher == b.finisher && a.chunk == b.chunk;
}

exl3_plan as_force(const Plan &pl) {
  exl3_plan f;
  f.parts = pl.parts;
  f.groups = pl.groups;
  f.mode = pl.mode;
  f.bm = pl.bm;
  f.decoder = pl.decoder;
  f.unit = pl.unit;
  f.launches = 0;
  f.wg_cols = pl.half ? 64 : 128;
  f.workspace = 0;
  return f;
}

// Candidate schedules for M rows: the planner's, then every valid mix of
// decoder, rows per tile (the planner's tier, one and two below, one above),
// mode, unit and workgroup width, without repeats.
std::vector<Plan> tune_candidates(const exl3_weight *w, int32_t M) {
  std::vector<Plan> out;
  Plan base;
  if (make_plan(w, M, nullptr, &base) != EXL3_OK) return out;
  out.push_back(base);
  auto add = [&](const exl3_plan &f) {
    Plan pl;
    if (make_plan(w, M, &f, &pl) != EXL3_OK) return;
    for (const Plan &q : out)
      if (same_schedule(q, pl)) return;
    out.push_back(pl);
  };
  std::vector<int32_t> bms;
  for (int32_t b : {base.bm / 4, base.bm / 2, base.bm, base.bm * 2})
    if (b >= 16 && b <= 512) bms.push_back(b);
  const int32_t decoders[] = {EXL3_DECODER_ALU, EXL3_DECODER_TABLE, EXL3_DECODER_DENSE};
  for (int32_t dec : decoders) {
    if (dec == EXL3_DECODER_DENSE && M < 256) continue;
    for (int32_t bm : bms) {
      if (dec != EXL3_DECODER_ALU && bm != bms[0]) continue;  // those decoders fix their own tile
      for (int32_t mode : {EXL3_MODE_AUTO, EXL3_MODE_FUSED, EXL3_MODE_SLABS})
        for (int32_t unit : {-1, 1})
          for (int32_t cols : {-1, 64}) {
            exl3_plan f;
            f.parts = base.parts;
            f.groups = base.groups;
            f.mode = mode;
            f.bm = dec == EXL3_DECODER_ALU ? bm : -1;
            f.decoder = dec;
            f.unit = unit;
            f.launches = 0;
            f.wg_cols = cols;
            f.workspace = 0;
            add(f);
          }
    }
  }
  return out;
}

}  // namespace

extern "C" {

int32_t exl3_abi_version(void) { return EXL3_ABI_VERSION; }

const char *exl3_status_str(exl3_status s) {
  switch (s) {
    case EXL3_OK: return "EXL3_OK";
    case EXL3_ERR_INVALID_ARG: return "EXL3_ERR_INVALID_ARG";
    case EXL3_ERR_UNSUPPORTED: return "EXL3_ERR_UNSUPPORTED";
    case EXL3_ERR_WORKSPACE: return "EXL3_ERR_WORKSPACE";
    case EXL3_ERR_LAUNCH: return "EXL3_ERR_LAUNCH";
  }
  return "EXL3_ERR_UNKNOWN";
}

const char *exl3_last_error(void) { return g_last_error; }

exl3_status exl3_input_transform(const void *x, int32_t x_dtype, int32_t M, int32_t K, const uint16_t *suh,
                                 int32_t n_shards, uint16_t *x_rot, void *stream) {
  return input_transform_checked(x, x_dtype, false, M, K, suh, n_shards, x_rot, stream);
}

exl3_status exl3_input_transform_swiglu(const void *gate_up, int32_t dtype, int32_t M, int32_t K,
                                        const uint16_t *suh, int32_t n_shards, uint16_t *x_rot, void *stream) {
  return input_transform_checked(gate_up, dtype, true, M, K, suh, n_shards, x_rot, stream);
}

size_t exl3_workspace_bytes_ex(const exl3_weight *w, int32_t M, const exl3_plan *force) {
  clear_error();
  if (validate_weight(w, false, false) != EXL3_OK) return 0;
  if (M < 0 || M > MAX_M) {
    fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 0..%d", M, MAX_M);
    return 0;
  }
  Plan pl;
  if (plan_for(w, M, force, &pl) != EXL3_OK) return 0;
  return pl.workspace;
}

size_t exl3_workspace_bytes(const exl3_weight *w, int32_t M) { return exl3_workspace_bytes_ex(w, M, nullptr); }

exl3_status exl3_plan_query(const exl3_weight *w, int32_t M, exl3_plan *plan) {
  return exl3_plan_query_ex(w, M, nullptr, plan);
}

exl3_status exl3_plan_query_ex(const exl3_weight *w, int32_t M, const exl3_plan *force, exl3_plan *plan) {
  clear_error();
  exl3_status st = validate_weight(w, false, false);
  if (st != EXL3_OK) return st;
  if (plan == nullptr) return fail(EXL3_ERR_INVALID_ARG, "plan (host output) is NULL");
  if (M < 0 || M > MAX_M) return fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 0..%d", M, MAX_M);
  Plan pl;
  if ((st = plan_for(w, M, force, &pl)) != EXL3_OK) return st;
  plan->parts = pl.parts;
  plan->groups = pl.groups;
  plan->mode = pl.mode;
  plan->bm = pl.bm;
  plan->decoder = pl.decoder;
  plan->unit = pl.unit;
  plan->launches = pl.launches;
  plan->wg_cols = pl.half ? 64 : 128;
  plan->workspace = pl.workspace;
  return EXL3_OK;
}

exl3_status exl3_linear_ex(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                           void *workspace, size_t workspace_bytes, void *stream, const exl3_plan *force) {
  clear_error();
  exl3_status st = validate_weight(w, true, false);
  if (st != EXL3_OK) return st;
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "y_dtype=%d, must be 0 (fp16) or 1 (bf16)", y_dtype);
  if (M < 0) return fail(EXL3_ERR_INVALID_ARG, "M=%d is negative", M);
  if (M > MAX_M) return fail(EXL3_ERR_UNSUPPORTED, "M=%d exceeds the supported %d", M, MAX_M);
  Plan pl;
  if ((st = plan_for(w, M, force, &pl)) != EXL3_OK) return st;
  if (M == 0) return EXL3_OK;
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
  if (pl.workspace > 0) {
    if (workspace == nullptr || workspace_bytes < pl.workspace)
      return fail(EXL3_ERR_WORKSPACE, "workspace of %zu bytes at %p; this plan needs %zu (short by %zu)",
                  workspace_bytes, workspace, pl.workspace,
                  pl.workspace > workspace_bytes ? pl.workspace - workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(EXL3_ERR_INVALID_ARG, "workspace=%p is not 16-byte aligned", workspace);
  }

  uint32_t *counters = static_cast<uint32_t *>(workspace);
  float *slabs = pl.workspace > 0 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.slab_off) : nullptr;
  uint16_t *dense =
      pl.decoder == EXL3_DECODER_DENSE ? reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + pl.dense_off)
                                       : nullptr;
  return run_linear(w, x_rot, M, y, y_dtype, counters, slabs, dense, pl, (hipStream_t)stream, true);
}

}  // extern "C"

namespace {

// The GEMM stage of a plan, in row chunks of pl.chunk rows: partials to
// `slabs` in slab mode, then, if `with_output` and in slab mode, the ordered
// part sum + output transform (in the GEMM's last workgroup of each tile when
// the plan has the finisher, else as a second kernel).
exl3_status run_linear(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                       uint32_t *counters, float *slabs, uint16_t *dense, const Plan &pl, hipStream_t s,
                       bool with_output, const int32_t *block_expert, int64_t expert_trellis, int32_t n_experts,
                       const void *x_in, bool x_in_bf16, int dense_which) {
  exl3::GemmParams p;
  std::memset(&p, 0, sizeof p);
  p.x_in = static_cast<const uint16_t *>(x_in);
  p.suh_in = w->suh;
  p.x_in_bf16 = x_in_bf16 ? 1 : 0;
  p.block_expert = block_expert;
  p.n_experts = n_experts;
  p.expert_trellis = expert_trellis;
  p.trellis = w->trellis;
  p.x_rot = x_rot;
  p.svh = w->svh;
  p.bias = w->bias;
  p.y = y;
  p.slabs = slabs;
  p.counters = with_output && pl.finisher ? counters : nullptr;
  p.M = M;
  p.K = w->K;
  p.N = w->N;
  p.parts = pl.parts;
  p.unit = pl.unit;
  p.fold_q = pl.parts / pl.groups / pl.unit;  // slabs per group
  p.slab_mode = pl.mode == EXL3_MODE_SLABS ? 1 : 0;
  p.out_bf16 = y_dtype == EXL3_BF16 ? 1 : 0;
  p.n_shards = w->n_shards;
  int32_t end = 0;
  for (int s = 0; s < w->n_shards; ++s) {
    end += w->shard_n[s] / 128;
    p.shard_end_blk[s] = end;
  }
  const int32_t n_units = p.slab_mode ? pl.parts / pl.unit : 1;
  hipError_t e;
  // dense_which: 3 dequantizes into `dense`, then runs both GEMM launches;
  // 1 or 2 (the dense GEMM hook) runs only that launch over `dense` as given
  if (pl.decoder == EXL3_DECODER_DENSE && dense_which == 3) {
    exl3::DecodeParams dp;
    dp.trellis = w->trellis;
    dp.wq = dense;
    dp.K = w->K;
    dp.N = w->N;
    if ((e = exl3::launch_dequant(w->bits, w->codebook, dp, s)) != hipSuccess) return launch_error(e, "dequant launch");
  }
  p.dense = dense;
  for (int32_t r0 = 0; r0 < M; r0 += pl.chunk) {
    p.row_base = r0;
    p.row_end = std::min(M, r0 + pl.chunk);
    if (pl.decoder == EXL3_DECODER_DENSE) {
      // one dimension of tiles (column blocks x 256-row tiles), ordered
      // inside the kernel; units on y
      const int32_t rows = p.row_end - p.row_base;
      const dim3 grid((unsigned)(w->N / 128 * ((rows + 255) / 256)), (unsigned)n_units, 1);
      int cus = 0;
      if ((e = device_cus(&cus)) != hipSuccess) return launch_error(e, "device query");
      const int bulk = pl.multi ? -1 : dense_bulk_tiles(w, rows, n_units, cus);
      e = exl3::launch_gemm_dense(pl.multi, p, grid, bulk, dense_which, s);
      if (e != hipSuccess) return launch_error(e, "dense GEMM launch");
    } else if (pl.decoder == EXL3_DECODER_TABLE) {
      int cus = 0;
      if ((e = device_cus(&cus)) != hipSuccess) return launch_error(e, "device query");
      const int64_t units = (int64_t)(w->N / 128) * n_units;
      const int grid = (int)std::min<int64_t>(cus, units);
      e = exl3::launch_gemm_table(w->bits, w->codebook, p, grid, s);
      if (e != hipSuccess) return launch_error(e, "table GEMM launch");
    } else {
      const dim3 grid((unsigned)(w->N / 128 * (pl.half ? 2 : 1)), (unsigned)n_units,
                      (unsigned)((p.row_end - p.row_base + pl.bm - 1) / pl.bm));
      e = exl3::launch_gemm(w->bits, w->codebook, pl.bm, pl.quads, pl.half, pl.multi, p, grid, s);
      if (e != hipSuccess) return launch_error(e, "trellis GEMM launch");
    }
    if (p.slab_mode && with_output && p.counters == nullptr) {
      e = exl3::launch_epilogue(p.slabs, n_units, p.fold_q, p.row_base, p.row_end, w->N, w->svh, w->bias, y,
                                p.out_bf16 != 0, s);
      if (e != hipSuccess) return launch_error(e, "part-sum epilogue launch");
    }
  }
  return EXL3_OK;
}

}  // namespace

extern "C" {

exl3_status exl3_linear(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                        void *workspace, size_t workspace_bytes, void *stream) {
  return exl3_linear_ex(w, x_rot, M, y, y_dtype, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

// The whole layer in one call: the rotation runs inside the GEMM when the
// plan's kernel is the small-tile kernel, every stage of a quad's K range
// has a stage slot there (one launch, no x~ in memory), and a workgroup's
// share of the rotation is short; otherwise the input transform writes x~
// into the workspace, after the plan's own part.  Every workgroup of a row
// tile rotates that tile's rows over its quads' K ranges again, ahead of
// its first product: at most 16 (row, stage) 128-blocks per quad, i.e. one
// pass of the 16-lane groups of a four-wave quad or two of a two-wave one,
// save more than the separate launch costs (measured at 1 to 64 rows on
// 1024- to 4096-wide layers: about 1.4 us saved at one pass per wave, 0.5
// us at two, break-even at three, a loss from four).
bool rotation_in_gemm(const exl3_weight *w, const Plan &pl, int32_t M) {
  if (pl.decoder != EXL3_DECODER_ALU || pl.bm > 64) return false;
  const int64_t kb = w->K / 128;
  const int64_t parts_per_quad = pl.quads > 1 ? 1 : pl.unit;
  const int64_t stages = (parts_per_quad * kb + pl.parts - 1) / pl.parts;  // the longest quad's
  if (stages > exl3::small_tile_slots(w->bits, pl.bm / 16, pl.half ? 2 : 4, pl.quads)) return false;
  return std::min<int64_t>(pl.bm, M) * stages <= 16;
}

// x_rot goes after everything the plan uses and never inside the arrival
// counters, which stay zero between calls even where the plan needs none.
size_t forward_x_rot_offset(const Plan &pl) {
  return (std::max(pl.workspace, (size_t)EXL3_WORKSPACE_COUNTER_BYTES) + 255) & ~(size_t)255;
}

size_t forward_workspace(const exl3_weight *w, int32_t M, const Plan &pl) {
  if (M == 0 || rotation_in_gemm(w, pl, M)) return pl.workspace;
  return forward_x_rot_offset(pl) + (size_t)w->n_shards * (size_t)M * (size_t)w->K * 2;
}

}  // namespace

extern "C" {

size_t exl3_forward_workspace_bytes(const exl3_weight *w, int32_t M) {
  clear_error();
  if (validate_weight(w, false, false) != EXL3_OK) return 0;
  if (M < 0 || M > MAX_M) {
    fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 0..%d", M, MAX_M);
    return 0;
  }
  Plan pl;
  if (plan_for(w, M, nullptr, &pl) != EXL3_OK) return 0;
  return forward_workspace(w, M, pl);
}

exl3_status exl3_forward(const exl3_weight *w, const void *x, int32_t x_dtype, int32_t M, void *y, int32_t y_dtype,
                         void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  exl3_status st = validate_weight(w, true, true);
  if (st != EXL3_OK) return st;
  if (x_dtype != EXL3_F16 && x_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "x_dtype=%d, must be 0 (fp16) or 1 (bf16)", x_dtype);
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "y_dtype=%d, must be 0 (fp16) or 1 (bf16)", y_dtype);
  if (M < 0) return fail(EXL3_ERR_INVALID_ARG, "M=%d is negative", M);
  if (M > MAX_M) return fail(EXL3_ERR_UNSUPPORTED, "M=%d exceeds the supported %d", M, MAX_M);
  Plan pl;
  if ((st = plan_for(w, M, nullptr, &pl)) != EXL3_OK) return st;
  if (M == 0) return EXL3_OK;
  if ((st = check_ptr(x, "x")) != EXL3_OK) return st;
  if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
  const size_t need = forward_workspace(w, M, pl);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(EXL3_ERR_WORKSPACE, "workspace of %zu bytes at %p; this call needs %zu (short by %zu)",
                  workspace_bytes, workspace, need, need > workspace_bytes ? need - workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(EXL3_ERR_INVALID_ARG, "workspace=%p is not 16-byte aligned", workspace);
  }
  uint32_t *counters = static_cast<uint32_t *>(workspace);
  float *slabs = pl.workspace > 0 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.slab_off) : nullptr;
  uint16_t *dense =
      pl.decoder == EXL3_DECODER_DENSE ? reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + pl.dense_off)
                                       : nullptr;
  const hipStream_t s = (hipStream_t)stream;
  if (rotation_in_gemm(w, pl, M))
    return run_linear(w, nullptr, M, y, y_dtype, counters, slabs, dense, pl, s, true, nullptr, 0, 0, x,
                      x_dtype == EXL3_BF16);
  uint16_t *x_rot = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + forward_x_rot_offset(pl));
  const hipError_t e = exl3::launch_input_transform(x, x_dtype == EXL3_BF16, false, M, w->K, w->suh, w->n_shards,
                                                    x_rot, s);
  if (e != hipSuccess) return launch_error(e, "input transform launch");
  return run_linear(w, x_rot, M, y, y_dtype, counters, slabs, dense, pl, s, true);
}

size_t exl3_tune_workspace_bytes(const exl3_weight *w, int32_t M) {
  clear_error();
  if (validate_weight(w, false, false) != EXL3_OK) return 0;
  if (M < 1 || M > MAX_M) {
    fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 1..%d", M, MAX_M);
    return 0;
  }
  size_t need = 0;
  for (const Plan &pl : tune_candidates(w, M)) need = std::max(need, pl.workspace);
  clear_error();  // candidates the planner refuses are skipped, not errors
  return need;
}

exl3_status exl3_tune_set(const exl3_weight *w, int32_t M, const exl3_plan *plan) {
  clear_error();
  exl3_status st = validate_weight(w, false, false);
  if (st != EXL3_OK) return st;
  if (plan == nullptr) return fail(EXL3_ERR_INVALID_ARG, "plan is NULL");
  if (M < 1 || M > MAX_M) return fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 1..%d", M, MAX_M);
  Plan pl, base;
  if ((st = make_plan(w, M, plan, &pl)) != EXL3_OK) return st;
  if ((st = make_plan(w, M, nullptr, &base)) != EXL3_OK) return st;
  if (pl.parts != base.parts || pl.groups != base.groups)
    return fail(EXL3_ERR_INVALID_ARG, "a tuned schedule keeps the shape's tree: parts=%d groups=%d, the shape has %d/%d",
                pl.parts, pl.groups, base.parts, base.groups);
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tuned[tune_key(w, M)] = as_force(pl);
  return EXL3_OK;
}

void exl3_tune_clear(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tuned.clear();
}

exl3_status exl3_tune(const exl3_weight *ws, int32_t n_w, const uint16_t *x_rot, int32_t M, void *y,
                      int32_t y_dtype, void *workspace, size_t workspace_bytes, int32_t reps, void *stream,
                      exl3_plan *best) {
  clear_error();
  if (ws == nullptr) return fail(EXL3_ERR_INVALID_ARG, "weight views are NULL");
  if (n_w < 1 || n_w > 65536) return fail(EXL3_ERR_INVALID_ARG, "n_w=%d, must be 1..65536", n_w);
  const exl3_weight *w = ws;
  exl3_status st = validate_weight(w, true, false);
  if (st != EXL3_OK) return st;
  for (int32_t c = 1; c < n_w; ++c) {
    if ((st = validate_weight(&ws[c], true, false)) != EXL3_OK) return st;
    bool same = ws[c].K == w->K && ws[c].N == w->N && ws[c].bits == w->bits && ws[c].codebook == w->codebook &&
                ws[c].n_shards == w->n_shards;
    for (int s = 0; same && s < w->n_shards; ++s) same = ws[c].shard_n[s] == w->shard_n[s];
    if (!same) return fail(EXL3_ERR_INVALID_ARG, "weight copy %d has another shape than copy 0", c);
  }
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "y_dtype=%d, must be 0 (fp16) or 1 (bf16)", y_dtype);
  if (M < 1 || M > MAX_M) return fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 1..%d", M, MAX_M);
  if (reps < 1 || reps > 1000) return fail(EXL3_ERR_INVALID_ARG, "reps=%d, must be 1..1000", reps);
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
  if (workspace != nullptr && !aligned16(workspace))
    return fail(EXL3_ERR_INVALID_ARG, "workspace=%p is not 16-byte aligned", workspace);
  const hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess || cap != hipStreamCaptureStatusNone)
    return fail(EXL3_ERR_UNSUPPORTED, "cannot tune while the stream is being captured (it times with events and "
                "synchronizes); tune in eager warm-up, then capture");
  std::vector<Plan> cands = tune_candidates(w, M);
  clear_error();
  if (cands.empty()) return fail(EXL3_ERR_INVALID_ARG, "no schedule for this shape");
  hipEvent_t e0, e1;
  if ((e = hipEventCreate(&e0)) != hipSuccess) return launch_error(e, "event create");
  if ((e = hipEventCreate(&e1)) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return launch_error(e, "event create");
  }
  uint32_t *counters = static_cast<uint32_t *>(workspace);
  // Two passes over the candidates (each keeps its faster pass, so a clock
  // or cache drift during one pass does not decide), each timing at least
  // `reps` calls and at least 2 ms.
  std::vector<float> per_call(cands.size(), -1.f);
  for (int pass = 0; pass < 2 && st == EXL3_OK; ++pass) {
    for (size_t i = 0; i < cands.size(); ++i) {
      const Plan &pl = cands[i];
      if (pl.workspace > 0 && (workspace == nullptr || workspace_bytes < pl.workspace)) continue;
      float *slabs =
          pl.workspace > 0 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.slab_off) : nullptr;
      uint16_t *dense = pl.decoder == EXL3_DECODER_DENSE
                            ? reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + pl.dense_off)
                            : nullptr;
      auto timed = [&](int n, float *ms) -> exl3_status {
        if ((e = hipEventRecord(e0, s)) != hipSuccess) return launch_error(e, "event record");
        exl3_status r = EXL3_OK;
        for (int k = 0; k < n && r == EXL3_OK; ++k)
          r = run_linear(&ws[(k + 1) % n_w], x_rot, M, y, y_dtype, counters, slabs, dense, pl, s, true);
        if (r != EXL3_OK) return r;
        if ((e = hipEventRecord(e1, s)) != hipSuccess || (e = hipEventSynchronize(e1)) != hipSuccess)
          return launch_error(e, "event wait");
        if ((e = hipEventElapsedTime(ms, e0, e1)) != hipSuccess) return launch_error(e, "event time");
        return EXL3_OK;
      };
      float ms1 = 0.f, ms = 0.f;
      // one untimed call, one timed call to size the batch, then the batch
      if ((st = run_linear(w, x_rot, M, y, y_dtype, counters, slabs, dense, pl, s, true)) != EXL3_OK) break;
      if ((st = timed(1, &ms1)) != EXL3_OK) break;
      const int n = std::min(1000, std::max(reps, (int)(2.0f / std::max(ms1, 1e-4f)) + 1));
      if ((st = timed(n, &ms)) != EXL3_OK) break;
      const float t = ms / n;
      if (per_call[i] < 0.f || t < per_call[i]) per_call[i] = t;
    }
  }
  int best_i = -1;
  for (size_t i = 0; i < cands.size(); ++i)
    if (per_call[i] >= 0.f && (best_i < 0 || per_call[i] < per_call[best_i])) best_i = (int)i;
  const float base_ms = per_call[0], best_ms = best_i >= 0 ? per_call[best_i] : 0.f;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != EXL3_OK) return st;
  if (best_i < 0)
    return fail(EXL3_ERR_WORKSPACE, "no candidate schedule fits the %zu-byte workspace (exl3_tune_workspace_bytes "
                "gives the size that fits all)", workspace_bytes);
  // keep the planner's schedule unless a candidate beats it by more than 2%
  if (best_i != 0 && base_ms > 0.f && best_ms > 0.98f * base_ms) best_i = 0;
  const Plan &win = cands[best_i];
  {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tuned[tune_key(w, M)] = as_force(win);
  }
  if (best) {
    *best = as_force(win);
    best->launches = win.launches;
    best->workspace = win.workspace;
  }
  return EXL3_OK;
}

// ------------------------------------------------------ mixture of experts

int32_t exl3_moe_rows_max(int32_t T, int32_t topk, int32_t E, int32_t block) {
  if (T < 0 || topk < 1 || E < 1 || block < 1) return 0;
  const int64_t pairs = (int64_t)T * topk;
  const int64_t rows = pairs + std::min<int64_t>(E, pairs) * (block - 1);
  const int64_t r = (rows + block - 1) / block * block;
  return r > MAX_M ? 0 : (int32_t)r;
}

exl3_status exl3_moe_align(const int32_t *topk_ids, int32_t T, int32_t topk, int32_t E, int32_t block,
                           int32_t *row_pair, int32_t *block_expert, int32_t *pair_row, void *stream) {
  clear_error();
  if (T < 0 || topk < 1 || topk > 64) return fail(EXL3_ERR_INVALID_ARG, "T=%d topk=%d: T >= 0, topk 1..64", T, topk);
  if (E < 1 || E > 4096) return fail(EXL3_ERR_INVALID_ARG, "E=%d experts, must be 1..4096", E);
  if (block != 16 && block != 32 && block != 64)
    return fail(EXL3_ERR_INVALID_ARG, "block=%d rows, must be 16, 32 or 64 (a tile of the grouped GEMM)", block);
  const int32_t rows = exl3_moe_rows_max(T, topk, E, block);
  if (T > 0 && rows == 0)
    return fail(EXL3_ERR_UNSUPPORTED, "%d tokens x %d experts each need more than %d routed rows", T, topk, MAX_M);
  if (T == 0) return EXL3_OK;
  exl3_status st;
  if ((st = check_ptr(topk_ids, "topk_ids")) != EXL3_OK) return st;
  if ((st = check_ptr(row_pair, "row_pair")) != EXL3_OK) return st;
  if ((st = check_ptr(block_expert, "block_expert")) != EXL3_OK) return st;
  if ((st = check_ptr(pair_row, "pair_row")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_moe_align(topk_ids, T * topk, E, block, rows, row_pair, block_expert, pair_row,
                                              (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "moe align launch");
}

exl3_status exl3_moe_input_transform(const void *x, int32_t x_dtype, int32_t swiglu, int32_t T, int32_t K,
                                     const uint16_t *suh, int32_t n_shards, int32_t E, const int32_t *row_pair,
                                     const int32_t *block_expert, int32_t topk, int32_t block, int32_t rows,
                                     uint16_t *x_rot, void *stream) {
  clear_error();
  if (x_dtype != EXL3_F16 && x_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "x_dtype=%d, must be 0 (fp16) or 1 (bf16)", x_dtype);
  if (K <= 0 || K % 128 != 0 || K > MAX_KN)
    return fail(EXL3_ERR_INVALID_ARG, "K=%d must be a positive multiple of 128 up to %d", K, MAX_KN);
  if (n_shards < 1 || n_shards > EXL3_MAX_SHARDS)
    return fail(EXL3_ERR_INVALID_ARG, "n_shards=%d, must be 1..%d", n_shards, EXL3_MAX_SHARDS);
  if (E < 1 || E > 4096) return fail(EXL3_ERR_INVALID_ARG, "E=%d experts, must be 1..4096", E);
  if (block != 16 && block != 32 && block != 64) return fail(EXL3_ERR_INVALID_ARG, "block=%d, must be 16, 32 or 64", block);
  if (T < 0 || topk < 1) return fail(EXL3_ERR_INVALID_ARG, "T=%d topk=%d", T, topk);
  if (rows != exl3_moe_rows_max(T, topk, E, block))
    return fail(EXL3_ERR_INVALID_ARG, "rows=%d, the routed buffers of %d tokens x %d of %d experts in blocks of %d "
                "have %d", rows, T, topk, E, block, exl3_moe_rows_max(T, topk, E, block));
  if (T == 0) return EXL3_OK;
  exl3_status st;
  if ((st = check_ptr(x, "x")) != EXL3_OK) return st;
  if ((st = check_ptr(suh, "suh")) != EXL3_OK) return st;
  if ((st = check_ptr(row_pair, "row_pair")) != EXL3_OK) return st;
  if ((st = check_ptr(block_expert, "block_expert")) != EXL3_OK) return st;
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_input_transform(x, x_dtype == EXL3_BF16, swiglu != 0, rows, K, suh, n_shards,
                                                    x_rot, (hipStream_t)stream, row_pair, block_expert, topk, block, E);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "moe input transform launch");
}

}  // extern "C"

namespace {
// The grouped GEMM's plan: the shape's own tree on the ALU tiles with
// block-row tiles, with the output stage in the GEMM (fused, or the
// finishing workgroup): a separate output kernel would need each block's
// svh.
// Grouped calls on the table decoder: one fused unit per (16-row block,
// column block), the expert shape's own part tree folded in two levels in
// the kernel, no workspace.
exl3_status run_moe_table(const exl3_weight *w, int32_t E, const uint16_t *x_rot, int32_t rows,
                          const int32_t *block_expert, void *y, int32_t y_dtype, hipStream_t s) {
  exl3::GemmParams p;
  std::memset(&p, 0, sizeof p);
  const int32_t G = choose_groups(w->K, w->N, w->bits);
  const int32_t P = G * choose_q(w->K, w->N, G);
  p.trellis = w->trellis;
  p.x_rot = x_rot;
  p.svh = w->svh;
  p.bias = w->bias;
  p.y = y;
  p.M = rows;
  p.row_base = 0;
  p.row_end = rows;
  p.K = w->K;
  p.N = w->N;
  p.parts = P;
  p.unit = P;
  p.fold_q = P / G;  // parts per group
  p.slab_mode = 0;
  p.out_bf16 = y_dtype == EXL3_BF16 ? 1 : 0;
  p.n_shards = w->n_shards;
  int32_t end = 0;
  for (int i = 0; i < w->n_shards; ++i) {
    end += w->shard_n[i] / 128;
    p.shard_end_blk[i] = end;
  }
  p.block_expert = block_expert;
  p.n_experts = E;
  p.expert_trellis = (int64_t)w->K / 16 * (w->N / 16) * 16 * w->bits;
  int cus = 0;
  hipError_t e;
  if ((e = device_cus(&cus)) != hipSuccess) return launch_error(e, "device query");
  const int64_t units = (int64_t)(rows / 16) * (w->N / 128);
  const int grid = (int)std::min<int64_t>(cus, units);
  e = exl3::launch_gemm_table(w->bits, w->codebook, p, grid, s);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "grouped table GEMM launch");
}

exl3_status moe_plan(const exl3_weight *w, int32_t rows, int32_t block, Plan *pl) {
  exl3_plan f;
  f.parts = -1;
  f.groups = -1;
  f.mode = EXL3_MODE_AUTO;
  f.bm = block;
  f.decoder = EXL3_DECODER_ALU;
  f.unit = -1;
  f.launches = 0;
  f.wg_cols = -1;
  f.workspace = 0;
  exl3_status st = make_plan(w, rows, &f, pl);
  if (st != EXL3_OK) return st;
  if (pl->mode == EXL3_MODE_SLABS && !pl->finisher) {
    f.mode = EXL3_MODE_FUSED;
    if (make_plan(w, rows, &f, pl) != EXL3_OK)
      return fail(EXL3_ERR_UNSUPPORTED, "%d routed rows in blocks of %d: more tiles than the finishing counters "
                  "hold and no fused schedule for this tree; route fewer rows per call", rows, block);
  }
  return EXL3_OK;
}
}  // namespace

extern "C" {

size_t exl3_moe_workspace_bytes(const exl3_weight *w, int32_t rows, int32_t block) {
  clear_error();
  if (validate_weight(w, false, false) != EXL3_OK) return 0;
  if (rows < 0 || rows > MAX_M || (block != 16 && block != 32 && block != 64) || rows % block != 0) {
    fail(EXL3_ERR_INVALID_ARG, "rows=%d block=%d: rows a multiple of block (16, 32 or 64)", rows, block);
    return 0;
  }
  Plan pl;
  if (moe_plan(w, rows, block, &pl) != EXL3_OK) return 0;
  return pl.workspace;
}

exl3_status exl3_moe_linear(const exl3_weight *w, int32_t E, const uint16_t *x_rot, int32_t rows,
                            const int32_t *block_expert, int32_t block, void *y, int32_t y_dtype, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return exl3_moe_linear_ex(w, E, x_rot, rows, block_expert, block, y, y_dtype, workspace, workspace_bytes, stream,
                            EXL3_DECODER_AUTO);
}

exl3_status exl3_moe_linear_ex(const exl3_weight *w, int32_t E, const uint16_t *x_rot, int32_t rows,
                               const int32_t *block_expert, int32_t block, void *y, int32_t y_dtype, void *workspace,
                               size_t workspace_bytes, void *stream, int32_t decoder) {
  clear_error();
  exl3_status st = validate_weight(w, true, true);
  if (st != EXL3_OK) return st;
  if (E < 1 || E > 4096) return fail(EXL3_ERR_INVALID_ARG, "E=%d experts, must be 1..4096", E);
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "y_dtype=%d, must be 0 (fp16) or 1 (bf16)", y_dtype);
  if (block != 16 && block != 32 && block != 64) return fail(EXL3_ERR_INVALID_ARG, "block=%d, must be 16, 32 or 64", block);
  if (rows < 0 || rows > MAX_M || rows % block != 0)
    return fail(EXL3_ERR_INVALID_ARG, "rows=%d must be a multiple of block=%d (remainder %d)", rows, block,
                rows >= 0 ? rows % block : rows);
  if (decoder != EXL3_DECODER_AUTO && decoder != EXL3_DECODER_ALU && decoder != EXL3_DECODER_TABLE)
    return fail(EXL3_ERR_INVALID_ARG, "decoder=%d, must be -1 (auto), 0 (alu) or 1 (table)", decoder);
  const double stack_bytes = (double)E * w->K * (double)w->N * w->bits / 8.0;
  if (decoder == EXL3_DECODER_TABLE && block != 16)
    return fail(EXL3_ERR_UNSUPPORTED, "the grouped table decoder takes 16-row blocks; block=%d", block);
  if (decoder == EXL3_DECODER_TABLE && stack_bytes > TABLE_MAX_TRELLIS_BYTES)
    return fail(EXL3_ERR_UNSUPPORTED, "the table decoder reads at most %.0f trellis bytes; %d experts hold %.0f",
                TABLE_MAX_TRELLIS_BYTES, E, stack_bytes);
  const int64_t table_units = (int64_t)(rows / 16) * (w->N / 128);
  const bool use_table = decoder == EXL3_DECODER_TABLE ||
                         (decoder == EXL3_DECODER_AUTO && block == 16 && stack_bytes <= TABLE_MAX_TRELLIS_BYTES &&
                          table_units >= MOE_TABLE_MIN_UNITS);
  if (use_table) {
    if (rows == 0) return EXL3_OK;
    if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
    if ((st = check_ptr(block_expert, "block_expert")) != EXL3_OK) return st;
    if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
    return run_moe_table(w, E, x_rot, rows, block_expert, y, y_dtype, (hipStream_t)stream);
  }
  Plan pl;
  if ((st = moe_plan(w, rows, block, &pl)) != EXL3_OK) return st;
  if (rows == 0) return EXL3_OK;
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  if ((st = check_ptr(block_expert, "block_expert")) != EXL3_OK) return st;
  if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
  if (pl.workspace > 0) {
    if (workspace == nullptr || workspace_bytes < pl.workspace)
      return fail(EXL3_ERR_WORKSPACE, "workspace of %zu bytes; this plan needs %zu (short by %zu)", workspace_bytes,
                  pl.workspace, pl.workspace > workspace_bytes ? pl.workspace - workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(EXL3_ERR_INVALID_ARG, "workspace=%p is not 16-byte aligned", workspace);
  }
  uint32_t *counters = static_cast<uint32_t *>(workspace);
  float *slabs = pl.workspace > 0 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.slab_off) : nullptr;
  const int64_t expert_words = (int64_t)w->K / 16 * (w->N / 16) * 16 * w->bits;
  return run_linear(w, x_rot, rows, y, y_dtype, counters, slabs, nullptr, pl, (hipStream_t)stream, true, block_expert,
                    expert_words, E);
}

exl3_status exl3_moe_combine(const void *y_routed, int32_t dtype, const int32_t *pair_row, const float *topk_weights,
                             int32_t T, int32_t topk, int32_t N, void *out, void *stream) {
  clear_error();
  if (dtype != EXL3_F16 && dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "dtype=%d, must be 0 (fp16) or 1 (bf16)", dtype);
  if (T < 0 || topk < 1 || topk > 64) return fail(EXL3_ERR_INVALID_ARG, "T=%d topk=%d: T >= 0, topk 1..64", T, topk);
  if (N <= 0 || N % 2 != 0) return fail(EXL3_ERR_INVALID_ARG, "N=%d must be positive and even", N);
  if (T == 0) return EXL3_OK;
  exl3_status st;
  if ((st = check_ptr(y_routed, "y_routed")) != EXL3_OK) return st;
  if ((st = check_ptr(pair_row, "pair_row")) != EXL3_OK) return st;
  if ((st = check_ptr(topk_weights, "topk_weights")) != EXL3_OK) return st;
  if ((st = check_ptr(out, "out")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_moe_combine(y_routed, dtype == EXL3_BF16, pair_row, topk_weights, T, topk, N, out,
                                                (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "moe combine launch");
}

exl3_status exl3_debug_parts(const exl3_weight *w, const uint16_t *x_rot, int32_t M, float *z_parts,
                             size_t z_bytes, void *stream, const exl3_plan *force) {
  clear_error();
  exl3_status st = validate_weight(w, true, false);
  if (st != EXL3_OK) return st;
  if (M < 0) return fail(EXL3_ERR_INVALID_ARG, "M=%d is negative", M);
  if (M > MAX_M) return fail(EXL3_ERR_UNSUPPORTED, "M=%d exceeds the supported %d", M, MAX_M);
  exl3_plan f;
  if (force) f = *force;
  else {
    f.parts = -1;
    f.groups = -1;
    f.bm = -1;
    f.decoder = EXL3_DECODER_AUTO;
    f.unit = -1;
    f.launches = 0;
    f.wg_cols = -1;
    f.workspace = 0;
  }
  f.mode = EXL3_MODE_SLABS;
  if (f.unit <= 0) f.unit = 1;  // one slab per part unless asked otherwise
  Plan pl;
  if ((st = make_plan(w, M, &f, &pl)) != EXL3_OK) return st;
  if (M == 0) return EXL3_OK;
  pl.mode = EXL3_MODE_SLABS;  // also for one part
  pl.unit = pl.parts == 1 ? 1 : pl.unit;
  if (pl.bm == 512 && pl.unit > 1) pl.bm = 256;
  pl.quads = 1;
  pl.multi = pl.unit > 1;
  if (pl.decoder == EXL3_DECODER_ALU && pl.bm <= 64 && (pl.unit == 2 || pl.unit == 4) &&
      (w->K / 128) % pl.parts == 0) {
    pl.quads = pl.unit;
    pl.multi = false;
  }
  pl.chunk = M;
  pl.finisher = false;
  if (pl.decoder == EXL3_DECODER_ALU && (int64_t)M > (int64_t)MAX_GRID_Z * pl.bm)
    return fail(EXL3_ERR_UNSUPPORTED, "the part-sums hook runs one launch: M=%d rows in %d-row tiles exceed %d tiles",
                M, pl.bm, MAX_GRID_Z);
  pl.half = f.wg_cols == 64 && pl.decoder == EXL3_DECODER_ALU && pl.bm <= 64 && !pl.multi;
  const int32_t n_slabs = pl.parts / pl.unit;
  const size_t need = slab_bytes(n_slabs, M, w->N);
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  if ((st = check_ptr(z_parts, "z_parts")) != EXL3_OK) return st;
  if (z_bytes < need)
    return fail(EXL3_ERR_WORKSPACE, "z_parts holds %zu bytes; %d slabs of %d rows need %zu (short by %zu)", z_bytes,
                n_slabs, M, need, need - z_bytes);
  if (pl.decoder == EXL3_DECODER_DENSE)
    return fail(EXL3_ERR_UNSUPPORTED, "the part-sums hook runs the decoding kernels; decoder=dense needs a workspace");
  return run_linear(w, x_rot, M, nullptr, EXL3_BF16, nullptr, z_parts, nullptr, pl, (hipStream_t)stream, false);
}

exl3_status exl3_debug_codebook(int32_t codebook, uint16_t *out, void *stream) {
  clear_error();
  if (codebook < EXL3_CB_3INST || codebook > EXL3_CB_MUL1)
    return fail(EXL3_ERR_INVALID_ARG, "codebook=%d, must be 0..2", codebook);
  exl3_status st;
  if ((st = check_ptr(out, "out")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_debug_codebook(codebook, out, (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "codebook launch");
}

exl3_status exl3_debug_decode(const exl3_weight *w, uint16_t *wq, void *stream) {
  clear_error();
  exl3_status st = validate_weight(w, true, false);
  if (st != EXL3_OK) return st;
  if ((st = check_ptr(wq, "wq")) != EXL3_OK) return st;
  exl3::DecodeParams p;
  p.trellis = w->trellis;
  p.wq = wq;
  p.K = w->K;
  p.N = w->N;
  const hipError_t e = exl3::launch_debug_decode(w->bits, w->codebook, p, (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "decode launch");
}

exl3_status exl3_debug_dequant(const exl3_weight *w, uint16_t *frags, size_t frag_bytes, void *stream) {
  clear_error();
  exl3_status st = validate_weight(w, true, false);
  if (st != EXL3_OK) return st;
  if ((st = check_ptr(frags, "frags")) != EXL3_OK) return st;
  const size_t need = (size_t)w->K * (size_t)w->N * 2;
  if (frag_bytes < need)
    return fail(EXL3_ERR_WORKSPACE, "frags holds %zu bytes; K*N fp16 need %zu (short by %zu)", frag_bytes, need,
                need - frag_bytes);
  exl3::DecodeParams p;
  p.trellis = w->trellis;
  p.wq = frags;
  p.K = w->K;
  p.N = w->N;
  const hipError_t e = exl3::launch_dequant(w->bits, w->codebook, p, (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "dequant launch");
}

exl3_status exl3_debug_dense_gemm(const exl3_weight *w, const uint16_t *frags, size_t frag_bytes,
                                  const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype, int32_t which,
                                  int32_t *bulk_blocks, void *stream) {
  clear_error();
  exl3_status st = validate_weight(w, false, false);
  if (st != EXL3_OK) return st;
  if (which < 1 || which > 3) return fail(EXL3_ERR_INVALID_ARG, "which=%d, must be 1, 2 or 3", which);
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "y_dtype=%d, must be 0 (fp16) or 1 (bf16)", y_dtype);
  if (M < 1 || M > MAX_M) return fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 1..%d", M, MAX_M);
  exl3_plan f;
  f.parts = -1;
  f.groups = -1;
  f.mode = EXL3_MODE_AUTO;
  f.bm = -1;
  f.decoder = EXL3_DECODER_DENSE;
  f.unit = -1;
  f.launches = 0;
  f.wg_cols = -1;
  f.workspace = 0;
  Plan pl;
  if ((st = make_plan(w, M, &f, &pl)) != EXL3_OK) return st;
  if (pl.mode != EXL3_MODE_FUSED || pl.multi || pl.chunk < M)
    return fail(EXL3_ERR_UNSUPPORTED, "the dense GEMM hook runs one-part fused plans in one row chunk (mode=%d "
                "unit=%d chunk=%d)", pl.mode, pl.unit, pl.chunk);
  if ((st = check_ptr(frags, "frags")) != EXL3_OK) return st;
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
  const size_t need = (size_t)w->K * (size_t)w->N * 2;
  if (frag_bytes < need)
    return fail(EXL3_ERR_WORKSPACE, "frags holds %zu bytes; K*N fp16 need %zu (short by %zu)", frag_bytes, need,
                need - frag_bytes);
  int cus = 0;
  const hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return launch_error(e, "device query");
  if (bulk_blocks) *bulk_blocks = dense_tile_first_block(w, dense_bulk_tiles(w, M, 1, cus));
  return run_linear(w, x_rot, M, y, y_dtype, nullptr, nullptr, const_cast<uint16_t *>(frags), pl,
                    (hipStream_t)stream, true, nullptr, 0, 0, nullptr, false, which);
}

exl3_status exl3_debug_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  clear_error();
  exl3_status st;
  if (bytes == 0 || bytes % 16 != 0)
    return fail(EXL3_ERR_INVALID_ARG, "bytes=%zu, must be a positive multiple of 16", bytes);
  if ((st = check_ptr(buf, "buf")) != EXL3_OK) return st;
  if ((st = check_ptr(out, "out")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_stream_read(buf, bytes, out, (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "stream-read launch");
}

exl3_status exl3_debug_mfma_loop(int32_t iters, uint16_t one, float *out, void *stream) {
  clear_error();
  exl3_status st;
  if (iters < 1 || iters > (1 << 20)) return fail(EXL3_ERR_INVALID_ARG, "iters=%d, must be 1..%d", iters, 1 << 20);
  if ((st = check_ptr(out, "out")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_mfma_loop(iters, one, out, (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "mfma-loop launch");
}

exl3_status exl3_debug_decode_rate(const exl3_weight *w, uint32_t *out, void *stream) {
  clear_error();
  exl3_status st = validate_weight(w, true, false);
  if (st != EXL3_OK) return st;
  if ((st = check_ptr(out, "out")) != EXL3_OK) return st;
  exl3::DecodeParams p;
  p.trellis = w->trellis;
  p.wq = reinterpret_cast<uint16_t *>(out);
  p.K = w->K;
  p.N = w->N;
  const hipError_t e = exl3::launch_decode_rate(w->bits, w->codebook, p, (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "decode-rate launch");
}

exl3_status exl3_debug_epilogue(const float *z_parts, int32_t n_parts, int32_t groups, int32_t M,
                                const exl3_weight *w, void *y, int32_t y_dtype, void *stream) {
  clear_error();
  exl3_status st = validate_weight(w, false, false);
  if (st != EXL3_OK) return st;
  if (n_parts < 1 || n_parts > 4096) return fail(EXL3_ERR_INVALID_ARG, "n_parts=%d, must be 1..4096", n_parts);
  if (groups < 1 || n_parts % groups != 0)
    return fail(EXL3_ERR_INVALID_ARG, "groups=%d must be positive and divide n_parts=%d", groups, n_parts);
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "y_dtype=%d, must be 0 (fp16) or 1 (bf16)", y_dtype);
  if (M < 0 || M > MAX_M) return fail(EXL3_ERR_INVALID_ARG, "M=%d out of range 0..%d", M, MAX_M);
  if (M == 0) return EXL3_OK;
  if ((st = check_ptr(z_parts, "z_parts")) != EXL3_OK) return st;
  if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
  const hipError_t e = exl3::launch_epilogue(z_parts, n_parts, n_parts / groups, 0, M, w->N, w->svh, w->bias, y,
                                             y_dtype == EXL3_BF16, (hipStream_t)stream);
  return e == hipSuccess ? EXL3_OK : launch_error(e, "epilogue launch");
}

}  // extern "C"

namespace {

// A schedule of the layer's own part tree (so the same bits as exl3_linear)
// whose workspace fits `bytes`: the planner's when it fits; else, without
// dequantized fragments, partial slabs in row chunks within the space left
// after the counters; else the one-level fused fold where the tree has one;
// else slabs with smaller row tiles.  Every automatic tree fits a few MiB:
// groups that split into parts (the only trees with no fused schedule) come
// with fewer than 512 column-block x group pairs, 8 KB of slabs each per
// 16-row tile.
exl3_status scratch_plan(const exl3_weight *w, int32_t M, size_t bytes, Plan *out) {
  Plan pl;
  exl3_status st = plan_for(w, M, nullptr, &pl);
  if (st != EXL3_OK) return st;
  if (pl.workspace <= bytes) {
    *out = pl;
    return EXL3_OK;
  }
  const Plan want = pl;
  const double cap = (double)bytes - EXL3_WORKSPACE_COUNTER_BYTES;
  exl3_plan f;
  f.parts = want.parts;
  f.groups = want.groups;
  f.mode = EXL3_MODE_AUTO;
  f.bm = -1;
  f.decoder = want.decoder == EXL3_DECODER_DENSE ? EXL3_DECODER_ALU : want.decoder;
  f.unit = -1;
  f.launches = 0;
  f.wg_cols = -1;
  f.workspace = 0;
  auto fits = [&](const exl3_plan &g) { return make_plan(w, M, &g, &pl, cap) == EXL3_OK && pl.workspace <= bytes; };
  bool ok = fits(f);
  if (!ok) {
    f.mode = EXL3_MODE_FUSED;
    ok = fits(f);
  }
  const int32_t tiles[] = {256, 128, 64, 32, 16};
  for (int i = 0; !ok && i < 5; ++i) {
    f.mode = EXL3_MODE_SLABS;
    f.decoder = EXL3_DECODER_ALU;
    f.bm = tiles[i];
    ok = fits(f);
  }
  clear_error();
  if (!ok)
    return fail(EXL3_ERR_UNSUPPORTED,
                "no schedule of this layer's tree (%d parts, %d groups) fits the %zu-byte scratch at M=%d; the "
                "planner's needs %zu (over by %zu)", want.parts, want.groups, bytes, M, want.workspace,
                want.workspace - bytes);
  *out = pl;
  return EXL3_OK;
}

}  // namespace

namespace exl3 {

exl3_status linear_in_scratch(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                              void *scratch, size_t scratch_bytes, void *stream, bool launch) {
  clear_error();
  exl3_status st = validate_weight(w, true, false);
  if (st != EXL3_OK) return st;
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_BF16)
    return fail(EXL3_ERR_INVALID_ARG, "y_dtype=%d, must be 0 (fp16) or 1 (bf16)", y_dtype);
  if (M < 0) return fail(EXL3_ERR_INVALID_ARG, "M=%d is negative", M);
  if (M > MAX_M) return fail(EXL3_ERR_UNSUPPORTED, "M=%d exceeds the supported %d", M, MAX_M);
  Plan pl;
  if ((st = scratch_plan(w, M, scratch_bytes, &pl)) != EXL3_OK) return st;
  if (M == 0) return EXL3_OK;
  if ((st = check_ptr(x_rot, "x_rot")) != EXL3_OK) return st;
  if ((st = check_ptr(y, "y")) != EXL3_OK) return st;
  if (!launch) return EXL3_OK;
  uint32_t *counters = static_cast<uint32_t *>(scratch);
  float *slabs = pl.workspace > 0 ? reinterpret_cast<float *>(static_cast<char *>(scratch) + pl.slab_off) : nullptr;
  uint16_t *dense = pl.decoder == EXL3_DECODER_DENSE
                        ? reinterpret_cast<uint16_t *>(static_cast<char *>(scratch) + pl.dense_off)
                        : nullptr;
  return run_linear(w, x_rot, M, y, y_dtype, counters, slabs, dense, pl, (hipStream_t)stream, true);
}

exl3_status scratch_setup_error(hipError_t e, const char *what) { return launch_error(e, what); }

}  // namespace exl3
