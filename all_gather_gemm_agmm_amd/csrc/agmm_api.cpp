// C ABI, plan and scheduler of the all-gather matmul library (host side).
//
// The plan validates the problem (the tpu-inference page's `validate_inputs`
// raises on malformed inputs; here every rejection is a status code plus a
// message), picks tile shapes and the variant, and owns everything a run
// needs: the staged ring, split-K scratch, tile-order tables, a second
// stream and the events that sequence it.
//
// Staged pipeline (the single-GPU form of the Ascend tutorial's "Double
// Buffering" and "pvalue Parameter" sections): chunk c holds rows
// [c*R, (c+1)*R) of every shard (R = pvalue * tile rows, the last chunk
// clamped), laid out in slot c % nbuf as [num_shards][R][k].  The copy of
// chunk c runs on the plan's copy stream once the GEMM that last read its
// slot has finished (event `free`); the GEMM of chunk c runs on the caller's
// stream once the copy is done (event `ready`).  These two events per slot
// take the place of the tutorial's barrier_all per chunk and of the
// semaphores of the tpu-inference kernel.
//
// Calls on one plan are ordered with each other wherever they are enqueued:
// every call ends by recording the plan's `done` event on the caller's
// stream (after the internal streams have joined it), and the next call's
// stream waits on that event before any of its work, so no call overwrites
// ring slots or split-K partial sums a previous call on another stream is
// still reading (the tutorial's rule that a slot is not refilled before the
// chunk that reads it has been consumed).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "agmm.h"
#include "agmm_kernels.h"

namespace {

thread_local int g_status = AGMM_OK;
thread_local std::string g_msg;

int set_err(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_status = status;
  g_msg = buf;
  return status;
}

int ok() {
  g_status = AGMM_OK;
  g_msg.clear();
  return AGMM_OK;
}

int hip_err(hipError_t e, const char* what) {
  return set_err(AGMM_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

constexpr int64_t kDimLimit = int64_t(1) << 30;
// automatic transposed copy of B (stored k x n) from this many rows of m
constexpr int64_t kBtMinRows = 24576;
constexpr int kTimingPairs = 4096;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t elem_bytes(int dtype) { return dtype == AGMM_FP32 ? 4 : 2; }

int validate(int N, int64_t m_s, int64_t k, int64_t n, int dtype, int rt) {
  if (N < 1) return set_err(AGMM_ERR_INVALID_ARG, "num_shards must be >= 1 (got %d)", N);
  if (N > agmm::kMaxGroups)
    return set_err(AGMM_ERR_UNSUPPORTED, "num_shards %d exceeds the supported maximum %d", N,
                   agmm::kMaxGroups);
  if (m_s < 1 || k < 1 || n < 1)
    return set_err(AGMM_ERR_INVALID_ARG,
                   "sizes must be >= 1 (m_per_shard=%lld, k=%lld, n_local=%lld)", (long long)m_s,
                   (long long)k, (long long)n);
  if (dtype != AGMM_BF16 && dtype != AGMM_FP16 && dtype != AGMM_FP32)
    return set_err(AGMM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (rt != 0 && rt != 1) return set_err(AGMM_ERR_INVALID_ARG, "rhs_transpose must be 0 or 1");
  const int64_t m = (int64_t)N * m_s;
  if (m >= kDimLimit || k >= kDimLimit || n >= kDimLimit || m * k >= (int64_t(1) << 40) ||
      k * n >= (int64_t(1) << 40) || m * n >= (int64_t(1) << 40))
    return set_err(AGMM_ERR_UNSUPPORTED, "problem too large (m=%lld, k=%lld, n=%lld)",
                   (long long)m, (long long)k, (long long)n);
  return ok();
}

// bf16/fp16 rows that are not whole 16-byte vectors (k, or n for B stored
// k x n, not a multiple of 8) cannot be fed to the vector and direct-to-LDS
// loads: such problems run on zero-padded copies of A and B.
bool needs_pad(int dtype, int64_t k, int64_t n, int rt) {
  return dtype != AGMM_FP32 && (k % 8 != 0 || (!rt && n % 8 != 0));
}

int64_t round8(int64_t x) { return (x + 7) / 8 * 8; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// What the caller can set (agmm_plan_set_int keys).
struct Settings {
  int variant = AGMM_VARIANT_AUTO;
  int pvalue = 2;
  int nbuf = 2;
  int tile = -1;          // -1: automatic
  int splits = 0;         // 0: automatic
  int local_shard = 0;
  int order = 0;
  int group_m = 0;        // 0: chosen per launch shape (pick_group_m)
  int xcd_remap = 1;
  int copy_wgs = 0;
  int skinny_shape = -1;  // tile shape of the skinny kernel; -1 automatic
  int copy_engine = 0;    // copies beside a GEMM: 0 gather kernel (CUs), 1 SDMA engines
  int gather_out = 0;     // agmm_run_gather_out on fused/skinny plans: 0 automatic, 1 side copy, 2 sequential
  int64_t lda = 0, ldb = 0, ldc = 0;   // element strides between rows (0: dense)
  int gemm_streams = 2;   // staged: chunk GEMMs alternate over this many streams (1 or 2)
  int local_first = 0;    // staged: the local shard's rows first, straight from its buffer
  int debug_keep_slots = 0;
  int b_transpose = -1;   // B stored k x n: -1 automatic, 0 never, 1 always transposed per call
};

// Everything derived from the problem and the settings.
struct Layout {
  int variant_used = AGMM_VARIANT_FUSED;
  int tile_used = agmm::kTile256x256;
  int bm = 256, bn = 256;
  int skinny_shape_used = 5;
  // zero-padded operands (needs_pad): the GEMM runs on A [m][kp] in the ring
  // and on B [n][kp] (rhs_transpose) or [kp][np] in its own buffer
  bool padded = false;
  int64_t kp = 0, np = 0;
  // B stored k x n, transposed per call into the B copy: the GEMM then reads
  // B as n x k (its B fragments are single 16-byte LDS reads instead of two
  // transposing reads each)
  bool bt = false;
  size_t padb_bytes = 0;   // the B copy: zero-padded (padded) or transposed (bt)
  int64_t rows_per_chunk = 0;
  int num_chunks = 1;
  int nslots = 0;
  int splits_used = 1;
  int64_t k_per_split = 0;
  size_t slot_bytes = 0, ring_bytes = 0, part_bytes = 0;
  std::vector<int32_t> h_order;     // concatenated per-chunk row-block orders
  std::vector<int64_t> order_off;   // offset of chunk c's table
  std::vector<int32_t> order_len;

  static size_t up(size_t x) { return (x + 255) & ~size_t(255); }
  size_t order_bytes() const { return h_order.size() * sizeof(int32_t); }
  size_t total_bytes() const {
    return up(ring_bytes) + up(part_bytes) + up(padb_bytes) + up(order_bytes());
  }
};

// Where the plan's previous call recorded its `done` event.
enum DoneState { kDoneNone = 0, kDoneEager = 1, kDoneCaptured = 2 };

}  // namespace

struct agmm_plan {
  // problem
  int device = 0;
  int cu_count = 256;
  int N = 0;
  int64_t m_s = 0, k = 0, n = 0, m = 0;
  int dtype = 0;
  int rt = 0;
  Settings s;
  Layout L;
  // device resources: one allocation, 256-byte aligned pieces
  char* ws = nullptr;
  size_t ws_cap = 0;
  char* ring = nullptr;
  float* partials = nullptr;
  char* padb = nullptr;             // B copy: zero-padded (padded layouts) or transposed (bt)
  int32_t* d_order = nullptr;
  // last automatic group_m choice, keyed by the launch's block counts
  int64_t group_key_rb = -1, group_key_cb = -1;
  int group_auto = 4;
  hipStream_t copy_stream = nullptr;
  hipStream_t compute2 = nullptr;   // second GEMM stream: staged chunks alternate
  hipEvent_t ev_entry = nullptr;    // start of a call on the caller's stream
  hipEvent_t ev_side = nullptr;     // end of the copy stream's work
  hipEvent_t ev_c2 = nullptr;       // end of the second GEMM stream's work
  hipEvent_t ev_done = nullptr;     // end of the plan's previous call
  std::vector<hipEvent_t> ev_ready, ev_free;
  // ordering between calls
  int done_state = kDoneNone;
  unsigned long long done_capture_id = 0;
  hipStream_t done_stream = nullptr;
  bool captured = false;            // some call was captured into a graph
  unsigned long long staged_capture_id = 0;   // capture holding a staged call, or 0
  int broken = AGMM_OK;             // status that left the plan unusable, or AGMM_OK
  std::string broken_msg;
  // timing
  bool timing = false;
  std::vector<hipEvent_t> tev;      // 2 * kTimingPairs
  int tev_used = 0;
  std::mutex mu;
};

namespace {

bool is_f32(const agmm_plan* p) { return p->dtype == AGMM_FP32; }

int64_t lda_of(const agmm_plan* p) { return p->s.lda ? p->s.lda : p->k; }
int64_t ldb_of(const agmm_plan* p) { return p->s.ldb ? p->s.ldb : (p->rt ? p->k : p->n); }
int64_t ldc_of(const agmm_plan* p) { return p->s.ldc ? p->s.ldc : p->n; }

// Tile choice for the MFMA path: fewest rounds of workgroups over the CUs,
// weighted by the per-tile efficiency of the larger shapes.
int choose_tile(const agmm_plan* p, const Settings& s, int64_t m, bool bnk) {
  if (s.tile >= 0) return s.tile;
  struct Cand { int cfg; double eff; };
  // The 256x256 and 128x128 tiles run as the 64-deep part ring on 16x16x32
  // MFMAs unless k is short (its k-tiles would then be mostly padding).
  const bool deep = p->k >= 256;
  const int big = deep ? agmm::kTile256x256m16 : agmm::kTile256x256;
  const int small = deep ? agmm::kTile128x128m16 : agmm::kTile128x128;
  // 256x224 (B stored n x k only): 12.5% less work per tile, for launches
  // whose 256x256 tiles leave a partial last round that 224-column tiles fill
  // (8192 x 3584: 448 tiles, 1.75 rounds of 256 CUs, against 512 tiles, 2
  // rounds); on a tie the 256x256 tile stays.
  const Cand cands[] = {{big, 1.0}, {agmm::kTile256x128, 0.9}, {small, 0.8},
                        {agmm::kTile256x224m16, 0.98}};
  int best = big;
  double best_cost = 1e300;
  for (const Cand& c : cands) {
    if (c.cfg == agmm::kTile256x224m16 && !(deep && bnk)) continue;
    const int64_t bm = agmm::tile_bm(c.cfg), bn = agmm::tile_bn(c.cfg);
    const int64_t tiles = cdiv(m, bm) * cdiv(p->n, bn);
    const int64_t waves = cdiv(tiles, p->cu_count);
    const double cost = (double)waves * (double)(bm * bn) / c.eff;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = c.cfg;
    }
  }
  return best;
}

// Row blocks walked together by a launch of nrb x ncb output tiles.  The
// device order gives each of the 8 XCDs a contiguous range of logical tiles
// and walks groups of g row blocks column by column; the tiles of one XCD
// share its L2, so the choice is the g whose first XCD range touches the
// fewest distinct A row blocks plus B column blocks (4 wins ties).  E.g.
// 32 x 14 tiles: g = 8 touches 8 + 7 blocks against 4 + 14 for g = 4
// (measured 369-370 against 373 us on the 8x1024x8192 -> 3584 workload,
// about 1%); on 128 x 28 tiles every g touches 16 + 28 and 4 measured
// fastest (2819 against 2875 us for g = 8).
int pick_group_m(int64_t nrb, int64_t ncb) {
  const int64_t tiles = nrb * ncb;
  const int64_t per = std::min<int64_t>(tiles, cdiv(tiles, 8));
  int best = 4;
  int64_t best_cost = INT64_MAX;
  for (int g : {4, 8, 2, 16, 1}) {
    // tiles [0, per) walk groups of g row blocks (the last one shorter),
    // column by column: a group's first `take` tiles touch min(take, rows)
    // of its row blocks and its first ceil(take / rows) column blocks
    int64_t t = 0, rows = 0, cols = 0;
    for (int64_t grp = 0; t < per; ++grp) {
      const int64_t rh = std::min<int64_t>(nrb - grp * g, g);
      const int64_t take = std::min<int64_t>(rh * ncb, per - t);
      rows += std::min(take, rh);
      cols = std::max(cols, cdiv(take, rh));
      t += take;
    }
    if (rows + cols < best_cost) {
      best_cost = rows + cols;
      best = g;
    }
  }
  return best;
}

// Row-block visit order for a launch covering `groups` groups of `rpg` rows
// each, whose position t inside a group is shard row `row_off + t`.
void ring_order(const agmm_plan* p, const Settings& s, int64_t rpg, int64_t row_off, int bm,
                std::vector<int32_t>& out) {
  const int64_t rows = rpg * p->N;
  const int64_t nrb = cdiv(rows, bm);
  out.resize(nrb);
  for (int64_t b = 0; b < nrb; ++b) out[b] = (int32_t)b;
  if (s.order != 0 || p->N == 1) return;
  const int64_t half = (p->m_s + 1) / 2;  // first half of a shard: rows [0, half)
  std::vector<int64_t> key(nrb, 0);
  const int64_t N = p->N, r0 = s.local_shard;
  for (int64_t b = 0; b < nrb; ++b) {
    int64_t kmax = -1;
    const int64_t lo = b * bm, hi = std::min(rows, lo + bm);
    for (int64_t i = lo; i < hi; ++i) {
      const int64_t g = i / rpg;
      const int64_t t = row_off + (i - g * rpg);
      const bool top = t < half;
      const int64_t step = top ? ((g - r0) % N + N) % N : ((r0 - g) % N + N) % N;
      kmax = std::max(kmax, 2 * step + (top ? 0 : 1));
    }
    key[b] = kmax;
  }
  std::stable_sort(out.begin(), out.end(), [&](int32_t a, int32_t b) { return key[a] < key[b]; });
}

// Output tile (rows x columns) and waves of each skinny kernel shape.
struct SkinnyDims {
  int rows, cols, waves;
};
constexpr int kSkinnyShapes = 8;
SkinnyDims skinny_dims(int shape) {
  static const SkinnyDims d[kSkinnyShapes] = {{64, 16, 4}, {32, 32, 4}, {32, 16, 4}, {16, 32, 4},
                                              {64, 32, 4}, {32, 32, 8}, {64, 16, 8}, {64, 64, 4}};
  return d[shape >= 0 && shape < kSkinnyShapes ? shape : 5];
}

// Derive the launch layout of a plan from its problem and the settings:
// variant, tiles, chunks, split-K and sizes (not the tile-order tables).
// Host only; touches nothing of the plan and allocates nothing.
int derive_launch(const agmm_plan* p, const Settings& s, Layout& L) {
  const int64_t e = elem_bytes(p->dtype);
  // variant
  int v = s.variant;
  if (v == AGMM_VARIANT_AUTO) {
    if (is_f32(p)) v = AGMM_VARIANT_FUSED;
    else if (p->m <= 256) v = AGMM_VARIANT_SKINNY;
    else v = AGMM_VARIANT_FUSED;
  }
  if (is_f32(p) && v == AGMM_VARIANT_SKINNY) v = AGMM_VARIANT_FUSED;
  // fp32 rows that are not whole 16-byte vectors: the fp32 GEMM reads any
  // row length, but the gathering variants copy rows with 16-byte vectors,
  // so they gather zero-padded rows (k rounded up to 4) instead
  const bool f32_pad = is_f32(p) && (v == AGMM_VARIANT_STAGED || v == AGMM_VARIANT_UNFUSED) &&
                       (p->k * e) % 16 != 0;
  L.padded = needs_pad(p->dtype, p->k, p->n, p->rt) || f32_pad;
  L.kp = !L.padded ? p->k : is_f32(p) ? (p->k + 3) / 4 * 4 : round8(p->k);
  L.np = L.padded && !p->rt && !is_f32(p) ? round8(p->n) : p->n;
  // padded operands are gathered (with the zero fill) into the ring first:
  // every requested variant runs as gather-then-GEMM
  if (L.padded) v = AGMM_VARIANT_UNFUSED;
  L.variant_used = v;

  // B stored k x n: transposed once per call into the workspace when the
  // GEMM is large enough to repay it.  Measured on 8x4096x8192 -> 7168 bf16:
  // the GEMM takes 2700 us on B k x n and 2619 us on B n x k, the transpose
  // of the 117 MB B 44 us; the gain grows with m and breaks even near
  // m = 18K rows (a GEMM about 3% faster against a copy of 2 k n e bytes).
  L.bt = !is_f32(p) && !L.padded && !p->rt && v != AGMM_VARIANT_SKINNY &&
         (s.b_transpose > 0 || (s.b_transpose < 0 && p->k >= 256 && p->m >= kBtMinRows));
  const bool bnk = p->rt || L.bt;   // the GEMM reads B as n x k

  // tiles
  if (!is_f32(p) && s.tile >= 0 && agmm::tile_needs_bt(s.tile) && !bnk)
    return set_err(AGMM_ERR_UNSUPPORTED, "tile %d needs B stored n x k (rhs_transpose)", s.tile);
  if (is_f32(p)) {
    L.tile_used = -1;
    L.bm = L.bn = 64;
  } else {
    if (v == AGMM_VARIANT_SKINNY) {
      // B stored n x k, m <= 128: the skinny kernel (its tile shape and k
      // ranges below).  Measured per call in graph replay (us, skinny kernel
      // over whole k against the best split-K GEMM tile): m 128, n 1792,
      // k 4096: 11.8 / 16.4; m 128, n 512: 8.6 / 14.4; m 64, n 3584, k 8192:
      // 21.6 / 32.3.  For m 256 the
      // split-K 128x64 part ring was fastest (19.7 against 20.7 whole-k and
      // 24.8 for the 256x128 tile).  Split-K tiles put all of m in one row
      // block and split k over narrow column blocks, so that enough
      // workgroups stream B.
      if (s.tile >= 0) L.tile_used = s.tile;
      else if (p->rt) L.tile_used = p->m <= 128 ? agmm::kTileSkinny : agmm::kTile128x64r5;
      else L.tile_used = p->m <= 128 ? agmm::kTile128x128 : agmm::kTile256x128;
    } else if (v == AGMM_VARIANT_STAGED) {
      // tile chosen for one chunk's launch (pvalue tile-rows of every shard)
      const int64_t chunk_m = (int64_t)p->N * std::min<int64_t>(p->m_s, (int64_t)s.pvalue * 256);
      L.tile_used = choose_tile(p, s, chunk_m, bnk);
    } else {
      L.tile_used = choose_tile(p, s, p->m, bnk);
    }
    L.bm = agmm::tile_bm(L.tile_used);
    L.bn = agmm::tile_bn(L.tile_used);
  }

  // skinny tile shape: 32 x 32 with 8 waves (2-3% faster than 4 on four
  // skinny shapes), its k split to fill the CUs (below); 64 x 64 (4 waves,
  // k split to fill the CUs) where 32 x 32 tiles would take more than one
  // round of workgroups and 64 x 64 tiles take at most one.  Measured per
  // call in graph replay (us): 8x16x14336 -> 4096: 32 x 32 whole k 64.2,
  // 64 x 64 with 2 splits 41.7; 4x16x8192 -> 1024: whole k 19.0, 4 splits
  // 11.5; 8x16x4096 -> 512: 8.3, 4 splits 7.6; the skinny workload
  // 8x16x4096 -> 1792 (224 tiles): whole k 11.5, 64 x 64 with 4 splits 13.3.
  if (s.skinny_shape >= 0) {
    L.skinny_shape_used = s.skinny_shape;
  } else {
    const int64_t t32 = cdiv(p->m, 32) * cdiv(p->n, 32), t64 = cdiv(p->m, 64) * cdiv(p->n, 64);
    L.skinny_shape_used = t32 > p->cu_count && t64 <= p->cu_count ? 7 : 5;
  }

  // chunking (staged) / split-K
  L.rows_per_chunk = p->m_s;
  L.num_chunks = 1;
  L.nslots = 0;
  L.splits_used = 1;
  L.k_per_split = L.kp;
  L.ring_bytes = L.part_bytes = L.slot_bytes = L.padb_bytes = 0;
  if (v == AGMM_VARIANT_STAGED) {
    L.rows_per_chunk = std::min<int64_t>(p->m_s, (int64_t)s.pvalue * L.bm);
    L.num_chunks = (int)cdiv(p->m_s, L.rows_per_chunk);
    L.nslots = s.debug_keep_slots ? L.num_chunks : std::min(s.nbuf, L.num_chunks);
    L.slot_bytes = (size_t)p->N * L.rows_per_chunk * p->k * e;
    L.ring_bytes = L.slot_bytes * L.nslots;
  } else if (v == AGMM_VARIANT_UNFUSED) {
    L.nslots = 1;
    L.slot_bytes = (size_t)p->m * L.kp * e;
    L.ring_bytes = L.slot_bytes;
    if (L.padded) L.padb_bytes = (size_t)(p->rt ? p->n * L.kp : L.kp * L.np) * e;
  }
  if (L.bt) L.padb_bytes = (size_t)p->n * p->k * e;
  // split-K: skinny problems always, the other variants when one launch has
  // too few output tiles to give every CU a workgroup.  A power of two of k
  // ranges (multiples of the k granularity), chosen so that splits * tiles
  // still fits on the CUs; fp32 partial sums then a fixed-order reduction.
  // A staged plan's launches are its chunks, which run one after another on
  // the caller's stream and share one partials buffer.
  if (!is_f32(p)) {
    const int64_t launch_m = v == AGMM_VARIANT_STAGED ? (int64_t)p->N * L.rows_per_chunk : p->m;
    const int64_t tiles = cdiv(launch_m, L.bm) * cdiv(p->n, L.bn);
    int64_t want = s.splits;
    int64_t tiles_k = tiles;   // output tiles of one launch, for the automatic split
    int64_t min_k = v == AGMM_VARIANT_SKINNY ? agmm::kTileBK : 1024;   // shortest automatic k range
    if (L.tile_used == agmm::kTileSkinny) {
      // the skinny kernel's waves take a k range's 64-deep k-tiles round
      // robin: at least one each
      const SkinnyDims d = skinny_dims(L.skinny_shape_used);
      tiles_k = cdiv(launch_m, d.rows) * cdiv(p->n, d.cols);
      min_k = std::max<int64_t>(min_k, (int64_t)d.waves * agmm::kTileBK);
    }
    if (want <= 0) {
      want = 1;
      // workgroup slots: the CUs times the workgroups of this tile one CU
      // holds (the skinny rule keeps one per CU: more k ranges there only
      // add partial sums, measured slower on the 8x16x4096->1792 workload;
      // counting both slots of the two-per-CU 128x128 tile measured 37.5 ->
      // 34.9 us on 4x512x4096->1024)
      const int64_t slots = v == AGMM_VARIANT_SKINNY
                                ? p->cu_count
                                : (int64_t)p->cu_count * agmm::tile_occ(L.tile_used);
      if (v == AGMM_VARIANT_SKINNY || 2 * tiles_k <= slots) {
        // long enough k ranges that the partial sums stay small next to the
        // operand traffic (skinny problems have no other way to fill the GPU)
        while (want * 2 * tiles_k <= slots && L.kp / (want * 2) >= min_k) want *= 2;
      }
    }
    want = std::max<int64_t>(1, std::min<int64_t>(want, cdiv(L.kp, agmm::kTileBK)));
    L.k_per_split = cdiv(cdiv(L.kp, want), agmm::kTileBK) * agmm::kTileBK;
    L.splits_used = (int)cdiv(L.kp, L.k_per_split);
    // a staged plan's launches: its chunks and (local_first) the local shard's rows
    const int64_t part_m = v == AGMM_VARIANT_STAGED ? std::max<int64_t>(launch_m, p->m_s) : launch_m;
    if (L.splits_used > 1) L.part_bytes = (size_t)L.splits_used * part_m * p->n * sizeof(float);
  }
  return AGMM_OK;
}

// derive_launch plus the tile-order tables (one per chunk).
int derive(const agmm_plan* p, const Settings& s, Layout& L) {
  const int rc = derive_launch(p, s, L);
  if (rc != AGMM_OK) return rc;
  L.h_order.clear();
  L.order_off.clear();
  L.order_len.clear();
  std::vector<int32_t> tmp;
  for (int c = 0; c < L.num_chunks; ++c) {
    const int64_t rows_c = std::min<int64_t>(L.rows_per_chunk, p->m_s - (int64_t)c * L.rows_per_chunk);
    ring_order(p, s, rows_c, (int64_t)c * L.rows_per_chunk, L.bm, tmp);
    L.order_off.push_back((int64_t)L.h_order.size());
    L.order_len.push_back((int32_t)tmp.size());
    L.h_order.insert(L.h_order.end(), tmp.begin(), tmp.end());
  }
  return AGMM_OK;
}

// Wait until no enqueued work of the plan can still use its workspace.
int wait_idle(agmm_plan* p) {
  if (p->done_state == kDoneEager) {
    const hipError_t err = hipEventSynchronize(p->ev_done);
    if (err != hipSuccess) return hip_err(err, "hipEventSynchronize(done)");
  }
  return AGMM_OK;
}

int alloc_ws(agmm_plan* p, size_t bytes) {
  if (bytes == 0) return AGMM_OK;
  // test hook: AGMM_TEST_FAIL_ALLOC=<n> makes every workspace allocation of
  // more than n bytes fail (n = 0 or 1: all of them)
  if (const char* hook = std::getenv("AGMM_TEST_FAIL_ALLOC")) {
    const long long limit = std::atoll(hook);
    if (limit <= 1 || (long long)bytes > limit)
      return set_err(AGMM_ERR_OOM, "workspace allocation of %zu bytes failed (forced by test hook)",
                     bytes);
  }
  hipError_t err = hipMalloc(&p->ws, bytes);
  if (err != hipSuccess) {
    p->ws = nullptr;
    (void)hipGetLastError();
    return set_err(AGMM_ERR_OOM, "workspace allocation of %zu bytes failed: %s", bytes,
                   hipGetErrorString(err));
  }
  p->ws_cap = bytes;
  return AGMM_OK;
}

// Give the plan a new layout: derive it, make room in the workspace (the
// existing allocation is kept when the new layout fits in it), then commit
// the settings and layout and upload the tile-order tables.  On an error
// before the commit the plan keeps its previous settings, layout and a
// workspace of the previous size; if even that cannot be restored the plan
// is marked unusable and every later call on it fails.
int apply(agmm_plan* p, const Settings& s) {
  Layout L;
  int rc = derive(p, s, L);
  if (rc != AGMM_OK) return rc;
  rc = wait_idle(p);   // the previous call may still read the workspace
  if (rc != AGMM_OK) return rc;
  const size_t total = L.total_bytes();
  if (total > p->ws_cap) {
    const size_t old_cap = p->ws_cap;
    if (p->ws) hipFree(p->ws);
    p->ws = nullptr;
    p->ws_cap = 0;
    p->ring = nullptr;
    p->partials = nullptr;
    p->padb = nullptr;
    p->d_order = nullptr;
    rc = alloc_ws(p, total);
    if (rc != AGMM_OK) {
      const int st = g_status;
      const std::string msg = g_msg;
      // Restore a workspace for the layout the plan still has.
      if (alloc_ws(p, old_cap) != AGMM_OK) {
        p->broken = st;
        p->broken_msg = msg + "; the previous workspace could not be restored either";
      } else {
        char* q = p->ws;
        if (p->L.ring_bytes) { p->ring = q; q += Layout::up(p->L.ring_bytes); }
        if (p->L.part_bytes) { p->partials = reinterpret_cast<float*>(q); q += Layout::up(p->L.part_bytes); }
        if (p->L.padb_bytes) { p->padb = q; q += Layout::up(p->L.padb_bytes); }
        if (p->L.order_bytes()) {
          p->d_order = reinterpret_cast<int32_t*>(q);
          if (hipMemcpy(p->d_order, p->L.h_order.data(), p->L.order_bytes(), hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipGetLastError();
            p->broken = AGMM_ERR_HIP;
            p->broken_msg = msg + "; re-uploading the tile order failed";
          }
        }
      }
      return set_err(st, "%s", msg.c_str());
    }
  }
  // commit
  p->s = s;
  p->L = std::move(L);
  p->ring = nullptr;
  p->partials = nullptr;
  p->padb = nullptr;
  p->d_order = nullptr;
  char* q = p->ws;
  if (p->L.ring_bytes) { p->ring = q; q += Layout::up(p->L.ring_bytes); }
  if (p->L.part_bytes) { p->partials = reinterpret_cast<float*>(q); q += Layout::up(p->L.part_bytes); }
  if (p->L.padb_bytes) { p->padb = q; q += Layout::up(p->L.padb_bytes); }
  if (p->L.order_bytes()) {
    p->d_order = reinterpret_cast<int32_t*>(q);
    const hipError_t err = hipMemcpy(p->d_order, p->L.h_order.data(), p->L.order_bytes(), hipMemcpyHostToDevice);
    if (err != hipSuccess) {
      p->broken = AGMM_ERR_HIP;
      p->broken_msg = std::string("uploading the tile order failed: ") + hipGetErrorString(err);
      return hip_err(err, "hipMemcpy(tile order)");
    }
  }
  // events for the ring
  const size_t want_ev = (size_t)std::max(p->L.nslots, 1);
  while (p->ev_ready.size() < want_ev) {
    hipEvent_t a, b;
    hipError_t err = hipEventCreateWithFlags(&a, hipEventDisableTiming);
    if (err != hipSuccess) return hip_err(err, "hipEventCreate");
    err = hipEventCreateWithFlags(&b, hipEventDisableTiming);
    if (err != hipSuccess) { hipEventDestroy(a); return hip_err(err, "hipEventCreate"); }
    p->ev_ready.push_back(a);
    p->ev_free.push_back(b);
  }
  return ok();
}

// One call's view of the caller's stream.
struct Call {
  hipStream_t s = nullptr;
  bool capturing = false;
  unsigned long long capture_id = 0;
};

// Start a call: refuse an unusable plan, find out whether the stream is being
// captured into a graph, and order the call after the plan's previous one.
// Across a capture boundary (a call captured into a graph after eager calls,
// or an eager call after a captured one) no event links them: waiting on an
// event recorded on the other side of the boundary is not allowed while a
// stream is capturing, and a captured call's work happens at each replay;
// the caller's streams order graph replays against other work.
int enter(agmm_plan* p, hipStream_t s, Call& c) {
  if (p->broken != AGMM_OK) return set_err(p->broken, "plan is unusable: %s", p->broken_msg.c_str());
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  unsigned long long id = 0;
  hipError_t err = hipStreamGetCaptureInfo(s, &st, &id);
  if (err != hipSuccess) return hip_err(err, "hipStreamGetCaptureInfo");
  if (st == hipStreamCaptureStatusInvalidated)
    return set_err(AGMM_ERR_HIP, "the stream's graph capture has been invalidated");
  c.s = s;
  c.capturing = st == hipStreamCaptureStatusActive;
  c.capture_id = c.capturing ? id : 0;
  if (c.capturing) p->captured = true;
  const bool linked = p->done_state == kDoneEager
                          ? !c.capturing
                          : (p->done_state == kDoneCaptured && c.capturing && p->done_capture_id == id);
  if (linked && p->done_stream != s) {
    err = hipStreamWaitEvent(s, p->ev_done, 0);
    if (err != hipSuccess) return hip_err(err, "hipStreamWaitEvent(done)");
  }
  return AGMM_OK;
}

// End a call that enqueued work: every internal stream has joined `c.s`.
int leave(agmm_plan* p, const Call& c) {
  const hipError_t err = hipEventRecord(p->ev_done, c.s);
  if (err != hipSuccess) return hip_err(err, "hipEventRecord(done)");
  p->done_state = c.capturing ? kDoneCaptured : kDoneEager;
  p->done_capture_id = c.capture_id;
  p->done_stream = c.s;
  return AGMM_OK;
}

agmm::RowMap shard_rows(const agmm_plan* p, const void* const* shards) {
  agmm::RowMap r{};
  for (int g = 0; g < p->N; ++g) r.a_group[g] = shards[g];
  r.a_ld = lda_of(p);
  r.rows_per_group = (int32_t)p->m_s;
  r.num_groups = p->N;
  r.c_group_rows = p->m_s;
  r.c_row_off = 0;
  return r;
}

agmm::RowMap dense_rows(const void* a, int64_t rows, int64_t ld) {
  agmm::RowMap r{};
  r.a_group[0] = a;
  r.a_ld = ld;
  r.rows_per_group = (int32_t)rows;
  r.num_groups = 1;
  r.c_group_rows = 0;
  r.c_row_off = 0;
  return r;
}

agmm::GemmProblem base_problem(agmm_plan* p, const agmm::RowMap& rows, int64_t m_launch,
                               const void* B, void* C, int chunk) {
  agmm::GemmProblem g{};
  g.rows = rows;
  g.m = (int32_t)m_launch;
  g.n = (int32_t)p->n;
  g.k = (int32_t)p->k;
  g.b = p->L.bt ? p->padb : B;
  g.ldb = p->L.bt ? p->k : ldb_of(p);
  g.c = C;
  g.ldc = ldc_of(p);
  g.order.num_rb = (int32_t)cdiv(m_launch, p->L.bm);
  g.order.num_cb = (int32_t)cdiv(p->n, p->L.bn);
  if (p->s.group_m > 0) {
    g.order.group_m = p->s.group_m;
  } else {
    if (p->group_key_rb != g.order.num_rb || p->group_key_cb != g.order.num_cb) {
      p->group_auto = pick_group_m(g.order.num_rb, g.order.num_cb);
      p->group_key_rb = g.order.num_rb;
      p->group_key_cb = g.order.num_cb;
    }
    g.order.group_m = p->group_auto;
  }
  g.order.xcd_remap = p->s.xcd_remap;
  g.order.rb_order = nullptr;
  if (chunk >= 0 && p->d_order && chunk < (int)p->L.order_off.size() &&
      p->L.order_len[chunk] == g.order.num_rb)
    g.order.rb_order = p->d_order + p->L.order_off[chunk];
  g.splits = 1;
  g.k_per_split = (int32_t)p->k;
  return g;
}

// Split-K for a launch: the plan's k ranges, when its partials buffer holds
// this launch's [splits][m][n] sums (a launch larger than the ones the plan
// sized it for, e.g. agmm_run_gathered on a staged plan, runs unsplit).
void with_splits(const agmm_plan* p, agmm::GemmProblem& g) {
  if (p->L.splits_used > 1 && p->partials &&
      (size_t)p->L.splits_used * (size_t)g.m * (size_t)p->n * sizeof(float) <= p->L.part_bytes) {
    g.splits = p->L.splits_used;
    g.k_per_split = (int32_t)p->L.k_per_split;
    g.partials = p->partials;
  }
}

int launch_gemm(agmm_plan* p, const Call& c, agmm::GemmProblem& g, hipStream_t s) {
  // timing events are recorded eagerly only (inside a capture they would
  // time nothing)
  const bool timed = p->timing && !c.capturing && p->tev_used + 2 <= (int)p->tev.size();
  if (timed) hipEventRecord(p->tev[p->tev_used], s);
  hipError_t err;
  if (is_f32(p)) err = agmm::launch_gemm_f32(g, p->rt != 0, s);
  else if (p->L.tile_used == agmm::kTileSkinny)
    err = agmm::launch_skinny_fullk(g, p->dtype, p->L.skinny_shape_used, s);
  else err = agmm::launch_gemm_mfma(g, p->L.tile_used, p->dtype, p->rt != 0 || p->L.bt, s);
  if (err != hipSuccess) return hip_err(err, "GEMM launch");
  if (timed) {
    hipEventRecord(p->tev[p->tev_used + 1], s);
    p->tev_used += 2;
  }
  return AGMM_OK;
}

int check_ptrs(agmm_plan* p, const void* const* shards, const void* B, const void* C) {
  if (!p) return set_err(AGMM_ERR_INVALID_ARG, "plan is NULL");
  if (!shards) return set_err(AGMM_ERR_INVALID_ARG, "shard_ptrs is NULL");
  for (int r = 0; r < p->N; ++r) {
    if (!shards[r]) return set_err(AGMM_ERR_INVALID_ARG, "shard_ptrs[%d] is NULL", r);
    if (!aligned16(shards[r]))
      return set_err(AGMM_ERR_UNSUPPORTED, "shard_ptrs[%d] is not 16-byte aligned", r);
  }
  if (!B) return set_err(AGMM_ERR_INVALID_ARG, "B is NULL");
  if (!C) return set_err(AGMM_ERR_INVALID_ARG, "C is NULL");
  if (!aligned16(B)) return set_err(AGMM_ERR_UNSUPPORTED, "B is not 16-byte aligned");
  if (!aligned16(C)) return set_err(AGMM_ERR_UNSUPPORTED, "C is not 16-byte aligned");
  return AGMM_OK;
}

int gather_chunk(agmm_plan* p, const void* const* shards, int64_t row0, int64_t rows, void* dst,
                 int64_t dst_group_rows, int max_wgs, hipStream_t s) {
  agmm::GatherProblem g{};
  for (int r = 0; r < p->N; ++r) g.src_group[r] = shards[r];
  g.num_groups = p->N;
  g.src_row0 = row0;
  g.rows = rows;
  g.row_bytes = p->k * (int64_t)elem_bytes(p->dtype);
  g.src_ld_bytes = lda_of(p) * (int64_t)elem_bytes(p->dtype);
  g.dst = dst;
  g.dst_group_rows = dst_group_rows;
  hipError_t err = agmm::launch_gather(g, max_wgs, s);
  if (err != hipSuccess) return hip_err(err, "gather launch");
  return AGMM_OK;
}

// The same bit copy on the SDMA engines (hipMemcpyDeviceToDeviceNoCU): no
// compute unit takes part, so it runs beside a GEMM that fills every CU's
// register file without slowing it.  Needs dense shard rows (each shard's
// chunk is then one contiguous range).
int gather_chunk_sdma(agmm_plan* p, const void* const* shards, int64_t row0, int64_t rows,
                      void* dst, int64_t dst_group_rows, hipStream_t s) {
  const size_t row_bytes = (size_t)p->k * elem_bytes(p->dtype);
  for (int g = 0; g < p->N; ++g) {
    const char* src = static_cast<const char*>(shards[g]) + (size_t)row0 * row_bytes;
    char* d = static_cast<char*>(dst) + (size_t)g * dst_group_rows * row_bytes;
    hipError_t err = hipMemcpyAsync(d, src, (size_t)rows * row_bytes, hipMemcpyDeviceToDeviceNoCU, s);
    if (err != hipSuccess) return hip_err(err, "hipMemcpyAsync(gather on SDMA)");
  }
  return AGMM_OK;
}

// Element-granular copy of rows with zero fill (launch_pad_copy), for rows
// that are not whole 16-byte vectors.
int pad_copy(const agmm_plan* p, const void* const* groups, int ngroups, int64_t src_rows,
             int64_t src_ld, int64_t cols, int64_t rows, void* dst, int64_t dst_group_rows,
             int64_t dst_ld, int64_t dst_cols, hipStream_t s) {
  agmm::PadCopyProblem c{};
  for (int g = 0; g < ngroups; ++g) c.src_group[g] = groups[g];
  c.num_groups = ngroups;
  c.elem_bytes = (int32_t)elem_bytes(p->dtype);
  c.src_row0 = 0;
  c.src_rows = src_rows;
  c.src_ld = src_ld;
  c.cols = cols;
  c.rows = rows;
  c.dst = dst;
  c.dst_group_rows = dst_group_rows;
  c.dst_ld = dst_ld;
  c.dst_cols = dst_cols;
  const hipError_t err = agmm::launch_pad_copy(c, s);
  if (err != hipSuccess) return hip_err(err, "pad copy launch");
  return AGMM_OK;
}

// The gathered operand [m][k] (dense rows) from the shards: the vector
// gather copy when rows are whole 16-byte vectors, else element by element.
int gather_rows(agmm_plan* p, const void* const* shards, void* dst, int max_wgs, hipStream_t s) {
  const int64_t e = elem_bytes(p->dtype);
  if ((p->k * e) % 16 == 0 && (lda_of(p) * e) % 16 == 0)
    return gather_chunk(p, shards, 0, p->m_s, dst, p->m_s, max_wgs, s);
  return pad_copy(p, shards, p->N, p->m_s, lda_of(p), p->k, p->m_s, dst, p->m_s, p->k, p->k, s);
}

// A padded layout's run: A (from the shards, or from a gathered [m][k]
// buffer) into the ring as [m][kp] and B into its buffer, both zero-filled,
// then the GEMM over kp (the zeros add nothing to any sum).
int run_padded(agmm_plan* p, const Call& c, const void* const* shards, const void* gathered,
               const void* B, void* C);

// Whether a copy goes to the SDMA engines: only when the plan asks for them
// (copy_engine 1), the copy runs beside a GEMM (`overlaps`), the shard rows
// are dense and the caller's stream is not being captured into a graph (the
// capture keeps the kernel copy, whose graph form is tested).  Measured on
// MI355X: alone, an SDMA copy moves ~1.16 TB/s and leaves the CUs free; but
// in the staged pipeline beside the chunk GEMMs the chunks arrive too late
// (workload 5: 5.26 ms against 3.47 ms with the kernel copy), so the kernel
// copy stays the default.
bool copy_on_sdma(const agmm_plan* p, const Call& c, bool overlaps) {
  return p->s.copy_engine == 1 && overlaps && lda_of(p) == p->k && !c.capturing &&
         (p->k * (int64_t)elem_bytes(p->dtype)) % 16 == 0;
}

// Fork: `other` waits for everything enqueued so far on the caller's stream.
int fork_to(agmm_plan* p, const Call& c, hipStream_t other) {
  hipError_t err = hipEventRecord(p->ev_entry, c.s);
  if (err == hipSuccess) err = hipStreamWaitEvent(other, p->ev_entry, 0);
  if (err != hipSuccess) return hip_err(err, "stream fork");
  return AGMM_OK;
}

// Join: the caller's stream waits for everything enqueued so far on `other`.
int join_from(const Call& c, hipStream_t other, hipEvent_t ev) {
  hipError_t err = hipEventRecord(ev, other);
  if (err == hipSuccess) err = hipStreamWaitEvent(c.s, ev, 0);
  if (err != hipSuccess) return hip_err(err, "stream join");
  return AGMM_OK;
}

// The chunk loop of the staged pipeline (the streams are forked and joined
// by run_staged).
int staged_chunks(agmm_plan* p, const Call& c, const void* const* shards, const void* B, void* C,
                  void* gathered, bool alt, bool local_first) {
  hipStream_t s = c.s;
  hipError_t err;
  const int64_t e = elem_bytes(p->dtype);
  const int r0 = p->s.local_shard;
  if (local_first) {
    agmm::RowMap rm{};
    rm.a_group[0] = shards[r0];
    rm.a_ld = lda_of(p);
    rm.rows_per_group = (int32_t)p->m_s;
    rm.num_groups = 1;
    rm.c_group_rows = 0;
    rm.c_row_off = (int64_t)r0 * p->m_s;
    agmm::GemmProblem g = base_problem(p, rm, p->m_s, B, C, -1);
    with_splits(p, g);
    const int rc = launch_gemm(p, c, g, s);
    if (rc != AGMM_OK) return rc;
  }
  for (int ch = 0; ch < p->L.num_chunks; ++ch) {
    const int slot = ch % p->L.nslots;
    const int64_t row0 = (int64_t)ch * p->L.rows_per_chunk;
    const int64_t rows_c = std::min<int64_t>(p->L.rows_per_chunk, p->m_s - row0);
    // destination of shard g's rows of this chunk: dst + g * dst_group_rows rows
    char* dst = gathered ? static_cast<char*>(gathered) + (size_t)row0 * p->k * e
                         : p->ring + (size_t)slot * p->L.slot_bytes;
    const int64_t dst_group_rows = gathered ? p->m_s : rows_c;
    if (!gathered && ch >= p->L.nslots) {
      err = hipStreamWaitEvent(p->copy_stream, p->ev_free[slot], 0);
      if (err != hipSuccess) return hip_err(err, "hipStreamWaitEvent(free)");
    }
    // Every chunk's copy is sized to the whole GPU unless the plan sets
    // copy_wgs: the GEMM holds all of a CU's registers, so a copy held to
    // one workgroup per CU mostly waits for CUs the GEMM leaves idle
    // (measured: 496 -> ~467 us on the 8x1024x8192 -> 3584 workload, 3244
    // -> ~3180 us on 8x4096x8192 -> 7168, pvalue 2, two slots).  With
    // copy_engine 1 the copies after the first go to the SDMA engines.
    int rc;
    if (copy_on_sdma(p, c, ch > 0)) {
      rc = gather_chunk_sdma(p, shards, row0, rows_c, dst, dst_group_rows, p->copy_stream);
    } else {
      rc = gather_chunk(p, shards, row0, rows_c, dst, dst_group_rows, p->s.copy_wgs, p->copy_stream);
    }
    if (rc != AGMM_OK) return rc;
    if ((err = hipEventRecord(p->ev_ready[slot], p->copy_stream)) != hipSuccess)
      return hip_err(err, "hipEventRecord(ready)");
    // chunks alternate streams; with local_first chunk 0 takes the second
    // stream, beside the local GEMM on the caller's
    hipStream_t cs = (alt && ((ch & 1) == (local_first ? 0 : 1))) ? p->compute2 : s;
    if ((err = hipStreamWaitEvent(cs, p->ev_ready[slot], 0)) != hipSuccess)
      return hip_err(err, "hipStreamWaitEvent(ready)");
    if (!local_first) {
      agmm::RowMap rm{};
      for (int g = 0; g < p->N; ++g) rm.a_group[g] = dst + (size_t)g * dst_group_rows * p->k * e;
      rm.a_ld = p->k;
      rm.rows_per_group = (int32_t)rows_c;
      rm.num_groups = p->N;
      rm.c_group_rows = p->m_s;
      rm.c_row_off = row0;
      agmm::GemmProblem g = base_problem(p, rm, rows_c * p->N, B, C, ch);
      with_splits(p, g);
      rc = launch_gemm(p, c, g, cs);
      if (rc != AGMM_OK) return rc;
    } else {
      // the other shards, as the runs [0, r0) and (r0, N) of consecutive
      // shards (C rows are linear in the shard index within a run)
      const int lo_hi[2][2] = {{0, r0}, {r0 + 1, p->N}};
      for (const auto& run : lo_hi) {
        const int lo = run[0], cnt = run[1] - run[0];
        if (cnt <= 0) continue;
        agmm::RowMap rm{};
        for (int j = 0; j < cnt; ++j) rm.a_group[j] = dst + (size_t)(lo + j) * dst_group_rows * p->k * e;
        rm.a_ld = p->k;
        rm.rows_per_group = (int32_t)rows_c;
        rm.num_groups = cnt;
        rm.c_group_rows = p->m_s;
        rm.c_row_off = (int64_t)lo * p->m_s + row0;
        agmm::GemmProblem g = base_problem(p, rm, rows_c * cnt, B, C, -1);
        with_splits(p, g);
        rc = launch_gemm(p, c, g, cs);
        if (rc != AGMM_OK) return rc;
      }
    }
    if (!gathered && (err = hipEventRecord(p->ev_free[slot], cs)) != hipSuccess)
      return hip_err(err, "hipEventRecord(free)");
  }
  return AGMM_OK;
}

// Staged pipeline.  With `gathered` == nullptr the chunks go through the
// plan's ring of slots; otherwise each chunk is copied to its final place in
// the caller's [m, k] buffer (no slot is reused, so no copy waits for a GEMM).
// The copy stream (and the second GEMM stream) fork from the caller's stream
// at entry and always join it again before the call returns.
int run_staged(agmm_plan* p, const Call& c, const void* const* shards, const void* B, void* C,
               void* gathered = nullptr) {
  // Odd chunks' GEMMs run on a second stream, so the workgroups of chunk c+1
  // take the CUs chunk c's workgroups leave (each chunk's launch is usually
  // a partial round); only the ring-slot events order them.  With split-K the
  // chunks share one partials buffer and stay on the caller's stream.
  // The local shard's rows need no copy (tpu-inference `all_gather_matmul`:
  // a device multiplies its own x block while the ring brings the others):
  // with local_first their GEMM runs first, from the shard buffer, on the
  // caller's stream beside chunk 0's copy, and the chunk GEMMs cover the
  // other shards' rows only.
  // Off by default: measured neutral on 8x1024x8192 -> 3584 (435 us), 1%
  // faster on 8x4096x8192 -> 7168, slower where the launches are small
  // (4x512x4096 -> 1024: 62 -> 75 us; with one chunk, 28 -> 43 us on
  // 8x16x4096 -> 1792, so it is never used with a single chunk).
  // Under graph capture only the staged forms whose replays are tested are
  // accepted: one staged call per captured graph, with no ring slot refilled
  // within the call (at most as many chunks as slots; the gathered-output
  // form never refills one).  A process once ended in a segmentation fault
  // while capturing several staged calls of a plan that refills slots into
  // one graph, and that case was never shown to be safe, so it is refused
  // before anything is enqueued.
  if (c.capturing) {
    if (!gathered && p->L.num_chunks > p->L.nslots)
      return set_err(AGMM_ERR_UNSUPPORTED,
                     "staged plan with %d chunks over %d ring slots: not under graph capture "
                     "(at most as many chunks as slots: raise nbuf or pvalue)",
                     p->L.num_chunks, p->L.nslots);
    if (p->staged_capture_id == c.capture_id)
      return set_err(AGMM_ERR_UNSUPPORTED,
                     "a staged call of this plan is already in this graph capture (one per graph)");
    p->staged_capture_id = c.capture_id;
  }
  const bool local_first = p->s.local_first && p->N > 1 && p->L.num_chunks > 1;
  const bool alt = p->s.gemm_streams == 2 && p->L.splits_used == 1 && (p->L.num_chunks > 1 || local_first);
  int rc = fork_to(p, c, p->copy_stream);
  if (rc != AGMM_OK) return rc;
  // The second GEMM stream needs no wait on the call's entry in an eager
  // call: each GEMM it runs first waits for its chunk's `ready` event, which
  // the copy stream records after its own wait on the entry.  Under graph
  // capture it is forked from the caller's stream explicitly.
  if (alt && c.capturing) {
    const hipError_t err = hipStreamWaitEvent(p->compute2, p->ev_entry, 0);
    if (err != hipSuccess) rc = hip_err(err, "hipStreamWaitEvent");
  }
  if (rc == AGMM_OK) rc = staged_chunks(p, c, shards, B, C, gathered, alt, local_first);
  // Join whatever was enqueued, also after an error.  After a complete chunk
  // loop an eager call needs no join of the copy stream: its work is the
  // chunk copies in order, and the last chunk's GEMM (on the caller's
  // stream, or on the second GEMM stream joined below) waited for the last
  // copy's `ready` event; one cross-stream wait fewer per call.  Under graph
  // capture every forked stream is joined explicitly.
  const bool copies_awaited = rc == AGMM_OK && p->L.num_chunks >= 1 && !c.capturing;
  const int rj = copies_awaited ? AGMM_OK : join_from(c, p->copy_stream, p->ev_side);
  const int rj2 = alt ? join_from(c, p->compute2, p->ev_c2) : AGMM_OK;
  if (rc != AGMM_OK) return rc;
  return rj != AGMM_OK ? rj : rj2;
}

int run_padded(agmm_plan* p, const Call& c, const void* const* shards, const void* gathered,
               const void* B, void* C) {
  const Layout& L = p->L;
  int rc = gathered
               ? pad_copy(p, &gathered, 1, p->m, p->k, p->k, p->m, p->ring, p->m, L.kp, L.kp, c.s)
               : pad_copy(p, shards, p->N, p->m_s, lda_of(p), p->k, p->m_s, p->ring, p->m_s, L.kp, L.kp, c.s);
  if (rc != AGMM_OK) return rc;
  rc = p->rt ? pad_copy(p, &B, 1, p->n, ldb_of(p), p->k, p->n, p->padb, p->n, L.kp, L.kp, c.s)
             : pad_copy(p, &B, 1, p->k, ldb_of(p), p->n, L.kp, p->padb, L.kp, L.np, L.np, c.s);
  if (rc != AGMM_OK) return rc;
  agmm::GemmProblem g = base_problem(p, dense_rows(p->ring, p->m, L.kp), p->m, p->padb, C, -1);
  g.k = (int32_t)L.kp;
  g.ldb = p->rt ? L.kp : L.np;
  with_splits(p, g);
  return launch_gemm(p, c, g, c.s);
}

// The transposed copy of B (plans with L.bt): B^T [n][k] into the B copy on
// the caller's stream, ahead of every GEMM of the call.
int transpose_b(agmm_plan* p, const void* B, hipStream_t s) {
  if (!p->L.bt) return AGMM_OK;
  const hipError_t err = agmm::launch_transpose16(B, ldb_of(p), p->k, p->n, p->padb, s);
  return err == hipSuccess ? AGMM_OK : hip_err(err, "B transpose launch");
}

// agmm_run's work, after enter().
int run_plan(agmm_plan* p, const Call& c, const void* const* shard_ptrs, const void* B, void* C) {
  int rc;
  if (p->L.padded) return run_padded(p, c, shard_ptrs, nullptr, B, C);
  rc = transpose_b(p, B, c.s);
  if (rc != AGMM_OK) return rc;
  switch (p->L.variant_used) {
    case AGMM_VARIANT_FUSED:
    case AGMM_VARIANT_SKINNY: {
      agmm::GemmProblem g = base_problem(p, shard_rows(p, shard_ptrs), p->m, B, C, 0);
      with_splits(p, g);
      return launch_gemm(p, c, g, c.s);
    }
    case AGMM_VARIANT_UNFUSED: {
      rc = gather_chunk(p, shard_ptrs, 0, p->m_s, p->ring, p->m_s, 0, c.s);
      if (rc != AGMM_OK) return rc;
      agmm::GemmProblem g = base_problem(p, dense_rows(p->ring, p->m, p->k), p->m, B, C, -1);
      with_splits(p, g);
      return launch_gemm(p, c, g, c.s);
    }
    case AGMM_VARIANT_STAGED:
      return run_staged(p, c, shard_ptrs, B, C);
    default:
      return set_err(AGMM_ERR_INVALID_ARG, "plan has no valid variant");
  }
}

// A call that enqueues work: enter, body, leave.
template <class F>
int guarded(agmm_plan* p, hipStream_t s, F&& body) {
  Call c;
  int rc = enter(p, s, c);
  if (rc != AGMM_OK) return rc;
  rc = body(c);
  const int rl = leave(p, c);
  if (rc != AGMM_OK) return rc;
  return rl != AGMM_OK ? rl : ok();
}

}  // namespace

extern "C" {

int agmm_plan_validate(int num_shards, int64_t m_per_shard, int64_t k, int64_t n_local, int dtype,
                       int rhs_transpose) {
  return validate(num_shards, m_per_shard, k, n_local, dtype, rhs_transpose);
}

agmm_plan_t agmm_plan_create(int num_shards, int64_t m_per_shard, int64_t k, int64_t n_local,
                             int dtype, int rhs_transpose) {
  if (validate(num_shards, m_per_shard, k, n_local, dtype, rhs_transpose) != AGMM_OK)
    return nullptr;
  agmm_plan* p = new (std::nothrow) agmm_plan();
  if (!p) {
    set_err(AGMM_ERR_OOM, "out of host memory");
    return nullptr;
  }
  p->N = num_shards;
  p->m_s = m_per_shard;
  p->k = k;
  p->n = n_local;
  p->m = (int64_t)num_shards * m_per_shard;
  p->dtype = dtype;
  p->rt = rhs_transpose;
  hipError_t err = hipGetDevice(&p->device);
  if (err != hipSuccess) {
    hip_err(err, "hipGetDevice");
    delete p;
    return nullptr;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) == hipSuccess &&
      cus > 0)
    p->cu_count = cus;
  err = hipStreamCreateWithFlags(&p->copy_stream, hipStreamNonBlocking);
  if (err == hipSuccess) err = hipStreamCreateWithFlags(&p->compute2, hipStreamNonBlocking);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&p->ev_entry, hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&p->ev_side, hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&p->ev_c2, hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&p->ev_done, hipEventDisableTiming);
  if (err != hipSuccess) {
    hip_err(err, "creating the plan's streams and events");
    const int st = g_status;
    const std::string msg = g_msg;
    agmm_plan_destroy(p);
    set_err(st, "%s", msg.c_str());
    return nullptr;
  }
  if (apply(p, Settings{}) != AGMM_OK) {
    const int st = g_status;
    const std::string msg = g_msg;
    agmm_plan_destroy(p);
    set_err(st, "%s", msg.c_str());
    return nullptr;
  }
  ok();
  return p;
}

int agmm_plan_set_int(agmm_plan_t p, const char* key, int64_t v) {
  if (!p) return set_err(AGMM_ERR_INVALID_ARG, "plan is NULL");
  if (!key) return set_err(AGMM_ERR_INVALID_ARG, "key is NULL");
  std::lock_guard<std::mutex> lk(p->mu);
  if (p->broken != AGMM_OK) return set_err(p->broken, "plan is unusable: %s", p->broken_msg.c_str());
  // A graph that captured a call holds the workspace addresses and tile
  // tables of the plan's current layout; changing it would leave that graph
  // reading freed or rewritten memory.
  if (p->captured)
    return set_err(AGMM_ERR_UNSUPPORTED,
                   "the plan has been captured into a graph; its settings are fixed (create a new plan)");
  const std::string k(key);
  Settings s = p->s;
  auto bad = [&]() {
    return set_err(AGMM_ERR_INVALID_ARG, "value %lld out of range for key '%s'", (long long)v, key);
  };
  if (k == "variant") {
    if (v < AGMM_VARIANT_AUTO || v > AGMM_VARIANT_SKINNY) return bad();
    s.variant = (int)v;
  } else if (k == "pvalue") {
    if (v < 1 || v > (1 << 20)) return bad();
    s.pvalue = (int)v;
  } else if (k == "nbuf") {
    if (v < 1 || v > 64) return bad();
    s.nbuf = (int)v;
  } else if (k == "tile") {
    if (v < -1 || v >= agmm::kTileCount) return bad();
    s.tile = (int)v;
  } else if (k == "splits") {
    if (v < 0 || v > 4096) return bad();
    s.splits = (int)v;
  } else if (k == "local_shard") {
    if (v < 0 || v >= p->N) return bad();
    s.local_shard = (int)v;
  } else if (k == "order") {
    if (v != 0 && v != 1) return bad();
    s.order = (int)v;
  } else if (k == "group_m") {
    if (v < 0 || v > 1 << 20) return bad();
    s.group_m = (int)v;
  } else if (k == "xcd_remap") {
    if (v != 0 && v != 1) return bad();
    s.xcd_remap = (int)v;
  } else if (k == "local_first") {
    if (v != 0 && v != 1) return bad();
    s.local_first = (int)v;
  } else if (k == "gemm_streams") {
    if (v < 1 || v > 2) return bad();
    s.gemm_streams = (int)v;
  } else if (k == "lda" || k == "ldb" || k == "ldc") {
    // 0 restores the dense default; otherwise at least the row length, and
    // A / B rows 16-byte aligned for the vector and direct-to-LDS loads
    // (not needed where the rows go through the element-granular padded copy)
    const int64_t e = elem_bytes(p->dtype);
    const int64_t row = k == "lda" ? p->k : k == "ldc" ? p->n : (p->rt ? p->k : p->n);
    const bool any_ld = k == "ldc" || needs_pad(p->dtype, p->k, p->n, p->rt);
    if (v != 0 && (v < row || v >= kDimLimit || (!any_ld && (v * e) % 16 != 0))) return bad();
    (k == "lda" ? s.lda : k == "ldb" ? s.ldb : s.ldc) = v;
  } else if (k == "copy_wgs") {
    if (v < 0 || v > 1 << 20) return bad();
    s.copy_wgs = (int)v;
  } else if (k == "skinny_shape") {
    if (v < -1 || v >= kSkinnyShapes) return bad();
    s.skinny_shape = (int)v;
  } else if (k == "copy_engine") {
    if (v < 0 || v > 1) return bad();
    s.copy_engine = (int)v;
  } else if (k == "gather_out") {
    if (v < 0 || v > 2) return bad();
    s.gather_out = (int)v;
  } else if (k == "debug_keep_slots") {
    if (v != 0 && v != 1) return bad();
    s.debug_keep_slots = (int)v;
  } else if (k == "b_transpose") {
    if (v < -1 || v > 1) return bad();
    s.b_transpose = (int)v;
  } else {
    return set_err(AGMM_ERR_INVALID_ARG, "unknown key '%s'", key);
  }
  return apply(p, s);
}

int agmm_plan_get_int(agmm_plan_t p, const char* key, int64_t* value) {
  if (!p || !key || !value) return set_err(AGMM_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(p->mu);
  const std::string k(key);
  const Settings& s = p->s;
  const Layout& L = p->L;
  int64_t v;
  if (k == "variant") v = s.variant;
  else if (k == "variant_used") v = L.variant_used;
  else if (k == "pvalue") v = s.pvalue;
  else if (k == "nbuf") v = s.nbuf;
  else if (k == "tile") v = L.tile_used;
  else if (k == "splits") v = L.splits_used;
  else if (k == "local_shard") v = s.local_shard;
  else if (k == "order") v = s.order;
  else if (k == "group_m") v = s.group_m;
  else if (k == "group_m_used")   // for a launch over the whole problem
    v = s.group_m > 0 ? s.group_m : pick_group_m(cdiv(p->m, L.bm), cdiv(p->n, L.bn));
  else if (k == "xcd_remap") v = s.xcd_remap;
  else if (k == "copy_wgs") v = s.copy_wgs;
  else if (k == "copy_engine") v = s.copy_engine;
  else if (k == "gather_out") v = s.gather_out;
  else if (k == "skinny_shape") v = L.skinny_shape_used;
  else if (k == "lda") v = lda_of(p);
  else if (k == "ldb") v = ldb_of(p);
  else if (k == "ldc") v = ldc_of(p);
  else if (k == "gemm_streams") v = s.gemm_streams;
  else if (k == "local_first") v = s.local_first;
  else if (k == "debug_keep_slots") v = s.debug_keep_slots;
  else if (k == "b_transpose") v = s.b_transpose;
  else if (k == "b_transposed") v = L.bt ? 1 : 0;
  else if (k == "num_chunks") v = L.num_chunks;
  else if (k == "rows_per_chunk") v = L.rows_per_chunk;
  else if (k == "num_slots") v = L.nslots;
  else if (k == "tile_bm") v = L.bm;
  else if (k == "tile_bn") v = L.bn;
  else if (k == "k_per_split") v = L.k_per_split;
  else if (k == "num_row_blocks") v = L.order_len.empty() ? 0 : L.order_len[0];
  else if (k == "cu_count") v = p->cu_count;
  else if (k == "captured") v = p->captured ? 1 : 0;
  else if (k == "usable") v = p->broken == AGMM_OK ? 1 : 0;
  else return set_err(AGMM_ERR_INVALID_ARG, "unknown key '%s'", key);
  *value = v;
  return ok();
}

size_t agmm_plan_workspace_bytes(agmm_plan_t p) { return p ? p->ws_cap : 0; }

const void* agmm_plan_slot_ptr(agmm_plan_t p, int slot) {
  if (!p || !p->ring || slot < 0 || slot >= p->L.nslots) return nullptr;
  return p->ring + (size_t)slot * p->L.slot_bytes;
}

int agmm_plan_tile_order(agmm_plan_t p, int chunk, int32_t* out, int capacity) {
  if (!p || !out || chunk < 0 || chunk >= (int)p->L.order_len.size()) {
    set_err(AGMM_ERR_INVALID_ARG, "bad arguments to agmm_plan_tile_order");
    return -1;
  }
  const int len = p->L.order_len[chunk];
  if (capacity < len) {
    set_err(AGMM_ERR_INVALID_ARG, "capacity %d < %d row blocks", capacity, len);
    return -1;
  }
  std::memcpy(out, p->L.h_order.data() + p->L.order_off[chunk], sizeof(int32_t) * len);
  ok();
  return len;
}

int agmm_run(agmm_plan_t p, const void* const* shard_ptrs, const void* B, void* C, void* stream) {
  int rc = check_ptrs(p, shard_ptrs, B, C);
  if (rc != AGMM_OK) return rc;
  std::lock_guard<std::mutex> lk(p->mu);
  return guarded(p, static_cast<hipStream_t>(stream),
                 [&](const Call& c) { return run_plan(p, c, shard_ptrs, B, C); });
}

int agmm_plan_autotune(agmm_plan_t p, const void* const* shard_ptrs, const void* B, void* C,
                       void* stream, int iters, double* best_ms) {
  int rc = check_ptrs(p, shard_ptrs, B, C);
  if (rc != AGMM_OK) return rc;
  if (iters < 1 || iters > 1000) return set_err(AGMM_ERR_INVALID_ARG, "iters must be in [1, 1000]");
  std::lock_guard<std::mutex> lk(p->mu);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cst = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cst) != hipSuccess) return hip_err(hipGetLastError(), "hipStreamIsCapturing");
  if (cst != hipStreamCaptureStatusNone || p->captured)
    return set_err(AGMM_ERR_UNSUPPORTED,
                   "autotuning times real runs and reconfigures the plan: not under graph capture, "
                   "nor on a plan a graph has captured");
  Call c;
  rc = enter(p, s, c);
  if (rc != AGMM_OK) return rc;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  if (err != hipSuccess) {
    if (e0) hipEventDestroy(e0);
    return hip_err(err, "hipEventCreate");
  }
  // time the current configuration: warm-up run, then `iters` runs
  auto time_current = [&](double& ms) -> int {
    int r = run_plan(p, c, shard_ptrs, B, C);
    if (r != AGMM_OK) return r;
    if (hipEventRecord(e0, s) != hipSuccess) return hip_err(hipGetLastError(), "hipEventRecord");
    for (int i = 0; i < iters && r == AGMM_OK; ++i) r = run_plan(p, c, shard_ptrs, B, C);
    if (r != AGMM_OK) return r;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
      return hip_err(hipGetLastError(), "hipEventSynchronize");
    float f = 0.f;
    hipEventElapsedTime(&f, e0, e1);
    ms = (double)f / iters;
    return AGMM_OK;
  };
  // the runs above are all on `s`; apply() waits for the plan's last call,
  // so mark `s` as where it happened
  auto mark_done = [&]() { return leave(p, c); };
  // let the clocks settle before the first candidate is timed (they take
  // more than ~10 ms of load to ramp; the first timing would otherwise lose)
  {
    const auto t0 = std::chrono::steady_clock::now();
    do {
      rc = run_plan(p, c, shard_ptrs, B, C);
      if (rc == AGMM_OK && hipStreamSynchronize(s) != hipSuccess)
        rc = hip_err(hipGetLastError(), "hipStreamSynchronize");
    } while (rc == AGMM_OK &&
             std::chrono::steady_clock::now() - t0 < std::chrono::milliseconds(100));
  }
  double best = 1e300;
  if (rc == AGMM_OK && is_f32(p)) {
    rc = time_current(best);
  } else if (rc == AGMM_OK) {
    const Settings base = p->s;
    Settings best_s = base;
    // candidate settings of the plan's variant; configurations that resolve
    // to the same (tile, splits, group) are timed once
    std::vector<int> tiles = {agmm::kTile256x256m16, agmm::kTile256x256r5, agmm::kTile256x256,
                              agmm::kTile256x128,    agmm::kTile128x128m16, agmm::kTile128x128r5,
                              agmm::kTile128x128};
    if (p->rt || p->L.bt) {   // tiles that read B as n x k only
      tiles.insert(tiles.begin(), agmm::kTile256x224m16);
      if (p->rt) tiles.insert(tiles.begin(), agmm::kTileSkinny);
      tiles.push_back(agmm::kTile128x64r5);
      tiles.push_back(agmm::kTile128x64);
      tiles.push_back(agmm::kTile128x64s8);
    }
    const int splits_c[] = {0, 1, 2, 4, 8};
    const int groups_c[] = {4, 8};
    std::vector<std::array<int, 4>> seen;
    struct Timed {
      double ms;
      Settings s;
    };
    std::vector<Timed> timed;
    // the skinny tile also over its 32 x 32 and 64 x 64 shapes
    const int shapes_skinny[] = {5, 7}, shapes_other[] = {-1};
    // a candidate whose workspace could not be allocated, with the previous
    // one not restorable either, leaves the plan unusable: stop there
    for (int t : tiles)
      for (int sh : t == agmm::kTileSkinny ? std::vector<int>(std::begin(shapes_skinny), std::end(shapes_skinny))
                                           : std::vector<int>(std::begin(shapes_other), std::end(shapes_other)))
      for (int sp : splits_c)
        for (int gm : groups_c) {
          if (p->broken != AGMM_OK) continue;
          Settings s2 = base;
          s2.tile = t;
          s2.splits = sp;
          s2.group_m = gm;
          if (sh >= 0) s2.skinny_shape = sh;
          if (mark_done() != AGMM_OK || apply(p, s2) != AGMM_OK) continue;
          // the skinny kernel has its own tile order (no group_m)
          const bool sk = p->L.tile_used == agmm::kTileSkinny;
          const std::array<int, 4> key = {p->L.tile_used, p->L.splits_used, sk ? -1 : p->s.group_m,
                                          sk ? p->L.skinny_shape_used : -1};
          if (std::find(seen.begin(), seen.end(), key) != seen.end()) continue;
          seen.push_back(key);
          double ms = 0;
          if (time_current(ms) != AGMM_OK) {
            (void)hipGetLastError();
            continue;
          }
          timed.push_back({ms, s2});
        }
    // A few runs per candidate leave a few percent of noise (clock and power
    // drift on this GPU), more than the gap between the best candidates: the
    // best three are timed again, three rounds each, interleaved, and the
    // lowest mean over the rounds wins.
    std::sort(timed.begin(), timed.end(),
              [](const Timed& a, const Timed& b) { return a.ms < b.ms; });
    if (timed.size() > 3) timed.resize(3);
    std::vector<double> sum(timed.size(), 0.0);
    std::vector<int> cnt(timed.size(), 0);
    for (int round = 0; round < 3 && timed.size() > 1 && p->broken == AGMM_OK; ++round)
      for (size_t i = 0; i < timed.size() && p->broken == AGMM_OK; ++i) {
        double ms = 0;
        if (mark_done() != AGMM_OK || apply(p, timed[i].s) != AGMM_OK) continue;
        if (time_current(ms) != AGMM_OK) {
          (void)hipGetLastError();
          continue;
        }
        sum[i] += ms;
        ++cnt[i];
      }
    for (size_t i = 0; i < timed.size(); ++i) {
      const double ms = cnt[i] > 0 ? sum[i] / cnt[i] : timed[i].ms;
      if (ms < best) {
        best = ms;
        best_s = timed[i].s;
      }
    }
    rc = mark_done();
    if (rc == AGMM_OK && p->broken == AGMM_OK) rc = apply(p, best_s);
    else if (p->broken != AGMM_OK) rc = set_err(p->broken, "plan is unusable: %s", p->broken_msg.c_str());
    if (rc == AGMM_OK && best >= 1e300) rc = set_err(AGMM_ERR_HIP, "no candidate configuration ran");
  }
  const int rl = leave(p, c);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (rc != AGMM_OK) return rc;
  if (rl != AGMM_OK) return rl;
  if (best_ms) *best_ms = best;
  return ok();
}

int agmm_gather(agmm_plan_t p, const void* const* shard_ptrs, void* gathered, void* stream) {
  if (!p) return set_err(AGMM_ERR_INVALID_ARG, "plan is NULL");
  if (!shard_ptrs) return set_err(AGMM_ERR_INVALID_ARG, "shard_ptrs is NULL");
  if (!gathered) return set_err(AGMM_ERR_INVALID_ARG, "gathered is NULL");
  if (!aligned16(gathered)) return set_err(AGMM_ERR_UNSUPPORTED, "gathered is not 16-byte aligned");
  for (int r = 0; r < p->N; ++r) {
    if (!shard_ptrs[r]) return set_err(AGMM_ERR_INVALID_ARG, "shard_ptrs[%d] is NULL", r);
    if (!aligned16(shard_ptrs[r]))
      return set_err(AGMM_ERR_UNSUPPORTED, "shard_ptrs[%d] is not 16-byte aligned", r);
  }
  std::lock_guard<std::mutex> lk(p->mu);
  // no workspace is used: nothing to order against the plan's other calls
  const int rc = gather_rows(p, shard_ptrs, gathered, 0, static_cast<hipStream_t>(stream));
  return rc == AGMM_OK ? ok() : rc;
}

int agmm_run_gathered(agmm_plan_t p, const void* gathered, const void* B, void* C, void* stream) {
  if (!p) return set_err(AGMM_ERR_INVALID_ARG, "plan is NULL");
  if (!gathered || !B || !C) return set_err(AGMM_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned16(gathered) || !aligned16(B) || !aligned16(C))
    return set_err(AGMM_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  std::lock_guard<std::mutex> lk(p->mu);
  return guarded(p, static_cast<hipStream_t>(stream), [&](const Call& c) {
    if (p->L.padded) return run_padded(p, c, nullptr, gathered, B, C);
    const int rtb = transpose_b(p, B, c.s);
    if (rtb != AGMM_OK) return rtb;
    agmm::GemmProblem g = base_problem(p, dense_rows(gathered, p->m, p->k), p->m, B, C, -1);
    with_splits(p, g);
    return launch_gemm(p, c, g, c.s);
  });
}

int agmm_run_gather_out(agmm_plan_t p, const void* const* shard_ptrs, const void* B, void* C,
                        void* gathered, void* stream) {
  int rc = check_ptrs(p, shard_ptrs, B, C);
  if (rc != AGMM_OK) return rc;
  if (!gathered) return set_err(AGMM_ERR_INVALID_ARG, "gathered is NULL");
  if (!aligned16(gathered)) return set_err(AGMM_ERR_UNSUPPORTED, "gathered is not 16-byte aligned");
  std::lock_guard<std::mutex> lk(p->mu);
  return guarded(p, static_cast<hipStream_t>(stream), [&](const Call& c) -> int {
    const int copy_wgs = p->s.copy_wgs > 0 ? p->s.copy_wgs : p->cu_count;
    if (p->L.padded) {
      // the gathered output keeps rows of k elements; the GEMM runs on the
      // padded copies
      const int r = gather_rows(p, shard_ptrs, gathered, 0, c.s);
      return r != AGMM_OK ? r : run_padded(p, c, shard_ptrs, nullptr, B, C);
    }
    const int rtb = transpose_b(p, B, c.s);
    if (rtb != AGMM_OK) return rtb;
    switch (p->L.variant_used) {
      case AGMM_VARIANT_STAGED:
        return run_staged(p, c, shard_ptrs, B, C, gathered);
      case AGMM_VARIANT_UNFUSED: {
        // the gather is the first half of this variant anyway
        int r = gather_chunk(p, shard_ptrs, 0, p->m_s, gathered, p->m_s, 0, c.s);
        if (r != AGMM_OK) return r;
        agmm::GemmProblem g = base_problem(p, dense_rows(gathered, p->m, p->k), p->m, B, C, -1);
        with_splits(p, g);
        return launch_gemm(p, c, g, c.s);
      }
      default: {
        // fused / skinny / fp32.  Sequential (the automatic choice): gather
        // into `gathered` on the caller's stream, then the GEMM reads it (same
        // tile and k order: the same C as from the shards).  Measured (ms per
        // call, sequential against the copy beside the GEMM on the CUs / on
        // the SDMA engines): 8x4096x8192 -> 7168 bf16 2.995 / 3.357 / 3.104
        // (the chip is power-limited under MFMA load, so a concurrent copy
        // slows the GEMM by more than the copy costs alone); 8x16x4096 ->
        // 1792 bf16 (eager) 0.032 / 0.101 / 0.119.
        const bool sequential = p->s.gather_out != 1;
        if (sequential) {
          int r = gather_rows(p, shard_ptrs, gathered, 0, c.s);
          if (r != AGMM_OK) return r;
          agmm::GemmProblem g = base_problem(p, dense_rows(gathered, p->m, p->k), p->m, B, C, 0);
          with_splits(p, g);
          return launch_gemm(p, c, g, c.s);
        }
        // side copy: the GEMM reads the shards on the caller's stream while
        // the copy stream writes the gathered operand; the caller's stream
        // then waits for the copy
        int r = fork_to(p, c, p->copy_stream);
        if (r != AGMM_OK) return r;
        r = copy_on_sdma(p, c, true)
                ? gather_chunk_sdma(p, shard_ptrs, 0, p->m_s, gathered, p->m_s, p->copy_stream)
                : gather_rows(p, shard_ptrs, gathered, copy_wgs, p->copy_stream);
        if (r == AGMM_OK) {
          agmm::GemmProblem g = base_problem(p, shard_rows(p, shard_ptrs), p->m, B, C, 0);
          with_splits(p, g);
          r = launch_gemm(p, c, g, c.s);
        }
        const int rj = join_from(c, p->copy_stream, p->ev_side);
        return r != AGMM_OK ? r : rj;
      }
    }
  });
}

int agmm_plan_timing_begin(agmm_plan_t p) {
  if (!p) return set_err(AGMM_ERR_INVALID_ARG, "plan is NULL");
  std::lock_guard<std::mutex> lk(p->mu);
  while (p->tev.size() < 2 * (size_t)kTimingPairs) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return hip_err(err, "hipEventCreate");
    p->tev.push_back(e);
  }
  p->tev_used = 0;
  p->timing = true;
  return ok();
}

int agmm_plan_timing_read(agmm_plan_t p, double* total_ms, int64_t* launches) {
  if (!p || !total_ms || !launches) return set_err(AGMM_ERR_INVALID_ARG, "NULL argument");
  std::lock_guard<std::mutex> lk(p->mu);
  double sum = 0.0;
  for (int i = 0; i + 1 < p->tev_used; i += 2) {
    hipError_t err = hipEventSynchronize(p->tev[i + 1]);
    if (err != hipSuccess) return hip_err(err, "hipEventSynchronize");
    float ms = 0.0f;
    err = hipEventElapsedTime(&ms, p->tev[i], p->tev[i + 1]);
    if (err != hipSuccess) return hip_err(err, "hipEventElapsedTime");
    sum += ms;
  }
  *total_ms = sum;
  *launches = p->tev_used / 2;
  return ok();
}

int agmm_plan_timing_end(agmm_plan_t p) {
  if (!p) return set_err(AGMM_ERR_INVALID_ARG, "plan is NULL");
  std::lock_guard<std::mutex> lk(p->mu);
  p->timing = false;
  return ok();
}

void agmm_plan_destroy(agmm_plan_t p) {
  if (!p) return;
  {
    std::lock_guard<std::mutex> lk(p->mu);
    // the plan's own work: its last call (which the internal streams joined)
    // and anything still queued on the internal streams
    if (p->done_state == kDoneEager && p->ev_done) hipEventSynchronize(p->ev_done);
    if (p->copy_stream) hipStreamSynchronize(p->copy_stream);
    if (p->compute2) hipStreamSynchronize(p->compute2);
    (void)hipGetLastError();
  }
  if (p->ws) hipFree(p->ws);
  for (hipEvent_t e : p->ev_ready) hipEventDestroy(e);
  for (hipEvent_t e : p->ev_free) hipEventDestroy(e);
  for (hipEvent_t e : p->tev) hipEventDestroy(e);
  for (hipEvent_t e : {p->ev_entry, p->ev_side, p->ev_c2, p->ev_done})
    if (e) hipEventDestroy(e);
  if (p->compute2) hipStreamDestroy(p->compute2);
  if (p->copy_stream) hipStreamDestroy(p->copy_stream);
  delete p;
}

int agmm_run_noalloc(int num_shards, int64_t m_per_shard, int64_t k, int64_t n_local, int dtype,
                     int rhs_transpose, const void* const* shard_ptrs, const void* B, void* C,
                     void* stream) {
  static_assert(AGMM_NOALLOC_SCRATCH_BYTES == agmm::kNoallocScratchBytes, "scratch size");
  int rc = validate(num_shards, m_per_shard, k, n_local, dtype, rhs_transpose);
  if (rc != AGMM_OK) return rc;
  // a plan on the stack: the problem and a default launch layout, no
  // workspace, no streams, no events, no tile-order table
  agmm_plan p;
  p.N = num_shards;
  p.m_s = m_per_shard;
  p.k = k;
  p.n = n_local;
  p.m = (int64_t)num_shards * m_per_shard;
  p.dtype = dtype;
  p.rt = rhs_transpose;
  p.s.b_transpose = 0;   // the transposed copy of B needs a plan's workspace
  rc = check_ptrs(&p, shard_ptrs, B, C);
  if (rc != AGMM_OK) return rc;
  hipError_t err = hipGetDevice(&p.device);
  if (err != hipSuccess) return hip_err(err, "hipGetDevice");
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p.device) == hipSuccess && cus > 0)
    p.cu_count = cus;
  rc = derive_launch(&p, p.s, p.L);
  if (rc != AGMM_OK) return rc;
  if (p.L.padded)
    return set_err(AGMM_ERR_UNSUPPORTED,
                   "rows that are not whole 16-byte vectors run on padded copies, which need a "
                   "plan's workspace (use a plan)");
  if (p.L.variant_used != AGMM_VARIANT_FUSED && p.L.variant_used != AGMM_VARIANT_SKINNY)
    return set_err(AGMM_ERR_UNSUPPORTED, "agmm_run_noalloc runs the fused and skinny paths only");
  if (p.L.part_bytes > AGMM_NOALLOC_SCRATCH_BYTES)
    return set_err(AGMM_ERR_UNSUPPORTED,
                   "this problem's split-K partial sums need %zu bytes of scratch; the "
                   "no-allocation entry point has %zu (use a plan)",
                   p.L.part_bytes, (size_t)AGMM_NOALLOC_SCRATCH_BYTES);
  if (p.L.part_bytes > 0) {
    void* scratch = nullptr;
    err = agmm::noalloc_scratch(&scratch);
    if (err != hipSuccess) return hip_err(err, "locating the no-allocation scratch");
    p.partials = static_cast<float*>(scratch);
  }
  // every partial sum a launch reads was written by that launch's own split
  // workgroups first, so the scratch needs no clearing between calls
  Call c;
  c.s = static_cast<hipStream_t>(stream);
  agmm::GemmProblem g = base_problem(&p, shard_rows(&p, shard_ptrs), p.m, B, C, -1);
  with_splits(&p, g);
  rc = launch_gemm(&p, c, g, c.s);
  return rc == AGMM_OK ? ok() : rc;
}

int agmm_last_status(void) { return g_status; }

const char* agmm_last_error(void) { return g_msg.c_str(); }

const char* agmm_version(void) { return "agmm 0.2.0 (gfx950)"; }

}  // extern "C"
