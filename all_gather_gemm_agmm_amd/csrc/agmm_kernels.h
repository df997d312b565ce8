// Internal interface between the plan/scheduler (agmm_api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/agmm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace agmm {

// Largest number of shard buffers one call can name.  The pointer table
// travels in the kernel arguments (8 bytes per entry).
constexpr int kMaxGroups = 64;

constexpr int kDtypeBf16 = 0;
constexpr int kDtypeFp16 = 1;
constexpr int kDtypeFp32 = 2;

// Row mapping shared by every kernel that reads the gathered operand.
//
// A launch covers m = num_groups * rows_per_group logical rows.  Logical row
// i belongs to group g = i / rows_per_group at position t = i % rows_per_group:
//   its A row starts at  a_group[g] + t * a_ld            (elements)
//   its C row is         g * c_group_rows + c_row_off + t
// The fused path passes the shard pointers themselves (one group per shard);
// a ring slot or the fully gathered buffer is described the same way.
struct RowMap {
  const void* a_group[kMaxGroups];
  int64_t a_ld;            // elements between consecutive rows of one group
  int32_t rows_per_group;  // rows of each group covered by this launch
  int32_t num_groups;
  int64_t c_group_rows;    // C rows between the starts of consecutive groups
  int64_t c_row_off;       // C row of position t = 0 inside each group
};

// Order in which workgroups visit output tiles.
struct TileOrder {
  const int32_t* rb_order;  // device table: visit order of row blocks (nullptr = natural)
  int32_t num_rb;           // row blocks  (ceil(m / BM))
  int32_t num_cb;           // column blocks (ceil(n / BN))
  int32_t group_m;          // row blocks walked together for L2 reuse
  int32_t xcd_remap;        // 1: keep consecutive tiles on one XCD
};

struct GemmProblem {
  RowMap rows;
  TileOrder order;
  int32_t m, n, k;
  const void* b;
  int64_t ldb;             // elements between rows of B as stored
  void* c;
  int64_t ldc;             // elements between rows of C
  // split-K (used when splits > 1): partial sums, then a reduction kernel
  int32_t splits;
  int32_t k_per_split;     // multiple of kTileBK
  float* partials;         // [splits][m][n] fp32 scratch
};

// Tile shapes compiled for the MFMA kernels.  Each one is reached by the
// plan's automatic choice or by the autotuner's candidate list.
enum TileCfg : int {
  kTile256x256 = 0,      // 4 waves, 128x128 per wave, 32-deep k-tiles in a 4-stage ring (k < 256)
  kTile128x128 = 1,      // 64x64 per wave, two workgroups per CU
  kTile256x128 = 2,      // 128x64 per wave, two workgroups per CU
  kTile128x64 = 3,       // 4 waves, 64x32 per wave; B stored n x k only
  kTile128x64s8 = 4,     // 8-stage LDS ring (whole short k ranges in flight); B stored n x k only
  kTile256x256r5 = 5,    // 64-deep k-tiles in a ring of 5 operand slots (whole L2 lines per load)
  kTile128x128r5 = 6,    // same ring, 128x128, two workgroups per CU
  kTile128x64r5 = 7,     // same ring, 128x64; B stored n x k only
  kTile256x256m16 = 8,   // part ring, 256x256, on 16x16x32 MFMAs (automatic for k >= 256)
  kTile128x128m16 = 9,   // part ring, 128x128, on 16x16x32 MFMAs
  kTileSkinny = 10,      // narrow tiles over all of k or k ranges, wave-private LDS rings (launch_skinny_fullk); B n x k only
  kTile256x224m16 = 11,  // part ring, 256x224 on 16x16x32 MFMAs (7 column blocks per wave); B n x k only
  kTileCount = 12,
};
// Tiles that read B only as stored n x k (rhs_transpose).
constexpr bool tile_needs_bt(int cfg) {
  return cfg == kTile128x64 || cfg == kTile128x64s8 || cfg == kTile128x64r5 || cfg == kTileSkinny ||
         cfg == kTile256x224m16;
}
int tile_bm(int cfg);
int tile_bn(int cfg);
int tile_bk(int cfg);
int tile_occ(int cfg);   // workgroups of this tile that fit on one CU
// k granularity of split-K ranges (a multiple of every configuration's depth)
constexpr int kTileBK = 64;

// bf16/fp16 MFMA GEMM (16-bit inputs, fp32 accumulate, output in the input dtype).
// With p.splits > 1 this is two launches on `stream`: fp32 partial sums per
// k range, then their fixed-order sum and cast.
hipError_t launch_gemm_mfma(const GemmProblem& p, int tile_cfg, int dtype, bool rhs_transpose,
                            hipStream_t stream);

// Skinny-m kernel (tile kTileSkinny, B stored n x k): small output tiles
// (32 x 32 by default), each over the whole of k in one workgroup (one
// launch), or with p.splits > 1 over one of p.splits k ranges of
// p.k_per_split elements (a multiple of 64) into p.partials [splits][m][n]
// fp32, then launch_splitk_reduce.  C rows through the row map.
// `shape` selects the tile: 0: 64 x 16, 1: 32 x 32, 2: 32 x 16, 3: 16 x 32,
// 4: 64 x 32, 7: 64 x 64 (rows x columns) with 4 waves; 5: 32 x 32 and 6:
// 64 x 16 with 8 waves (the LDS shared out over twice as many, half as
// deep, rings).
hipError_t launch_skinny_fullk(const GemmProblem& p, int dtype, int shape, hipStream_t stream);

// Fixed-order sum of p.partials [p.splits][p.m][p.n] fp32 (split 0 first),
// cast to the output dtype and stored to C through the row map.
hipError_t launch_splitk_reduce(const GemmProblem& p, int dtype, hipStream_t stream);

// fp32 inputs, fp64 accumulate, fp32 output (any shape).
hipError_t launch_gemm_f32(const GemmProblem& p, bool rhs_transpose, hipStream_t stream);

// Bit copy of rows into a dense destination:
//   dst[(g * dst_group_rows + t) * row_bytes ...] = src_group[g][(src_row0 + t) * src_ld_bytes ...]
// for g < num_groups, t < rows.  row_bytes % 16 == 0 and src_ld_bytes % 16 == 0
// (src_ld_bytes == 0: row_bytes), all pointers 16-byte aligned.
struct GatherProblem {
  const void* src_group[kMaxGroups];
  int32_t num_groups;
  int64_t src_row0;
  int64_t rows;
  int64_t row_bytes;
  int64_t src_ld_bytes;    // bytes between source rows (0: row_bytes)
  void* dst;
  int64_t dst_group_rows;
};
hipError_t launch_gather(const GatherProblem& p, int max_workgroups, hipStream_t stream);

// Element-granular copy of rows for rows that are not whole 16-byte vectors
// (any row length and strides), with zero fill:
//   dst[(g * dst_group_rows + t) * dst_ld + c] =
//       (t < src_rows && c < cols) ? src_group[g][(src_row0 + t) * src_ld + c] : 0
// for g < num_groups, t < rows, c < dst_cols.  Strides and lengths in
// elements of elem_bytes (2 or 4) bytes; pointers aligned to an element.
struct PadCopyProblem {
  const void* src_group[kMaxGroups];
  int32_t num_groups;
  int32_t elem_bytes;
  int64_t src_row0;
  int64_t src_rows;        // rows of each group that exist in the source (the rest are zeros)
  int64_t src_ld;
  int64_t cols;            // elements of a source row that are copied
  int64_t rows;            // rows written per group
  void* dst;
  int64_t dst_group_rows;
  int64_t dst_ld;
  int64_t dst_cols;        // elements written per row (zeros past cols)
};
hipError_t launch_pad_copy(const PadCopyProblem& p, hipStream_t stream);

// Transpose of a 16-bit matrix: out[c * rows + r] = in[r * ld_in + c] for
// r < rows, c < cols.  rows, cols and ld_in multiples of 8, both pointers
// 16-byte aligned (else hipErrorInvalidValue, nothing launched).
hipError_t launch_transpose16(const void* in, int64_t ld_in, int64_t rows, int64_t cols, void* out,
                              hipStream_t stream);

// Size of the device scratch of the no-allocation entry point (one per GPU,
// held for the life of the process; equal to AGMM_NOALLOC_SCRATCH_BYTES).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
// Device address of the current GPU's scratch (looked up on the first call
// on each device, then cached).
hipError_t noalloc_scratch(void** ptr);

}  // namespace agmm
