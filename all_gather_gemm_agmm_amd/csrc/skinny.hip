// Skinny-m all-gather matmul on gfx950: C[m, n] = concat_r(A_r) @ B^T for
// small m (a few shards of a few rows, decode-like) with B stored n x k
// (tpu-inference "all_gather_matmul.py", `_do_mxu` with rhs_transpose: the
// dot_general contracts dimension 1 of both operands; fp32 accumulation over
// the k blocks, cast to the input dtype at the end).
//
// At these shapes the work is one pass over B, and a CU streams its operands
// at a fixed rate (about 26 bytes per clock here: the L2 reads one CU keeps
// in flight, over their latency), so the time is set by the bytes one CU
// reads.  Each workgroup takes a narrow tile (32 x 32 by default) over the
// whole of k when that gives every CU a workgroup: m = 128, n = 1792 gives
// 224 workgroups, each reading 256 KiB of B and 256 KiB of A (A's 1 MiB is
// shared by all workgroups through L2; B comes from HBM once, its column
// block shared by the 4 row blocks on one XCD).  No partials, one launch.
// With fewer tiles than CUs, or (64 x 64) to halve the bytes per CU where
// 32 x 32 tiles would take several rounds, the skinny_splitk_kernel form
// takes one of several k ranges and writes its fp32 sums; a second launch
// adds the ranges in a fixed order.
//
//  * The waves (4 or 8) take the k-tiles (64 deep) round robin and
//    accumulate separately; each streams its own k-tiles through a private
//    ring of LDS slots (160 KiB shared out; e.g. 5 slots of A 4 KiB + B 4 KiB
//    per wave for the 32 x 32 tile with 4 waves) with global -> LDS DMA, so the
//    main loop has no workgroup barrier: each wave waits only for its own
//    loads (vmcnt), and every slot is in flight (a slot is refilled as soon
//    as its k-tile has been read into registers).
//  * v_mfma_f32_16x16x32 with the B fragment first: each 16-lane group g
//    holds k elements [8g, 8g + 8) of a k32 step; 4 row blocks x 1 column
//    block per wave.  LDS rows of 128 bytes, chunk c of row r at
//    c ^ swz(r) (swz: bit 1 of r -> bit 0, bit 2 -> bit 2, bit 3 -> bit 1),
//    free of bank conflicts for these 16-row x 4-chunk fragment reads.
//  * The two row halves of a column block sit on the same XCD (workgroups
//    are dispatched round robin over the 8 XCDs; each XCD gets a contiguous
//    range of logical tiles), so B is fetched from HBM once.
//  * The wave partials are summed in LDS in wave order (fixed), cast with
//    round-to-nearest-even and stored through the row map.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "agmm_kernels.h"

namespace agmm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char_t;

// 16 zero bytes: the source of every out-of-range 16-byte chunk.
__device__ __attribute__((aligned(64))) const uint32_t sk_zero16[16] = {0};

constexpr int kKT = 64;                   // k elements per k-tile

// Shape of one tile configuration: ROWS x COLS outputs, 1 KiB DMAs per
// k-tile (8 rows of 128 bytes each), as many ring slots as fit in a wave's
// LDS share.
template <int ROWS, int COLS, int WAVES>
struct Shape {
  static constexpr int kWaves = WAVES;
  static constexpr int kWaveLds = 160 * 1024 / WAVES;   // LDS per wave: all 160 KiB shared out
  static constexpr int kRows = ROWS, kCols = COLS;
  static constexpr int kALoads = ROWS / 8, kBLoads = COLS / 8;
  static constexpr int kLoads = kALoads + kBLoads;
  static constexpr int kSlotBytes = kLoads * 1024;
  static constexpr int kSlots = kWaveLds / kSlotBytes < 8 ? kWaveLds / kSlotBytes : 8;
  static constexpr int kWaveBytes = kSlots * kSlotBytes;
  static_assert(ROWS % 16 == 0 && COLS % 16 == 0, "16x16 MFMA blocks");
  static_assert(kSlots >= 2, "ring");
  static_assert(kWaves * kWaveBytes <= 160 * 1024, "LDS");
  static_assert(kSlots * kLoads < 64, "loads in flight exceed vmcnt");
};

template <int DT>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t b, u32x4_t a, f32x4_t c) {
  if constexpr (DT == kDtypeBf16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                   __builtin_bit_cast(bf16x8_t, a), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, b),
                                                  __builtin_bit_cast(f16x8_t, a), c, 0, 0, 0);
  }
}

template <int DT>
__device__ __forceinline__ uint16_t to16(float v) {
  if constexpr (DT == kDtypeBf16) {
    __bf16 a = (__bf16)v;
    return __builtin_bit_cast(uint16_t, a);
  } else {
    _Float16 a = (_Float16)v;
    return __builtin_bit_cast(uint16_t, a);
  }
}

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 1) | (r & 4) | ((r >> 2) & 2); }

// One global -> LDS DMA: lane i writes bytes [16i, 16i + 16) of the 1 KiB
// block at LDS address `lds_addr` (wave-uniform).  Inline assembly so that
// the compiler does not wait for every such load before each LDS read; the
// kernel waits for exactly the k-tile it reads next.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "m0");
}

// vmcnt(n), other counters untouched (gfx9 encoding); nothing is scheduled
// or moved across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Logical row r of the row map -> (group, position), exact for r < 2^24.
__device__ __forceinline__ void split_row(int r, int rpg, float inv, int& g, int& t) {
  g = (int)((float)r * inv);
  t = r - g * rpg;
  if (t < 0) { --g; t += rpg; }
  if (t >= rpg) { ++g; t -= rpg; }
}

// vmcnt(after * kLoads) for a wave-uniform `after` in [0, kMax]
template <int kLoads, int kMax>
__device__ __forceinline__ void wait_tiles(int after) {
  if constexpr (kMax <= 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= kMax) wait_vmcnt<kMax * kLoads>();
    else wait_tiles<kLoads, kMax - 1>(after);
  }
}

// One output tile over one k range: the whole of k, or (SPLIT) k range
// `split` of p.splits, whose fp32 sums go to p.partials[split][row][col].
template <int DT, int ROWS, int COLS, int WAVES, bool SPLIT>
__device__ __forceinline__ void skinny_body(const GemmProblem& p) {
  using S = Shape<ROWS, COLS, WAVES>;
  constexpr int kWaves = S::kWaves, kThreads = 64 * WAVES;
  constexpr int kRows = S::kRows, kCols = S::kCols, kALoads = S::kALoads, kBLoads = S::kBLoads;
  constexpr int kLoads = S::kLoads, kSlotBytes = S::kSlotBytes, kSlots = S::kSlots;
  constexpr int kWaveBytes = S::kWaveBytes;
  constexpr int FM = kRows / 16, FN = kCols / 16;
  __shared__ __attribute__((aligned(1024))) char smem[kWaves * kWaveBytes];
  // the shard table is staged in the last 512 bytes of LDS (the last slot of
  // the last wave, first written after the barrier that follows its use)
  const char** s_groups = reinterpret_cast<const char**>(smem + kWaves * kWaveBytes - kMaxGroups * 8);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.m, N = p.n, K = p.k;
  const int RB = (M + kRows - 1) / kRows, CB = (N + kCols - 1) / kCols;
  // logical unit: XCD x (= workgroup id mod 8) gets a contiguous range, row
  // blocks fastest, so the row blocks of one column block share an XCD;
  // then column blocks, then k ranges (an XCD's units share few A slices)
  int tile, split = 0;
  {
    const int T = RB * CB * (SPLIT ? p.splits : 1), wg = blockIdx.x;
    const int xcd = wg & 7, local = wg >> 3, per = T >> 3, rem = T & 7;
    const int u = xcd * per + (xcd < rem ? xcd : rem) + local;
    tile = u % (RB * CB);
    if constexpr (SPLIT) split = u / (RB * CB);
  }
  const int rb = tile % RB, cb = tile / RB;
  const int row0 = rb * kRows, n0 = cb * kCols;
  // k range [kb, kend): multiples of the k-tile except at the end of k
  const int kb = SPLIT ? split * p.k_per_split : 0;
  const int kend = SPLIT ? min(K, kb + p.k_per_split) : K;
  const int nkt = kend > kb ? (kend - kb + kKT - 1) / kKT : 0;
  const int rpg = p.rows.rows_per_group;
  const float inv = 1.0f / (float)rpg;

  if (tid < p.rows.num_groups) s_groups[tid] = static_cast<const char*>(p.rows.a_group[tid]);
  __syncthreads();

  // DMA sources of this lane: A rows row0 + 8q + lane/8 (q < 8), B columns
  // n0 + 8q + lane/8 (q < 2); chunk (lane % 8) ^ swz(row) of each k-tile.
  const char* asrc[kALoads];
  uint32_t a_ok = 0;
#pragma unroll
  for (int q = 0; q < kALoads; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int gr = row0 + r;
    int g, t;
    split_row(gr, rpg, inv, g, t);
    g = min(max(g, 0), p.rows.num_groups - 1);
    const int c = (lane & 7) ^ swz(r);
    asrc[q] = s_groups[g] + ((int64_t)t * p.rows.a_ld + 8 * c) * 2;   // read only when gr < M
    a_ok |= (uint32_t)(gr < M) << q;
  }
  const char* bsrc[kBLoads];
  uint32_t b_ok = 0;
#pragma unroll
  for (int q = 0; q < kBLoads; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int gn = n0 + r;
    const int c = (lane & 7) ^ swz(r);
    bsrc[q] = static_cast<const char*>(p.b) + ((int64_t)gn * p.ldb + 8 * c) * 2;   // read only when gn < N
    b_ok |= (uint32_t)(gn < N) << q;
  }

  __syncthreads();   // every lane has read the shard table
  char* ring = smem + wave * kWaveBytes;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_char_t*)ring;

  // this wave's k-tiles: wave, wave + 4, ...
  const int nt = nkt > wave ? (nkt - wave + kWaves - 1) / kWaves : 0;
  auto issue = [&](int j) {   // k-tile number j of this wave into slot j % kSlots
    const int kk = kb + (wave + kWaves * j) * kKT;
    const uint32_t dst = ring_lds + (j % kSlots) * kSlotBytes;
#pragma unroll
    for (int q = 0; q < kALoads; ++q) {
      const int r = 8 * q + (lane >> 3);
      const int ke = kk + 8 * ((lane & 7) ^ swz(r));
      const void* src = (((a_ok >> q) & 1u) && ke < kend) ? (const void*)(asrc[q] + (int64_t)kk * 2)
                                                       : (const void*)sk_zero16;
      dma16(src, dst + q * 1024);
    }
#pragma unroll
    for (int q = 0; q < kBLoads; ++q) {
      const int r = 8 * q + (lane >> 3);
      const int ke = kk + 8 * ((lane & 7) ^ swz(r));
      const void* src = (((b_ok >> q) & 1u) && ke < kend) ? (const void*)(bsrc[q] + (int64_t)kk * 2)
                                                       : (const void*)sk_zero16;
      dma16(src, dst + (kALoads + q) * 1024);
    }
  };

  // fragment offsets: lane (g4, i16) reads row i16 of a 16-row block, chunk
  // 4 * step + g4
  const int g4 = lane >> 4, i16 = lane & 15;
  int a_off[FM], a_x[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int r = 16 * f + i16;
    a_off[f] = r * 128;
    a_x[f] = g4 ^ swz(r);
  }
  int b_off[FN], b_x[FN];   // B rows follow the A rows in a slot
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int r = 16 * f + i16;
    b_off[f] = (kRows + r) * 128;
    b_x[f] = g4 ^ swz(r);
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  // every slot in flight: k-tiles 0 .. kSlots-1 first, then slot j % kSlots
  // is refilled with k-tile j + kSlots as soon as k-tile j has been read
  const int pre = nt < kSlots ? nt : kSlots;
  for (int j = 0; j < pre; ++j) issue(j);
  for (int j = 0; j < nt; ++j) {
    // k-tiles issued after j and still allowed in flight
    wait_tiles<kLoads, kSlots - 1>(min(kSlots - 1, nt - 1 - j));
    const char* slot = ring + (j % kSlots) * kSlotBytes;
    // all of k-tile j's fragments into registers, the slot's refill issued,
    // then the MFMAs: the ring stays full while they run
    u32x4_t bf[2][FN], af[2][FM];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int f = 0; f < FN; ++f)
        bf[st][f] = *reinterpret_cast<const u32x4_t*>(slot + b_off[f] + (((4 * st) ^ b_x[f]) << 4));
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[st][i] = *reinterpret_cast<const u32x4_t*>(slot + a_off[i] + (((4 * st) ^ a_x[i]) << 4));
    }
    if (j + kSlots < nt) {
      lds_reads_done();   // k-tile j's fragments are in registers: its slot is free
      issue(j + kSlots);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f) acc[i][f] = mfma16<DT>(bf[st][f], af[st][i], acc[i][f]);
  }
  wait_vmcnt<0>();
  lds_reads_done();

  // wave partials -> own ring region: [ROWS][COLS] fp32, row stride COLS + 4
  // floats; lane (g4, i16) holds C[16i + i16][16f + 4 g4 .. +3] of block (i, f)
  constexpr int RLD = kCols + 4;
  static_assert(kRows * RLD * 4 <= kWaveBytes, "partial tile fits the wave's ring");
  float* red = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
      *reinterpret_cast<f32x4_t*>(red + (16 * i + i16) * RLD + 16 * f + 4 * g4) = acc[i][f];
  __syncthreads();
  // ROWS x COLS outputs, 4 consecutive columns per thread and pass
  constexpr int E4 = kRows * kCols / 4;
#pragma unroll
  for (int e4 = tid; e4 < E4; e4 += kThreads) {
  const int row = e4 / (kCols / 4), c4 = (e4 % (kCols / 4)) * 4;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(smem) + row * RLD + c4);
#pragma unroll
  for (int w = 1; w < kWaves; ++w)
    v += *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(smem + w * kWaveBytes) +
                                           row * RLD + c4);
  const int gr = row0 + row, gc = n0 + c4;
  if constexpr (SPLIT) {
    // fp32 sums of this k range, rows in launch order (the reduction maps
    // them to C)
    if (gr < M) {
      float* prow = p.partials + ((int64_t)split * M + gr) * N;
      if (gc + 3 < N && (N % 4) == 0) {
        *reinterpret_cast<f32x4_t*>(prow + gc) = v;
      } else {
        if (gc + 0 < N) prow[gc + 0] = v[0];
        if (gc + 1 < N) prow[gc + 1] = v[1];
        if (gc + 2 < N) prow[gc + 2] = v[2];
        if (gc + 3 < N) prow[gc + 3] = v[3];
      }
    }
    continue;
  }
  if (gr < M) {
    int g, t;
    split_row(gr, rpg, inv, g, t);
    uint16_t* crow = static_cast<uint16_t*>(p.c) + ((int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t) * p.ldc;
    const uint16_t o0 = to16<DT>(v[0]), o1 = to16<DT>(v[1]), o2 = to16<DT>(v[2]), o3 = to16<DT>(v[3]);
    if (gc + 3 < N && (p.ldc % 4) == 0) {
      *reinterpret_cast<u32x2_t*>(crow + gc) =
          u32x2_t{(uint32_t)o0 | ((uint32_t)o1 << 16), (uint32_t)o2 | ((uint32_t)o3 << 16)};
    } else {
      if (gc + 0 < N) crow[gc + 0] = o0;
      if (gc + 1 < N) crow[gc + 1] = o1;
      if (gc + 2 < N) crow[gc + 2] = o2;
      if (gc + 3 < N) crow[gc + 3] = o3;
    }
  }
  }
}

template <int DT, int ROWS, int COLS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void skinny_fullk_kernel(GemmProblem p) {
  skinny_body<DT, ROWS, COLS, WAVES, false>(p);
}

template <int DT, int ROWS, int COLS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void skinny_splitk_kernel(GemmProblem p) {
  skinny_body<DT, ROWS, COLS, WAVES, true>(p);
}

}  // namespace

template <int ROWS, int COLS, int WAVES = 4>
hipError_t launch_shape(const GemmProblem& p, int dtype, hipStream_t stream) {
  const int64_t tiles = (int64_t)((p.m + ROWS - 1) / ROWS) * ((p.n + COLS - 1) / COLS);
  const bool split = p.splits > 1;
  if (tiles * (split ? p.splits : 1) > (int64_t(1) << 30)) return hipErrorInvalidValue;
  if (split && (p.partials == nullptr || p.k_per_split < kKT || p.k_per_split % kKT != 0 ||
                (int64_t)p.splits * p.k_per_split < p.k))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles * (split ? p.splits : 1))), block(64 * WAVES);
  if (split) {
    if (dtype == kDtypeBf16)
      hipLaunchKernelGGL((skinny_splitk_kernel<kDtypeBf16, ROWS, COLS, WAVES>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((skinny_splitk_kernel<kDtypeFp16, ROWS, COLS, WAVES>), grid, block, 0, stream, p);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_splitk_reduce(p, dtype, stream);
  }
  if (dtype == kDtypeBf16)
    hipLaunchKernelGGL((skinny_fullk_kernel<kDtypeBf16, ROWS, COLS, WAVES>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((skinny_fullk_kernel<kDtypeFp16, ROWS, COLS, WAVES>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_skinny_fullk(const GemmProblem& p, int dtype, int shape, hipStream_t stream) {
  if (dtype != kDtypeBf16 && dtype != kDtypeFp16) return hipErrorInvalidValue;
  if (p.m < 1 || p.n < 1 || p.k < 1 || p.m >= (1 << 24) || p.rows.num_groups < 1 ||
      p.rows.num_groups > kMaxGroups)
    return hipErrorInvalidValue;
  switch (shape) {
    case 0: return launch_shape<64, 16>(p, dtype, stream);
    case 1: return launch_shape<32, 32>(p, dtype, stream);
    case 2: return launch_shape<32, 16>(p, dtype, stream);
    case 3: return launch_shape<16, 32>(p, dtype, stream);
    case 4: return launch_shape<64, 32>(p, dtype, stream);
    case 5: return launch_shape<32, 32, 8>(p, dtype, stream);
    case 6: return launch_shape<64, 16, 8>(p, dtype, stream);
    case 7: return launch_shape<64, 64>(p, dtype, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace agmm
