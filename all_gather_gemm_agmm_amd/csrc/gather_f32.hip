// Gather copy and the fp32-input GEMM of the all-gather matmul (gfx950).
//
// Gather: the staged path first copies each shard's rows into a dense buffer
// (a ring slot, or the whole gathered operand for the unfused path).  This is
// the single-GPU stand-in for the pages' data movement: the tpu-inference
// kernel's HBM->VMEM x copies per received shard (`_all_gather_kernel`, the
// local x copies), and the Ascend tutorial's phase-2 local copy of A into the
// symmetric buffer in COMM_BLOCK tiles ("Two-Phase Pipeline").  Here it is a
// plain bit copy with 16-byte vector loads/stores, several in flight per lane.
//
// fp32 GEMM: the same contraction for fp32 inputs.  The products of two fp32
// values are exact in fp64 and the sum runs in fp64, then the result is
// rounded once to fp32; an fp32 accumulator cannot meet a 1e-5 relative bound
// on outputs near zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "agmm_kernels.h"

namespace agmm {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;

// Work items of the gather: one workgroup copies 256 consecutive 16-byte
// chunks of one row (rows of at least 256 chunks), or whole rows packed
// 256 / chunks-per-row to a workgroup (shorter rows).
struct CopyShape {
  int64_t cpr;     // 16-byte chunks per row
  int64_t bpr;     // workgroup items per row (long rows), else 0
  int64_t rpw;     // rows per workgroup item (short rows), else 0
  int64_t items;
};

__host__ __device__ inline CopyShape copy_shape(const GatherProblem& p) {
  CopyShape c;
  c.cpr = p.row_bytes >> 4;
  const int64_t rows_total = p.rows * p.num_groups;
  if (c.cpr >= kCopyThreads) {
    c.bpr = (c.cpr + kCopyThreads - 1) / kCopyThreads;
    c.rpw = 0;
    c.items = rows_total * c.bpr;
  } else {
    c.bpr = 0;
    c.rpw = c.cpr > 0 ? kCopyThreads / c.cpr : 0;
    c.items = c.rpw > 0 ? (rows_total + c.rpw - 1) / c.rpw : 0;
  }
  return c;
}

// One 16-byte chunk per thread.  A grid of one workgroup per item sweeps
// the source and the destination front to back, 4 KiB per workgroup
// (measured on an 8 x 64 MiB -> 512 MiB gather: 162 us, 6.6 TB/s of
// traffic, against 182-190 us for four chunks per thread a quarter of the
// copy apart, and 184 us for a grid-stride loop over 8192 workgroups); a
// capped grid (max_workgroups) walks the items in strides.
// NT: non-temporal stores, for copies larger than the 256 MiB MALL; a
// smaller copy keeps ordinary stores (128 MiB: 41.5 against 42.0 us with
// NT), its destination still fits the MALL for the GEMM that reads it.
template <bool NT>
__global__ __launch_bounds__(kCopyThreads) void gather_kernel(GatherProblem p) {
  const CopyShape cs = copy_shape(p);
  const int64_t src_ld = p.src_ld_bytes ? p.src_ld_bytes : p.row_bytes;
  const int64_t rows_total = p.rows * p.num_groups;
  const int tid = threadIdx.x;
  // short rows: this thread's row within the item and chunk within the row
  const int64_t r_in = cs.rpw > 0 ? tid / cs.cpr : 0;
  const int64_t c_short = cs.rpw > 0 ? tid - r_in * cs.cpr : 0;
  for (int64_t it = blockIdx.x; it < cs.items; it += gridDim.x) {
    int64_t row, c;
    if (cs.bpr > 0) {
      row = it / cs.bpr;
      c = (it - row * cs.bpr) * kCopyThreads + tid;
      if (c >= cs.cpr) continue;
    } else {
      if (r_in >= cs.rpw) continue;
      row = it * cs.rpw + r_in;
      c = c_short;
      if (row >= rows_total) continue;
    }
    const int64_t g = row / p.rows;
    const int64_t t = row - g * p.rows;
    const char* src = static_cast<const char*>(p.src_group[g]) + (p.src_row0 + t) * src_ld + (c << 4);
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
    u32x4_t* d = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.dst) + (g * p.dst_group_rows + t) * p.row_bytes +
                                            (c << 4));
    if constexpr (NT) __builtin_nontemporal_store(v, d);
    else *d = v;
  }
}

// Element-granular row copy with zero fill (rows that are not whole 16-byte
// vectors: a k or n that is not a multiple of 8 16-bit elements).  Each
// thread assembles one 16-byte chunk of a destination row from element
// loads (consecutive threads take consecutive chunks, so a wave reads and
// writes contiguous runs) and stores it whole when the destination row is
// 16-byte aligned, element by element otherwise.
template <int E>
__global__ __launch_bounds__(256) void pad_copy_kernel(PadCopyProblem p) {
  typedef typename std::conditional<E == 2, uint16_t, uint32_t>::type elem_t;
  constexpr int V = 16 / E;                  // elements per 16-byte chunk
  const int64_t chunks = (p.dst_cols + V - 1) / V;
  const int64_t per_group = chunks * p.rows;
  const int64_t total = per_group * p.num_groups;
  const bool vec_rows = ((p.dst_ld * E) % 16) == 0 && (reinterpret_cast<uintptr_t>(p.dst) & 15) == 0;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = u / per_group;
    const int64_t rem = u - g * per_group;
    const int64_t t = rem / chunks;
    const int64_t c0 = (rem - t * chunks) * V;
    const elem_t* src = static_cast<const elem_t*>(p.src_group[g]) + (p.src_row0 + t) * p.src_ld;
    const bool row_ok = t < p.src_rows;
    elem_t v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = (row_ok && c0 + j < p.cols) ? src[c0 + j] : elem_t(0);
    elem_t* dst = static_cast<elem_t*>(p.dst) + (g * p.dst_group_rows + t) * p.dst_ld + c0;
    if (vec_rows && c0 + V <= p.dst_cols) {
      u32x4_t w;
      __builtin_memcpy(&w, v, 16);
      *reinterpret_cast<u32x4_t*>(dst) = w;
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (c0 + j < p.dst_cols) dst[j] = v[j];
    }
  }
}

// fp32 GEMM: 64x64 output tile per workgroup, 256 threads, each thread a 4x4
// block; 16-deep k slices staged in LDS as double.
constexpr int kF32Tile = 64;
constexpr int kF32K = 16;

template <bool BT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmProblem p) {
  __shared__ double sa[kF32K][kF32Tile + 1];
  __shared__ double sb[kF32K][kF32Tile + 1];
  const int tid = threadIdx.x;
  const int M = p.m, N = p.n, K = p.k;
  const int num_cb = p.order.num_cb;
  const int tile = blockIdx.x;
  const int rbi = tile / num_cb;
  const int cb = tile - rbi * num_cb;
  const int rb = p.order.rb_order ? p.order.rb_order[rbi] : rbi;
  const int m0 = rb * kF32Tile, n0 = cb * kF32Tile;
  const int tr = tid / 16, tc = tid % 16;  // this thread: rows tr*4.., cols tc*4..

  // Row sources for the A loads: thread loads A rows m0 + (tid / 16) * 4 + i.
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < K; k0 += kF32K) {
    // A tile: 64 rows x 16 k -> 1024 values, 4 per thread.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + q * 256;
      const int r = idx / kF32K, kk = idx % kF32K;
      const int gi = m0 + r, gk = k0 + kk;
      double v = 0.0;
      if (gi < M && gk < K) {
        const int g = gi / p.rows.rows_per_group;
        const int t = gi - g * p.rows.rows_per_group;
        v = (double)static_cast<const float*>(p.rows.a_group[g])[(int64_t)t * p.rows.a_ld + gk];
      }
      sa[kk][r] = v;
    }
    // B tile: 16 k x 64 n.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + q * 256;
      int kk, c;
      if (BT) { c = idx / kF32K; kk = idx % kF32K; }
      else { kk = idx / kF32Tile; c = idx % kF32Tile; }
      const int gk = k0 + kk, gn = n0 + c;
      double v = 0.0;
      if (gk < K && gn < N) {
        const float* b = static_cast<const float*>(p.b);
        v = BT ? (double)b[(int64_t)gn * p.ldb + gk] : (double)b[(int64_t)gk * p.ldb + gn];
      }
      sb[kk][c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32K; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sa[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sb[kk][tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gi = m0 + tr * 4 + i;
    if (gi >= M) continue;
    const int g = gi / p.rows.rows_per_group;
    const int t = gi - g * p.rows.rows_per_group;
    const int64_t crow = (int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t;
    float* cp = static_cast<float*>(p.c) + crow * p.ldc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tc * 4 + j;
      if (gn < N) cp[gn] = (float)acc[i][j];
    }
  }
}

// 16-bit transpose: out[c][r] = in[r][c] for r < rows, c < cols (in: row
// stride ld_in elements; out: dense rows of `rows` elements).  Each wave
// covers a 64 x 64 tile; lane (8 * rb + cb) loads the 8 x 8 block at rows
// 8rb.., columns 8cb.. as 8 row pieces of 16 bytes (a wave's loads cover 8
// whole 128-byte row segments per instruction), transposes it in registers
// and stores 8 output row pieces of 16 bytes (again 128-byte segments per
// instruction).  rows and cols are multiples of 8, so a block is either
// wholly inside or wholly outside.  The source is read once (non-temporal
// loads); the destination keeps ordinary stores, so the GEMM that reads it
// next finds it in the MALL.
constexpr int kTrWaves = 4;
__global__ __launch_bounds__(64 * kTrWaves) void transpose16_kernel(const uint16_t* __restrict__ in,
                                                                    int64_t ld_in, int64_t rows,
                                                                    int64_t cols, int64_t tiles_c,
                                                                    int64_t tiles,
                                                                    uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * kTrWaves + (threadIdx.x >> 6);
  if (tile >= tiles) return;
  const int64_t tr = tile / tiles_c, tc = tile - tr * tiles_c;
  const int64_t r0 = tr * 64 + (lane >> 3) * 8, c0 = tc * 64 + (lane & 7) * 8;
  if (r0 >= rows || c0 >= cols) return;
  u32x4_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(in + (r0 + i) * ld_in + c0));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // output row c0 + j: element i is v[i] element j (16-bit half j & 1 of
    // 32-bit word j / 2); word d packs elements 2d (low half) and 2d + 1
    u32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = v[2 * d][j >> 1], hi = v[2 * d + 1][j >> 1];
      o[d] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    *reinterpret_cast<u32x4_t*>(out + (c0 + j) * rows + r0) = o;
  }
}

}  // namespace

hipError_t launch_gather(const GatherProblem& p, int max_workgroups, hipStream_t stream) {
  const int64_t total = (p.row_bytes >> 4) * p.rows * p.num_groups;
  if (total == 0) return hipSuccess;
  const CopyShape cs = copy_shape(p);
  int64_t wgs = cs.items;
  if (max_workgroups > 0 && wgs > max_workgroups) wgs = max_workgroups;
  if (wgs > (int64_t(1) << 30)) wgs = int64_t(1) << 30;   // larger copies stride
  if (wgs < 1) wgs = 1;
  constexpr int64_t kMallBytes = int64_t(256) << 20;
  if (total * 16 > kMallBytes)
    hipLaunchKernelGGL(gather_kernel<true>, dim3((unsigned)wgs), dim3(kCopyThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(gather_kernel<false>, dim3((unsigned)wgs), dim3(kCopyThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_pad_copy(const PadCopyProblem& p, hipStream_t stream) {
  if ((p.elem_bytes != 2 && p.elem_bytes != 4) || p.num_groups < 1 || p.num_groups > kMaxGroups ||
      p.rows < 0 || p.dst_cols < p.cols || p.dst_ld < p.dst_cols || p.cols < 0)
    return hipErrorInvalidValue;
  const int64_t chunks = (p.dst_cols + 16 / p.elem_bytes - 1) / (16 / p.elem_bytes);
  const int64_t total = chunks * p.rows * p.num_groups;
  if (total == 0) return hipSuccess;
  const int64_t wgs = std::min<int64_t>((total + 255) / 256, 8192);
  if (p.elem_bytes == 2)
    hipLaunchKernelGGL(pad_copy_kernel<2>, dim3((unsigned)wgs), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(pad_copy_kernel<4>, dim3((unsigned)wgs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_transpose16(const void* in, int64_t ld_in, int64_t rows, int64_t cols, void* out,
                              hipStream_t stream) {
  if (rows % 8 != 0 || cols % 8 != 0 || ld_in % 8 != 0 || ld_in < cols || rows < 0 || cols < 0 ||
      (reinterpret_cast<uintptr_t>(in) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 15) != 0)
    return hipErrorInvalidValue;
  const int64_t tiles_c = (cols + 63) / 64;
  const int64_t tiles = ((rows + 63) / 64) * tiles_c;
  if (tiles == 0) return hipSuccess;
  const int64_t wgs = (tiles + kTrWaves - 1) / kTrWaves;
  hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)wgs), dim3(64 * kTrWaves), 0, stream,
                     static_cast<const uint16_t*>(in), ld_in, rows, cols, tiles_c, tiles,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmProblem& p, bool rhs_transpose, hipStream_t stream) {
  const int ntiles = p.order.num_rb * p.order.num_cb;
  if (ntiles == 0) return hipSuccess;
  if (rhs_transpose)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(ntiles), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(ntiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace agmm
