// bf16 / fp16 MFMA GEMM for the all-gather matmul on gfx950 (CDNA4).
//
// Computes, for the logical rows described by a RowMap (shard buffers, a ring
// slot or the fully gathered operand),
//     C[row, :] = A[row, :] @ B          (B stored k x n)
//     C[row, :] = A[row, :] @ B^T        (rhs_transpose: B stored n x k)
// with fp32 accumulation and a round-to-nearest-even cast to the input dtype
// (tpu-inference "all_gather_matmul.py", `_do_mxu`: jnp.dot / dot_general with
// preferred_element_type=float32 accumulated over bk slices, cast with
// astype(x.dtype) on the last slice; Triton-distributed-Ascend
// "AllGather-GEMM" kernel listing: fp32 accumulator over K blocks, cast on
// store).
//
// Design (MI355X-native, not a translation of either page):
//  * 256 threads = 4 waves of 64 lanes, 2x2 waves per output tile.
//  * v_mfma_f32_32x32x16_{bf16,f16}: the B tile is the MFMA's first operand
//    and the A tile its second, so each lane ends up owning 4 consecutive
//    output columns of one row (8-byte packed stores in the epilogue).
//  * A and k-contiguous B tiles go global -> LDS directly
//    (global_load_lds_dwordx4, no register staging).  B stored k x n is
//    loaded to registers in 8x8 blocks, transposed in registers and written
//    to LDS in the same k-contiguous layout.
//  * LDS rows are 64 elements (128 bytes, 8 chunks of 16 bytes); chunk c of
//    row r sits at position c ^ ((r ^ (r >> 3)) & 7), which keeps both the
//    MFMA fragment reads and the transposed B writes free of bank conflicts.
//  * Two LDS stages: the loads of k-tile i+1 are in flight while the MFMAs of
//    k-tile i run.
//  * Rows past m, columns past n and k past the end are fed from a zero
//    block, so ragged tails need no masking inside the main loop.
//  * Tile order: XCD-aware remap of the workgroup id, grouped row blocks for
//    L2 reuse, then the plan's row-block visit order (ring order from the
//    local shard, or natural order).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "agmm_kernels.h"

namespace agmm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 zero bytes: the source of every out-of-range 16-byte chunk.
__device__ __attribute__((aligned(64))) const uint32_t g_zero_chunk[16] = {0};

constexpr int kThreads = 256;
constexpr int kBK = kTileBK;        // 64 elements = 128 bytes per LDS row
constexpr int kRowBytes = kBK * 2;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int DT>
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (DT == kDtypeBf16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// fp32 -> 16-bit storage, round to nearest even (subnormals kept for fp16).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == kDtypeBf16) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  } else {
    _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
}

template <int DT>
__device__ __forceinline__ uint16_t cvt1(float v) {
  if constexpr (DT == kDtypeBf16) {
    __bf16 a = (__bf16)v;
    return __builtin_bit_cast(uint16_t, a);
  } else {
    _Float16 a = (_Float16)v;
    return __builtin_bit_cast(uint16_t, a);
  }
}

__device__ __forceinline__ void load_lds16(const void* gsrc, char* lds_base_uniform) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_base_uniform, 16, 0, 0);
}

// Logical tile visited by this workgroup.
__device__ __forceinline__ void tile_coords(const TileOrder& o, int wg, int nwg, int& rb, int& cb) {
  if (o.xcd_remap) {
    // Workgroups are dispatched round-robin over the 8 XCDs; give XCD x a
    // contiguous range of logical tiles so neighbours share its L2.
    const int xcd = wg & 7, local = wg >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    wg = xcd * per + (xcd < rem ? xcd : rem) + local;
  }
  const int gsz = o.group_m * o.num_cb;
  const int grp = wg / gsz;
  const int first = grp * o.group_m;
  const int rows_here = min(o.num_rb - first, o.group_m);
  const int in = wg - grp * gsz;
  const int rbi = first + in % rows_here;
  cb = in / rows_here;
  rb = o.rb_order ? o.rb_order[rbi] : rbi;
}

template <int BM, int BN, int DT, bool BT>
struct GemmTile {
  static constexpr int WM = 2, WN = 2;
  static constexpr int TM = BM / WM, TN = BN / WN;     // per-wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;     // 32x32 MFMA blocks per wave
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BN * kRowBytes;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int A_IPW = BM / 32;                // 8-row load instructions per wave for A
  static constexpr int B_IPW = BN / 32;                // same for k-contiguous B
  static constexpr int NN_BLOCKS = 8 * (BN / 8);       // 8x8 blocks of a k x n B tile
  static constexpr int NN_PER_THREAD = (NN_BLOCKS + kThreads - 1) / kThreads;
  static_assert(FM >= 1 && FN >= 1, "tile too small");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int BM, int BN, int DT, bool BT, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_mfma_kernel(GemmProblem p) {
  using T = GemmTile<BM, BN, DT, BT>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;

  const int M = p.m, N = p.n, K = p.k;
  const int ntiles = p.order.num_rb * p.order.num_cb;
  int wg = blockIdx.x;
  int split = 0;
  if constexpr (SPLIT) {
    split = wg / ntiles;
    wg -= split * ntiles;
  }
  int rb, cb;
  tile_coords(p.order, wg, ntiles, rb, cb);
  const int m0 = rb * BM, n0 = cb * BN;

  int k_begin = 0, k_end = K;
  if constexpr (SPLIT) {
    k_begin = split * p.k_per_split;
    k_end = min(K, k_begin + p.k_per_split);
  }
  const int nk = (k_end - k_begin + kBK - 1) / kBK;

  const char* zero = reinterpret_cast<const char*>(g_zero_chunk);

  // ---- per-lane global sources for the direct-to-LDS loads -------------------
  // Load instruction j of this wave fills LDS rows (wave*IPW + j)*8 + lane/8,
  // position lane%8, which holds logical chunk (lane%8) ^ swz(row).
  const int lrow8 = lane >> 3, lpos = lane & 7;
  const char* a_src[T::A_IPW];
  int a_kc[T::A_IPW];  // element offset of this lane's chunk inside a k-tile
  uint32_t a_ok = 0;
#pragma unroll
  for (int j = 0; j < T::A_IPW; ++j) {
    const int r = (wave * T::A_IPW + j) * 8 + lrow8;
    const int c = lpos ^ swz(r);
    a_kc[j] = c * 8;
    const int gi = m0 + r;
    a_src[j] = zero;
    if (gi < M) {
      const int g = gi / p.rows.rows_per_group;
      const int t = gi - g * p.rows.rows_per_group;
      a_src[j] = static_cast<const char*>(p.rows.a_group[g]) + ((int64_t)t * p.rows.a_ld + c * 8) * 2;
      a_ok |= 1u << j;
    }
  }
  const char* b_src[BT ? T::B_IPW : 1];
  int b_kc[BT ? T::B_IPW : 1];
  uint32_t b_ok = 0;
  if constexpr (BT) {
#pragma unroll
    for (int j = 0; j < T::B_IPW; ++j) {
      const int r = (wave * T::B_IPW + j) * 8 + lrow8;
      const int c = lpos ^ swz(r);
      b_kc[j] = c * 8;
      const int gn = n0 + r;
      b_src[j] = zero;
      if (gn < N) {
        b_src[j] = static_cast<const char*>(p.b) + ((int64_t)gn * p.ldb + c * 8) * 2;
        b_ok |= 1u << j;
      }
    }
  }

  // B stored k x n: each thread owns 8x8 blocks (8 k rows x 8 n columns).
  u32x4_t nn_regs[T::NN_PER_THREAD][8];

  auto issue_a = [&](char* stage, int k0) {
    const bool full = (k0 + kBK <= k_end);
#pragma unroll
    for (int j = 0; j < T::A_IPW; ++j) {
      const bool ok = ((a_ok >> j) & 1) && (full || (k0 + a_kc[j] < k_end));
      const char* src = ok ? a_src[j] + (int64_t)k0 * 2 : zero;
      load_lds16(src, stage + (wave * T::A_IPW + j) * 1024);
    }
  };
  auto issue_b_direct = [&](char* stage, int k0) {
    const bool full = (k0 + kBK <= k_end);
#pragma unroll
    for (int j = 0; j < T::B_IPW; ++j) {
      const bool ok = ((b_ok >> j) & 1) && (full || (k0 + b_kc[j] < k_end));
      const char* src = ok ? b_src[j] + (int64_t)k0 * 2 : zero;
      load_lds16(src, stage + T::A_BYTES + (wave * T::B_IPW + j) * 1024);
    }
  };
  auto load_b_nn = [&](int k0) {
#pragma unroll
    for (int q = 0; q < T::NN_PER_THREAD; ++q) {
      const int blk = tid + q * kThreads;
      const int nb = blk % (BN / 8), kb = blk / (BN / 8);
      const int gn = n0 + nb * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gk = k0 + kb * 8 + i;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (blk < T::NN_BLOCKS && gk < k_end && gn < N)
          v = *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.b) +
                                                ((int64_t)gk * p.ldb + gn) * 2);
        nn_regs[q][i] = v;
      }
    }
  };
  auto store_b_nn = [&](char* stage) {
    char* bs = stage + T::A_BYTES;
#pragma unroll
    for (int q = 0; q < T::NN_PER_THREAD; ++q) {
      const int blk = tid + q * kThreads;
      if (blk < T::NN_BLOCKS) {
        const int nb = blk % (BN / 8), kb = blk / (BN / 8);
        // Transpose the 8x8 block of 16-bit values: out[j] gathers element j
        // of rows 0..7 (8 consecutive k of column n0 + nb*8 + j).
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int w = j >> 1, sh = (j & 1) * 16;
          u32x4_t o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (nn_regs[q][2 * e][w] >> sh) & 0xFFFFu;
            const uint32_t hi = (nn_regs[q][2 * e + 1][w] >> sh) & 0xFFFFu;
            o[e] = lo | (hi << 16);
          }
          const int r = nb * 8 + j;
          *reinterpret_cast<u32x4_t*>(bs + r * kRowBytes + ((kb ^ swz(r)) << 4)) = o;
        }
      }
    }
  };

  // ---- LDS fragment read offsets -------------------------------------------
  const int hi = lane >> 5, l32 = lane & 31;
  int a_off[T::FM], a_x[T::FM], b_off[T::FN], b_x[T::FN];
#pragma unroll
  for (int f = 0; f < T::FM; ++f) {
    const int r = wm * T::TM + f * 32 + l32;
    a_off[f] = r * kRowBytes;
    a_x[f] = hi ^ swz(r);
  }
#pragma unroll
  for (int f = 0; f < T::FN; ++f) {
    const int r = wn * T::TN + f * 32 + l32;
    b_off[f] = T::A_BYTES + r * kRowBytes;
    b_x[f] = hi ^ swz(r);
  }

  f32x16_t acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Fragments for k-substep s+1 are read from LDS while the MFMAs of
  // substep s run (two register sets).
  auto read_frags = [&](const char* stage, int s, u32x4_t* af, u32x4_t* bfr) {
#pragma unroll
    for (int f = 0; f < T::FM; ++f)
      af[f] = *reinterpret_cast<const u32x4_t*>(stage + a_off[f] + (((2 * s) ^ a_x[f]) << 4));
#pragma unroll
    for (int f = 0; f < T::FN; ++f)
      bfr[f] = *reinterpret_cast<const u32x4_t*>(stage + b_off[f] + (((2 * s) ^ b_x[f]) << 4));
  };
  auto compute = [&](const char* stage) {
    u32x4_t af[2][T::FM], bfr[2][T::FN];
    read_frags(stage, 0, af[0], bfr[0]);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      if (s + 1 < kBK / 16) read_frags(stage, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc[i][j] = mfma32<DT>(bfr[s & 1][j], af[s & 1][i], acc[i][j]);
    }
  };

  // ---- main loop -------------------------------------------------------------
  char* stage0 = smem;
  char* stage1 = smem + T::STAGE_BYTES;
  if (nk > 0) {
    issue_a(stage0, k_begin);
    if constexpr (BT) {
      issue_b_direct(stage0, k_begin);
    } else {
      load_b_nn(k_begin);
      store_b_nn(stage0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = (kt & 1) ? stage1 : stage0;
    char* nxt = (kt & 1) ? stage0 : stage1;
    const bool more = (kt + 1 < nk);
    const int k1 = k_begin + (kt + 1) * kBK;
    if (more) {
      issue_a(nxt, k1);
      if constexpr (BT) issue_b_direct(nxt, k1);
      else load_b_nn(k1);
    }
    compute(cur);
    if constexpr (!BT) {
      if (more) store_b_nn(nxt);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------
  // acc[i][j][4q + e] holds C[m0 + wm*TM + i*32 + l32][n0 + wn*TN + j*32 + 8q + 4hi + e].
  if constexpr (!SPLIT) {
    const bool vec_ok = (N % 4) == 0 && (p.ldc % 4) == 0;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int gi = m0 + wm * T::TM + i * 32 + l32;
      if (gi >= M) continue;
      const int g = gi / p.rows.rows_per_group;
      const int t = gi - g * p.rows.rows_per_group;
      const int64_t crow = (int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t;
      uint16_t* cp = static_cast<uint16_t*>(p.c) + crow * p.ldc;
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gn = n0 + wn * T::TN + j * 32 + 8 * q + 4 * hi;
          const f32x16_t& a = acc[i][j];
          if (vec_ok && gn + 3 < N) {
            u32x2_t v;
            v[0] = pack2<DT>(a[4 * q + 0], a[4 * q + 1]);
            v[1] = pack2<DT>(a[4 * q + 2], a[4 * q + 3]);
            *reinterpret_cast<u32x2_t*>(cp + gn) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e < N) cp[gn + e] = cvt1<DT>(a[4 * q + e]);
          }
        }
      }
    }
  } else {
    // Split-K: fp32 partial tile, then the last workgroup of this tile sums
    // the partials in split order (fixed, so results are reproducible) and
    // writes the cast result.
    float* part = p.partials + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int gi = m0 + wm * T::TM + i * 32 + l32;
      if (gi >= M) continue;
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gn = n0 + wn * T::TN + j * 32 + 8 * q + 4 * hi;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gn + e < N) part[(int64_t)gi * N + gn + e] = acc[i][j][4 * q + e];
        }
      }
    }
    __threadfence();
    __syncthreads();
    __shared__ int s_last;
    const int tile = rb * p.order.num_cb + cb;
    if (tid == 0) {
      const int prev = atomicAdd(&p.counters[tile], 1);
      s_last = (prev == p.splits - 1);
    }
    __syncthreads();
    if (s_last) {
      __threadfence();
      const int rows = min(BM, M - m0), cols = min(BN, N - n0);
      for (int idx = tid; idx < rows * cols; idx += kThreads) {
        const int r = idx / cols, cc = idx - r * cols;
        const int gi = m0 + r, gn = n0 + cc;
        float s = 0.0f;
        for (int sp = 0; sp < p.splits; ++sp)
          s += __builtin_nontemporal_load(p.partials + ((int64_t)sp * M + gi) * N + gn);
        const int g = gi / p.rows.rows_per_group;
        const int t = gi - g * p.rows.rows_per_group;
        const int64_t crow = (int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t;
        static_cast<uint16_t*>(p.c)[crow * p.ldc + gn] = cvt1<DT>(s);
      }
      if (tid == 0) p.counters[tile] = 0;
    }
  }
}

template <int BM, int BN, int DT, bool BT>
hipError_t launch_one(const GemmProblem& p, hipStream_t stream) {
  const int ntiles = p.order.num_rb * p.order.num_cb;
  if (p.splits > 1) {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, DT, BT, true>), dim3(ntiles * p.splits),
                       dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, DT, BT, false>), dim3(ntiles), dim3(kThreads), 0,
                       stream, p);
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_tile(const GemmProblem& p, int dtype, bool bt, hipStream_t s) {
  if (dtype == kDtypeBf16)
    return bt ? launch_one<BM, BN, kDtypeBf16, true>(p, s) : launch_one<BM, BN, kDtypeBf16, false>(p, s);
  return bt ? launch_one<BM, BN, kDtypeFp16, true>(p, s) : launch_one<BM, BN, kDtypeFp16, false>(p, s);
}

}  // namespace

int tile_bm(int cfg) { return cfg == kTile128x128 ? 128 : 256; }
int tile_bn(int cfg) { return cfg == kTile256x256 ? 256 : 128; }

hipError_t launch_gemm_mfma(const GemmProblem& p, int tile_cfg, int dtype, bool rhs_transpose,
                            hipStream_t stream) {
  if (dtype != kDtypeBf16 && dtype != kDtypeFp16) return hipErrorInvalidValue;
  switch (tile_cfg) {
    case kTile256x256: return launch_tile<256, 256>(p, dtype, rhs_transpose, stream);
    case kTile128x128: return launch_tile<128, 128>(p, dtype, rhs_transpose, stream);
    case kTile256x128: return launch_tile<256, 128>(p, dtype, rhs_transpose, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace agmm
