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
//  * 4 waves of 64 lanes per workgroup, 2 x 2 over the output tile.
//  * Two main-loop forms:
//      - the part ring (gemm_m16_kernel, and gemm_mfma_kernel with
//        kLoopParts): 64-deep k-tiles, LDS split into 5 slots that each hold
//        one operand of one k-tile, so 2.5 k-tiles are resident and every
//        load fetches whole 128-byte lines; one barrier per k-tile;
//      - the stage ring (gemm_mfma_kernel, kLoopStages): 32-deep k-tiles in
//        3-8 whole stages, for short k.
//  * MFMAs: v_mfma_f32_16x16x32 (gemm_m16_kernel, the default for k >= 256;
//    it holds a higher clock than the 32x32x16 form for the same work on this
//    power-limited chip) or v_mfma_f32_32x32x16 (gemm_mfma_kernel), always
//    with the B fragment as the first operand.
//  * Every operand tile goes global -> LDS directly (lane i of a wave writes
//    bytes [16i, 16i+16) of a 1 KiB LDS block, so the LDS swizzle is chosen
//    by which global chunk each lane fetches); each wave waits only for the
//    k-tile it reads next (partial vmcnt).  gemm_m16_kernel loads interior
//    tiles whose rows lie in one shard through buffer descriptors
//    (buffer_load_dwordx4 ... lds: scalar base and k offset, fixed 32-bit
//    lane offsets); other tiles use global_load_lds_dwordx4 with 64-bit lane
//    addresses.
//  * k-contiguous tiles (A, and B when stored n x k) and n-contiguous B
//    tiles (B stored k x n, transposed on the way out by ds_read_b64_tr_b16)
//    use XOR swizzles measured free of LDS bank conflicts for each form's
//    fragment reads.
//  * Rows past m, columns past n and k past the end are fed from a zero
//    block, so ragged tails need no masking inside the main loop; interior
//    tiles take an unmasked loop.
//  * Tile order: XCD-aware remap of the workgroup id, grouped row blocks for
//    L2 reuse, then the plan's row-block visit order (ring order from the
//    local shard, or natural order).
//  * Epilogue: round-to-nearest-even cast, C staged through LDS and stored
//    as whole rows with 16-byte lanes (interior tiles), or fp32 partial sums
//    for split-K followed by a fixed-order reduction launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "agmm_kernels.h"

namespace agmm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// 16 zero bytes: the source of every out-of-range 16-byte chunk.
__device__ __attribute__((aligned(64))) const uint32_t g_zero_chunk[16] = {0};


// Position of 16-byte chunk groups in a k-contiguous LDS row (BK elements,
// 2*BK bytes).  Both choices were measured free of LDS bank conflicts for
// the MFMA fragment reads on gfx950 (64 banks, 16 lanes per ds_read_b128
// cycle).
template <int BK>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (BK == 32) return (row >> 2) & 3;
  else return (row ^ (row >> 3)) & 7;
}
__device__ __forceinline__ int swz_n(int krow) {
  // 0, 4, 10, 14 for krow % 4 = 0..3
  const int r = krow & 3;
  return (r << 2) ^ ((r >> 1) << 1);
}

// Swizzles of the 16x16x32-MFMA kernel.  Its fragment reads differ from the
// 32x32x16 ones: a ds_read_b128 covers 16 rows x 4 chunks (lane 16g + i
// reads row i, chunk g) instead of 32 rows x 2 chunks, and a transposed B
// read covers k-rows 8g + 0..3 for g = 0..3.  Rocprof counters showed the
// 32x32 swizzles costing this kernel LDS bank-conflict stalls on ~16% of
// its cycles (against 0.3% in the 32x32 kernel).  Both patterns agree with
// the LDS serving a b128 read in passes of lanes 8p..8p+7 with
// 32+8p..32+8p+7, and a b64 read in passes of 32 lanes.  Under that
// grouping:
//  * k-contiguous rows of 128 bytes: chunk c of row r at c ^ swz_k16(r).
//    A pass reads 8 consecutive rows x chunks {g, g ^ 2}; the 4 rows of one
//    parity (one 128-byte bank half) get swizzles 0, 1, 4, 5 (first 8 rows
//    of 16) or 2, 3, 6, 7 (last 8), so the 8 chunks they need are distinct.
//    Any 16 consecutive rows use 8 distinct swizzles per parity as well.
//  * n-contiguous B k-rows: the 32x32 swizzle of k-row r (by r % 4), plus
//    a flip of chunk bit 1 for k-rows with bit 3 set, which puts k-rows r
//    and r + 8 (read in the same pass) on disjoint bank sets.
__device__ __forceinline__ int swz_k16(int row) {
  return ((row >> 1) & 1) | (row & 4) | ((row >> 2) & 2);
}
__device__ __forceinline__ int swz_n16(int krow) { return swz_n(krow) ^ ((krow >> 2) & 2); }

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

// One 16-byte-per-lane global -> LDS load: lane i of the wave writes bytes
// [16i, 16i+16) of the 1 KiB LDS block at `lds_block` (wave-uniform).
// Issued as inline assembly on purpose: the compiler cannot tell which LDS
// bytes such a load writes, so it would otherwise wait for every one of
// them (vmcnt(0)) before the next LDS read anywhere in the kernel, which
// defeats the multi-stage pipeline.  The kernel instead waits explicitly for
// exactly the k-tile it is about to read (wait_vmcnt + barrier).
__device__ __forceinline__ void load_lds16(const void* gsrc, char* lds_block) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char_t*)lds_block);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds)
               : "m0");
}

// Same, with the LDS destination given as a 32-bit LDS address (no generic
// pointer conversion per load).
__device__ __forceinline__ void load_lds16_at(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "m0");
}

// Buffer-descriptor form of the same load: the 64-bit base sits in the
// scalar descriptor, each lane adds a 32-bit offset (`voff`) and the wave a
// scalar one (`soff`).  Interior tiles use it: their per-lane offsets stay
// fixed over the k loop, so a load costs no vector address arithmetic (the
// flat form adds a 64-bit k offset to every lane's pointer per load), and the
// descriptor's record count bounds every lane's offset.  LDS placement is the
// flat form's: lane i writes bytes [16i, 16i+16) of a 1 KiB block.
// The load goes into block R (0..3) of a 4 KiB LDS group: the instruction's
// offset field, R KiB, moves the LDS destination and the memory address
// alike, so `voff` is the lane's offset less R KiB.  With SET the load first
// writes the group's base into M0; without it M0 must already hold that
// base (the previous load of the group set it, and nothing between writes
// M0).  Writing M0 right before a DMA load costs the issuing wave about nine
// cycles beside its MFMA stream, against about one for the load alone
// (measured on MI355X), so one write serves four loads.
template <int R, bool SET>
__device__ __forceinline__ void load_lds16_buf_grp(const u32x4_t& rsrc, uint32_t voff, uint32_t soff,
                                                   uint32_t group_lds) {
  static_assert(R >= 0 && R < 4, "block of a 4 KiB group");
  if constexpr (SET)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen offset:%4 lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(group_lds)),
                   "s"(__builtin_amdgcn_readfirstlane(soff)), "n"(R * 1024)
                 : "m0");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "n"(R * 1024)
                 : "memory");
}

// Load j of a part: block j % 4 of group j / 4; M0 is written at the first
// block of each group.  A part's loads are issued in increasing j with no
// other M0 write between them.
__device__ __forceinline__ void load_lds16_buf_j(int j, const u32x4_t& rsrc, uint32_t voff_shifted,
                                                 uint32_t soff, uint32_t part_lds) {
  const uint32_t grp = part_lds + (uint32_t)(j & ~3) * 1024u;
  switch (j & 3) {
    case 0: load_lds16_buf_grp<0, true>(rsrc, voff_shifted, soff, grp); break;
    case 1: load_lds16_buf_grp<1, false>(rsrc, voff_shifted, soff, grp); break;
    case 2: load_lds16_buf_grp<2, false>(rsrc, voff_shifted, soff, grp); break;
    default: load_lds16_buf_grp<3, false>(rsrc, voff_shifted, soff, grp); break;
  }
}

// Raw buffer descriptor (stride 0, so the record count is in bytes) over
// `bytes` bytes from `base`; the last word is the gfx9 data-format word.
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* base, uint64_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  r[3] = 0x00020000u;
  return r;
}

__device__ __forceinline__ u32x2_t read_tr(const char* p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds_char_t*)p);
  return __builtin_bit_cast(u32x2_t, v);
}

// vmcnt(n) with the other counters left alone (gfx9 encoding).
// The scheduling barrier keeps the wait where it is written: the compiler
// would otherwise hoist it above independent MFMAs and stall them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the release/acquire fence of __syncthreads():
// that fence would also wait for the in-flight global->LDS loads of the
// next k-tiles.  Completion of the loads a k-tile needs is awaited
// explicitly (wait_vmcnt) before this barrier; the empty asm statements keep
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
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

// Main-loop forms.
//   kLoopStages:   ring of NST stages, each one k-tile of A and B.
//   kLoopParts:    ring of NST slots, each holding one operand of one k-tile
//                  ("part"); the parts alternate A, B, A, B, ...  With an odd
//                  slot count this keeps 2.5 k-tiles of 64-deep operands in
//                  LDS, i.e. 128-byte row pieces per load (a whole L2 line)
//                  with a load depth that whole stages could not fit.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};
template <int V>
struct IntTag {
  static constexpr int value = V;
};

constexpr int kLoopStages = 0;
constexpr int kLoopParts = 2;

template <int BM, int BN, int BK, int DT, bool BT, int NST, int WAVES, int LOOP = kLoopStages>
struct GemmTile {
  static constexpr int kStages = NST;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = 2, WN = WAVES / 2;      // wave grid over the output tile
  static constexpr int TM = BM / WM, TN = BN / WN;     // per-wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;     // 32x32 MFMA blocks per wave
  static constexpr int KROW = BK * 2;                  // bytes of a k-contiguous LDS row
  static constexpr int CPR = BK / 8;                   // 16-byte chunks per such row
  static constexpr int RPI = 1024 / KROW;              // rows one 1 KiB load instruction fills
  static constexpr int SUB = BK / 16;                  // k16 MFMA substeps per k-tile
  static constexpr int A_BYTES = BM * KROW;
  static constexpr int B_BYTES = BN * KROW;            // same size in both B layouts
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int PART_BYTES = A_BYTES > B_BYTES ? A_BYTES : B_BYTES;
  static constexpr int LDS_BYTES = LOOP == kLoopParts ? kStages * PART_BYTES : kStages * STAGE_BYTES;
  static constexpr int A_IPW = A_BYTES / 1024 / WAVES; // 1 KiB load instructions per wave
  static constexpr int B_IPW = B_BYTES / 1024 / WAVES;
  static constexpr int LOADS = A_IPW + B_IPW;          // per wave per k-tile
  static constexpr int B_ROW = BN * 2;                 // bytes of an n-contiguous k-row
  // Where in a k-tile the workgroup synchronises: in the middle when at
  // least 3 stages leave a tile of slack, else at the end of the tile.
  static constexpr bool MID_SYNC = NST >= 3;
  static constexpr int SYNC_SUB = MID_SYNC ? SUB / 2 : SUB;
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(WAVES == 4 || WAVES == 8, "waves");
  static_assert(FM >= 1 && FN >= 1, "tile too small");
  static_assert(A_IPW >= 1 && B_IPW >= 1, "tile too small for the load split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LOOP == kLoopParts || (NST - 1) * LOADS < 64, "vmcnt range");
  static_assert(NST >= 2 && NST <= 8, "stages");
  // part ring: 5 slots (parts 2t, 2t+1 = A, B of k-tile t live in slots
  // (2t) % 5 and (2t+1) % 5), at most 2 A parts and one B part in flight
  static_assert(LOOP != kLoopParts || (NST == 5 && A_IPW >= B_IPW && SUB >= 2 && 2 * A_IPW + B_IPW < 64),
                "part ring layout");
};

template <int BM, int BN, int BK, int DT, bool BT, bool SPLIT, int NST, int WAVES, int OCC, int LOOP>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void gemm_mfma_kernel(GemmProblem p) {
  using T = GemmTile<BM, BN, BK, DT, BT, NST, WAVES, LOOP>;
  constexpr int kBK = BK;
  constexpr int kStages = T::kStages;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS block addresses stay scalar
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

  // ---- per-lane global sources of the direct-to-LDS loads -------------------
  // k-contiguous tiles: instruction j of this wave fills LDS rows
  // (wave*IPW + j)*RPI + lane/CPR, position lane%CPR, which holds chunk
  // (lane%CPR) ^ swz_k(row).
  const char* a_src[T::A_IPW];
  int a_kc[T::A_IPW];
  uint32_t a_ok = 0;
#pragma unroll
  for (int j = 0; j < T::A_IPW; ++j) {
    const int r = (wave * T::A_IPW + j) * T::RPI + lane / T::CPR;
    const int c = (lane % T::CPR) ^ swz_k<BK>(r);
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
  const char* b_src[T::B_IPW];
  int b_kc[T::B_IPW];   // BT: element offset in k; !BT: k-row inside the tile
  uint32_t b_ok = 0;
#pragma unroll
  for (int j = 0; j < T::B_IPW; ++j) {
    b_src[j] = zero;
    if constexpr (BT) {
      const int r = (wave * T::B_IPW + j) * T::RPI + lane / T::CPR;
      const int c = (lane % T::CPR) ^ swz_k<BK>(r);
      b_kc[j] = c * 8;
      const int gn = n0 + r;
      if (gn < N) {
        b_src[j] = static_cast<const char*>(p.b) + ((int64_t)gn * p.ldb + c * 8) * 2;
        b_ok |= 1u << j;
      }
    } else {
      // n-contiguous k-rows of BN*2 bytes: byte (wave*IPW + j)*1024 + lane*16
      const int byte = (wave * T::B_IPW + j) * 1024 + lane * 16;
      const int kr = byte / T::B_ROW;
      const int pos = (byte % T::B_ROW) >> 4;
      const int c = pos ^ swz_n(kr);
      b_kc[j] = kr;
      const int gn = n0 + c * 8;
      if (gn < N) {
        b_src[j] = static_cast<const char*>(p.b) + ((int64_t)kr * p.ldb + gn) * 2;
        b_ok |= 1u << j;
      }
    }
  }

  // Branch-free issue of one k-tile: lanes whose row/column is out of range,
  // or whose chunk lies past k_end (ragged k, or a k-tile past the end that
  // the uniform pipeline still issues), fetch the zero block instead.
  auto issue_a = [&](char* sa, int k0) {
    const int64_t a_step = (int64_t)k0 * 2;
#pragma unroll
    for (int j = 0; j < T::A_IPW; ++j) {
      const bool ok = ((a_ok >> j) & 1) && (k0 + a_kc[j] < k_end);
      load_lds16(ok ? a_src[j] + a_step : zero, sa + (wave * T::A_IPW + j) * 1024);
    }
  };
  auto issue_b = [&](char* sb, int k0) {
    const int64_t b_step = BT ? (int64_t)k0 * 2 : (int64_t)k0 * p.ldb * 2;
#pragma unroll
    for (int j = 0; j < T::B_IPW; ++j) {
      const bool ok = ((b_ok >> j) & 1) && (k0 + b_kc[j] < k_end);
      load_lds16(ok ? b_src[j] + b_step : zero, sb + (wave * T::B_IPW + j) * 1024);
    }
  };
  auto issue = [&](int stage, int k0) {
    char* sa = smem + stage * T::STAGE_BYTES;
    issue_a(sa, k0);
    issue_b(sa + T::A_BYTES, k0);
  };

  // ---- LDS fragment read offsets -------------------------------------------
  const int hi = lane >> 5, l32 = lane & 31;
  int a_off[T::FM], a_x[T::FM];
#pragma unroll
  for (int f = 0; f < T::FM; ++f) {
    const int r = wm * T::TM + f * 32 + l32;
    a_off[f] = r * T::KROW;
    a_x[f] = hi ^ swz_k<BK>(r);
  }
  // BT: k-contiguous rows like A.  !BT: ds_read_b64_tr_b16 source lanes.
  // Lane i of 16-lane group G reads k-row 16s + 8*(G/2) + 4*half + i/4 at
  // columns nb + 16*(G%2) + 4*(i%4) .. +3; the instruction hands lane
  // 16G + j element e of the 16x4 block read by lanes 4e + j/4, i.e.
  // B[16s + 8*(G/2) + 4*half + e][nb + 16*(G%2) + j].
  int b_off[T::FN], b_x[T::FN];
  if constexpr (BT) {
#pragma unroll
    for (int f = 0; f < T::FN; ++f) {
      const int r = wn * T::TN + f * 32 + l32;
      b_off[f] = r * T::KROW;
      b_x[f] = hi ^ swz_k<BK>(r);
    }
  }
  const int tr_g = lane >> 4, tr_i = lane & 15;
  const int tr_krow = 8 * (tr_g >> 1) + (tr_i >> 2);        // + 16s + 4*half
  const int tr_swz = swz_n(tr_krow);                        // k-row % 4 is the same for every s/half
  int tr_n[T::FN];
#pragma unroll
  for (int f = 0; f < T::FN; ++f) tr_n[f] = wn * T::TN + f * 32 + 16 * (tr_g & 1) + 4 * (tr_i & 3);

  f32x16_t acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Fragments of k16 substep s from the A operand at `sa` and the B operand at `sb`.
  auto read_frags2 = [&](const char* sa, const char* sb, int s, u32x4_t* af, u32x4_t* bfr) {
    // in the order mfma_block consumes them: B0, A0 .. A(FM-1), B1 .. B(FN-1)
    auto read_b = [&](int f) {
      if constexpr (BT) {
        bfr[f] = *reinterpret_cast<const u32x4_t*>(sb + b_off[f] + (((2 * s) ^ b_x[f]) << 4));
      } else {
        const int n = tr_n[f];
        const int pos = (n >> 3) ^ tr_swz;
        const int within = (n & 7) * 2;
        const char* p0 = sb + (16 * s + tr_krow) * T::B_ROW + (pos << 4) + within;
        const u32x2_t lo = read_tr(p0);
        const u32x2_t hi2 = read_tr(p0 + 4 * T::B_ROW);
        bfr[f] = u32x4_t{lo[0], lo[1], hi2[0], hi2[1]};
      }
    };
    read_b(0);
#pragma unroll
    for (int f = 0; f < T::FM; ++f)
      af[f] = *reinterpret_cast<const u32x4_t*>(sa + a_off[f] + (((2 * s) ^ a_x[f]) << 4));
#pragma unroll
    for (int f = 1; f < T::FN; ++f) read_b(f);
  };
  auto read_frags = [&](const char* stage, int s, u32x4_t* af, u32x4_t* bfr) {
    read_frags2(stage, stage + T::A_BYTES, s, af, bfr);
  };
  // B fragment outermost: the j-th group of MFMAs needs only B0..Bj and the
  // A fragments, which arrive in that order.
  auto mfma_block = [&](const u32x4_t* af, const u32x4_t* bfr) {
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int i = 0; i < T::FM; ++i) acc[i][j] = mfma32<DT>(bfr[j], af[i], acc[i][j]);
  };
  constexpr int kMfmaPerSub = T::FM * T::FN;
  constexpr int kReadsPerSub = T::FM + (BT ? T::FN : 2 * T::FN);

  // ---- main loop, part ring ----------------------------------------------------
  // Slot q % 5 receives part q: A of k-tile q/2 for even q, B for odd q.
  // Parts 0-3 are issued up front.  During k-tile t:
  //   substeps 0 .. SUB-2: the loads of part 2t+4 (A of t+2) are spread over
  //     the MFMAs, into the slot of B of t-1 (free since the previous sync);
  //   substep SUB-1: each wave waits for its own loads of parts 2t+2, 2t+3
  //     (k-tile t+1; part 2t+4 may still be in flight) and for its LDS reads
  //     of k-tile t; one barrier; then part 2t+5 (B of t+2) goes into the
  //     slot of A of t, and the fragments of k-tile t+1 are read while the
  //     last MFMAs of k-tile t run.
  // Spreading the loads keeps the L1/L2 request stream even instead of one
  // burst per k-tile from every CU at once.  Past the end the parts fetch
  // zeros into slots nobody reads again, so the vmcnt arithmetic is the same
  // in every iteration.
  if constexpr (LOOP == kLoopParts) {
    constexpr int L = T::A_IPW;                       // load instructions per A part per wave
    constexpr int LB = T::B_IPW;                      // ... per B part
    constexpr int PB = T::PART_BYTES;
    constexpr int SPREAD = T::SUB - 1;                // substeps that carry A loads
    // Interior tiles (every row and column in range, whole k-tiles) load
    // without per-lane masks: the source is the lane's row pointer plus a
    // uniform k offset, and k-tiles past the end re-read the last k-tile
    // (valid memory; those slots are never read).  Edge tiles redirect
    // out-of-range chunks to the zero block.
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N) && ((k_end - k_begin) % kBK == 0) && nk > 0;
    auto ring = [&](auto tag) {
      constexpr bool FAST = decltype(tag)::value;
      auto a_addr = [&](int j, int t) -> const char* {
        if constexpr (FAST) {
          const int kk = k_begin + (t < nk ? t : nk - 1) * kBK;
          return a_src[j] + (int64_t)kk * 2;
        } else {
          const int kk = k_begin + t * kBK;
          const bool ok = ((a_ok >> j) & 1) && (kk + a_kc[j] < k_end);
          return ok ? a_src[j] + (int64_t)kk * 2 : zero;
        }
      };
      auto b_addr = [&](int j, int t) -> const char* {
        if constexpr (FAST) {
          const int kk = k_begin + (t < nk ? t : nk - 1) * kBK;
          return b_src[j] + (BT ? (int64_t)kk * 2 : (int64_t)kk * p.ldb * 2);
        } else {
          const int kk = k_begin + t * kBK;
          const bool ok = ((b_ok >> j) & 1) && (kk + b_kc[j] < k_end);
          return ok ? b_src[j] + (BT ? (int64_t)kk * 2 : (int64_t)kk * p.ldb * 2) : zero;
        }
      };
      const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t*)smem;
      const uint32_t lds_a = lds0 + wave * (T::A_IPW * 1024);
      const uint32_t lds_b = lds0 + wave * (T::B_IPW * 1024);
      auto put_a = [&](int slot, int t, int j0, int j1) {
#pragma unroll
        for (int j = j0; j < j1; ++j) load_lds16_at(a_addr(j, t), lds_a + slot * PB + j * 1024);
      };
      auto put_b = [&](int slot, int t) {
#pragma unroll
        for (int j = 0; j < T::B_IPW; ++j) load_lds16_at(b_addr(j, t), lds_b + slot * PB + j * 1024);
      };
      u32x4_t fa[2][T::FM], fb[2][T::FN];
      put_a(0, 0, 0, L);
      put_b(1, 0);
      put_a(2, 1, 0, L);
      put_b(3, 1);
      wait_vmcnt<L + LB>();
      block_barrier();
      read_frags2(smem, smem + PB, 0, fa[0], fb[0]);
      int sa_slot = 0, sb_slot = 1;   // slots of A and B of k-tile it
      for (int it = 0; it < nk; ++it) {
        const char* sa = smem + sa_slot * PB;
        const char* sb = smem + sb_slot * PB;
        const int a_new = sb_slot + 3 >= 5 ? sb_slot - 2 : sb_slot + 3;   // slot of B of it-1
        const int na = sa_slot + 2 >= 5 ? sa_slot - 3 : sa_slot + 2;
        const int nb = sb_slot + 2 >= 5 ? sb_slot - 3 : sb_slot + 2;
#pragma unroll
        for (int s = 0; s < T::SUB; ++s) {
          int nv;
          if (s == T::SUB - 1) {
            wait_vmcnt<L>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            block_barrier();
            read_frags2(smem + na * PB, smem + nb * PB, 0, fa[0], fb[0]);
            put_b(sa_slot, it + 2);
            nv = LB;
          } else {
            const int j0 = s * L / SPREAD, j1 = (s + 1) * L / SPREAD;
            read_frags2(sa, sb, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            put_a(a_new, it + 2, j0, j1);
            nv = j1 - j0;
          }
          mfma_block(fa[s & 1], fb[s & 1]);
          // interleave: MFMA, LDS read, ... (all reads first: the next
          // substep waits on them), then MFMA, global->LDS load(s), ...
          constexpr int nr = kReadsPerSub < kMfmaPerSub ? kReadsPerSub : kMfmaPerSub;
          const int left = kMfmaPerSub - nr;
#pragma unroll
          for (int q = 0; q < nr; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int q = 0; q < left; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
            for (int r = q * nv / left; r < (q + 1) * nv / left; ++r)
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
        sa_slot = na;
        sb_slot = nb;
      }
    };
    if (interior) ring(BoolTag<true>{});
    else ring(BoolTag<false>{});
  } else {
  // ---- main loop ---------------------------------------------------------------
  // Fragment registers alternate between two sets: the LDS reads of substep
  // s+1 are in flight while the MFMAs of substep s run.  Once per k-tile the
  // workgroup synchronises ("sync"): each wave waits for its own loads of
  // the next k-tile (vmcnt), then a barrier makes that tile complete in LDS
  // and guarantees every wave is done with the stage the next issue reuses;
  // right after it the loads of a further k-tile are issued.
  //   MID_SYNC (>= 3 stages): sync in the middle of tile `it`, issue tile
  //     it+NST-1 into the stage of tile it-1; the reads of tile it+1 start
  //     during the last substep of tile it.
  //   2 stages: sync at the end of tile `it`, issue tile it+2 into the stage
  //     of tile it.
  // Every iteration issues exactly one k-tile of loads (past the end they
  // fetch zeros into a stage nobody reads again), so the vmcnt arithmetic is
  // the same in every iteration and the loop body has no branches.
  u32x4_t fa[2][T::FM], fb[2][T::FN];
  constexpr int kPre = T::MID_SYNC ? kStages - 1 : kStages;   // tiles issued up front
#pragma unroll
  for (int t = 0; t < kPre; ++t) issue(t, k_begin + t * kBK);
  wait_vmcnt<(kPre - 1) * T::LOADS>();
  block_barrier();
  read_frags(smem, 0, fa[0], fb[0]);
  int st_cur = 0;                              // stage of tile it
  int st_new = T::MID_SYNC ? kStages - 1 : 0;  // stage the next issue fills
  int t_new = kPre;                            // k-tile the next issue loads
  for (int it = 0; it < nk; ++it) {
    const char* cur = smem + st_cur * T::STAGE_BYTES;
    const int st_next = (st_cur + 1 == kStages) ? 0 : st_cur + 1;
#pragma unroll
    for (int s = 0; s < T::SUB; ++s) {
      if (s == T::SYNC_SUB) {
        wait_vmcnt<(kStages - 3 > 0 ? kStages - 3 : 0) * T::LOADS>();
        block_barrier();
        issue(st_new, k_begin + t_new * kBK);
      }
      if (s + 1 < T::SUB) read_frags(cur, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
      else if (T::MID_SYNC) read_frags(smem + st_next * T::STAGE_BYTES, 0, fa[0], fb[0]);
      mfma_block(fa[s & 1], fb[s & 1]);
      // interleave: MFMA, global->LDS load (right after a sync), ...,
      // then MFMA, LDS read, MFMA, LDS read, ..., then the remaining MFMAs
      const int nv = (s == T::SYNC_SUB) ? (T::LOADS < kMfmaPerSub ? T::LOADS : kMfmaPerSub) : 0;
      const int left = kMfmaPerSub - nv;
      const int nr = kReadsPerSub < left ? kReadsPerSub : left;
#pragma unroll
      for (int q = 0; q < nv; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < nr; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < left - nr; ++q) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if constexpr (!T::MID_SYNC) {
      wait_vmcnt<0>();
      block_barrier();
      issue(st_new, k_begin + t_new * kBK);
      read_frags(smem + st_next * T::STAGE_BYTES, 0, fa[0], fb[0]);
    }
    st_cur = st_next;
    st_new = (st_new + 1 == kStages) ? 0 : st_new + 1;
    ++t_new;
  }
  }
  // No LDS-bound load may still be in flight when the workgroup retires.
  wait_vmcnt<0>();

  // ---- epilogue --------------------------------------------------------------
  // acc[i][j][4q + e] holds C[m0 + wm*TM + i*32 + l32][n0 + wn*TN + j*32 + 8q + 4hi + e].
  //
  // Interior tiles with 16-byte aligned C rows go through LDS: every wave
  // writes its converted sub-tile into a [BM][BN] staging tile (16-byte
  // chunk c of row r at position c ^ (r % chunks-per-row), which spreads
  // the 32 rows one ds_write touches over the banks), then the workgroup
  // writes C row by row, 16 bytes per lane and whole rows per group of
  // lanes, instead of 16-byte pieces of 32 different rows per store.
  constexpr int kRowB = BN * 2;            // bytes of a staged C row
  constexpr int kChunks = kRowB / 16;      // 16-byte chunks per row
  static_assert(T::LDS_BYTES >= BM * kRowB, "LDS too small to stage the C tile");
  static_assert((kChunks & (kChunks - 1)) == 0 && T::THREADS % kChunks == 0, "staging layout");
  bool staged = false;
  if constexpr (!SPLIT) {
    staged = (m0 + BM <= M) && (n0 + BN <= N) && (p.ldc % 8) == 0 &&
             ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
  }
  if (staged) {
    block_barrier();   // every wave's fragment reads and LDS-bound loads are done
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int r = wm * T::TM + i * 32 + l32;
      char* row = smem + r * kRowB;
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * T::TN + j * 32 + 8 * q;          // first column of the chunk
          const int pos = (c >> 3) ^ (r & (kChunks - 1));
          const f32x16_t& a = acc[i][j];
          u32x2_t v;
          v[0] = pack2<DT>(a[4 * q + 0], a[4 * q + 1]);
          v[1] = pack2<DT>(a[4 * q + 2], a[4 * q + 3]);
          *reinterpret_cast<u32x2_t*>(row + pos * 16 + hi * 8) = v;
        }
      }
    }
    block_barrier();
    constexpr int kRowsPerPass = T::THREADS / kChunks;
    const int ch = tid % kChunks;
    int r = tid / kChunks;
    int gi = m0 + r;
    int g = gi / p.rows.rows_per_group;
    int t = gi - g * p.rows.rows_per_group;
    uint16_t* cbase = static_cast<uint16_t*>(p.c) + n0 + ch * 8;
#pragma unroll 4
    for (; r < BM; r += kRowsPerPass) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + r * kRowB + ((ch ^ (r & (kChunks - 1))) << 4));
      const int64_t crow = (int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(cbase + crow * p.ldc));   // C is not re-read: keep L2 for A and B
      t += kRowsPerPass;
      while (t >= p.rows.rows_per_group) {
        t -= p.rows.rows_per_group;
        ++g;
      }
    }
  } else if constexpr (!SPLIT) {
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
    // Split-K: this workgroup's fp32 partial tile goes to partials[split];
    // splitk_reduce_kernel sums the splits afterwards.
    float* part = p.partials + (int64_t)split * M * N;
    const bool vec_ok = (N % 4) == 0;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int gi = m0 + wm * T::TM + i * 32 + l32;
      if (gi >= M) continue;
      float* prow = part + (int64_t)gi * N;
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gn = n0 + wn * T::TN + j * 32 + 8 * q + 4 * hi;
          const f32x16_t& a = acc[i][j];
          if (vec_ok && gn + 3 < N) {
            *reinterpret_cast<f32x4_t*>(prow + gn) =
                f32x4_t{a[4 * q + 0], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e < N) prow[gn + e] = a[4 * q + e];
          }
        }
      }
    }
  }
}

// acc += B-fragment x A-fragment on one 16x16 block, accumulator tied to its
// AGPRs.  Written as inline assembly because the compiler gives the builtin
// for this shape a separate destination and copies every accumulator once
// per use (four register moves per MFMA); with the operand tied read-write
// the 64 accumulators of a 128x128 sub-tile stay in place.  Being opaque to
// the hazard recognizer, the caller keeps the rules the compiler would:
// fragment registers come straight from LDS reads (waitcnt covers those),
// and the accumulators are touched by no other instruction between the
// mfma16_drain() calls around the main loop.
template <int DT>
__device__ __forceinline__ void mfma16(f32x4_t& c, const u32x4_t& b, const u32x4_t& a) {
  if constexpr (DT == kDtypeBf16)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
  else
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
}

template <int DT>
__device__ __forceinline__ f32x4_t mfma16_builtin(u32x4_t b, u32x4_t a, f32x4_t c) {
  if constexpr (DT == kDtypeBf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                   __builtin_bit_cast(bf16x8_t, a), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, b),
                                                  __builtin_bit_cast(f16x8_t, a), c, 0, 0, 0);
}

// Wait states between MFMAs and any other instruction that reads or writes
// their accumulators (more than the longest MFMA-to-VALU dependency).  The
// empty statements tie every accumulator on both sides, so no read or write
// of one can be placed across the wait.
template <int FM, int FN>
__device__ __forceinline__ void mfma16_drain(f32x4_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// Part-ring GEMM on v_mfma_f32_16x16x32_{bf16,f16}: the tiles, LDS layouts,
// part ring, synchronisation, load paths and epilogue of the part-ring form
// of gemm_mfma_kernel, with each wave's sub-tile computed as 16x16 blocks and
// a 64-deep k-tile as two k32 steps.  With random bf16 operands the chip is
// power-limited, and this instruction holds a higher clock than the 32x32x16
// one for the same work (measured raw MFMA throughput on MI355X: 1.88 against
// 1.65 PFLOP/s, 1.97 against 1.64 GHz).
// Fragments (lane l, g = l / 16, i = l % 16), B is the first operand:
//   A (second operand): A[m = i][k = 8g .. 8g+7] of a 16-row block
//   B (first operand):  B[k = 8g .. 8g+7][n = i] of a 16-column block
//   result:             C[m = i][n = 4g .. 4g+3] of the 16x16 block
template <int BM, int BN, int BK, int DT, bool BT, bool SPLIT, int WAVES, int OCC>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void gemm_m16_kernel(GemmProblem p) {
  using T = GemmTile<BM, BN, BK, DT, BT, 5, WAVES, kLoopParts>;
  constexpr int kBK = BK;
  constexpr int FM = T::TM / 16, FN = T::TN / 16;   // 16x16 blocks per wave
  constexpr int STEPS = BK / 32;                    // k32 steps per k-tile
  static_assert(BK == 64, "two k32 steps per k-tile");
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // ---- per-lane global sources (same LDS layout as gemm_mfma_kernel) -------
  const char* a_src[T::A_IPW];
  int a_kc[T::A_IPW];
  uint32_t a_ok = 0;
#pragma unroll
  for (int j = 0; j < T::A_IPW; ++j) {
    const int r = (wave * T::A_IPW + j) * T::RPI + lane / T::CPR;
    const int c = (lane % T::CPR) ^ swz_k16(r);
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
  const char* b_src[T::B_IPW];
  int b_kc[T::B_IPW];
  uint32_t b_ok = 0;
#pragma unroll
  for (int j = 0; j < T::B_IPW; ++j) {
    b_src[j] = zero;
    if constexpr (BT) {
      const int r = (wave * T::B_IPW + j) * T::RPI + lane / T::CPR;
      const int c = (lane % T::CPR) ^ swz_k16(r);
      b_kc[j] = c * 8;
      const int gn = n0 + r;
      if (gn < N) {
        b_src[j] = static_cast<const char*>(p.b) + ((int64_t)gn * p.ldb + c * 8) * 2;
        b_ok |= 1u << j;
      }
    } else {
      const int byte = (wave * T::B_IPW + j) * 1024 + lane * 16;
      const int kr = byte / T::B_ROW;
      const int pos = (byte % T::B_ROW) >> 4;
      const int c = pos ^ swz_n16(kr);
      b_kc[j] = kr;
      const int gn = n0 + c * 8;
      if (gn < N) {
        b_src[j] = static_cast<const char*>(p.b) + ((int64_t)kr * p.ldb + gn) * 2;
        b_ok |= 1u << j;
      }
    }
  }

  // ---- buffer-descriptor sources (interior tiles whose rows lie in one
  // shard; see load_lds16_buf) ---------------------------------------------
  // A: base = first row of the tile at k_begin, lane offset = row * lda + its
  // chunk; B (n x k) likewise by tile column; B (k x n): base = k_begin row at
  // column n0, lane offset = k-row * ldb + its chunk.  The k offset of k-tile
  // t is a scalar: 128 bytes per k-tile (A, B n x k) or 64 rows of B (k x n).
  // Each record count is the tile's whole extent from its base (lane plus
  // scalar offsets), which must stay below 4 GiB.
  const int g0 = m0 / p.rows.rows_per_group;
  const int row0 = m0 - g0 * p.rows.rows_per_group;
  const int64_t kspan = (int64_t)(k_end - k_begin) * 2;
  const int64_t a_span = (int64_t)(BM - 1) * p.rows.a_ld * 2 + kspan;
  const int64_t b_span = BT ? (int64_t)(BN - 1) * p.ldb * 2 + kspan
                            : (int64_t)(k_end - k_begin - 1) * p.ldb * 2 + BN * 2;
  // Load j of a wave lands in block j % 4 of its 4 KiB LDS group, reached
  // through the instruction's offset field, so its lane offsets are stored
  // less (j % 4) KiB.  Wave 0's first lane has the smallest offset of load j:
  // row 8j (A, B n x k: 8 rows per load) or k-row floor(1 KiB j / B_ROW)
  // (B k x n), so row strides of at least 64 elements (A, B n x k) and
  // 512 / floor(1 KiB / B_ROW) elements (B k x n) keep every shifted offset
  // non-negative; interior tiles always meet them (k, ldb >= a 64-deep
  // k-tile; ldb >= n >= BN).
  const bool shift_ok = p.rows.a_ld >= 64 &&
                        (BT ? p.ldb >= 64 : (int64_t)p.ldb * 2 * (1024 / T::B_ROW) >= 1024);
  const bool buf_ok = (row0 + BM <= p.rows.rows_per_group) && a_span < (1ll << 32) && b_span < (1ll << 32) &&
                      shift_ok;
  u32x4_t rsrc_a{}, rsrc_b{};
  uint32_t a_voff[T::A_IPW], b_voff[T::B_IPW];
  if (buf_ok) {
    rsrc_a = buffer_rsrc(static_cast<const char*>(p.rows.a_group[g0]) +
                             ((int64_t)row0 * p.rows.a_ld + k_begin) * 2, (uint64_t)a_span);
    rsrc_b = buffer_rsrc(static_cast<const char*>(p.b) +
                             (BT ? (int64_t)n0 * p.ldb + k_begin : (int64_t)k_begin * p.ldb + n0) * 2,
                         (uint64_t)b_span);
  }
#pragma unroll
  for (int j = 0; j < T::A_IPW; ++j) {
    const int r = (wave * T::A_IPW + j) * T::RPI + lane / T::CPR;
    const int c = (lane % T::CPR) ^ swz_k16(r);
    a_voff[j] = (uint32_t)(((int64_t)r * p.rows.a_ld + c * 8) * 2 - (j & 3) * 1024);
  }
#pragma unroll
  for (int j = 0; j < T::B_IPW; ++j) {
    if constexpr (BT) {
      const int r = (wave * T::B_IPW + j) * T::RPI + lane / T::CPR;
      const int c = (lane % T::CPR) ^ swz_k16(r);
      b_voff[j] = (uint32_t)(((int64_t)r * p.ldb + c * 8) * 2 - (j & 3) * 1024);
    } else {
      const int byte = (wave * T::B_IPW + j) * 1024 + lane * 16;
      const int kr = byte / T::B_ROW;
      const int c = ((byte % T::B_ROW) >> 4) ^ swz_n16(kr);
      b_voff[j] = (uint32_t)(((int64_t)kr * p.ldb + c * 8) * 2 - (j & 3) * 1024);
    }
  }

  // ---- LDS fragment offsets --------------------------------------------------
  const int g4 = lane >> 4, i16 = lane & 15;
  int a_off[FM], a_x[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int r = wm * T::TM + f * 16 + i16;
    a_off[f] = r * T::KROW;
    a_x[f] = g4 ^ swz_k16(r);          // chunk (4*step + g4) sits at (4*step) ^ a_x
  }
  int b_off[FN], b_x[FN];
  if constexpr (BT) {
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int r = wn * T::TN + f * 16 + i16;
      b_off[f] = r * T::KROW;
      b_x[f] = g4 ^ swz_k16(r);
    }
  }
  // k x n B: lane i of 16-lane group G reads k-row 32*step + 8G + 4*half + i/4,
  // columns nb + 4*(i%4) .. +3; ds_read_b64_tr_b16 then hands lane 16G + j
  // element e of B[32*step + 8G + 4*half + e][nb + j]
  const int tr_krow = 8 * g4 + (i16 >> 2);
  const int tr_swz = swz_n16(tr_krow);
  int tr_n[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) tr_n[f] = wn * T::TN + f * 16 + 4 * (i16 & 3);

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;

  // A fragments of k32 step `st`, and B fragments of one half of the wave's
  // column blocks of step `st`: half 0 is blocks [0, FH0), half 1 [FH0, FN)
  // (FH0 = FH1 when FN is even; 4 and 3 for the 7 blocks of a 112-column
  // sub-tile)
  auto read_a = [&](const char* sa, int st, u32x4_t* af) {
#pragma unroll
    for (int f = 0; f < FM; ++f)
      af[f] = *reinterpret_cast<const u32x4_t*>(sa + a_off[f] + (((4 * st) ^ a_x[f]) << 4));
  };
  constexpr int FH0 = (FN + 1) / 2, FH1 = FN - FH0;   // column blocks of each half
  static_assert(FH1 >= 1, "two halves of column blocks");
  auto read_b = [&](const char* sb, int st, int h, u32x4_t* bfr) {
#pragma unroll
    for (int q = 0; q < (h ? FH1 : FH0); ++q) {
      const int f = (h ? FH0 : 0) + q;
      if constexpr (BT) {
        bfr[q] = *reinterpret_cast<const u32x4_t*>(sb + b_off[f] + (((4 * st) ^ b_x[f]) << 4));
      } else {
        const int n = tr_n[f];
        const int pos = (n >> 3) ^ tr_swz;
        const char* p0 = sb + (32 * st + tr_krow) * T::B_ROW + (pos << 4) + (n & 7) * 2;
        const u32x2_t lo = read_tr(p0);
        const u32x2_t hi2 = read_tr(p0 + 4 * T::B_ROW);
        bfr[q] = u32x4_t{lo[0], lo[1], hi2[0], hi2[1]};
      }
    }
  };
  auto read_a_one = [&](const char* sa, int st, int f) -> u32x4_t {
    return *reinterpret_cast<const u32x4_t*>(sa + a_off[f] + (((4 * st) ^ a_x[f]) << 4));
  };
  auto read_b_one = [&](const char* sb, int st, int f) -> u32x4_t {
    if constexpr (BT) {
      return *reinterpret_cast<const u32x4_t*>(sb + b_off[f] + (((4 * st) ^ b_x[f]) << 4));
    } else {
      const int n = tr_n[f];
      const int pos = (n >> 3) ^ tr_swz;
      const char* p0 = sb + (32 * st + tr_krow) * T::B_ROW + (pos << 4) + (n & 7) * 2;
      const u32x2_t lo = read_tr(p0);
      const u32x2_t hi2 = read_tr(p0 + 4 * T::B_ROW);
      return u32x4_t{lo[0], lo[1], hi2[0], hi2[1]};
    }
  };
  // Interior tiles of the one-workgroup-per-CU shape, whose accumulators fill
  // the AGPRs, use the tied form; edge tiles (more live registers for their
  // masks) and the smaller shape the builtin, whose hazards the compiler
  // tracks itself.
  constexpr bool kTied = OCC == 1;
  auto mfma_half = [&](auto tied, const u32x4_t* af, const u32x4_t* bfr, int h) {
    const int c0 = h ? FH0 : 0;
#pragma unroll
    for (int q = 0; q < (h ? FH1 : FH0); ++q)
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (kTied && decltype(tied)::value) mfma16<DT>(acc[i][c0 + q], bfr[q], af[i]);
        else acc[i][c0 + q] = mfma16_builtin<DT>(bfr[q], af[i], acc[i][c0 + q]);
      }
  };
  constexpr int kMfmaHalf0 = FM * FH0, kMfmaHalf1 = FM * FH1;   // MFMAs of each half

  // ---- main loop: the part ring (see gemm_mfma_kernel) -----------------------
  constexpr int L = T::A_IPW;
  constexpr int LB = T::B_IPW;
  constexpr int PB = T::PART_BYTES;
  constexpr int SPREAD = STEPS - 1;
  const bool interior = (m0 + BM <= M) && (n0 + BN <= N) && ((k_end - k_begin) % kBK == 0) && nk > 0;
  // load modes: 0 edge tiles (masked flat loads), 1 interior (flat), 2
  // interior in one shard (buffer descriptors)
  auto ring = [&](auto tag) {
    constexpr int MODE = decltype(tag)::value;
    constexpr bool FAST = MODE >= 1;
    auto a_addr = [&](int j, int t) -> const char* {
      if constexpr (FAST) {
        const int kk = k_begin + (t < nk ? t : nk - 1) * kBK;
        return a_src[j] + (int64_t)kk * 2;
      } else {
        const int kk = k_begin + t * kBK;
        const bool ok = ((a_ok >> j) & 1) && (kk + a_kc[j] < k_end);
        return ok ? a_src[j] + (int64_t)kk * 2 : zero;
      }
    };
    auto b_addr = [&](int j, int t) -> const char* {
      if constexpr (FAST) {
        const int kk = k_begin + (t < nk ? t : nk - 1) * kBK;
        return b_src[j] + (BT ? (int64_t)kk * 2 : (int64_t)kk * p.ldb * 2);
      } else {
        const int kk = k_begin + t * kBK;
        const bool ok = ((b_ok >> j) & 1) && (kk + b_kc[j] < k_end);
        return ok ? b_src[j] + (BT ? (int64_t)kk * 2 : (int64_t)kk * p.ldb * 2) : zero;
      }
    };
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t*)smem;
    const uint32_t lds_a = lds0 + wave * (T::A_IPW * 1024);
    const uint32_t lds_b = lds0 + wave * (T::B_IPW * 1024);
    // scalar k offsets of k-tile t (k-tiles past the end re-read the last)
    auto a_soff = [&](int t) -> uint32_t { return (uint32_t)((t < nk ? t : nk - 1) * kBK * 2); };
    auto b_soff = [&](int t) -> uint32_t {
      return (uint32_t)((int64_t)(t < nk ? t : nk - 1) * kBK * 2 * (BT ? 1 : p.ldb));
    };
    auto put_a = [&](int slot, int t, int j0, int j1) {
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        if constexpr (MODE == 2) load_lds16_buf_j(j, rsrc_a, a_voff[j], a_soff(t), lds_a + slot * PB);
        else load_lds16_at(a_addr(j, t), lds_a + slot * PB + j * 1024);
      }
    };
    auto put_b_one = [&](int slot, int t, int j) {
      if constexpr (MODE == 2) load_lds16_buf_j(j, rsrc_b, b_voff[j], b_soff(t), lds_b + slot * PB);
      else load_lds16_at(b_addr(j, t), lds_b + slot * PB + j * 1024);
    };
    auto put_b = [&](int slot, int t) {
#pragma unroll
      for (int j = 0; j < T::B_IPW; ++j) put_b_one(slot, t, j);
    };
    // Four half-steps per k-tile, (step, half) = (0,0) (0,1) (1,0) (1,1):
    //   (0,0) MFMAs A0 x Ba; reads Bb = B(step 0, half 1)
    //   (0,1) MFMAs A0 x Bb; reads A1 = A(step 1), Ba = B(step 1, half 0)
    //   (1,0) MFMAs A1 x Ba; reads Bb = B(step 1, half 1)
    //   (1,1) sync; MFMAs A1 x Bb; reads A0, Ba of the next k-tile
    // Every read of this k-tile's slots is issued before the sync, which also
    // waits for them (lgkmcnt), so the loads after it may overwrite them.
    // A part loads ride on half-steps 0-2, the B part on half-step 3.
    u32x4_t A0[FM], A1[FM], Ba[FH0], Bb[FH0];
    if constexpr (kTied && FAST) mfma16_drain(acc);
    put_a(0, 0, 0, L);
    put_b(1, 0);
    put_a(2, 1, 0, L);
    put_b(3, 1);
    wait_vmcnt<L + LB>();
    block_barrier();
    read_b(smem + PB, 0, 0, Ba);
    read_a(smem, 0, A0);
    int sa_slot = 0, sb_slot = 1;
    auto interleave = [&](int nmfma, int nread, int nload) {
      // MFMA / LDS read pairs first (the next half-step waits on the reads),
      // then the global->LDS loads spread over the remaining MFMAs
      const int nr = nread < nmfma ? nread : nmfma;
      const int left = nmfma - nr;
#pragma unroll
      for (int q = 0; q < nr; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < left; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int r = q * nload / left; r < (q + 1) * nload / left; ++r)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    };
    constexpr int kReadsB0 = BT ? FH0 : 2 * FH0, kReadsB1 = BT ? FH1 : 2 * FH1;   // LDS reads per B half
    if constexpr (kTied && FAST) {
      // The compiler cannot see the tied MFMAs as MFMAs, so the interleaving
      // is written out and pinned: after MFMA number x of a half-step comes
      // its share of the other work (an LDS fragment read per MFMA first,
      // the next half-step needs them; then the global->LDS loads spread
      // over the remaining MFMAs), each group fenced from the next.
      auto half = [&](const u32x4_t* af, const u32x4_t* bfr, int h, int nread, int nload, auto&& op) {
        const int c0 = h ? FH0 : 0, nm = h ? kMfmaHalf1 : kMfmaHalf0;
#pragma unroll
        for (int q = 0; q < (h ? FH1 : FH0); ++q)
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int x = q * FM + i;
            mfma16<DT>(acc[i][c0 + q], bfr[q], af[i]);
            if (x < nread) {
              op(x);
            } else {
              const int left = nm - nread, y = x - nread;
#pragma unroll
              for (int r = y * nload / left; r < (y + 1) * nload / left; ++r) op(nread + r);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      };
      constexpr int L0 = L / 3, L1 = (2 * L) / 3 - L / 3, L2 = L - (2 * L) / 3;
      // one LDS read per MFMA, and MFMAs left over for the loads
      static_assert(FH1 + (L0 > 0 ? 1 : 0) <= kMfmaHalf0 && FM + FH0 < kMfmaHalf1, "reads per MFMA");
      for (int it = 0; it < nk; ++it) {
        const char* sa = smem + sa_slot * PB;
        const char* sb = smem + sb_slot * PB;
        const int a_new = sb_slot + 3 >= 5 ? sb_slot - 2 : sb_slot + 3;   // slot of B of it-1
        const int na = sa_slot + 2 >= 5 ? sa_slot - 3 : sa_slot + 2;
        const int nb = sb_slot + 2 >= 5 ? sb_slot - 3 : sb_slot + 2;
        // (0,0): MFMAs A0 x Ba; reads Bb (step 0, half 1); A loads 0 .. L0-1
        half(A0, Ba, 0, FH1, L0, [&](int k) {
          if (k < FH1) Bb[k] = read_b_one(sb, 0, FH0 + k);
          else put_a(a_new, it + 2, k - FH1, k - FH1 + 1);
        });
        // (0,1): MFMAs A0 x Bb; reads A1 (step 1), Ba (step 1, half 0); A loads L0 ..
        half(A0, Bb, 1, FM + FH0, L1, [&](int k) {
          if (k < FM) A1[k] = read_a_one(sa, 1, k);
          else if (k < FM + FH0) Ba[k - FM] = read_b_one(sb, 1, k - FM);
          else put_a(a_new, it + 2, L0 + k - FM - FH0, L0 + k - FM - FH0 + 1);
        });
        // (1,0): MFMAs A1 x Ba; reads Bb (step 1, half 1); the last A loads
        half(A1, Ba, 0, FH1, L2, [&](int k) {
          if (k < FH1) Bb[k] = read_b_one(sb, 1, FH0 + k);
          else put_a(a_new, it + 2, L0 + L1 + k - FH1, L0 + L1 + k - FH1 + 1);
        });
        // (1,1): sync; MFMAs A1 x Bb; reads Ba, A0 of the next k-tile; B loads
        wait_vmcnt<L>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        block_barrier();
        const char* sa2 = smem + na * PB;
        const char* sb2 = smem + nb * PB;
        half(A1, Bb, 1, FH0 + FM, LB, [&](int k) {
          if (k < FH0) Ba[k] = read_b_one(sb2, 0, k);
          else if (k < FH0 + FM) A0[k - FH0] = read_a_one(sa2, 0, k - FH0);
          else put_b_one(sa_slot, it + 2, k - FH0 - FM);
        });
        sa_slot = na;
        sb_slot = nb;
      }
    } else
    for (int it = 0; it < nk; ++it) {
      const char* sa = smem + sa_slot * PB;
      const char* sb = smem + sb_slot * PB;
      const int a_new = sb_slot + 3 >= 5 ? sb_slot - 2 : sb_slot + 3;   // slot of B of it-1
      const int na = sa_slot + 2 >= 5 ? sa_slot - 3 : sa_slot + 2;
      const int nb = sb_slot + 2 >= 5 ? sb_slot - 3 : sb_slot + 2;
      constexpr int L0 = L / 3, L1 = (2 * L) / 3 - L / 3, L2 = L - (2 * L) / 3;
      // (0,0)
      read_b(sb, 0, 1, Bb);
      put_a(a_new, it + 2, 0, L0);
      mfma_half(tag, A0, Ba, 0);
      interleave(kMfmaHalf0, kReadsB1, L0);
      // (0,1)
      read_a(sa, 1, A1);
      read_b(sb, 1, 0, Ba);
      put_a(a_new, it + 2, L0, L0 + L1);
      mfma_half(tag, A0, Bb, 1);
      interleave(kMfmaHalf1, FM + kReadsB0, L1);
      // (1,0)
      read_b(sb, 1, 1, Bb);
      put_a(a_new, it + 2, L0 + L1, L);
      mfma_half(tag, A1, Ba, 0);
      interleave(kMfmaHalf0, kReadsB1, L2);
      // (1,1)
      wait_vmcnt<L>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      block_barrier();
      read_b(smem + nb * PB, 0, 0, Ba);
      read_a(smem + na * PB, 0, A0);
      put_b(sa_slot, it + 2);
      mfma_half(tag, A1, Bb, 1);
      interleave(kMfmaHalf1, kReadsB0 + FM, LB);
      sa_slot = na;
      sb_slot = nb;
    }
    if constexpr (kTied && FAST) mfma16_drain(acc);
  };
  if (interior && buf_ok) ring(IntTag<2>{});
  else if (interior) ring(IntTag<1>{});
  else ring(IntTag<0>{});
  wait_vmcnt<0>();

  // ---- epilogue: acc[i][j][e] = C[m0 + wm*TM + 16i + i16][n0 + wn*TN + 16j + 4g4 + e]
  const int hi = g4 & 1;   // which half of a 16-byte (8-column) chunk
  constexpr int kRowB = BN * 2;
  constexpr int kChunks = kRowB / 16;
  // staged C rows: chunk c of row r at c ^ (r mod kSwz), kSwz the largest
  // power of two dividing the chunks per row (so positions stay in the row)
  constexpr int kSwz = kChunks & -kChunks;
  static_assert(T::LDS_BYTES >= BM * kRowB, "LDS too small to stage the C tile");
  bool staged = false;
  if constexpr (!SPLIT) {
    staged = (m0 + BM <= M) && (n0 + BN <= N) && (p.ldc % 8) == 0 &&
             ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
  }
  if (staged) {
    block_barrier();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * T::TM + i * 16 + i16;
      char* row = smem + r * kRowB;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c = wn * T::TN + j * 16 + 4 * g4;
        const int pos = (c >> 3) ^ (r & (kSwz - 1));
        u32x2_t v;
        v[0] = pack2<DT>(acc[i][j][0], acc[i][j][1]);
        v[1] = pack2<DT>(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2_t*>(row + pos * 16 + hi * 8) = v;
      }
    }
    block_barrier();
    constexpr int kRowsPerPass = T::THREADS / kChunks;   // threads past whole rows stay idle
    const int ch = tid % kChunks;
    int r = tid < kRowsPerPass * kChunks ? tid / kChunks : BM;
    int gi = m0 + r;
    int g = gi / p.rows.rows_per_group;
    int t = gi - g * p.rows.rows_per_group;
    uint16_t* cbase = static_cast<uint16_t*>(p.c) + n0 + ch * 8;
#pragma unroll 4
    for (; r < BM; r += kRowsPerPass) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + r * kRowB + ((ch ^ (r & (kSwz - 1))) << 4));
      const int64_t crow = (int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(cbase + crow * p.ldc));
      t += kRowsPerPass;
      while (t >= p.rows.rows_per_group) {
        t -= p.rows.rows_per_group;
        ++g;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int gi = m0 + wm * T::TM + i * 16 + i16;
      if (gi >= M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int gn = n0 + wn * T::TN + j * 16 + 4 * g4;
        const f32x4_t& a = acc[i][j];
        if constexpr (SPLIT) {
          float* prow = p.partials + ((int64_t)split * M + gi) * N;
          if ((N % 4) == 0 && gn + 3 < N) {
            *reinterpret_cast<f32x4_t*>(prow + gn) = a;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e < N) prow[gn + e] = a[e];
          }
        } else {
          const int g = gi / p.rows.rows_per_group;
          const int t = gi - g * p.rows.rows_per_group;
          uint16_t* cp = static_cast<uint16_t*>(p.c) + ((int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t) * p.ldc;
          if ((N % 4) == 0 && (p.ldc % 4) == 0 && gn + 3 < N) {
            u32x2_t v;
            v[0] = pack2<DT>(a[0], a[1]);
            v[1] = pack2<DT>(a[2], a[3]);
            *reinterpret_cast<u32x2_t*>(cp + gn) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e < N) cp[gn + e] = cvt1<DT>(a[e]);
          }
        }
      }
    }
  }
}

// Sum of the split-K partials in split order 0, 1, ..., S-1 (fixed, so the
// result does not depend on which workgroup finished first), cast to the
// output dtype, scattered to C rows through the row map.  Four consecutive
// columns per thread.
template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmProblem p) {
  const int M = p.m, N = p.n;
  const int n4 = (N + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * n4) return;
  const int row = (int)(idx / n4);
  const int col = (int)(idx - (int64_t)row * n4) * 4;
  const int g = row / p.rows.rows_per_group;
  const int t = row - g * p.rows.rows_per_group;
  const int64_t crow = (int64_t)g * p.rows.c_group_rows + p.rows.c_row_off + t;
  uint16_t* cp = static_cast<uint16_t*>(p.c) + crow * p.ldc;
  const int64_t plane = (int64_t)M * N;
  const float* src = p.partials + (int64_t)row * N + col;
  if ((N % 4) == 0) {
    // Up to 8 partial vectors are loaded before any is added, then added in
    // split order.
    f32x4_t s = *reinterpret_cast<const f32x4_t*>(src);
    for (int sp0 = 1; sp0 < p.splits; sp0 += 8) {
      f32x4_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (sp0 + q < p.splits) v[q] = *reinterpret_cast<const f32x4_t*>(src + (sp0 + q) * plane);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (sp0 + q < p.splits) s += v[q];
    }
    u32x2_t v;
    v[0] = pack2<DT>(s[0], s[1]);
    v[1] = pack2<DT>(s[2], s[3]);
    if ((p.ldc % 4) == 0) {
      *reinterpret_cast<u32x2_t*>(cp + col) = v;
    } else {
      for (int e = 0; e < 4; ++e) cp[col + e] = cvt1<DT>(s[e]);
    }
  } else {
    for (int e = 0; e < 4 && col + e < N; ++e) {
      float s = src[e];
      for (int sp = 1; sp < p.splits; ++sp) s += src[sp * plane + e];
      cp[col + e] = cvt1<DT>(s);
    }
  }
}

template <int BM, int BN, int BK, int DT, bool BT, int NST, int WAVES, int OCC, int LOOP = kLoopStages>
hipError_t launch_one(const GemmProblem& p, hipStream_t stream) {
  const int ntiles = p.order.num_rb * p.order.num_cb;
  if (p.splits > 1) {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, DT, BT, true, NST, WAVES, OCC, LOOP>),
                       dim3(ntiles * p.splits), dim3(64 * WAVES), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t work = (int64_t)p.m * ((p.n + 3) / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<DT>), dim3((unsigned)((work + 255) / 256)), dim3(256),
                       0, stream, p);
  } else {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, DT, BT, false, NST, WAVES, OCC, LOOP>),
                       dim3(ntiles), dim3(64 * WAVES), 0, stream, p);
  }
  return hipGetLastError();
}

template <int BM, int BN, int BK, int NST, int WAVES, int OCC, int LOOP = kLoopStages>
hipError_t launch_tile(const GemmProblem& p, int dtype, bool bt, hipStream_t s) {
  if (dtype == kDtypeBf16)
    return bt ? launch_one<BM, BN, BK, kDtypeBf16, true, NST, WAVES, OCC, LOOP>(p, s)
              : launch_one<BM, BN, BK, kDtypeBf16, false, NST, WAVES, OCC, LOOP>(p, s);
  return bt ? launch_one<BM, BN, BK, kDtypeFp16, true, NST, WAVES, OCC, LOOP>(p, s)
            : launch_one<BM, BN, BK, kDtypeFp16, false, NST, WAVES, OCC, LOOP>(p, s);
}

template <int BM, int BN, int BK, int DT, bool BT, int WAVES, int OCC>
hipError_t launch_m16_one(const GemmProblem& p, hipStream_t stream) {
  const int ntiles = p.order.num_rb * p.order.num_cb;
  if (p.splits > 1) {
    hipLaunchKernelGGL((gemm_m16_kernel<BM, BN, BK, DT, BT, true, WAVES, OCC>),
                       dim3(ntiles * p.splits), dim3(64 * WAVES), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t work = (int64_t)p.m * ((p.n + 3) / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<DT>), dim3((unsigned)((work + 255) / 256)), dim3(256),
                       0, stream, p);
  } else {
    hipLaunchKernelGGL((gemm_m16_kernel<BM, BN, BK, DT, BT, false, WAVES, OCC>),
                       dim3(ntiles), dim3(64 * WAVES), 0, stream, p);
  }
  return hipGetLastError();
}

// B stored n x k only (tiles whose B rows are not a power-of-two of chunks)
template <int BM, int BN, int BK, int WAVES, int OCC>
hipError_t launch_m16_bt(const GemmProblem& p, int dtype, hipStream_t s) {
  return dtype == kDtypeBf16 ? launch_m16_one<BM, BN, BK, kDtypeBf16, true, WAVES, OCC>(p, s)
                             : launch_m16_one<BM, BN, BK, kDtypeFp16, true, WAVES, OCC>(p, s);
}

template <int BM, int BN, int BK, int WAVES, int OCC>
hipError_t launch_m16(const GemmProblem& p, int dtype, bool bt, hipStream_t s) {
  if (dtype == kDtypeBf16)
    return bt ? launch_m16_one<BM, BN, BK, kDtypeBf16, true, WAVES, OCC>(p, s)
              : launch_m16_one<BM, BN, BK, kDtypeBf16, false, WAVES, OCC>(p, s);
  return bt ? launch_m16_one<BM, BN, BK, kDtypeFp16, true, WAVES, OCC>(p, s)
            : launch_m16_one<BM, BN, BK, kDtypeFp16, false, WAVES, OCC>(p, s);
}

}  // namespace

// Compiled tile configurations: output tile, k-depth of an LDS stage,
// stages in the LDS ring, waves per workgroup, waves per SIMD.
struct TileInfo { int bm, bn, bk, stages, waves, occ; };
constexpr TileInfo kTiles[kTileCount] = {
    {256, 256, 32, 4, 4, 1},   // kTile256x256:      128 KiB LDS, 3 k-tiles in flight
    {128, 128, 32, 4, 4, 2},   // kTile128x128:      64 KiB, two workgroups per CU
    {256, 128, 32, 3, 4, 2},   // kTile256x128:      72 KiB, two workgroups per CU
    {128, 64, 32, 4, 4, 1},    // kTile128x64:       48 KiB; B stored n x k only (skinny m)
    {128, 64, 32, 8, 4, 1},    // kTile128x64s8:     96 KiB, 7 k-tiles in flight; B n x k only
    {256, 256, 64, 5, 4, 1},   // kTile256x256r5:    160 KiB part ring, 64-deep k-tiles
    {128, 128, 64, 5, 4, 2},   // kTile128x128r5:    80 KiB part ring, two workgroups per CU
    {128, 64, 64, 5, 4, 2},    // kTile128x64r5:     80 KiB part ring; B stored n x k only
    {256, 256, 64, 5, 4, 1},   // kTile256x256m16:   part ring on 16x16x32 MFMAs
    {128, 128, 64, 5, 4, 2},   // kTile128x128m16:   same, two workgroups per CU
    {32, 32, 64, 4, 8, 1},     // kTileSkinny:       skinny kernel, whole k (launch_skinny_fullk)
    {256, 224, 64, 5, 4, 1},   // kTile256x224m16:   16x16x32 part ring, 7 column blocks per wave; B n x k only
};

constexpr bool all_tiles_described() {
  for (const TileInfo& t : kTiles)
    if (t.bm <= 0 || t.bn <= 0 || t.bk <= 0 || t.waves <= 0 || t.occ <= 0) return false;
  return true;
}
static_assert(all_tiles_described(), "every tile configuration needs its row of kTiles");

int tile_bm(int cfg) { return kTiles[cfg].bm; }
int tile_bn(int cfg) { return kTiles[cfg].bn; }
int tile_bk(int cfg) { return kTiles[cfg].bk; }
int tile_occ(int cfg) { return kTiles[cfg].occ; }

hipError_t launch_gemm_mfma(const GemmProblem& p, int tile_cfg, int dtype, bool rhs_transpose,
                            hipStream_t stream) {
  if (dtype != kDtypeBf16 && dtype != kDtypeFp16) return hipErrorInvalidValue;
  // an n-contiguous B tile of 64 columns is too narrow for its LDS swizzle
  if (tile_needs_bt(tile_cfg) && !rhs_transpose) return hipErrorInvalidValue;
  switch (tile_cfg) {
    case kTile256x256: return launch_tile<256, 256, 32, 4, 4, 1>(p, dtype, rhs_transpose, stream);
    case kTile128x128: return launch_tile<128, 128, 32, 4, 4, 2>(p, dtype, rhs_transpose, stream);
    case kTile256x128: return launch_tile<256, 128, 32, 3, 4, 2>(p, dtype, rhs_transpose, stream);
    case kTile128x64:
      return dtype == kDtypeBf16 ? launch_one<128, 64, 32, kDtypeBf16, true, 4, 4, 1>(p, stream)
                                 : launch_one<128, 64, 32, kDtypeFp16, true, 4, 4, 1>(p, stream);
    case kTile128x64s8:
      return dtype == kDtypeBf16 ? launch_one<128, 64, 32, kDtypeBf16, true, 8, 4, 1>(p, stream)
                                 : launch_one<128, 64, 32, kDtypeFp16, true, 8, 4, 1>(p, stream);
    case kTile256x256r5:
      return launch_tile<256, 256, 64, 5, 4, 1, kLoopParts>(p, dtype, rhs_transpose, stream);
    case kTile128x128r5:
      return launch_tile<128, 128, 64, 5, 4, 2, kLoopParts>(p, dtype, rhs_transpose, stream);
    case kTile128x64r5:
      return dtype == kDtypeBf16 ? launch_one<128, 64, 64, kDtypeBf16, true, 5, 4, 2, kLoopParts>(p, stream)
                                 : launch_one<128, 64, 64, kDtypeFp16, true, 5, 4, 2, kLoopParts>(p, stream);
    case kTile256x256m16: return launch_m16<256, 256, 64, 4, 1>(p, dtype, rhs_transpose, stream);
    case kTile128x128m16: return launch_m16<128, 128, 64, 4, 2>(p, dtype, rhs_transpose, stream);
    case kTile256x224m16: return launch_m16_bt<256, 224, 64, 4, 1>(p, dtype, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_splitk_reduce(const GemmProblem& p, int dtype, hipStream_t stream) {
  if (dtype != kDtypeBf16 && dtype != kDtypeFp16) return hipErrorInvalidValue;
  if (p.splits < 1 || p.partials == nullptr) return hipErrorInvalidValue;
  const int64_t blocks = ((int64_t)p.m * ((p.n + 3) / 4) + 255) / 256;
  if (blocks < 1 || blocks > INT32_MAX) return hipErrorInvalidValue;
  if (dtype == kDtypeBf16)
    hipLaunchKernelGGL((splitk_reduce_kernel<kDtypeBf16>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<kDtypeFp16>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace agmm
