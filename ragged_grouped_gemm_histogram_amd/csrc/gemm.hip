// Persistent grouped GEMM over ragged per-expert row blocks, bf16 MFMA with
// fp32 accumulation, for the two projections of a SwiGLU expert (OLMo report,
// Eq 13):
//
//   up:   h_buf[rows_e]  = bf16( SiLU(bf16(G)) * bf16(U) ),  [G | U] = x_perm[rows_e] * W_ug[e]^T
//   down: y_perm[rows_e] = bf16( h_buf[rows_e] * W_down[e] )
//
// OLMo report Sec 9.2 / Fig 37: the offsets stay on the device; one grouped
// kernel walks the tiles of every expert's problem. Here each workgroup
// rebuilds the problem list from the device offsets in LDS (expert e owns
// sorted rows [offsets[e], offsets[e+1]); its pointers are affine in e and
// offsets[e]), then takes output tiles in a static round-robin until none is
// left. Empty experts contribute no tile; rows past an expert's block, columns
// past N and the K remainder are masked with zeros on load and skipped on
// store.
//
// Tile: BM rows x BN weight rows, K stepped by 64 through double-buffered LDS
// (global -> registers -> LDS while the previous stage feeds the MFMAs).
// 4 waves in a 2x2 grid, each owning (BM/2) x (BN/2) outputs as 32x32 blocks
// of v_mfma_f32_32x32x16_bf16. The MFMA is issued with the weight fragment as
// its first operand, so each lane ends up holding four consecutive output
// columns of one output row; the epilogue packs them to bf16, stages the tile
// through LDS and writes whole 16-byte chunks.
//
// For the up projection the BN weight rows of a tile are BN/2 gate rows
// followed by the BN/2 matching up rows (W_ug is gate-then-up, chunked), so a
// lane holds each gate value and its up value in the same register slot and
// SwiGLU is applied in registers. For the down projection W_down [h, d] is
// N-contiguous: each thread loads an 8(k) x 8(n) block and transposes it in
// registers so that LDS always holds K-contiguous rows.

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int BK = 64;         // K per stage: 8 chunks of 16 bytes per tile row
constexpr int kChunksK = BK / 8;
constexpr int kGroupM = 8;     // m-tiles per group in the tile order (operand reuse in L2)

template <int BM, int BN, bool GATED>
struct Tile {
  static constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int OUTW = GATED ? BN / 2 : BN;  // output columns per tile
  static constexpr int OUT_CPR = OUTW / 8;          // 16-byte chunks per output row
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int A_LOADS = BM * kChunksK / kThreads;  // 16-byte chunks per thread per stage
  static constexpr int B_LOADS = BN * kChunksK / kThreads;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must split into 32x32 blocks over a 2x2 wave grid");
  static_assert(BM * OUTW * 2 <= LDS_BYTES, "epilogue tile must fit in the stage buffers");
  static_assert((OUT_CPR & (OUT_CPR - 1)) == 0, "output chunk count must be a power of two");
  static_assert(!GATED || FN % 2 == 0, "gated tiles pair gate and up blocks");
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// v_perm_b32 byte select: result bytes [b0 b1 a0 a1] (lo halves) or [b2 b3 a2 a3] (hi halves).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(a, b, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(a, b, 0x07060302u); }

// Map a persistent workgroup to a logical worker so that consecutive logical
// workers (which take consecutive tiles) sit on one XCD: workgroups are
// dealt to the 8 XCDs round-robin.
__device__ __forceinline__ int logical_worker() {
  const int G = gridDim.x, b = blockIdx.x;
  if (G % 8 != 0) return b;
  return (b % 8) * (G / 8) + b / 8;
}

template <int BM, int BN, bool GATED, bool B_NMAJOR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ W, int64_t w_expert_stride,
    int64_t ldw, int64_t gate_up_rows, int64_t N, int64_t K, const int32_t* __restrict__ offsets, int E,
    int64_t cap_rows, uint16_t* __restrict__ out, int64_t ldo) {
  using C = Tile<BM, BN, GATED>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int seg_lo[MOE_MAX_EXPERTS];
  __shared__ int seg_rows[MOE_MAX_EXPERTS];
  __shared__ int mt_prefix[MOE_MAX_EXPERTS + 1];
  __shared__ int scan_tmp[kThreads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- problem list from the device offsets (clamped: no access outside the buffers)
  constexpr int kPer = (MOE_MAX_EXPERTS + kThreads - 1) / kThreads;
  int mt_local[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    int mt = 0;
    if (e < E) {
      int64_t lo = offsets[e], hi = offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > cap_rows ? cap_rows : lo);
      hi = hi < lo ? lo : (hi > cap_rows ? cap_rows : hi);
      seg_lo[e] = (int)lo;
      seg_rows[e] = (int)(hi - lo);
      mt = (int)((hi - lo + BM - 1) / BM);
    }
    mt_local[i] = mt;
    sum += mt;
  }
  scan_tmp[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? scan_tmp[tid - off] : 0;
    __syncthreads();
    scan_tmp[tid] += add;
    __syncthreads();
  }
  {
    int run = scan_tmp[tid] - sum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid * kPer + i;
      if (e < E) mt_prefix[e] = run;
      run += mt_local[i];
    }
    if (tid == kThreads - 1) mt_prefix[E] = scan_tmp[kThreads - 1];
  }
  __syncthreads();

  const int total_mt = mt_prefix[E];
  const int64_t n_tiles = GATED ? (N + C::OUTW - 1) / C::OUTW : (N + BN - 1) / BN;
  const int64_t total_tiles = (int64_t)total_mt * n_tiles;
  const int nk = (int)((K + BK - 1) / BK);

  unsigned char* As = smem;                   // [2][BM][BK] swizzled
  unsigned char* Bs = smem + 2 * C::A_BYTES;  // [2][BN][BK] swizzled

  for (int64_t t = logical_worker(); t < total_tiles; t += gridDim.x) {
    // ---- tile -> (expert, m-tile, n-tile); groups of kGroupM m-tiles sweep all n-tiles
    const int64_t group_span = (int64_t)kGroupM * n_tiles;
    const int64_t group = t / group_span;
    const int64_t in_group = t - group * group_span;
    const int64_t g0 = group * kGroupM;
    const int gsize = (int)((total_mt - g0) < kGroupM ? (total_mt - g0) : kGroupM);
    const int64_t nt = in_group / gsize;
    const int gm = (int)(g0 + (in_group - nt * gsize));
    int lo_e = 0, hi_e = E;  // largest e with mt_prefix[e] <= gm
    while (hi_e - lo_e > 1) {
      const int mid = (lo_e + hi_e) >> 1;
      if (mt_prefix[mid] <= gm) lo_e = mid; else hi_e = mid;
    }
    const int e = lo_e;
    const int mi = gm - mt_prefix[e];
    const int64_t row0 = (int64_t)seg_lo[e] + (int64_t)mi * BM;  // first sorted row of the tile
    const int rows_valid = min(BM, seg_rows[e] - mi * BM);
    const uint16_t* Wexp = W + (int64_t)e * w_expert_stride;
    const int64_t n0 = nt * (GATED ? C::OUTW : BN);  // first output column

    // ---- global -> register loaders
    u32x4 ra[C::A_LOADS];
    u32x4 rb[C::B_LOADS];
    auto load_a = [&](int kt) {
      const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int idx = i * kThreads + tid;
        const int r = idx / kChunksK, c = idx % kChunksK;
        const int64_t kk = k0 + c * 8;
        ra[i] = (r < rows_valid && kk < K)
                    ? *reinterpret_cast<const u32x4*>(A + (row0 + r) * lda + kk)
                    : zero4();
      }
    };
    auto load_b = [&](int kt) {
      const int64_t k0 = (int64_t)kt * BK;
      if constexpr (!B_NMAJOR) {
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
          const int idx = i * kThreads + tid;
          const int r = idx / kChunksK, c = idx % kChunksK;
          int64_t wrow, ncol;
          if constexpr (GATED) {
            const int half = r / (BN / 2);
            ncol = n0 + (r - half * (BN / 2));
            wrow = ncol + half * gate_up_rows;
          } else {
            ncol = n0 + r;
            wrow = ncol;
          }
          const int64_t kk = k0 + c * 8;
          rb[i] = (ncol < N && kk < K) ? *reinterpret_cast<const u32x4*>(Wexp + wrow * ldw + kk) : zero4();
        }
      } else {
        // 8(k) x 8(n) block per thread: rows k0+kb*8+i, columns n0+nb*8 .. +8
        static_assert(!B_NMAJOR || C::B_LOADS == 8, "transposing loader covers the tile with one 8x8 block per thread");
        const int nb = tid % (BN / 8), kb = tid / (BN / 8);
        const int64_t ncol = n0 + nb * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t kk = k0 + kb * 8 + i;
          rb[i] = (ncol < N && kk < K) ? *reinterpret_cast<const u32x4*>(Wexp + kk * ldw + ncol) : zero4();
        }
      }
    };
    auto store_stage = [&](int buf) {
      unsigned char* as = As + buf * C::A_BYTES;
      unsigned char* bs = Bs + buf * C::B_BYTES;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int idx = i * kThreads + tid;
        const int r = idx / kChunksK, c = idx % kChunksK;
        *reinterpret_cast<u32x4*>(as + r * (BK * 2) + swz(r, c) * 16) = ra[i];
      }
      if constexpr (!B_NMAJOR) {
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
          const int idx = i * kThreads + tid;
          const int r = idx / kChunksK, c = idx % kChunksK;
          *reinterpret_cast<u32x4*>(bs + r * (BK * 2) + swz(r, c) * 16) = rb[i];
        }
      } else {
        const int nb = tid % (BN / 8), kb = tid / (BN / 8);
        // rb[i] holds k = kb*8+i, n = nb*8 .. +8 (dword j: n = 2j, 2j+1).
        // Column n = nb*8 + m needs dword p = (k = 2p, 2p+1) of its 8 k values.
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          u32x4 v;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t a = rb[2 * p + 1][m >> 1], b = rb[2 * p][m >> 1];
            v[p] = (m & 1) ? hi_halves(a, b) : lo_halves(a, b);
          }
          const int r = nb * 8 + m;
          *reinterpret_cast<u32x4*>(bs + r * (BK * 2) + swz(r, kb) * 16) = v;
        }
      }
    };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // weight-tile row of the wave's fn-th 32-row block
    auto b_block_row = [&](int fn) {
      if constexpr (GATED) {
        constexpr int half_fn = C::FN / 2;
        const int half = fn / half_fn, sub = fn % half_fn;
        return half * (BN / 2) + wn * (BN / 4) + sub * 32;
      } else {
        return wn * (BN / 2) + fn * 32;
      }
    };

    load_a(0);
    load_b(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) {
        load_a(kt + 1);
        load_b(kt + 1);
      }
      const unsigned char* as = As + buf * C::A_BYTES;
      const unsigned char* bs = Bs + buf * C::B_BYTES;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int chunk = 2 * ks + (lane >> 5);
        bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int r = wm * C::WTM + i * 32 + (lane & 31);
          af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(as + r * (BK * 2) + swz(r, chunk) * 16));
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int r = b_block_row(j) + (lane & 31);
          bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bs + r * (BK * 2) + swz(r, chunk) * 16));
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store_stage(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: registers -> bf16 tile in LDS (swizzled 16-byte chunks) -> global
    // acc[i][j][4q+s] is output row (wm*WTM + i*32 + lane%32), column
    // (block column base + 8q + 4*(lane/32) + s).
    unsigned char* ot = smem;  // [BM][OUTW] bf16
    constexpr int OUT_ROW_BYTES = C::OUTW * 2;
    const int half_lane = lane >> 5;
    if constexpr (GATED) {
      constexpr int half_fn = C::FN / 2;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm * C::WTM + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < half_fn; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float hv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const float g = bf16_bits_to_f32(f32_to_bf16_bits(acc[i][j][4 * q + s]));
              const float u = bf16_bits_to_f32(f32_to_bf16_bits(acc[i][j + half_fn][4 * q + s]));
              hv[s] = g / (1.0f + __expf(-g)) * u;
            }
            const int col = wn * (BN / 4) + j * 32 + 8 * q + 4 * half_lane;
            const int c = col >> 3;
            uint2 pk{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            *reinterpret_cast<uint2*>(ot + r * OUT_ROW_BYTES + ((c ^ (r & (C::OUT_CPR - 1))) * 16) + (col & 7) * 2) = pk;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm * C::WTM + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wn * C::WTN + j * 32 + 8 * q + 4 * half_lane;
            const int c = col >> 3;
            uint2 pk{pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]),
                     pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
            *reinterpret_cast<uint2*>(ot + r * OUT_ROW_BYTES + ((c ^ (r & (C::OUT_CPR - 1))) * 16) + (col & 7) * 2) = pk;
          }
        }
      }
    }
    __syncthreads();
    constexpr int kStoreIters = BM * C::OUT_CPR / kThreads;
#pragma unroll
    for (int it = 0; it < kStoreIters; ++it) {
      const int idx = it * kThreads + tid;
      const int r = idx / C::OUT_CPR, c = idx % C::OUT_CPR;
      const int64_t col = n0 + c * 8;
      if (r < rows_valid && col < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(ot + r * OUT_ROW_BYTES + ((c ^ (r & (C::OUT_CPR - 1))) * 16));
        *reinterpret_cast<u32x4*>(out + (row0 + r) * ldo + col) = v;
      }
    }
    __syncthreads();  // LDS is reused by the next tile's first stage
  }
}

template <int BM, int BN, bool GATED, bool B_NMAJOR>
hipError_t launch_grouped(const uint16_t* A, int64_t lda, const uint16_t* W, int64_t w_expert_stride, int64_t ldw,
                          int64_t gate_up_rows, int64_t N, int64_t K, const int32_t* offsets, int E, int64_t cap_rows,
                          uint16_t* out, int64_t ldo, hipStream_t stream) {
  using C = Tile<BM, BN, GATED>;
  auto kern = grouped_gemm_kernel<BM, BN, GATED, B_NMAJOR>;
  static bool attr_set[64] = {};
  const int dev = current_device();
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (st != hipSuccess) return st;
    attr_set[dev] = true;
  }
  const int grid = device_cu_count(dev);  // one 128 KB-LDS workgroup per CU
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), C::LDS_BYTES, stream, A, lda, W, w_expert_stride, ldw,
                     gate_up_rows, N, K, offsets, E, cap_rows, out, ldo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_up_swiglu(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                 int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf,
                                 hipStream_t stream) {
  // A = x_perm [cap, d] (K = d); weights [E, 2h, d], gate rows n, up rows h + n; out h_buf [cap, h]
  return launch_grouped<128, 256, true, false>(x_perm, d, w_ug, 2 * h * d, d, h, h, d, offsets, E, cap_rows, h_buf, h,
                                               stream);
}

hipError_t launch_gemm_down(const uint16_t* h_buf, const int32_t* offsets, const uint16_t* w_down, int64_t cap_rows,
                            int64_t d, int64_t h, int32_t E, uint16_t* y_perm, hipStream_t stream) {
  // A = h_buf [cap, h] (K = h); weights [E, h, d] N-contiguous; out y_perm [cap, d]
  return launch_grouped<128, 256, false, true>(h_buf, h, w_down, h * d, d, 0, d, h, offsets, E, cap_rows, y_perm, d,
                                               stream);
}

}  // namespace moe
