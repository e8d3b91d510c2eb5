// Persistent grouped GEMMs over ragged per-expert row blocks, bf16 MFMA with
// fp32 accumulation. The forward's two projections of a SwiGLU expert (OLMo
// report, Eq 13):
//
//   up:   h_buf[rows_e]  = bf16( SiLU(bf16(G)) * bf16(U) ),  [G | U] = x_perm[rows_e] * W_ug[e]^T
//   down: y_perm[rows_e] = bf16( h_buf[rows_e] * W_down[e] )
//
// and, with the same kernels, any plain grouped projection and its input
// gradient (Eq 15's Dgrad is forward-shaped); the weight gradient, which
// contracts over the ragged rows, has its own kernel further down. The up
// projection can also store its bf16 pre-activation [G | U] for the backward.
//
// OLMo report Sec 9.2 / Fig 37: the offsets stay on the device; one grouped
// kernel walks the tiles of every expert's problem. Here each workgroup
// rebuilds the problem list from the device offsets in LDS (expert e owns
// sorted rows [offsets[e], offsets[e+1]); its pointers are affine in e and
// offsets[e]), then takes output tiles in a static round-robin until none is
// left. Empty experts contribute no tile; rows past an expert's block and
// columns past N are never stored. The A rows of the up projection can be
// gathered from the token matrix through the dispatch order instead of a
// permuted copy.
//
// Tiles are 32x32 blocks of v_mfma_f32_32x32x16_bf16 per wave. The MFMA takes
// the weight fragment as its first operand, so each lane ends up holding four
// consecutive output columns of one output row; the epilogue packs them to
// bf16, stages the tile through LDS and writes 16-byte chunks. For the up
// projection the BN weight rows of a tile are BN/2 gate rows followed by the
// BN/2 matching up rows (W_ug is gate-then-up, chunked), so a lane holds each
// gate value and its up value in the same register slot and SwiGLU is applied
// in registers.
//
// Two main loops:
//  * pipelined (K % 8 == 0): global -> LDS direct loads
//    (global_load_lds_dwordx4) into a ring of 64-deep stages, one barrier per
//    stage, the next 16-deep slice's fragments read under the current slice's
//    MFMAs; 256 x 256 tiles on 8 waves with a 2-slot ring for large expert
//    blocks, 128 x 256 tiles on 8 waves with a 3-slot ring otherwise.
//    N-contiguous weights (W_down [h, d]) land in LDS as they are in memory
//    and their fragments come from the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16).
//    With K not a multiple of 64 the same loop loads through buffer resources and
//    the chunks of its last stage at k >= K get an offset past the resource's
//    range, so they stage zeros for both operands.
//  * register-staged (any K % 8 == 0, operands too large for the pipelined
//    loop's 32-bit offsets): global -> registers -> LDS with zero fill for the K
//    remainder, double-buffered, 128 x 256 tiles on 4 waves; N-contiguous blocks
//    of 8(k) x 8(n) are transposed in registers.

#include <atomic>
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int BK = 64;         // K per stage: 8 chunks of 16 bytes per tile row
constexpr int kChunksK = BK / 8;
constexpr int kGroupM = 8;     // m-tiles per group in the tile order (operand reuse in L2)

#define LDS_AS __attribute__((address_space(3)))
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Tile geometry: BM x BN weight rows per workgroup, WGM x WGN waves, NST LDS stages.
template <int BM_, int BN_, int WGM_, int WGN_, int NST_, bool GATED_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, NST = NST_;
  static constexpr bool GATED = GATED_;
  static constexpr int NWAVES = WGM * WGN, THREADS = 64 * NWAVES;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int OUTW = GATED ? BN / 2 : BN;  // output columns per tile
  static constexpr int OUT_CPR = OUTW / 8;          // 16-byte chunks per output row
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NST * STAGE_BYTES;
  static constexpr int A_LOADS = BM * kChunksK / THREADS;  // register path: 16-byte chunks per thread
  static constexpr int B_LOADS = BN * kChunksK / THREADS;
  static constexpr int A_OPS = A_BYTES / 1024 / NWAVES;  // pipelined path: 1 KB wave loads per wave per stage
  static constexpr int B_OPS = B_BYTES / 1024 / NWAVES;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must split into 32x32 blocks");
  static_assert(BM * OUTW * 2 <= LDS_BYTES, "epilogue tile must fit in the stage buffers");
  static_assert((OUT_CPR & (OUT_CPR - 1)) == 0, "output chunk count must be a power of two");
  static_assert(!GATED || FN % 2 == 0, "gated tiles pair gate and up blocks");
  static_assert(A_BYTES % (1024 * NWAVES) == 0 && B_BYTES % (1024 * NWAVES) == 0, "stage must split into wave loads");
};

struct GemmArgs {
  const uint16_t* A;        // activations: [cap_rows, K], or token rows [a_tokens, K] when a_rows is set
  int64_t lda;
  const int32_t* a_rows;    // optional: sorted row p reads A row a_rows[p] / a_k (the fused permuted gather)
  int a_k;
  int64_t a_tokens;
  const uint16_t* W;        // expert weights
  int64_t w_expert_stride;  // elements between experts
  int64_t ldw;              // row pitch of a weight matrix
  int64_t gate_up_rows;     // gated: row offset of the up block (h); unused otherwise
  int64_t N;                // output columns
  int64_t K;
  const int32_t* offsets;   // [E+1]
  int E;
  int64_t cap_rows;
  uint16_t* out;            // [cap_rows, N], row pitch ldo
  int64_t ldo;
  uint16_t* u_out = nullptr;  // gated only, optional: the pre-activation U = [G | Up], [cap_rows, 2N], pitch 2N
};

template <int THREADS>
struct ProblemList {
  int seg_lo[MOE_MAX_EXPERTS];
  int seg_rows[MOE_MAX_EXPERTS];
  int mt_prefix[MOE_MAX_EXPERTS + 1];
  int scan_tmp[THREADS / 64];  // one total per wave
};

struct TileCoord {
  int e;
  int mi;
  int64_t row0;     // first sorted row of the tile
  int rows_valid;   // rows of the tile inside the expert's block
  int64_t n0;       // first output column
};

// K-contiguous tile rows are 128 B (8 chunks of 16 B). LDS has 64 banks (256 B
// per cycle), so two rows share a bank window and a 16-lane read group spans 16
// rows: chunk c of row r is kept at position c ^ ((r / 2) % 8), which gives the
// 16 rows of a group 16 distinct (window half, position) pairs.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// N-contiguous rows (W_down tiles) are BN*2 bytes. A 32-lane half of a transpose
// read touches 4 rows x 4 consecutive chunks; chunk c of row k is kept at
// c ^ (4 * (k % 4)), which spreads those 16 chunks over the 16 bank positions.
__device__ __forceinline__ int swz_n(int krow, int chunk) { return chunk ^ (4 * (krow & 3)); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// v_perm_b32 byte select: result bytes [b0 b1 a0 a1] (lo halves) or [b2 b3 a2 a3] (hi halves).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(a, b, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(a, b, 0x07060302u); }

// One 16-byte chunk per lane from base + off (bytes) into LDS[lds_addr + 16 * lane]: a
// wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte offset (M0 holds the
// wave's LDS base).
__device__ __forceinline__ void dma16_off(uint64_t base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// One 16-byte chunk per lane through a buffer resource into LDS[lds_addr + 16 * lane]: a lane whose
// offset lies past the resource's range reads nothing and stages zeros.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, uint32_t soff, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);  // the same in every lane: M0 takes it from an SGPR
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(soff), "s"(lds_addr)
               : "memory", "m0");
}

// A 64-bit value every lane holds the same value of, moved to SGPRs.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A pointer every lane holds the same value of, moved to SGPRs.
__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// vmcnt(N) together with lgkmcnt(0): this wave's own LDS reads are complete
// too, whatever order the compiler left them in, before a barrier after which
// other waves may overwrite the slot those reads came from.
//
// EXACT: issue it as the compiler's own s_waitcnt, so that its wait bookkeeping knows every
// earlier LDS read is complete and adds no wait of its own for them behind newer reads.
// s_waitcnt's immediate on gfx9: vmcnt in bits [3:0] and [15:14], expcnt in [6:4] (7: no
// wait), lgkmcnt in [11:8].
template <int N, bool EXACT = false>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (EXACT) __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" : : : "memory"); }

// Barrier for LDS hand-offs only: this wave's LDS accesses are complete, its
// global stores may still be in flight (a full __syncthreads would wait for
// their write acknowledgements too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

// Scheduling hint for one K slice: spread READS LDS reads (the next slice's
// fragments) between the MFMAS matrix instructions of the current one, so the
// reads' latency hides behind matrix work instead of stalling the next slice.
template <int MFMAS, int READS>
__device__ __forceinline__ void interleave_reads() {
  constexpr int kPer = MFMAS / READS > 0 ? MFMAS / READS : 1;
  constexpr int kPairs = READS < MFMAS ? READS : MFMAS;
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
  }
  if constexpr (MFMAS > kPairs * kPer) __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - kPairs * kPer, 0);
  if constexpr (READS > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, READS - kPairs, 0);
}

// Map a persistent workgroup to a logical worker so that consecutive logical
// workers (which take consecutive tiles) sit on one XCD: workgroups are
// dealt to the 8 XCDs round-robin.
__device__ __forceinline__ int logical_worker() {
  const int G = gridDim.x, b = blockIdx.x;
  if (G % 8 != 0) return b;
  return (b % 8) * (G / 8) + b / 8;
}

// Problem list from the device offsets, clamped so no access leaves the buffers:
// per expert its first row, its row count and the prefix of its m-tile counts.
template <int BM, int THREADS>
__device__ void build_problem_list(const GemmArgs& g, ProblemList<THREADS>& pl) {
  const int tid = threadIdx.x;
  constexpr int kPer = (MOE_MAX_EXPERTS + THREADS - 1) / THREADS;
  int mt_local[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    int mt = 0;
    if (e < g.E) {
      int64_t lo = g.offsets[e], hi = g.offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > g.cap_rows ? g.cap_rows : lo);
      hi = hi < lo ? lo : (hi > g.cap_rows ? g.cap_rows : hi);
      pl.seg_lo[e] = (int)lo;
      pl.seg_rows[e] = (int)(hi - lo);
      mt = (int)((hi - lo + BM - 1) / BM);
    }
    mt_local[i] = mt;
    sum += mt;
  }
  // Exclusive prefix of the per-thread sums: an inclusive scan inside each wave (shuffles), the
  // waves' totals through LDS, then each thread adds the totals of the waves before it.
  constexpr int kWaves = THREADS / 64;
  const int lane = tid & 63, wave = tid >> 6;
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(incl, off, 64);
    if (lane >= off) incl += up;
  }
  if (lane == 63) pl.scan_tmp[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int v = pl.scan_tmp[w];
    before += w < wave ? v : 0;
    total += v;
  }
  int run = before + incl - sum;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    if (e < g.E) pl.mt_prefix[e] = run;
    run += mt_local[i];
  }
  if (tid == 0) pl.mt_prefix[g.E] = total;
  __syncthreads();
}

// Tile t -> (expert, m-tile, n-tile). Groups of GM consecutive m-tiles
// sweep every n-tile before the next group starts, so tiles that run at the
// same time share A rows and weight rows.
template <int BM, int TILE_N, int THREADS>
__device__ __forceinline__ TileCoord tile_coord(int64_t t, int64_t n_tiles, int total_mt, int E,
                                                const ProblemList<THREADS>& pl, int group_m = kGroupM) {
  const int kGroupM = group_m;
  const int64_t group_span = (int64_t)kGroupM * n_tiles;
  const int64_t group = t / group_span;
  const int64_t in_group = t - group * group_span;
  const int64_t g0 = group * kGroupM;
  const int gsize = (int)((total_mt - g0) < kGroupM ? (total_mt - g0) : kGroupM);
  const int64_t nt = in_group / gsize;
  const int gm = (int)(g0 + (in_group - nt * gsize));
  int lo_e = 0, hi_e = E;  // largest e with mt_prefix[e] <= gm: the non-empty expert owning m-tile gm
  while (hi_e - lo_e > 1) {
    const int mid = (lo_e + hi_e) >> 1;
    if (pl.mt_prefix[mid] <= gm) lo_e = mid; else hi_e = mid;
  }
  // every lane holds the same coordinates (LDS reads of the problem list): keep them in scalar
  // registers, where the epilogue's buffer descriptor and the load bases need them
  TileCoord c;
  c.e = __builtin_amdgcn_readfirstlane(lo_e);
  c.mi = __builtin_amdgcn_readfirstlane(gm - pl.mt_prefix[lo_e]);
  c.row0 = uniform_i64((int64_t)pl.seg_lo[lo_e] + (int64_t)c.mi * BM);
  c.rows_valid = __builtin_amdgcn_readfirstlane(min(BM, pl.seg_rows[lo_e] - c.mi * BM));
  c.n0 = uniform_i64(nt * TILE_N);
  return c;
}

// weight-tile row of a wave's fn-th 32-row block (gated: the first FN/2 blocks are gate rows,
// the rest the matching up rows, BN/2 further down)
template <class C>
__device__ __forceinline__ int b_block_row(int wn, int fn) {
  if constexpr (C::GATED) {
    constexpr int half_fn = C::FN / 2;
    const int half = fn / half_fn, sub = fn % half_fn;
    return half * (C::BN / 2) + wn * (C::BN / 2 / C::WGN) + sub * 32;
  } else {
    return wn * C::WTN + fn * 32;
  }
}

// SiLU(g) * u of the bf16-rounded gate and up values, in fp32 with the hardware
// exponential and reciprocal (a few fp32 ulps, far below the bf16 rounding of the result).
__device__ __forceinline__ float swiglu(float gv, float uv) { return gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv; }

// threadIdx.x, through an opaque register move when OPAQUE: the epilogues' LDS and global
// addresses are fixed per lane, so the compiler otherwise computes them once before the tile
// loop and keeps them (about 60 registers) live through every main loop. The 256-row tiles with
// a plain (256-column) output need those registers for the second fragment set, and the
// U-keeping and weight-gradient launches to avoid spilling; the other tiles are faster with the
// addresses kept.
template <bool OPAQUE>
__device__ __forceinline__ int epilogue_tid() {
  int tid = threadIdx.x;
  if constexpr (OPAQUE) asm volatile("" : "+v"(tid));
  return tid;
}
template <class C>
constexpr bool kOpaqueEpilogue = !C::GATED && C::BM == 256;

// Registers -> bf16 tile in LDS (swizzled 16-byte chunks) -> global. For the
// gated projection, SwiGLU is applied here: g and u are rounded to bf16 first,
// then SiLU(g) * u is evaluated in fp32 with the hardware exponential and
// reciprocal (a few fp32 ulps, far below the bf16 rounding of the result).
// acc[i][j][4q+s] is output row (wm*WTM + i*32 + lane%32), column
// (block column base + 8q + 4*(lane/32) + s).
template <class C>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[C::FM][C::FN], unsigned char* smem, const GemmArgs& g,
                                         const TileCoord& tc) {
  constexpr int BM = C::BM, BN = C::BN;
  const int tid = epilogue_tid<kOpaqueEpilogue<C>>(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  unsigned char* ot = smem;  // [BM][OUTW] bf16
  constexpr int OUT_ROW_BYTES = C::OUTW * 2;
  const int half_lane = lane >> 5;
  if constexpr (C::GATED) {
    constexpr int half_fn = C::FN / 2;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int r = wm * C::WTM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < half_fn; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // g and u rounded to bf16 two at a time (one packed convert per pair)
          float hv[4];
#pragma unroll
          for (int s = 0; s < 4; s += 2) {
            const uint32_t g2 = pack_bf16x2(acc[i][j][4 * q + s], acc[i][j][4 * q + s + 1]);
            const uint32_t u2 = pack_bf16x2(acc[i][j + half_fn][4 * q + s], acc[i][j + half_fn][4 * q + s + 1]);
            hv[s] = swiglu(bf16_bits_to_f32(g2 & 0xFFFFu), bf16_bits_to_f32(u2 & 0xFFFFu));
            hv[s + 1] = swiglu(bf16_bits_to_f32(g2 >> 16), bf16_bits_to_f32(u2 >> 16));
          }
          const int col = wn * (BN / 2 / C::WGN) + j * 32 + 8 * q + 4 * half_lane;
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
  lds_barrier();
  // Thread tid takes chunk tid % OUT_CPR of rows tid / OUT_CPR + RSTEP * it: all its LDS reads
  // first, then the stores (one read's latency instead of one per store). The stores go through a
  // buffer resource that ends at the tile's last valid row, and a column past N gets an offset
  // past the end: the hardware drops those stores, so no branch separates them.
  constexpr int kStoreIters = BM * C::OUT_CPR / C::THREADS;
  constexpr int RSTEP = C::THREADS / C::OUT_CPR;
  static_assert(C::THREADS % C::OUT_CPR == 0, "a thread keeps one chunk column");
  const int c = tid % C::OUT_CPR, r0 = tid / C::OUT_CPR;
  u32x4 v[kStoreIters];
#pragma unroll
  for (int it = 0; it < kStoreIters; ++it) {
    const int r = r0 + RSTEP * it;
    v[it] = *reinterpret_cast<const u32x4*>(ot + r * OUT_ROW_BYTES + ((c ^ (r & (C::OUT_CPR - 1))) * 16));
  }
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      g.out + tc.row0 * g.ldo, (short)0, (int)((int64_t)tc.rows_valid * g.ldo * 2), 0x00020000);
  const int64_t col = tc.n0 + c * 8;
  const uint32_t col_off = col < g.N ? (uint32_t)(col * 2) : 0x80000000u;
  const uint32_t row_bytes = (uint32_t)(g.ldo * 2);
#pragma unroll
  for (int it = 0; it < kStoreIters; ++it) {
    const uint32_t off = (uint32_t)(r0 + RSTEP * it) * row_bytes + col_off;
    // Plain outputs (the down projection's y_perm, 256-column tiles) go out as non-temporal
    // stores: this launch never reads them back, and allocating them in L2 would evict operand
    // lines (-2% on the down projection in the zipf64 step, -8% back to back).
    __builtin_amdgcn_raw_buffer_store_b128(v[it], rsrc, off, 0, C::GATED ? 0 : 2 /* nt */);
  }
  lds_barrier();  // LDS is reused by the next tile
}

// Gated epilogue that also stores the pre-activation U = [G | Up] ([cap, 2N], pitch 2N). The
// bf16 U tile (BN/2 gate columns, then the BN/2 matching up columns) is staged in LDS; then each
// thread takes a gate chunk and its up chunk (8 columns each), stores both to U and the 8 SwiGLU
// values (the same rounding and arithmetic as the plain epilogue) to the output, so the
// accumulators are dead once the tile is staged.
template <class C>
__device__ __forceinline__ void epilogue_save_u(const f32x16 (&acc)[C::FM][C::FN], unsigned char* smem,
                                                const GemmArgs& g, const TileCoord& tc) {
  static_assert(C::GATED, "U exists for the gated projection only");
  constexpr int BM = C::BM, BN = C::BN;
  constexpr int U_CPR = BN / 8, U_ROW_BYTES = BN * 2, HALF = U_CPR / 2;
  static_assert(BM * U_ROW_BYTES <= C::LDS_BYTES, "U tile must fit in the stage buffers");
  const int tid = epilogue_tid<true>(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int half_lane = lane >> 5;
  unsigned char* ut = smem;  // [BM][BN] bf16
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int r = wm * C::WTM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = b_block_row<C>(wn, j) + 8 * q + 4 * half_lane;
        const int c = col >> 3;
        uint2 pk{pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]),
                 pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
        *reinterpret_cast<uint2*>(ut + r * U_ROW_BYTES + ((c ^ (r & (U_CPR - 1))) * 16) + (col & 7) * 2) = pk;
      }
    }
  }
  lds_barrier();
  // As the plain epilogue: thread tid takes gate chunk tid % HALF of rows tid / HALF + RSTEP * it,
  // all its LDS reads first, then U and H stores through buffer resources that end at the tile's
  // last valid row (columns past N get an offset past the end).
  const int64_t ldu = 2 * g.N;
  constexpr int kIters = BM * HALF / C::THREADS;
  constexpr int RSTEP = C::THREADS / HALF;
  static_assert(C::THREADS % HALF == 0, "a thread keeps one chunk column");
  const int c = tid % HALF, r0 = tid / HALF;
  u32x4 gv[kIters], uv[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int r = r0 + RSTEP * it;
    gv[it] = *reinterpret_cast<const u32x4*>(ut + r * U_ROW_BYTES + ((c ^ (r & (U_CPR - 1))) * 16));
    uv[it] = *reinterpret_cast<const u32x4*>(ut + r * U_ROW_BYTES + (((c + HALF) ^ (r & (U_CPR - 1))) * 16));
  }
  const __amdgpu_buffer_rsrc_t u_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      g.u_out + tc.row0 * ldu, (short)0, (int)((int64_t)tc.rows_valid * ldu * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t h_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      g.out + tc.row0 * g.ldo, (short)0, (int)((int64_t)tc.rows_valid * g.ldo * 2), 0x00020000);
  const int64_t col = tc.n0 + c * 8;
  const bool col_ok = col < g.N;
  const uint32_t u_col = col_ok ? (uint32_t)(col * 2) : 0x80000000u;
  const uint32_t h_col = col_ok ? (uint32_t)(col * 2) : 0x80000000u;
  const uint32_t up_bytes = (uint32_t)(g.N * 2);
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const uint32_t r = (uint32_t)(r0 + RSTEP * it);
    const uint32_t u_off = r * (uint32_t)(ldu * 2) + u_col;
    __builtin_amdgcn_raw_buffer_store_b128(gv[it], u_rsrc, u_off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(uv[it], u_rsrc, col_ok ? u_off + up_bytes : u_off, 0, 0);
    u32x4 hv;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float h0 = swiglu(bf16_bits_to_f32(gv[it][w] & 0xFFFFu), bf16_bits_to_f32(uv[it][w] & 0xFFFFu));
      const float h1 = swiglu(bf16_bits_to_f32(gv[it][w] >> 16), bf16_bits_to_f32(uv[it][w] >> 16));
      hv[w] = pack_bf16x2(h0, h1);
    }
    __builtin_amdgcn_raw_buffer_store_b128(hv, h_rsrc, r * (uint32_t)(g.ldo * 2) + h_col, 0, 0);
  }
  lds_barrier();  // LDS is reused by the next tile
}

// ============================================================================
// Pipelined main loop: direct global -> LDS loads into an NST-stage ring.
// ============================================================================
template <class C, bool B_NMAJOR, bool SAVE_U, bool KTAIL = false>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_pipe_kernel(GemmArgs g) {
  constexpr int BN = C::BN, NST = C::NST;
  constexpr int OPS = C::A_OPS + C::B_OPS;
  static_assert(OPS * (NST - 1) < 64, "outstanding wave loads must fit the vmcnt counter");
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  static_assert(!B_NMAJOR || BN * 2 <= 1024, "N-major tile rows must not exceed one wave load");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ ProblemList<C::THREADS> pl;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int wm_u = __builtin_amdgcn_readfirstlane(wm);  // the same, as a scalar: branches on it stay uniform

  build_problem_list<C::BM>(g, pl);
  const int total_mt = pl.mt_prefix[g.E];
  constexpr int TILE_N = C::GATED ? C::OUTW : BN;
  const int64_t n_tiles = (g.N + TILE_N - 1) / TILE_N;
  const int64_t total_tiles = (int64_t)total_mt * n_tiles;
  const int nk = (int)(KTAIL ? (g.K + BK - 1) / BK : g.K / BK);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // N-contiguous weights (the down projection) with at most 12 n-tiles: one m-tile per group, so the 32
  // consecutive tiles an XCD runs at once cover every n-tile of a few row tiles and most row tiles' A rows
  // are fetched into one XCD's L2 only (1-2% faster than groups of eight on the zipf64, Qwen3-shaped and
  // square workloads, 8 and 12 n-tiles). With more n-tiles that window would hold one or two row tiles
  // and no weight tile twice (16 n-tiles: 2% slower; 320: 18% slower), so groups of eight stay.
  const int group_m = (B_NMAJOR && n_tiles <= 12) ? 1 : kGroupM;
  for (int64_t t = logical_worker(); t < total_tiles; t += gridDim.x) {
    const TileCoord tc = tile_coord<C::BM, TILE_N>(t, n_tiles, total_mt, g.E, pl, group_m);
    const uint16_t* Wexp = g.W + (int64_t)tc.e * g.w_expert_stride;

    // Source of each lane's 16-byte chunk for k0 = 0, as a byte offset from a
    // wave-uniform base (the host guarantees the offsets fit in 32 bits). A wave
    // load fills 1 KB of LDS (lane l -> bytes [16l, 16l+16)), so the swizzle is
    // applied by choosing which global chunk each lane fetches. Rows past the
    // expert's block and columns past N are pointed at valid rows/columns: they
    // only feed outputs that are never stored.
    const uint64_t a_base = uniform_addr(g.a_rows != nullptr ? g.A : g.A + tc.row0 * g.lda);
    uint32_t a_off[C::A_OPS];
    if (g.a_rows != nullptr) {
      // Fused gather: the lane's dispatch slots of all its A loads are fetched together (one
      // memory round trip instead of one per load), then mapped to token rows with 32-bit
      // arithmetic (slot / k; slots < 2^31, and a tile exists only when there is at least one
      // slot). Bit-identical; the zipf64 gate/up GEMM 1.8% faster, the whole step 0.7%.
      int32_t slot[C::A_OPS];
      const int32_t* rows = g.a_rows + tc.row0;
#pragma unroll
      for (int t2 = 0; t2 < C::A_OPS; ++t2) {
        const int r = 8 * (wave + C::NWAVES * t2) + (lane >> 3);
        slot[t2] = rows[r < tc.rows_valid ? r : tc.rows_valid - 1];
      }
      const uint32_t last = (uint32_t)(g.a_tokens * g.a_k) - 1u;
#pragma unroll
      for (int t2 = 0; t2 < C::A_OPS; ++t2) {
        const int r = 8 * (wave + C::NWAVES * t2) + (lane >> 3);
        const int c = swz(r, lane & 7);  // the swizzle is an involution: position -> logical chunk
        const uint32_t s = slot[t2] < 0 ? 0u : min((uint32_t)slot[t2], last);
        const uint32_t token = s / (uint32_t)g.a_k;
        a_off[t2] = (uint32_t)(((int64_t)token * g.lda + c * 8) * 2);
      }
    } else {
#pragma unroll
      for (int t2 = 0; t2 < C::A_OPS; ++t2) {
        const int r = 8 * (wave + C::NWAVES * t2) + (lane >> 3);
        const int c = swz(r, lane & 7);
        const int rr = r < tc.rows_valid ? r : tc.rows_valid - 1;
        a_off[t2] = (uint32_t)(((int64_t)rr * g.lda + c * 8) * 2);
      }
    }
    const uint64_t b_base = uniform_addr(Wexp);
    uint32_t b_off[C::B_OPS];
#pragma unroll
    for (int t2 = 0; t2 < C::B_OPS; ++t2) {
      const int j = wave + C::NWAVES * t2;
      if constexpr (!B_NMAJOR) {
        const int r = 8 * j + (lane >> 3);
        const int c = swz(r, lane & 7);
        int64_t n, wrow;
        if constexpr (C::GATED) {
          const int half = r >= BN / 2 ? 1 : 0;
          n = tc.n0 + (r - half * (BN / 2));
          if (n >= g.N) n = tc.n0;
          wrow = n + half * g.gate_up_rows;
        } else {
          n = tc.n0 + r;
          if (n >= g.N) n = tc.n0;
          wrow = n;
        }
        b_off[t2] = (uint32_t)((wrow * g.ldw + c * 8) * 2);
      } else {
        // 64 k-rows of BN columns, chunk positions swizzled by swz_n
        constexpr int kRowsPerOp = 1024 / (BN * 2);
        constexpr int kChunksRow = BN / 8;
        const int r = j * kRowsPerOp + lane / kChunksRow;
        const int c = swz_n(r, lane % kChunksRow);
        int64_t col = tc.n0 + c * 8;
        if (col >= g.N) col = tc.n0;
        b_off[t2] = (uint32_t)(((int64_t)r * g.ldw + col) * 2);
      }
    }
    const uint64_t b_step = (uint64_t)(B_NMAJOR ? BK * g.ldw : BK) * 2;
    // K not a multiple of 64: every load goes through a buffer resource, and in the last stage the
    // chunks at k >= K get an offset past the resource's range, so they stage zeros (both operands).
    uint32_t a_tail_off[KTAIL ? C::A_OPS : 1], b_tail_off[KTAIL ? C::B_OPS : 1];
    __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc;
    if constexpr (KTAIL) {
      const int k_last = (nk - 1) * BK;
#pragma unroll
      for (int t2 = 0; t2 < C::A_OPS; ++t2) {
        const int r = 8 * (wave + C::NWAVES * t2) + (lane >> 3);
        a_tail_off[t2] = k_last + swz(r, lane & 7) * 8 < g.K ? a_off[t2] : 0x80000000u;
      }
#pragma unroll
      for (int t2 = 0; t2 < C::B_OPS; ++t2) {
        const int j = wave + C::NWAVES * t2;
        int kk;
        if constexpr (!B_NMAJOR) {
          const int r = 8 * j + (lane >> 3);
          kk = k_last + swz(r, lane & 7) * 8;
        } else {
          constexpr int kRowsPerOp = 1024 / (BN * 2);
          kk = k_last + j * kRowsPerOp + lane / (BN / 8);
        }
        b_tail_off[t2] = kk < g.K ? b_off[t2] : 0x80000000u;
      }
      const int64_t a_range = g.a_rows != nullptr ? g.a_tokens * g.lda * 2 : (int64_t)tc.rows_valid * g.lda * 2;
      a_rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(a_base), (short)0, (int)a_range, 0x00020000);
      b_rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(b_base), (short)0,
                                                 (int)(g.w_expert_stride * 2), 0x00020000);
    }
    // Loads of stage kt, the ones with index % parts == part (issue(kt) issues them all).
    auto issue_part = [&](int kt, int part, int parts) {
      const uint32_t sa = lds0 + (uint32_t)((kt % NST) * C::STAGE_BYTES);
      const uint32_t sb = sa + C::A_BYTES;
      const uint32_t wave_lds = __builtin_amdgcn_readfirstlane((uint32_t)wave * 1024u);
      if constexpr (KTAIL) {
        const bool last = kt == nk - 1;
        const uint32_t a_soff = __builtin_amdgcn_readfirstlane((uint32_t)kt * (BK * 2));
        const uint32_t b_soff = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)kt * b_step));
#pragma unroll
        for (int t2 = 0; t2 < C::A_OPS; ++t2)
          if (t2 % parts == part)
            dma16_buf(a_rsrc, last ? a_tail_off[t2] : a_off[t2], a_soff, sa + wave_lds + (uint32_t)(C::NWAVES * t2 * 1024));
#pragma unroll
        for (int t2 = 0; t2 < C::B_OPS; ++t2)
          if (t2 % parts == part)
            dma16_buf(b_rsrc, last ? b_tail_off[t2] : b_off[t2], b_soff, sb + wave_lds + (uint32_t)(C::NWAVES * t2 * 1024));
      } else {
        const uint64_t ak = a_base + (uint64_t)kt * (BK * 2);
        const uint64_t bk = b_base + (uint64_t)kt * b_step;
#pragma unroll
        for (int t2 = 0; t2 < C::A_OPS; ++t2)
          if (t2 % parts == part) dma16_off(ak, a_off[t2], sa + wave_lds + (uint32_t)(C::NWAVES * t2 * 1024));
#pragma unroll
        for (int t2 = 0; t2 < C::B_OPS; ++t2)
          if (t2 % parts == part) dma16_off(bk, b_off[t2], sb + wave_lds + (uint32_t)(C::NWAVES * t2 * 1024));
      }
    };
    auto issue = [&](int kt) { issue_part(kt, 0, 1); };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragments of one 16-deep K slice: A rows of the wave tile and B columns.
    // Two register sets: the slice the MFMAs consume and the next one, read
    // from LDS while those MFMAs run.
    bf16x8 af[2][C::FM], bfr[2][C::FN];
    auto load_frags = [&](int set, int slot, int ks) {
      const unsigned char* as = smem + slot * C::STAGE_BYTES;
      const unsigned char* bs = as + C::A_BYTES;
      const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm * C::WTM + i * 32 + (lane & 31);
        af[set][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(as + r * (BK * 2) + swz(r, chunk) * 16));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if constexpr (!B_NMAJOR) {
          const int r = b_block_row<C>(wn, j) + (lane & 31);
          bfr[set][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bs + r * (BK * 2) + swz(r, chunk) * 16));
        } else {
          // lane l gets k = 16ks + 8(l/32) + 0..7 of column nb0 + l%32: two transpose reads of
          // 4 k each; in a 16-lane group lane j points at k-row j/4, columns 4(j%4)..+3.
          // the swizzle depends on the k-row only through krow % 4, which ks and q
          // leave unchanged: one lane address plus a constant slice offset
          const int nb0 = wn * C::WTN + j * 32;
          const int c = (nb0 >> 3) + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
          const int kr = 8 * (lane >> 5) + ((lane & 15) >> 2);
          const unsigned char* lane_p = bs + kr * (BN * 2) + swz_n(kr, c) * 16 + (lane & 1) * 8;
          uint2 part[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const v4i16 v =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(lane_p + (ks * 16 + 4 * q) * (BN * 2)));
            part[q] = __builtin_bit_cast(uint2, v);
          }
          bfr[set][j] = __builtin_bit_cast(bf16x8, u32x4{part[0].x, part[0].y, part[1].x, part[1].y});
        }
      }
    };
    // B-fragment-major order: the first MFMAs of a slice need the A fragments (read first) and
    // one B fragment, so the B reads issued last have the most matrix work to hide behind.
    auto mfmas = [&](int set) {
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[set][j], af[set][i], acc[i][j], 0, 0, 0);
    };
    // The next slice's fragments are read during the current slice's MFMAs (two register
    // sets, `load_frags` into the set the MFMAs do not use). The 256x256 tiles with a plain
    // (256-column) output fit the second set only with their epilogue addresses kept out of the
    // main loop (kOpaqueEpilogue); there it makes the down projection 2% (zipf64) and 5%
    // (square) faster than reading each slice just before its MFMAs, bit-identical.
    //
    // Stage kt is complete for this wave once only the later stages already issued are still
    // in flight; after the barrier it is complete for every wave, and every wave has finished
    // reading the stage before it. The hand-off waits through the compiler's own s_waitcnt and
    // the last stage is peeled (see stage_body): the stage's MFMAs after the hand-off then wait
    // for nothing (1-3% faster on the zipf64, square and Qwen3-shaped workloads, bit-identical).
    auto wait_stage = [&](int kt) {
      const int ahead = min(nk - 1, kt + NST - 2) - kt;  // stages issued after kt, still allowed in flight
      if (NST >= 4 && ahead >= 2) wait_vmcnt_lds<(NST >= 4 ? 2 : 0) * OPS, true>();
      else if (NST >= 3 && ahead >= 1) wait_vmcnt_lds<(NST >= 3 ? 1 : 0) * OPS, true>();
      else wait_vmcnt_lds<0, true>();
      bare_barrier();
    };

    // Waves w and w+4 share a SIMD. With a 2-slot ring, waves 4..7 issue their share of a
    // stage's loads one slice after waves 0..3 (at the start of the next stage instead of at
    // the hand-off): when both waves of a SIMD issue eight wave loads at once, both can stall on
    // load issue while neither issues MFMAs. Their loads still have three of the four slices to
    // land (issuing them two slices late instead was 10% slower). Bit-identical results; the
    // 256-row gate/up GEMM 2% faster on the zipf64 and square workloads, the down projection 2%
    // (zipf64) and 4% (square). The launch that also keeps U has no registers to spare for it
    // (the compiler spills).
    const bool late_issue = !SAVE_U && NST == 2 && C::NWAVES == 8 && wave >= 4;
    // A wave whose rows all lie past the expert's block (the last row tile of an expert) does no
    // matrix work: it keeps its share of every stage's loads and the barrier sequence of the waves
    // that compute (the same issues, waits and barriers as below), without fragment reads or MFMAs.
    // Its accumulators stay zero and feed no stored row.
    if (wm_u * C::WTM >= tc.rows_valid) {
      if constexpr (NST == 2) {
        issue(0);
        if (nk > 1) {
          issue(1);
          wait_vmcnt_lds<OPS, true>();
        } else {
          wait_vmcnt_lds<0, true>();
        }
        bare_barrier();
        for (int kt = 0; kt + 1 < nk; ++kt) {
          if (late_issue && kt > 0) issue(kt + 1);
          wait_vmcnt_lds<0, true>();
          bare_barrier();
          if (!late_issue && kt + 2 < nk) issue(kt + 2);
        }
      } else {
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
          if (s < nk) issue(s);
        for (int kt = 0; kt < nk; ++kt) {
          wait_stage(kt);
#pragma unroll
          for (int ks = 0; ks < BK / 16; ++ks)
            if (kt + NST - 1 < nk) issue_part(kt + NST - 1, ks, BK / 16);
        }
      }
    } else {
      // Both slots of a 2-slot ring are free at the tile start: fill them and wait for the first
      // only, so the second has a whole stage more to land (0.5-1.5% faster, bit-identical).
      if constexpr (NST == 2) {
        issue(0);
        if (nk > 1) {
          issue(1);
          wait_vmcnt_lds<OPS, true>();
          bare_barrier();
        } else {
          wait_stage(0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
          if (s < nk) issue(s);
        wait_stage(0);
      }
      load_frags(0, 0, 0);
      // One stage of the main loop; `last_c` marks the peeled last stage (no hand-off). Every
      // other stage hands off unconditionally, so no branch merges a path with pending fragment
      // reads into one without them (the compiler's wait bookkeeping stays exact).
      auto stage_body = [&](int kt, auto last_c) {
        constexpr bool kLast = decltype(last_c)::value;
        // The slot stage kt+NST-1 fills held stage kt-1, which every wave finished
        // reading before the barrier that made stage kt visible.
        // With a 3-slot ring (128-row tiles) the next stage's loads are spread over the four
        // slices; the 2-slot ring issues them a stage ahead (right after that barrier, inside the
        // previous stage's last slice; the second wave of each SIMD one slice later, see
        // late_issue; stage 1 at the tile start).
        constexpr int kParts = NST >= 3 ? BK / 16 : 1;
        const bool more = kt + NST - 1 < nk;
        const int slot = kt % NST;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          const int cur = ks & 1;
          if (more && ks < kParts && (NST > 2 || (late_issue && kt > 0))) issue_part(kt + NST - 1, ks, kParts);
          if (ks + 1 < BK / 16) {
            load_frags(cur ^ 1, slot, ks + 1);
            mfmas(cur);
            interleave_reads<C::FM * C::FN, C::FM + (B_NMAJOR ? 2 : 1) * C::FN>();
          } else {
            // The last slice's fragments are already in registers: hand the stage
            // off first (wait, barrier, refill of the slot just drained, reads of
            // the next stage's first slice) so that its MFMAs cover the barrier
            // and the read latency. The MFMAs stay outside the branch so the
            // accumulators keep one register assignment.
            if constexpr (!kLast) {
              wait_stage(kt + 1);
              if (NST == 2 && kt + 2 < nk && !late_issue) issue(kt + 2);
              load_frags(cur ^ 1, (kt + 1) % NST, 0);
            }
            mfmas(cur);
          }
        }
      };
      for (int kt = 0; kt + 1 < nk; ++kt) stage_body(kt, std::false_type{});
      stage_body(nk - 1, std::true_type{});
    }
    lds_barrier();  // every wave is done with the ring (all its loads were waited for) before the epilogue reuses it
    if constexpr (SAVE_U) epilogue_save_u<C>(acc, smem, g, tc);
    else epilogue<C>(acc, smem, g, tc);
  }
}

// ============================================================================
// Register-staged main loop: any K % 8 == 0 (zero fill of the K remainder).
// ============================================================================
template <class C, bool B_NMAJOR, bool SAVE_U>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_regs_kernel(GemmArgs g) {
  constexpr int BN = C::BN;
  static_assert(C::NST == 2, "register-staged loop double-buffers");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ ProblemList<C::THREADS> pl;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;

  build_problem_list<C::BM>(g, pl);
  const int total_mt = pl.mt_prefix[g.E];
  constexpr int TILE_N = C::GATED ? C::OUTW : BN;
  const int64_t n_tiles = (g.N + TILE_N - 1) / TILE_N;
  const int64_t total_tiles = (int64_t)total_mt * n_tiles;
  const int nk = (int)((g.K + BK - 1) / BK);

  unsigned char* As = smem;                   // [2][BM][BK] swizzled
  unsigned char* Bs = smem + 2 * C::A_BYTES;  // [2][BN][BK] swizzled

  for (int64_t t = logical_worker(); t < total_tiles; t += gridDim.x) {
    const TileCoord tc = tile_coord<C::BM, TILE_N>(t, n_tiles, total_mt, g.E, pl);
    const uint16_t* Wexp = g.W + (int64_t)tc.e * g.w_expert_stride;

    u32x4 ra[C::A_LOADS];
    u32x4 rb[C::B_LOADS];
    // Start of each of this thread's A rows (or -1 past the expert's block), fetched once per tile:
    // with the fused gather all the rows' dispatch slots are in flight together.
    int64_t a_row_start[C::A_LOADS];
    {
      int32_t slot[C::A_LOADS];
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int r = (i * C::THREADS + tid) / kChunksK;
        slot[i] = (g.a_rows != nullptr && r < tc.rows_valid) ? g.a_rows[tc.row0 + r] : 0;
      }
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int r = (i * C::THREADS + tid) / kChunksK;
        int64_t row = tc.row0 + r;
        if (g.a_rows != nullptr) {
          const int64_t cap = g.a_tokens * g.a_k;
          const int64_t sl = slot[i] < 0 ? 0 : (slot[i] >= cap ? cap - 1 : slot[i]);
          row = sl / g.a_k;
        }
        a_row_start[i] = r < tc.rows_valid ? row * g.lda : -1;
      }
    }
    auto load_a = [&](int kt) {
      const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int c = (i * C::THREADS + tid) % kChunksK;
        const int64_t kk = k0 + c * 8;
        ra[i] = (a_row_start[i] >= 0 && kk < g.K) ? *reinterpret_cast<const u32x4*>(g.A + a_row_start[i] + kk) : zero4();
      }
    };
    auto load_b = [&](int kt) {
      const int64_t k0 = (int64_t)kt * BK;
      if constexpr (!B_NMAJOR) {
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
          const int idx = i * C::THREADS + tid;
          const int r = idx / kChunksK, c = idx % kChunksK;
          int64_t wrow, ncol;
          if constexpr (C::GATED) {
            const int half = r / (BN / 2);
            ncol = tc.n0 + (r - half * (BN / 2));
            wrow = ncol + half * g.gate_up_rows;
          } else {
            ncol = tc.n0 + r;
            wrow = ncol;
          }
          const int64_t kk = k0 + c * 8;
          rb[i] = (ncol < g.N && kk < g.K) ? *reinterpret_cast<const u32x4*>(Wexp + wrow * g.ldw + kk) : zero4();
        }
      } else {
        // 8(k) x 8(n) block per thread: rows k0+kb*8+i, columns n0+nb*8 .. +8
        static_assert(!B_NMAJOR || (C::B_LOADS == 8 && (BK / 8) * (BN / 8) == C::THREADS),
                      "transposing loader covers the tile with one 8x8 block per thread");
        const int nb = tid % (BN / 8), kb = tid / (BN / 8);
        const int64_t ncol = tc.n0 + nb * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t kk = k0 + kb * 8 + i;
          rb[i] = (ncol < g.N && kk < g.K) ? *reinterpret_cast<const u32x4*>(Wexp + kk * g.ldw + ncol) : zero4();
        }
      }
    };
    auto store_stage = [&](int buf) {
      unsigned char* as = As + buf * C::A_BYTES;
      unsigned char* bs = Bs + buf * C::B_BYTES;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int idx = i * C::THREADS + tid;
        const int r = idx / kChunksK, c = idx % kChunksK;
        *reinterpret_cast<u32x4*>(as + r * (BK * 2) + swz(r, c) * 16) = ra[i];
      }
      if constexpr (!B_NMAJOR) {
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
          const int idx = i * C::THREADS + tid;
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
          const int r = b_block_row<C>(wn, j) + (lane & 31);
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
    if constexpr (SAVE_U) epilogue_save_u<C>(acc, smem, g, tc);
    else epilogue<C>(acc, smem, g, tc);
  }
}

// ============================================================================
// Wgrad: out[e] = A_e^T B_e, contracting over each expert's rows (Eq 15).
// A [cap_rows, P] and B [cap_rows, Q] are both row-major, so a K stage (64 of
// the expert's rows) lands in LDS row-contiguous for both operands and both
// MFMA fragments come from transpose reads, as the N-major weights of the
// forward do. The ragged contraction length is handled by clamping the rows a
// tail stage loads to the expert's last row and zeroing A's fragment entries
// past the block, so every product with a padded row is an exact zero.
//
// An expert with more than kWgradChunk rows is split along its rows into
// chunks of at most kWgradChunk: every chunk writes an fp32 partial gradient
// into the workspace and a second kernel sums an expert's partials in chunk
// order and rounds once to bf16 (deterministic, no atomics). Without the
// split the largest expert's tiles would each contract over all its rows and
// finish long after the rest of the grid.
// ============================================================================
struct WgradArgs {
  const uint16_t* A;  // [cap_rows, P]
  int64_t lda;
  const uint16_t* B;  // [cap_rows, Q]
  int64_t ldb;
  int64_t P, Q;       // out[e] is [P, Q]
  const int32_t* offsets;
  int32_t E;
  int64_t cap_rows;
  uint16_t* out;      // [E, P, Q]
  float* partial;     // [slots, P, Q] fp32 partial gradients of split experts
  int64_t slots;
};

// Per-expert row blocks, chunk counts and partial-slot bases from the device
// offsets (clamped as in the forward), in LDS. Experts are split in index
// order: slot_base[e] is the first partial slot of a split expert (-1 if the
// expert is not split). Identical in both Wgrad kernels.
struct WgradPlan {
  int lo[MOE_MAX_EXPERTS];
  int rows[MOE_MAX_EXPERTS];
  int chunks[MOE_MAX_EXPERTS];
  int slot_base[MOE_MAX_EXPERTS];
};

template <int THREADS>
__device__ void build_wgrad_plan(const WgradArgs& g, WgradPlan& pl) {
  for (int e = threadIdx.x; e < g.E; e += THREADS) {
    int64_t lo = g.offsets[e], hi = g.offsets[e + 1];
    lo = lo < 0 ? 0 : (lo > g.cap_rows ? g.cap_rows : lo);
    hi = hi < lo ? lo : (hi > g.cap_rows ? g.cap_rows : hi);
    const int rows = (int)(hi - lo);
    pl.lo[e] = (int)lo;
    pl.rows[e] = rows;
    pl.chunks[e] = rows > kWgradChunk ? (rows + kWgradChunk - 1) / kWgradChunk : 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int next = 0;
    for (int e = 0; e < g.E; ++e) {
      pl.slot_base[e] = pl.chunks[e] > 1 ? next : -1;
      if (pl.chunks[e] > 1) next += pl.chunks[e];
    }
  }
  __syncthreads();
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void grouped_wgrad_kernel(WgradArgs g) {
  constexpr int BM = C::BM, BN = C::BN, NST = C::NST;
  static_assert(!C::GATED && NST == 2, "plain output, double-buffered ring");
  static_assert(BM * 2 <= 1024 && BN * 2 <= 1024, "a stage row must fit one wave load");
  constexpr int OPS = C::A_OPS + C::B_OPS;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ WgradPlan pl;
  __shared__ int s_order[MOE_MAX_EXPERTS];
  __shared__ int s_item_end[MOE_MAX_EXPERTS];  // inclusive prefix of work items over s_order

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;

  build_wgrad_plan<C::THREADS>(g, pl);
  // Experts in descending row count (ties by index): dealing the largest
  // contractions first keeps the static round-robin schedule balanced.
  for (int e = tid; e < g.E; e += C::THREADS) {
    const int re = pl.rows[e];
    int rank = 0;
    for (int f = 0; f < g.E; ++f) {
      const int rf = pl.rows[f];
      rank += (rf > re || (rf == re && f < e)) ? 1 : 0;
    }
    s_order[rank] = e;
  }
  __syncthreads();
  const int64_t m_tiles = (g.P + BM - 1) / BM, n_tiles = (g.Q + BN - 1) / BN;
  const int per_chunk = (int)(m_tiles * n_tiles);  // output tiles of one expert (or one chunk of it)
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < g.E; ++i) {
      run += pl.chunks[s_order[i]] * per_chunk;
      s_item_end[i] = run;
    }
  }
  __syncthreads();
  const int total_items = __builtin_amdgcn_readfirstlane(s_item_end[g.E - 1]);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const GemmArgs ge{nullptr, 0, nullptr, 1, 0, nullptr, 0, 0, 0, g.Q, 0, nullptr, g.E, 0, g.out, g.Q};

  for (int64_t t = logical_worker(); t < total_items; t += gridDim.x) {
    int lo_i = 0, hi_i = g.E - 1;  // first position whose item range ends after t
    while (lo_i < hi_i) {
      const int mid = (lo_i + hi_i) >> 1;
      if (s_item_end[mid] > t) hi_i = mid; else lo_i = mid + 1;
    }
    const int pos = lo_i;
    const int64_t rem0 = t - (pos > 0 ? s_item_end[pos - 1] : 0);
    const int e = __builtin_amdgcn_readfirstlane(s_order[pos]);
    const int chunk = __builtin_amdgcn_readfirstlane((int)(rem0 / per_chunk));
    const int64_t rem = rem0 - (int64_t)chunk * per_chunk;
    const int lo = __builtin_amdgcn_readfirstlane(pl.lo[e] + chunk * kWgradChunk);
    const int all_rows = pl.rows[e] - chunk * kWgradChunk;
    const int rows = __builtin_amdgcn_readfirstlane(all_rows < kWgradChunk ? all_rows : kWgradChunk);
    const int slot_base = __builtin_amdgcn_readfirstlane(pl.slot_base[e]);
    const int64_t m0 = (rem / n_tiles) * BM, n0 = (rem % n_tiles) * BN;
    const int nk = (rows + BK - 1) / BK;

    // Per lane and wave load: stage row r (of 64) and the column chunk it fetches.
    constexpr int kRowsA = 1024 / (BM * 2), kChunksA = BM / 8;
    constexpr int kRowsB = 1024 / (BN * 2), kChunksB = BN / 8;
    int a_r[C::A_OPS], b_r[C::B_OPS];
    int a_col[C::A_OPS], b_col[C::B_OPS];  // P, Q < 2^24
#pragma unroll
    for (int t2 = 0; t2 < C::A_OPS; ++t2) {
      const int j = wave + C::NWAVES * t2;
      a_r[t2] = j * kRowsA + lane / kChunksA;
      const int64_t col = m0 + swz_n(a_r[t2], lane % kChunksA) * 8;
      a_col[t2] = (int)(col < g.P ? col : m0);
    }
#pragma unroll
    for (int t2 = 0; t2 < C::B_OPS; ++t2) {
      const int j = wave + C::NWAVES * t2;
      b_r[t2] = j * kRowsB + lane / kChunksB;
      const int64_t col = n0 + swz_n(b_r[t2], lane % kChunksB) * 8;
      b_col[t2] = (int)(col < g.Q ? col : n0);
    }
    auto issue = [&](int kt) {
      const uint32_t sa = lds0 + (uint32_t)((kt % NST) * C::STAGE_BYTES);
      const uint32_t sb = sa + C::A_BYTES;
      const int row0 = lo + kt * BK;
      const int left = rows - kt * BK;  // rows of this stage inside the block (>= 1)
      const uint64_t ab = uniform_addr(g.A + (int64_t)row0 * g.lda);
      const uint64_t bb = uniform_addr(g.B + (int64_t)row0 * g.ldb);
      const uint32_t wave_lds = __builtin_amdgcn_readfirstlane((uint32_t)wave * 1024u);
#pragma unroll
      for (int t2 = 0; t2 < C::A_OPS; ++t2) {
        const int r = a_r[t2] < left ? a_r[t2] : left - 1;
        dma16_off(ab, (uint32_t)(((int64_t)r * g.lda + a_col[t2]) * 2), sa + wave_lds + (uint32_t)(C::NWAVES * t2 * 1024));
      }
#pragma unroll
      for (int t2 = 0; t2 < C::B_OPS; ++t2) {
        const int r = b_r[t2] < left ? b_r[t2] : left - 1;
        dma16_off(bb, (uint32_t)(((int64_t)r * g.ldb + b_col[t2]) * 2), sb + wave_lds + (uint32_t)(C::NWAVES * t2 * 1024));
      }
    };
    // lane l gets k = 16ks + 8(l/32) + 0..7 of column cb + l%32 from a row-contiguous stage
    // region whose rows are ROWB bytes: two transpose reads of four k each.
    // The swizzle depends on the row only through row % 4, which ks and q leave
    // unchanged, so the slice offset is a constant added to one lane address.
    auto tr_frag = [&](const unsigned char* base, int rowb, int cb, int ks) {
      const int c = (cb >> 3) + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      const int kr = 8 * (lane >> 5) + ((lane & 15) >> 2);
      const unsigned char* lane_p = base + kr * rowb + swz_n(kr, c) * 16 + (lane & 1) * 8;
      uint2 part[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(lane_p + (ks * 16 + 4 * q) * rowb));
        part[q] = __builtin_bit_cast(uint2, v);
      }
      return u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
    };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
      issue(0);
      wait_vmcnt_lds<0>();
      bare_barrier();
    }
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) issue(kt + 1);
      const unsigned char* as = smem + (kt % NST) * C::STAGE_BYTES;
      const unsigned char* bs = as + C::A_BYTES;
      const int left = rows - kt * BK;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          u32x4 v = tr_frag(as, BM * 2, wm * C::WTM + i * 32, ks);
          if (left < BK) {  // tail stage: zero A entries of rows past the block
            const int k0 = ks * 16 + 8 * (lane >> 5);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t keep_lo = k0 + 2 * w < left ? 0x0000FFFFu : 0u;
              const uint32_t keep_hi = k0 + 2 * w + 1 < left ? 0xFFFF0000u : 0u;
              v[w] &= keep_lo | keep_hi;
            }
          }
          af[i] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j) bfr[j] = __builtin_bit_cast(bf16x8, tr_frag(bs, BN * 2, wn * C::WTN + j * 32, ks));
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) {
        wait_vmcnt_lds<0>();
        bare_barrier();
      }
    }
    (void)OPS;
    lds_barrier();  // every wave is done with the ring before the epilogue stages through it
    if (slot_base >= 0) {
      // A chunk of a split expert: fp32 partial straight from the accumulators. Lane l holds
      // row m0 + wm*WTM + 32i + l%32, columns n0 + wn*WTN + 32j + 8q + 4(l/32) + 0..3.
      const int64_t slot = slot_base + chunk;
      if (slot < g.slots) {
        float* dst = g.partial + slot * g.P * g.Q;
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          const int64_t row = m0 + wm * C::WTM + i * 32 + (lane & 31);
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t col = n0 + wn * C::WTN + j * 32 + 8 * q + 4 * (lane >> 5);
              if (row < g.P && col < g.Q) {
                const float4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                *reinterpret_cast<float4*>(dst + row * g.Q + col) = v;
              }
            }
        }
      }
    } else {
      TileCoord tc;
      tc.e = e;
      tc.mi = 0;
      tc.row0 = (int64_t)e * g.P + m0;
      tc.rows_valid = (int)(g.P - m0 < BM ? g.P - m0 : BM);
      tc.n0 = n0;
      epilogue<C>(acc, smem, ge, tc);
    }
  }
}

// Second Wgrad pass: each split expert's gradient is the sum of its chunk
// partials, taken in chunk order in fp32 and rounded once to bf16.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(WgradArgs g) {
  __shared__ WgradPlan pl;
  __shared__ int s_split[MOE_MAX_EXPERTS];
  __shared__ int s_nsplit;
  build_wgrad_plan<256>(g, pl);
  if (threadIdx.x == 0) {
    int n = 0;
    for (int e = 0; e < g.E; ++e)
      if (pl.slot_base[e] >= 0) s_split[n++] = e;
    s_nsplit = n;
  }
  __syncthreads();
  const int64_t groups = g.P * g.Q / 8;  // 8 consecutive elements per thread step (Q % 8 == 0)
  const int64_t total = (int64_t)s_nsplit * groups;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int se = (int)(i / groups);
    const int64_t el = (i - (int64_t)se * groups) * 8;
    const int e = s_split[se];
    const int base = pl.slot_base[e];
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < pl.chunks[e]; ++c) {
      if (base + c >= g.slots) break;
      const float* src = g.partial + (int64_t)(base + c) * g.P * g.Q + el;
      const float4 a = *reinterpret_cast<const float4*>(src);
      const float4 b = *reinterpret_cast<const float4*>(src + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *reinterpret_cast<u32x4*>(g.out + (int64_t)e * g.P * g.Q + el) = o;
  }
}

template <class C, typename Kern>
hipError_t launch_kernel(Kern kern, std::atomic<bool>* attr_done, const GemmArgs& g, hipStream_t stream) {
  const int dev = current_device();
  // Threads launching on one device may race to set the attribute the first time: setting it twice is harmless,
  // and the flag is atomic so that the race itself is well-defined.
  if (dev >= 0 && dev < 64 && !attr_done[dev].load(std::memory_order_acquire)) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                        C::LDS_BYTES);
    if (st != hipSuccess) return st;
    attr_done[dev].store(true, std::memory_order_release);
  }
  const int grid = device_cu_count(dev);  // one workgroup per CU: the LDS ring fills it
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, stream, g);
  return hipGetLastError();
}

// Tile configurations. Large expert blocks (mean rows per expert >= 384, and
// enough 256-row tiles to occupy the device) take 256 x 256 tiles on 8 waves
// (two per SIMD, so one wave's LDS and barrier waits overlap the other's MFMAs)
// with a 2-stage ring; smaller blocks take 128 x 256 tiles on 8 waves with a
// 3-stage ring, which wastes fewer rows on ragged tails. K not a multiple of 64 takes the same loop with its
// loads through buffer resources (the last stage's chunks past K staged as zeros; 40-43% faster than the
// register-staged loop at d = 2056, h = 776, bit-identical), unless an operand reaches 2 GiB; operands too large
// for that or for 32-bit load offsets take the register-staged loop.
// The gate/up tile puts its waves 4 x 2 (64 x 128 per wave: two gate and two up blocks each), 1-1.5% faster than
// 2 x 4 on the zipf64 and square workloads (bit-identical); the launch that also keeps U stays 2 x 4, where 4 x 2
// makes the compiler spill.
template <bool GATED, bool SAVE_U = false>
using BigTile = std::conditional_t<GATED && !SAVE_U, Tile<256, 256, 4, 2, 2, true>, Tile<256, 256, 2, 4, 2, GATED>>;
template <bool GATED>
using SmallTile = Tile<128, 256, 2, 4, 3, GATED>;
template <bool GATED>
using RegsTile = Tile<128, 256, 2, 2, 2, GATED>;

// The pipelined loop addresses its loads as 32-bit byte offsets from per-tile
// bases: A rows of one tile (or, gathered, the whole token matrix) and one
// expert's weights must each span less than 4 GiB.
inline bool offsets_fit_32(const GemmArgs& g) {
  constexpr int64_t kMax = 0xFFFFFFFFll;
  const int64_t a_span = g.a_rows != nullptr ? g.a_tokens * g.lda * 2 : (int64_t)256 * g.lda * 2;
  return a_span <= kMax && g.w_expert_stride * 2 <= kMax;
}

// The pipelined loop with a K remainder addresses its loads through buffer resources and marks the
// remainder's chunks with offset 2^31: A's span and one expert's weights must each stay below 2 GiB.
inline bool spans_below_2g(const GemmArgs& g) {
  constexpr int64_t kMax = 0x7FFFFFFFll;
  const int64_t a_span = g.a_rows != nullptr ? g.a_tokens * g.lda * 2 : (int64_t)256 * g.lda * 2;
  return a_span <= kMax && g.w_expert_stride * 2 <= kMax;
}

template <bool GATED, bool B_NMAJOR, bool SAVE_U, bool KTAIL>
hipError_t launch_pipe(const GemmArgs& g, hipStream_t stream);

template <bool GATED, bool B_NMAJOR, bool SAVE_U = false>
hipError_t launch_grouped(const GemmArgs& g, hipStream_t stream) {
  if (g.K % BK != 0 && spans_below_2g(g)) return launch_pipe<GATED, B_NMAJOR, SAVE_U, true>(g, stream);
  if (g.K % BK == 0 && offsets_fit_32(g)) return launch_pipe<GATED, B_NMAJOR, SAVE_U, false>(g, stream);
  static std::atomic<bool> done[64] = {};
  return launch_kernel<RegsTile<GATED>>(grouped_gemm_regs_kernel<RegsTile<GATED>, B_NMAJOR, SAVE_U>, done, g, stream);
}

template <bool GATED, bool B_NMAJOR, bool SAVE_U, bool KTAIL>
hipError_t launch_pipe(const GemmArgs& g, hipStream_t stream) {
  {
    // 256-row tiles need large expert blocks, and enough of them to occupy every CU: at most
    // cap_rows/256 + E row tiles exist whatever the offsets; when even that many cannot fill the
    // device, 128-row tiles (twice the tiles, a deeper ring) finish sooner. The host knows only
    // the mean rows per expert (cap_rows / E). From 384 on, 256-row tiles are faster. Below it an
    // expert's last tile decides: a 256-row tile costs about 1.6 of a 128-row one (its loads set
    // the stage time), so an expert of 129-256 rows is cheaper as one 256-row tile than as two
    // 128-row tiles, and one of 257-384 rows as three 128-row tiles than as two 256-row ones.
    // The down projection (N-contiguous weights) follows that count for a mean of 192-256 rows:
    // balanced 16-expert d = h = 4096 projections at 192 and 256 rows per expert 11-16% faster,
    // the same at 128 and 320, the Qwen3-shaped down projection 1-4% faster. The gate/up
    // projection keeps 128-row tiles below 384 (on the Qwen3-shaped workload 256-row tiles made
    // it 11% slower: an expert's tail then costs a whole 2048-deep tile).
    const int64_t tile_n = GATED ? BigTile<GATED>::OUTW : BigTile<GATED>::BN;
    const int64_t big_tiles = (g.cap_rows / BigTile<GATED>::BM + g.E) * ((g.N + tile_n - 1) / tile_n);
    const int64_t rows = g.cap_rows;
    const bool tall = rows >= (int64_t)384 * g.E ||
                      (!GATED && B_NMAJOR && rows >= (int64_t)192 * g.E && rows <= (int64_t)256 * g.E);
    if (tall && big_tiles >= device_cu_count(current_device())) {
      static std::atomic<bool> done[64] = {};
      using Big = BigTile<GATED, SAVE_U>;
      return launch_kernel<Big>(grouped_gemm_pipe_kernel<Big, B_NMAJOR, SAVE_U, KTAIL>, done, g, stream);
    }
    static std::atomic<bool> done[64] = {};
    return launch_kernel<SmallTile<GATED>>(grouped_gemm_pipe_kernel<SmallTile<GATED>, B_NMAJOR, SAVE_U, KTAIL>, done,
                                           g, stream);
  }
}

using WgradTile = Tile<256, 256, 2, 4, 2, false>;

}  // namespace

hipError_t launch_grouped_projection(const uint16_t* x, const int32_t* offsets, const uint16_t* w, bool w_out_in,
                                     int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* y,
                                     hipStream_t stream) {
  // Y_e = X_e W_e: A = x [cap, d_in] (K = d_in), N = d_out, out y [cap, d_out]
  if (!w_out_in) {
    // w [E, d_in, d_out]: K rows of N-contiguous columns (the down projection's layout)
    const GemmArgs g{x, d_in, nullptr, 1, 0, w, d_in * d_out, d_out, 0, d_out, d_in, offsets, E, cap_rows, y, d_out};
    return launch_grouped<false, true>(g, stream);
  }
  // w [E, d_out, d_in]: row n of the operand is W row n, K-contiguous (the gate/up layout, no activation)
  const GemmArgs g{x, d_in, nullptr, 1, 0, w, d_in * d_out, d_in, 0, d_out, d_in, offsets, E, cap_rows, y, d_out};
  return launch_grouped<false, false>(g, stream);
}

hipError_t launch_grouped_dgrad(const uint16_t* dy, const int32_t* offsets, const uint16_t* w, bool w_out_in,
                                int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dx,
                                hipStream_t stream) {
  // dX_e = dY_e W_e^T: A = dy [cap, d_out] (K = d_out), N = d_in, out dx [cap, d_in]
  if (!w_out_in) {
    // w [E, d_in, d_out]: row n of the operand is W_e row n, K-contiguous
    const GemmArgs g{dy, d_out, nullptr, 1, 0, w, d_in * d_out, d_out, 0, d_in, d_out, offsets, E, cap_rows, dx, d_in};
    return launch_grouped<false, false>(g, stream);
  }
  // w [E, d_out, d_in]: K rows of N-contiguous columns, as the down projection's weights
  const GemmArgs g{dy, d_out, nullptr, 1, 0, w, d_in * d_out, d_in, 0, d_in, d_out, offsets, E, cap_rows, dx, d_in};
  return launch_grouped<false, true>(g, stream);
}

int64_t wgrad_partial_slots(int64_t cap_rows) {
  // A split expert has more than kWgradChunk rows and at most rows / kWgradChunk + 1 < 2 rows / kWgradChunk
  // chunks, so all split experts together hold fewer than 2 * cap_rows / kWgradChunk chunks.
  return cap_rows > kWgradChunk ? (2 * cap_rows + kWgradChunk - 1) / kWgradChunk : 0;
}

hipError_t launch_grouped_wgrad(const uint16_t* x, const uint16_t* dy, const int32_t* offsets, bool w_out_in,
                                int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dw,
                                float* partial, hipStream_t stream) {
  // [E, d_in, d_out] = X^T dY per expert, or its transpose [E, d_out, d_in] = dY^T X
  const int64_t slots = wgrad_partial_slots(cap_rows);
  const WgradArgs g = !w_out_in ? WgradArgs{x, d_in, dy, d_out, d_in, d_out, offsets, E, cap_rows, dw, partial, slots}
                                : WgradArgs{dy, d_out, x, d_in, d_out, d_in, offsets, E, cap_rows, dw, partial, slots};
  static std::atomic<bool> done[64] = {};
  const int dev = current_device();
  if (dev >= 0 && dev < 64 && !done[dev]) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(grouped_wgrad_kernel<WgradTile>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, WgradTile::LDS_BYTES);
    if (st != hipSuccess) return st;
    done[dev] = true;
  }
  hipLaunchKernelGGL(grouped_wgrad_kernel<WgradTile>, dim3(device_cu_count(dev)), dim3(WgradTile::THREADS),
                     WgradTile::LDS_BYTES, stream, g);
  if (slots > 0) {
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(device_cu_count(dev) * 4), dim3(256), 0, stream, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_up_swiglu(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                 int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf,
                                 hipStream_t stream) {
  // A = x_perm [cap, d] (K = d); weights [E, 2h, d], gate rows n, up rows h + n; out h_buf [cap, h]
  const GemmArgs g{x_perm, d, nullptr, 1, 0, w_ug, 2 * h * d, d, h, h, d, offsets, E, cap_rows, h_buf, h};
  return launch_grouped<true, false>(g, stream);
}

hipError_t launch_gemm_up_swiglu_u(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                   int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf,
                                   uint16_t* u_buf, hipStream_t stream) {
  // as launch_gemm_up_swiglu, and the epilogue also stores U [cap, 2h]
  GemmArgs g{x_perm, d, nullptr, 1, 0, w_ug, 2 * h * d, d, h, h, d, offsets, E, cap_rows, h_buf, h};
  g.u_out = u_buf;
  return launch_grouped<true, false, true>(g, stream);
}

hipError_t launch_gemm_up_swiglu_gather(const uint16_t* x, const int32_t* perm, int64_t T, int32_t k,
                                        const int32_t* offsets, const uint16_t* w_ug, int64_t d, int64_t h, int32_t E,
                                        uint16_t* h_buf, hipStream_t stream) {
  // A rows are gathered: sorted row p reads x[perm[p] / k]
  const GemmArgs g{x, d, perm, k, T, w_ug, 2 * h * d, d, h, h, d, offsets, E, T * k, h_buf, h};
  return launch_grouped<true, false>(g, stream);
}

hipError_t launch_gemm_down(const uint16_t* h_buf, const int32_t* offsets, const uint16_t* w_down, int64_t cap_rows,
                            int64_t d, int64_t h, int32_t E, uint16_t* y_perm, hipStream_t stream) {
  // A = h_buf [cap, h] (K = h); weights [E, h, d] N-contiguous; out y_perm [cap, d]
  const GemmArgs g{h_buf, h, nullptr, 1, 0, w_down, h * d, d, 0, d, h, offsets, E, cap_rows, y_perm, d};
  return launch_grouped<false, true>(g, stream);
}

}  // namespace moe
