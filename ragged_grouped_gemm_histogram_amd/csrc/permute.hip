// Dispatch preparation on the device: histogram of kept expert ids, exclusive
// scan into int32 offsets, stable order + inverse map, and the permuted gather.
//
// OLMo report, Sec 9.2-9.3 / Fig 37: counts and cumulative offsets are produced
// and consumed on the GPU so the host never waits for them. halo notes: ids
// outside [0, E) are dropped before the sort, rows are sorted into contiguous
// per-expert blocks, and a sentinel-padded inverse map records where each slot
// went.
//
// Four launches (one workgroup for the first three when the dispatch is small, see
// permute_small_kernel; colscan and scatter in one launch when the table is at most
// 2^16 entries, see scan_scatter_kernel), none of which needs a count on the host:
//   1. hist     one block per chunk of 256 slots: LDS histogram -> table[e][chunk]
//   2. colscan  one block per expert: exclusive scan of that expert's row of
//               the table over chunks (in place) and its total -> counts[e]
//   3. scatter  one wave per chunk: offsets from counts (block 0 stores them),
//               then the chunk's slots in ascending order, each taking
//               offsets[e] + table[e][chunk] + (earlier slots of e in the chunk)
//   4. gather   x_perm[p] = x[perm[p] / k] for p < M, 16-byte vector copies
// Integer work only; the result is independent of scheduling (bit-exact).

#include <atomic>

#include "common.h"

// The per-chunk histogram table of moe_permute_noalloc, for callers that cannot allocate: a
// fixed array in the library's own device memory. Each GPU holds its own copy at its own
// address for as long as the process lives. In host code this name is only a stand-in for
// the symbol: the device address comes from hipGetSymbolAddress (see static_table below).
static __device__ __align__(256) int32_t scratch[moe::kStaticTableEntries];

namespace moe {
namespace {

constexpr int kHistThreads = kPermuteChunk;  // one slot per thread
constexpr int kScanThreads = 256;
constexpr int kGatherThreads = 256;

// chunk_major: table[c * E + e] (the two-launch path) instead of table[e * nchunks + c].
__global__ __launch_bounds__(kHistThreads) void hist_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                            int32_t* __restrict__ table, int64_t nchunks,
                                                            bool chunk_major) {
  __shared__ int h[MOE_MAX_EXPERTS];
  const int64_t c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kHistThreads) h[e] = 0;
  __syncthreads();
  const int64_t s = c * kPermuteChunk + threadIdx.x;
  if (s < S) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);  // LDS integer atomics: order-free
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kHistThreads)
    table[chunk_major ? c * E + e : (int64_t)e * nchunks + c] = h[e];
}

// Exclusive scan of one expert's per-chunk counts, in place; total -> counts[e].
__global__ __launch_bounds__(kScanThreads) void colscan_kernel(int32_t* __restrict__ table, int64_t nchunks,
                                                               int32_t* __restrict__ counts) {
  __shared__ int part[kScanThreads];
  const int e = blockIdx.x;
  int32_t* row = table + (int64_t)e * nchunks;
  constexpr int kItems = 4;
  int carry = 0;
  for (int64_t base = 0; base < nchunks; base += (int64_t)kScanThreads * kItems) {
    int v[kItems];
    int local = 0;
    const int64_t i0 = base + (int64_t)threadIdx.x * kItems;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      v[i] = (i0 + i < nchunks) ? row[i0 + i] : 0;
      local += v[i];
    }
    part[threadIdx.x] = local;
    __syncthreads();
    // Hillis-Steele inclusive scan of the per-thread sums.
    for (int off = 1; off < kScanThreads; off <<= 1) {
      const int add = (threadIdx.x >= off) ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    int run = carry + part[threadIdx.x] - local;  // exclusive prefix of this thread's first item
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      if (i0 + i < nchunks) row[i0 + i] = run;
      run += v[i];
    }
    const int tile_total = part[kScanThreads - 1];
    __syncthreads();
    carry += tile_total;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// One wave per chunk. Within each step of 64 slots, lanes holding the same
// expert id find each other with one ballot per id bit; the lowest such lane
// reserves a run of rows from the expert's LDS cursor, and every lane takes
// cursor + (number of lower lanes with its id). Slots therefore land in
// ascending slot order inside each expert block.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int id_bits,
                                                     const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ table, int64_t nchunks,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
  __shared__ int off_s[MOE_MAX_EXPERTS + 1];
  __shared__ int cursor[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x;
  const int64_t c = blockIdx.x;

  // offsets = exclusive scan of counts: each lane sums a run of 16 experts,
  // then a wave-wide inclusive scan of the run sums.
  constexpr int kPer = (MOE_MAX_EXPERTS + 63) / 64;
  int run[kPer];
  int local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane * kPer + i;
    run[i] = (e < E) ? counts[e] : 0;
    local += run[i];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(incl, off, 64);
    if (lane >= off) incl += up;
  }
  int acc = incl - local;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane * kPer + i;
    if (e < E) off_s[e] = acc;
    acc += run[i];
  }
  if (lane == 63) off_s[E] = incl;
  __syncthreads();
  if (c == 0) {
    for (int e = lane; e <= E; e += 64) offsets[e] = off_s[e];
  }
  if (c >= nchunks) return;

  for (int e = lane; e < E; e += 64) cursor[e] = off_s[e] + table[(int64_t)e * nchunks + c];
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int step = 0; step < kPermuteChunk / 64; ++step) {
    const int64_t s = c * kPermuteChunk + step * 64 + lane;
    const int e = (s < S) ? ids[s] : -1;
    const bool keep = (s < S) && ((unsigned)e < (unsigned)E);
    uint64_t same = __ballot(keep);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lt_mask);
    const int leader = keep ? (__ffsll((long long)same) - 1) : lane;
    int base = 0;
    if (keep && lane == leader) {
      base = cursor[e];
      cursor[e] = base + __popcll(same);
    }
    base = __shfl(base, leader, 64);
    if (s < S) {
      if (keep) {
        const int pos = base + rank;  // < offsets[e+1] <= S when ids are unchanged since the histogram
        if ((int64_t)pos < S) perm[pos] = (int32_t)s;
        inv[s] = pos;
      } else {
        inv[s] = -1;
      }
    }
    __syncthreads();  // the cursor updates of this step are visible to the next
  }
}

// The column scan and the scatter in one launch, for chunk-major tables of at most kFusedTable
// entries whose expert count is a power of two from 4 to 1024 (so E divides the 1024 entries a
// block reads per step, and every thread keeps the same four experts): block c (one chunk) reads
// the whole table in 16-byte loads (at most 256 KB, from L2), eight in flight per thread, and
// sums for every expert its entries before chunk c and its total; the totals become offsets and
// the block walks its chunk as scatter_kernel does. This costs less than a launch boundary and a
// second pass over the table. Block 0 also stores counts and offsets. Same order, same results
// as the three-launch path.
constexpr int kFusedThreads = 256;
constexpr int64_t kFusedTable = int64_t(1) << 16;

__global__ __launch_bounds__(kFusedThreads) void scan_scatter_kernel(const int32_t* __restrict__ ids, int64_t S,
                                                                     int E, int id_bits,
                                                                     const int32_t* __restrict__ table,
                                                                     int64_t nchunks, int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ perm,
                                                                     int32_t* __restrict__ inv) {
  __shared__ int off_s[MOE_MAX_EXPERTS + 1];
  __shared__ int cursor[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x;
  constexpr int kSteps = kPermuteChunk / 64;
  // this chunk's ids, loaded before the table so that both are in flight together
  int id_reg[kSteps];
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int64_t s = c * kPermuteChunk + step * 64 + lane;
    id_reg[step] = (wave == 0 && s < S) ? ids[s] : -1;
  }
  for (int e = tid; e < E; e += kFusedThreads) {
    off_s[e] = 0;
    cursor[e] = 0;
  }
  __syncthreads();
  // Thread tid reads 16-byte groups tid, tid + 256, ...: entries 4 tid + 1024 i, always experts
  // e0..e0+3 with e0 = 4 tid mod E, of chunk rows (4 tid + 1024 i) / E.
  const int4* t4 = reinterpret_cast<const int4*>(table);
  const int64_t n4 = nchunks * E / 4;
  const int e0 = (4 * tid) % E;
  int before[4] = {0, 0, 0, 0}, total[4] = {0, 0, 0, 0};
  constexpr int kBatch = 8;
  for (int64_t f0 = tid; f0 < n4; f0 += (int64_t)kFusedThreads * kBatch) {
    int4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t f = f0 + (int64_t)kFusedThreads * u;
      v[u] = f < n4 ? t4[f] : int4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t f = f0 + (int64_t)kFusedThreads * u;
      const bool early = (4 * f) / E < c;  // entries of a chunk before this one
      total[0] += v[u].x; total[1] += v[u].y; total[2] += v[u].z; total[3] += v[u].w;
      if (early) {
        before[0] += v[u].x; before[1] += v[u].y; before[2] += v[u].z; before[3] += v[u].w;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // LDS integer atomics: order-free
    if (total[q] != 0) atomicAdd(&off_s[e0 + q], total[q]);
    if (before[q] != 0) atomicAdd(&cursor[e0 + q], before[q]);
  }
  __syncthreads();
  if (wave == 0) {
    // offsets = exclusive scan of the totals: each lane sums a run of 16 experts, then a wave-wide scan
    constexpr int kPer = (MOE_MAX_EXPERTS + 63) / 64;
    int run[kPer];
    int local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane * kPer + i;
      run[i] = (e < E) ? off_s[e] : 0;
      local += run[i];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    int acc = incl - local;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane * kPer + i;
      if (e < E) {
        if (c == 0) counts[e] = run[i];
        off_s[e] = acc;
      }
      acc += run[i];
    }
    if (lane == 63) off_s[E] = incl;
  }
  __syncthreads();
  if (c == 0) {
    for (int e = tid; e <= E; e += kFusedThreads) offsets[e] = off_s[e];
  }
  for (int e = tid; e < E; e += kFusedThreads) cursor[e] += off_s[e];
  __syncthreads();
  if (wave != 0) return;  // one wave walks the chunk (no barrier below this point)
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int64_t s = c * kPermuteChunk + step * 64 + lane;
    const int e = id_reg[step];
    const bool keep = (s < S) && ((unsigned)e < (unsigned)E);
    uint64_t same = __ballot(keep);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lt_mask);
    const int leader = keep ? (__ffsll((long long)same) - 1) : lane;
    int base = 0;
    if (keep && lane == leader) {
      base = cursor[e];
      cursor[e] = base + __popcll(same);
    }
    base = __shfl(base, leader, 64);
    if (s < S) {
      if (keep) {
        const int pos = base + rank;  // < offsets[e+1] <= S when ids are unchanged since the histogram
        if ((int64_t)pos < S) perm[pos] = (int32_t)s;
        inv[s] = pos;
      } else {
        inv[s] = -1;
      }
    }
    // this step's cursor updates land before the next step's leaders read them (one wave: an LDS wait
    // and a compiler fence take the place of the workgroup barrier)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
    __builtin_amdgcn_wave_barrier();
  }
}

// Small dispatches (at most kSmallChunks chunks and kSmallTable table entries): the
// three steps above in one workgroup of 16 waves, the per-chunk table in LDS and
// workgroup barriers in place of kernel boundaries (for a few thousand slots each
// launch costs more than its work). Same table, same order, same results.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallChunks = 64;
constexpr int kSmallTable = 8192;  // E * nchunks entries, 32 KB of LDS

__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(const int32_t* __restrict__ ids, int64_t S,
                                                                      int E, int id_bits, int nchunks,
                                                                      int32_t* __restrict__ counts,
                                                                      int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ perm,
                                                                      int32_t* __restrict__ inv) {
  __shared__ int table[kSmallTable];  // [e][chunk]: counts, then starting positions
  __shared__ int off_s[MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int entries = E * nchunks;
  for (int i = tid; i < entries; i += kSmallThreads) table[i] = 0;
  __syncthreads();
  // 1. histogram per chunk (LDS integer atomics: order-free)
  for (int64_t s = tid; s < S; s += kSmallThreads) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&table[e * nchunks + (int)(s / kPermuteChunk)], 1);
  }
  __syncthreads();
  // 2. per expert: exclusive scan over chunks, total -> counts
  for (int e = tid; e < E; e += kSmallThreads) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = table[e * nchunks + c];
      table[e * nchunks + c] = run;
      run += v;
    }
    counts[e] = run;
    off_s[e] = run;  // the scan below turns the totals into offsets
  }
  __syncthreads();
  // offsets = exclusive scan of the totals, by the first wave (a run of 16 experts per lane)
  if (wave == 0) {
    constexpr int kPer = (MOE_MAX_EXPERTS + 63) / 64;
    int run[kPer];
    int local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane * kPer + i;
      run[i] = (e < E) ? off_s[e] : 0;
      local += run[i];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int up = __shfl_up(incl, off, 64);
      if (lane >= off) incl += up;
    }
    int acc = incl - local;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane * kPer + i;
      if (e < E) off_s[e] = acc;
      acc += run[i];
    }
    if (lane == 63) off_s[E] = incl;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kSmallThreads) offsets[e] = off_s[e];
  // 3. starting position of every (expert, chunk) run
  for (int i = tid; i < entries; i += kSmallThreads) table[i] += off_s[i / nchunks];
  __syncthreads();
  // 4. wave w walks chunks w, w + 16, ... in steps of 64 slots, as scatter_kernel does; the
  // loop bounds are the same for every wave so every wave meets every barrier.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < nchunks; c0 += kSmallWaves) {
    const int c = c0 + wave;
    for (int step = 0; step < kPermuteChunk / 64; ++step) {
      const int64_t s = (int64_t)c * kPermuteChunk + step * 64 + lane;
      const bool in = c < nchunks && s < S;
      const int e = in ? ids[s] : -1;
      const bool keep = in && ((unsigned)e < (unsigned)E);
      uint64_t same = __ballot(keep);
      for (int b = 0; b < id_bits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
      }
      const int rank = __popcll(same & lt_mask);
      const int leader = keep ? (__ffsll((long long)same) - 1) : lane;
      int base = 0;
      if (keep && lane == leader) {
        base = table[e * nchunks + c];
        table[e * nchunks + c] = base + __popcll(same);
      }
      base = __shfl(base, leader, 64);
      if (in) {
        if (keep) {
          const int pos = base + rank;
          if ((int64_t)pos < S) perm[pos] = (int32_t)s;
          inv[s] = pos;
        } else {
          inv[s] = -1;
        }
      }
      __syncthreads();  // this step's cursor updates are visible to the next
    }
  }
}

// x_perm[p] = x[perm[p] / k] for p < M = offsets[E]; 16-byte chunks.
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(const uint16_t* __restrict__ x,
                                                                const int32_t* __restrict__ perm,
                                                                const int32_t* __restrict__ offsets, int E,
                                                                int64_t S, int k, int64_t d,
                                                                uint16_t* __restrict__ x_perm) {
  int64_t M = offsets[E];
  M = M < 0 ? 0 : (M > S ? S : M);
  const int64_t cpr = d / 8;  // 16-byte chunks per row
  int rows_per_iter, r_local, ch0;
  if (cpr <= kGatherThreads) {
    rows_per_iter = kGatherThreads / (int)cpr;
    r_local = threadIdx.x / (int)cpr;
    ch0 = threadIdx.x - r_local * (int)cpr;
    if (r_local >= rows_per_iter) return;
  } else {
    rows_per_iter = 1;
    r_local = 0;
    ch0 = threadIdx.x;
  }
  const int ch_step = (cpr <= kGatherThreads) ? (int)cpr : kGatherThreads;
  for (int64_t row = (int64_t)blockIdx.x * rows_per_iter + r_local; row < M;
       row += (int64_t)gridDim.x * rows_per_iter) {
    int64_t slot = perm[row];
    slot = slot < 0 ? 0 : (slot >= S ? S - 1 : slot);
    const int64_t t = slot / k;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + t * d);
    u32x4* dst = reinterpret_cast<u32x4*>(x_perm + row * d);
    for (int64_t ch = ch0; ch < cpr; ch += ch_step) dst[ch] = __builtin_nontemporal_load(src + ch);
  }
}

int bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_table_addr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

hipError_t static_table(int dev, int32_t** table) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* p = g_table_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // First call on this device (the caller made it current): resolve the array's address on
    // it once. Two threads may both resolve it; they store the same value.
    void* addr = nullptr;
    const hipError_t st = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (st != hipSuccess) return st;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<int32_t*>(addr);
    g_table_addr[dev].store(p, std::memory_order_release);
  }
  *table = p;
  return hipSuccess;
}

hipError_t launch_permute(const uint16_t* x, const int32_t* ids, int64_t T, int32_t k, int64_t d, int32_t E,
                          uint16_t* x_perm, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                          int32_t* table, hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t nchunks = permute_chunks(S);
  if (nchunks <= kSmallChunks && (int64_t)E * nchunks <= kSmallTable) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), 0, stream, ids, S, E, bits_for(E),
                       (int)nchunks, counts, offsets, perm, inv);
  } else if ((int64_t)E * nchunks <= kFusedTable && E >= 4 && (E & (E - 1)) == 0 &&
             (reinterpret_cast<uintptr_t>(table) & 15) == 0) {
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nchunks), dim3(kHistThreads), 0, stream, ids, S, E, table,
                       nchunks, true);
    hipLaunchKernelGGL(scan_scatter_kernel, dim3((unsigned)nchunks), dim3(kFusedThreads), 0, stream, ids, S, E,
                       bits_for(E), table, nchunks, counts, offsets, perm, inv);
  } else {
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nchunks), dim3(kHistThreads), 0, stream, ids, S, E, table,
                       nchunks, false);
    hipLaunchKernelGGL(colscan_kernel, dim3(E), dim3(kScanThreads), 0, stream, table, nchunks, counts);
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nchunks), dim3(64), 0, stream, ids, S, E, bits_for(E), counts,
                       table, nchunks, offsets, perm, inv);
  }
  if (S > 0 && x_perm != nullptr) {  // no x_perm: the caller gathers inside the GEMM
    const int dev = current_device();
    const int64_t cpr = d / 8;
    const int64_t rpi = cpr <= kGatherThreads ? kGatherThreads / cpr : 1;
    int64_t blocks = (S + rpi - 1) / rpi;
    const int64_t cap = (int64_t)device_cu_count(dev) * 8;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(kGatherThreads), 0, stream, x, perm, offsets, E, S,
                       k, d, x_perm);
  }
  return hipGetLastError();
}

}  // namespace moe
