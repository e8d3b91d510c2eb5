// Atomic-free scatter-back (halo notes, permute/unpermute paragraph): the
// inverse map lists, for every token, the sorted rows that hold its expert
// outputs, so the combine is a gather plus a reduction and no two threads ever
// write the same element. Each thread owns 8 consecutive columns of one token
// and accumulates sum_j w[t,j] * y_perm[inv[t,j]] in fp32 registers, j
// ascending, skipping slots whose inverse-map entry is outside [0, T*k); the
// k gathered rows are never materialised.

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void unpermute_kernel(const uint16_t* __restrict__ y_perm,
                                                             const int32_t* __restrict__ inv,
                                                             const float* __restrict__ w, int64_t T, int k,
                                                             int64_t d, uint16_t* __restrict__ y) {
  const int64_t S = T * k;
  const int64_t cpr = d / 8;
  int rows_per_iter, r_local, ch0;
  if (cpr <= kThreads) {
    rows_per_iter = kThreads / (int)cpr;
    r_local = threadIdx.x / (int)cpr;
    ch0 = threadIdx.x - r_local * (int)cpr;
    if (r_local >= rows_per_iter) return;
  } else {
    rows_per_iter = 1;
    r_local = 0;
    ch0 = threadIdx.x;
  }
  const int ch_step = (cpr <= kThreads) ? (int)cpr : kThreads;
  for (int64_t t = (int64_t)blockIdx.x * rows_per_iter + r_local; t < T; t += (int64_t)gridDim.x * rows_per_iter) {
    for (int64_t ch = ch0; ch < cpr; ch += ch_step) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const int64_t p = inv[t * k + j];
        if (p < 0 || p >= S) continue;
        const float wt = w[t * k + j];
        const u32x4 v = *reinterpret_cast<const u32x4*>(y_perm + p * d + ch * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(wt, bf16_bits_to_f32(v[q] & 0xFFFFu), acc[2 * q]);
          acc[2 * q + 1] = fmaf(wt, bf16_bits_to_f32(v[q] >> 16), acc[2 * q + 1]);
        }
      }
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      *reinterpret_cast<u32x4*>(y + t * d + ch * 8) = o;
    }
  }
}

}  // namespace

hipError_t launch_unpermute(const uint16_t* y_perm, const int32_t* inv, const float* w, int64_t T, int32_t k,
                            int64_t d, uint16_t* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int dev = current_device();
  const int64_t cpr = d / 8;
  const int64_t rpi = cpr <= kThreads ? kThreads / cpr : 1;
  int64_t blocks = (T + rpi - 1) / rpi;
  const int64_t cap = (int64_t)device_cu_count(dev) * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, y_perm, inv, w, T, k, d, y);
  return hipGetLastError();
}

}  // namespace moe
