// Atomic-free scatter-back (halo notes, permute/unpermute paragraph): the
// inverse map lists, for every token, the sorted rows that hold its expert
// outputs, so the combine is a gather plus a reduction and no two threads ever
// write the same element. Each thread owns 8 consecutive columns of one token
// and accumulates sum_j w[t,j] * y_perm[inv[t,j]] in fp32 registers, j
// ascending, skipping slots whose inverse-map entry is outside [0, T*k); the
// k gathered rows are never materialised. With no weights (a null pointer)
// the same kernel is the backward of the forward's row gather: a token's
// gradient is the plain sum of its kept slots' rows.

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSlots = 8;  // row loads in flight per thread

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
      // slots in groups of kSlots: all of a group's row loads are issued before any is used
      for (int j0 = 0; j0 < k; j0 += kSlots) {
        u32x4 v[kSlots];
        float wt[kSlots];
#pragma unroll
        for (int jj = 0; jj < kSlots; ++jj) {
          const int j = j0 + jj;
          const int64_t p = j < k ? (int64_t)inv[t * k + j] : -1;
          const bool keep = p >= 0 && p < S;
          wt[jj] = keep ? (w != nullptr ? w[t * k + j] : 1.0f) : 0.0f;
          v[jj] = keep ? *reinterpret_cast<const u32x4*>(y_perm + p * d + ch * 8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int jj = 0; jj < kSlots; ++jj) {
          if (j0 + jj >= k) break;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = fmaf(wt[jj], bf16_bits_to_f32(v[jj][q] & 0xFFFFu), acc[2 * q]);
            acc[2 * q + 1] = fmaf(wt[jj], bf16_bits_to_f32(v[jj][q] >> 16), acc[2 * q + 1]);
          }
        }
      }
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      *reinterpret_cast<u32x4*>(y + t * d + ch * 8) = o;
    }
  }
}

// Backward of the weighted scatter-back, one wave per token: for every kept
// slot j, dy_perm[inv[t,j]] = bf16(w[t,j] * dy[t]) (each sorted row has one
// owner slot, so rows are written once and without atomics) and the routing
// weight gradient dw[t,j] = sum_c dy[t,c] * y_perm[inv[t,j],c], an fp32 dot
// product reduced across the wave; dropped slots get dw = 0.
__global__ __launch_bounds__(kThreads) void unpermute_backward_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ y_perm, const int32_t* __restrict__ inv,
    const float* __restrict__ w, int64_t T, int k, int64_t d, uint16_t* __restrict__ dy_perm, float* __restrict__ dw) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int64_t S = T * k;
  const int64_t cpr = d / 8;
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < T; t += nwaves) {
    for (int j = 0; j < k; ++j) {
      const int64_t p = inv[t * k + j];
      if (p < 0 || p >= S) {
        if (lane == 0) dw[t * k + j] = 0.f;
        continue;
      }
      const float wt = w[t * k + j];
      float dot = 0.f;
      for (int64_t ch = lane; ch < cpr; ch += 64) {
        const u32x4 g = *reinterpret_cast<const u32x4*>(dy + t * d + ch * 8);
        const u32x4 v = *reinterpret_cast<const u32x4*>(y_perm + p * d + ch * 8);
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g0 = bf16_bits_to_f32(g[q] & 0xFFFFu), g1 = bf16_bits_to_f32(g[q] >> 16);
          dot = fmaf(g0, bf16_bits_to_f32(v[q] & 0xFFFFu), dot);
          dot = fmaf(g1, bf16_bits_to_f32(v[q] >> 16), dot);
          o[q] = pack_bf16x2(wt * g0, wt * g1);
        }
        *reinterpret_cast<u32x4*>(dy_perm + p * d + ch * 8) = o;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
      if (lane == 0) dw[t * k + j] = dot;
    }
  }
}

// SwiGLU backward over the sorted rows [0, M), M = offsets[E] clamped to the
// capacity: with [g | up] = U and s = sigmoid(g) (hardware exponential and
// reciprocal, fp32), dG = dH * up * s * (1 + g * (1 - s)) and dUp = dH * g * s,
// each rounded to bf16. Each thread takes 8 consecutive columns of one row.
__global__ __launch_bounds__(kThreads) void swiglu_backward_kernel(const uint16_t* __restrict__ dh,
                                                                   const uint16_t* __restrict__ u,
                                                                   const int32_t* __restrict__ offsets, int E,
                                                                   int64_t cap_rows, int64_t h,
                                                                   uint16_t* __restrict__ du) {
  int64_t M = offsets[E];
  M = M < 0 ? 0 : (M > cap_rows ? cap_rows : M);
  const int64_t cpr = h / 8;
  const int64_t total = M * cpr;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / cpr, c = (i - r * cpr) * 8;
    const u32x4 gd = *reinterpret_cast<const u32x4*>(dh + r * h + c);
    const u32x4 gv = *reinterpret_cast<const u32x4*>(u + r * 2 * h + c);
    const u32x4 uv = *reinterpret_cast<const u32x4*>(u + r * 2 * h + h + c);
    u32x4 og, ou;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float dg[2], dup[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int sh = 16 * s2;
        const float d = bf16_bits_to_f32((gd[q] >> sh) & 0xFFFFu);
        const float g = bf16_bits_to_f32((gv[q] >> sh) & 0xFFFFu);
        const float up = bf16_bits_to_f32((uv[q] >> sh) & 0xFFFFu);
        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
        dg[s2] = d * up * sg * (1.0f + g * (1.0f - sg));
        dup[s2] = d * g * sg;
      }
      og[q] = pack_bf16x2(dg[0], dg[1]);
      ou[q] = pack_bf16x2(dup[0], dup[1]);
    }
    *reinterpret_cast<u32x4*>(du + r * 2 * h + c) = og;
    *reinterpret_cast<u32x4*>(du + r * 2 * h + h + c) = ou;
  }
}

}  // namespace

hipError_t launch_swiglu_backward(const uint16_t* dh, const uint16_t* u, const int32_t* offsets, int32_t E,
                                  int64_t cap_rows, int64_t h, uint16_t* du, hipStream_t stream) {
  if (cap_rows == 0) return hipSuccess;
  const int dev = current_device();
  int64_t blocks = (cap_rows * (h / 8) + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count(dev) * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(swiglu_backward_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, dh, u, offsets, E,
                     cap_rows, h, du);
  return hipGetLastError();
}

hipError_t launch_unpermute_backward(const uint16_t* dy, const uint16_t* y_perm, const int32_t* inv, const float* w,
                                     int64_t T, int32_t k, int64_t d, uint16_t* dy_perm, float* dw,
                                     hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int dev = current_device();
  constexpr int kWaves = kThreads / 64;
  int64_t blocks = (T + kWaves - 1) / kWaves;
  const int64_t cap = (int64_t)device_cu_count(dev) * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(unpermute_backward_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, dy, y_perm, inv, w,
                     T, k, d, dy_perm, dw);
  return hipGetLastError();
}

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
