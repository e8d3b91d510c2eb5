// Shared device helpers and host-side launch declarations for the MoE expert step.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe_grouped.h"

namespace moe {

// ---------------------------------------------------------------- device side

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bit pattern, round to nearest even (the compiler lowers the
// __bf16 conversion to the gfx950 hardware convert, which rounds to nearest even).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// Two fp32 values to a pair of bf16 (lo in the low half), round to nearest even: one packed
// convert (v_cvt_pk_bf16_f32) instead of two single converts, a shift and an or.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ------------------------------------------------------------------ host side

// Number of compute units of a device (cached per device).
int device_cu_count(int dev);

inline int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return dev;
}

// Permute: chunking of the dispatch slots for the per-chunk histogram table.
constexpr int kPermuteChunk = 256;  // slots per chunk (one wave walks it in 4 steps of 64)
inline int64_t permute_chunks(int64_t S) { return (S + kPermuteChunk - 1) / kPermuteChunk; }

hipError_t launch_permute(const uint16_t* x, const int32_t* ids, int64_t T, int32_t k, int64_t d, int32_t E,
                          uint16_t* x_perm, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                          int32_t* table, hipStream_t stream);

// Entries of the fixed per-device table behind moe_permute_noalloc (E * permute_chunks(T*k) int32
// at most; 4 MiB per device), and its device address on device `dev`, which must be current.
constexpr int64_t kStaticTableEntries = MOE_PERMUTE_NOALLOC_TABLE_ENTRIES;
hipError_t static_table(int dev, int32_t** table);

hipError_t launch_gemm_up_swiglu(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                 int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf,
                                 hipStream_t stream);

hipError_t launch_gemm_up_swiglu_u(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                   int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf,
                                   uint16_t* u_buf, hipStream_t stream);

hipError_t launch_gemm_up_swiglu_gather(const uint16_t* x, const int32_t* perm, int64_t T, int32_t k,
                                        const int32_t* offsets, const uint16_t* w_ug, int64_t d, int64_t h, int32_t E,
                                        uint16_t* h_buf, hipStream_t stream);

hipError_t launch_grouped_projection(const uint16_t* x, const int32_t* offsets, const uint16_t* w, bool w_out_in,
                                     int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* y,
                                     hipStream_t stream);
hipError_t launch_swiglu_backward(const uint16_t* dh, const uint16_t* u, const int32_t* offsets, int32_t E,
                                  int64_t cap_rows, int64_t h, uint16_t* du, hipStream_t stream);
hipError_t launch_grouped_dgrad(const uint16_t* dy, const int32_t* offsets, const uint16_t* w, bool w_out_in,
                                int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dx,
                                hipStream_t stream);
// Wgrad splits experts with more than kWgradChunk rows; their fp32 partials need
// wgrad_partial_slots(cap_rows) slots of d_in * d_out floats.
constexpr int kWgradChunk = 4096;
int64_t wgrad_partial_slots(int64_t cap_rows);
hipError_t launch_grouped_wgrad(const uint16_t* x, const uint16_t* dy, const int32_t* offsets, bool w_out_in,
                                int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dw,
                                float* partial, hipStream_t stream);
hipError_t launch_gemm_down(const uint16_t* h_buf, const int32_t* offsets, const uint16_t* w_down,
                            int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* y_perm,
                            hipStream_t stream);

hipError_t launch_unpermute_backward(const uint16_t* dy, const uint16_t* y_perm, const int32_t* inv, const float* w,
                                     int64_t T, int32_t k, int64_t d, uint16_t* dy_perm, float* dw,
                                     hipStream_t stream);
hipError_t launch_unpermute(const uint16_t* y_perm, const int32_t* inv, const float* w, int64_t T, int32_t k,
                            int64_t d, uint16_t* y, hipStream_t stream);

}  // namespace moe
