// C ABI of the MoE expert step: host-side validation, device check and launches.
// Nothing here allocates, synchronises or reads device data.

#include <atomic>
#include <cstring>

#include "common.h"

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
std::atomic<int> g_cus[kMaxDevices];

constexpr int64_t kMaxSlots = (int64_t(1) << 31) - 1;  // int32 row indices and offsets

bool load_props(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  if (g_arch[dev].load(std::memory_order_acquire) != 0) return true;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
  g_arch[dev].store(std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1, std::memory_order_release);
  return true;
}

moe_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !load_props(dev)) return MOE_ERR_UNSUPPORTED_DEVICE;
  return g_arch[dev].load(std::memory_order_acquire) == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

inline bool missing(const void* p, int64_t elems) { return elems > 0 && p == nullptr; }
inline bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }
inline bool bad_width(int64_t w) { return w < 8 || (w % 8) != 0 || w > (int64_t(1) << 24); }

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// The GEMM epilogues store a tile of up to 256 output rows through one buffer resource with 32-bit
// byte offsets (and an offset of 2^31 for columns past the end). The widest output row is U's 2h
// columns, so 256 * 2 * 2^20 * 2 bytes = 2^30 keeps every offset of a tile below 2^31.
constexpr int64_t kMaxGemmWidth = int64_t(1) << 20;

moe_status check_gemm_shape(int64_t cap_rows, int64_t d, int64_t h, int32_t E) {
  if (cap_rows < 0 || cap_rows > kMaxSlots || bad_width(d) || bad_width(h) || E < 1 || E > MOE_MAX_EXPERTS)
    return MOE_ERR_BAD_SHAPE;
  if (d > kMaxGemmWidth || h > kMaxGemmWidth) return MOE_ERR_BAD_SHAPE;
  return MOE_OK;
}

}  // namespace

int device_cu_count(int dev) {
  if (!load_props(dev)) return 256;
  const int n = g_cus[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS || T > kMaxSlots / k) return 0;
  return (size_t)permute_chunks(T * k) * (size_t)E * sizeof(int32_t);
}

moe_status moe_permute(const uint16_t* x, const int32_t* expert_ids, int64_t T, int32_t k, int64_t d, int32_t E,
                       uint16_t* x_perm, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_map,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS || bad_width(d) || T > kMaxSlots / k) return MOE_ERR_BAD_SHAPE;
  const int64_t S = T * k;
  const size_t need = moe_permute_workspace_bytes(T, k, E);
  // x_perm == NULL asks for no row gather (a later *_gather GEMM reads x through perm); x is then unused.
  if ((x_perm != nullptr && missing(x, T * d)) || missing(expert_ids, S) || missing(counts, E) ||
      missing(offsets, E + 1) || missing(perm, S) || missing(inv_map, S) || missing(workspace, (int64_t)need))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(x, 16) || misaligned(x_perm, 16) || misaligned(expert_ids, 4) || misaligned(counts, 4) ||
      misaligned(offsets, 4) || misaligned(perm, 4) || misaligned(inv_map, 4) || misaligned(workspace, 4))
    return MOE_ERR_MISALIGNED;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  const moe_status dev = check_device();
  if (dev != MOE_OK) return dev;
  (void)hipGetLastError();
  return launched(launch_permute(x, expert_ids, T, k, d, E, x_perm, counts, offsets, perm, inv_map,
                                 static_cast<int32_t*>(workspace), stream));
}

moe_status moe_permute_noalloc(const uint16_t* x, const int32_t* expert_ids, int64_t T, int32_t k, int64_t d,
                               int32_t E, uint16_t* x_perm, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv_map, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS || bad_width(d) || T > kMaxSlots / k) return MOE_ERR_BAD_SHAPE;
  const int64_t S = T * k;
  if ((int64_t)E * permute_chunks(S) > kStaticTableEntries) return MOE_ERR_TOO_LARGE;
  if ((x_perm != nullptr && missing(x, T * d)) || missing(expert_ids, S) || missing(counts, E) ||
      missing(offsets, E + 1) || missing(perm, S) || missing(inv_map, S))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(x, 16) || misaligned(x_perm, 16) || misaligned(expert_ids, 4) || misaligned(counts, 4) ||
      misaligned(offsets, 4) || misaligned(perm, 4) || misaligned(inv_map, 4))
    return MOE_ERR_MISALIGNED;
  const moe_status st = check_device();
  if (st != MOE_OK) return st;
  int dev = -1;
  int32_t* table = nullptr;
  if (hipGetDevice(&dev) != hipSuccess || static_table(dev, &table) != hipSuccess) return MOE_ERR_LAUNCH;
  (void)hipGetLastError();
  // Every table entry a call reads was written earlier in the same call (the histogram launch writes
  // all E x chunks entries before the scan and the scatter read them), so nothing needs clearing.
  return launched(launch_permute(x, expert_ids, T, k, d, E, x_perm, counts, offsets, perm, inv_map, table, stream));
}

moe_status moe_gemm_up_swiglu(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug, int64_t cap_rows,
                              int64_t d, int64_t h, int32_t E, uint16_t* h_buf, hipStream_t stream) {
  moe_status st = check_gemm_shape(cap_rows, d, h, E);
  if (st != MOE_OK) return st;
  if (missing(x_perm, cap_rows * d) || missing(offsets, E + 1) || missing(w_ug, (int64_t)E * 2 * h * d) ||
      missing(h_buf, cap_rows * h))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(x_perm, 16) || misaligned(w_ug, 16) || misaligned(h_buf, 16) || misaligned(offsets, 4))
    return MOE_ERR_MISALIGNED;
  if ((st = check_device()) != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_gemm_up_swiglu(x_perm, offsets, w_ug, cap_rows, d, h, E, h_buf, stream));
}

moe_status moe_gemm_up_swiglu_u(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf, uint16_t* u_buf,
                                hipStream_t stream) {
  moe_status st = check_gemm_shape(cap_rows, d, h, E);
  if (st != MOE_OK) return st;
  if (missing(x_perm, cap_rows * d) || missing(offsets, E + 1) || missing(w_ug, (int64_t)E * 2 * h * d) ||
      missing(h_buf, cap_rows * h) || missing(u_buf, cap_rows * 2 * h))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(x_perm, 16) || misaligned(w_ug, 16) || misaligned(h_buf, 16) || misaligned(u_buf, 16) ||
      misaligned(offsets, 4))
    return MOE_ERR_MISALIGNED;
  if ((st = check_device()) != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_gemm_up_swiglu_u(x_perm, offsets, w_ug, cap_rows, d, h, E, h_buf, u_buf, stream));
}

moe_status moe_gemm_up_swiglu_gather(const uint16_t* x, const int32_t* perm, int64_t T, int32_t k,
                                     const int32_t* offsets, const uint16_t* w_ug, int64_t d, int64_t h, int32_t E,
                                     uint16_t* h_buf, hipStream_t stream) {
  if (T < 0 || k < 1 || T > kMaxSlots / k) return MOE_ERR_BAD_SHAPE;
  const int64_t S = T * k;
  moe_status st = check_gemm_shape(S, d, h, E);
  if (st != MOE_OK) return st;
  if (missing(x, T * d) || missing(perm, S) || missing(offsets, E + 1) || missing(w_ug, (int64_t)E * 2 * h * d) ||
      missing(h_buf, S * h))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(x, 16) || misaligned(w_ug, 16) || misaligned(h_buf, 16) || misaligned(offsets, 4) ||
      misaligned(perm, 4))
    return MOE_ERR_MISALIGNED;
  if ((st = check_device()) != MOE_OK) return st;
  if (S == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_gemm_up_swiglu_gather(x, perm, T, k, offsets, w_ug, d, h, E, h_buf, stream));
}

moe_status moe_gemm_down(const uint16_t* h_buf, const int32_t* offsets, const uint16_t* w_down, int64_t cap_rows,
                         int64_t d, int64_t h, int32_t E, uint16_t* y_perm, hipStream_t stream) {
  moe_status st = check_gemm_shape(cap_rows, d, h, E);
  if (st != MOE_OK) return st;
  if (missing(h_buf, cap_rows * h) || missing(offsets, E + 1) || missing(w_down, (int64_t)E * h * d) ||
      missing(y_perm, cap_rows * d))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(h_buf, 16) || misaligned(w_down, 16) || misaligned(y_perm, 16) || misaligned(offsets, 4))
    return MOE_ERR_MISALIGNED;
  if ((st = check_device()) != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_gemm_down(h_buf, offsets, w_down, cap_rows, d, h, E, y_perm, stream));
}

moe_status grouped_swiglu_expert(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                 const uint16_t* w_down, int64_t cap_rows, int64_t d, int64_t h, int32_t E,
                                 uint16_t* h_buf, uint16_t* y_perm, hipStream_t stream) {
  moe_status st = check_gemm_shape(cap_rows, d, h, E);
  if (st != MOE_OK) return st;
  if (missing(w_down, (int64_t)E * h * d) || missing(y_perm, cap_rows * d)) return MOE_ERR_NULL_POINTER;
  if (misaligned(w_down, 16) || misaligned(y_perm, 16)) return MOE_ERR_MISALIGNED;
  st = moe_gemm_up_swiglu(x_perm, offsets, w_ug, cap_rows, d, h, E, h_buf, stream);
  if (st != MOE_OK) return st;
  return moe_gemm_down(h_buf, offsets, w_down, cap_rows, d, h, E, y_perm, stream);
}

moe_status grouped_swiglu_expert_gather(const uint16_t* x, const int32_t* perm, int64_t T, int32_t k,
                                        const int32_t* offsets, const uint16_t* w_ug, const uint16_t* w_down,
                                        int64_t d, int64_t h, int32_t E, uint16_t* h_buf, uint16_t* y_perm,
                                        hipStream_t stream) {
  if (T < 0 || k < 1 || T > kMaxSlots / k) return MOE_ERR_BAD_SHAPE;
  const int64_t S = T * k;
  moe_status st = check_gemm_shape(S, d, h, E);
  if (st != MOE_OK) return st;
  if (missing(w_down, (int64_t)E * h * d) || missing(y_perm, S * d)) return MOE_ERR_NULL_POINTER;
  if (misaligned(w_down, 16) || misaligned(y_perm, 16)) return MOE_ERR_MISALIGNED;
  st = moe_gemm_up_swiglu_gather(x, perm, T, k, offsets, w_ug, d, h, E, h_buf, stream);
  if (st != MOE_OK) return st;
  return moe_gemm_down(h_buf, offsets, w_down, S, d, h, E, y_perm, stream);
}

moe_status moe_unpermute(const uint16_t* y_perm, const int32_t* inv_map, const float* routing_w, int64_t T, int32_t k,
                         int64_t d, uint16_t* y, hipStream_t stream) {
  if (T < 0 || k < 1 || bad_width(d) || T > kMaxSlots / k) return MOE_ERR_BAD_SHAPE;
  const int64_t S = T * k;
  if (missing(y_perm, S * d) || missing(inv_map, S) || missing(routing_w, S) || missing(y, T * d))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(y_perm, 16) || misaligned(y, 16) || misaligned(inv_map, 4) || misaligned(routing_w, 4))
    return MOE_ERR_MISALIGNED;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_unpermute(y_perm, inv_map, routing_w, T, k, d, y, stream));
}

moe_status moe_grouped_projection(const uint16_t* x, const int32_t* offsets, const uint16_t* w, int32_t w_layout,
                                  int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* y,
                                  hipStream_t stream) {
  if (w_layout != MOE_W_IN_OUT && w_layout != MOE_W_OUT_IN) return MOE_ERR_BAD_SHAPE;
  moe_status st = check_gemm_shape(cap_rows, d_in, d_out, E);
  if (st != MOE_OK) return st;
  if (missing(x, cap_rows * d_in) || missing(offsets, E + 1) || missing(w, (int64_t)E * d_in * d_out) ||
      missing(y, cap_rows * d_out))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(x, 16) || misaligned(w, 16) || misaligned(y, 16) || misaligned(offsets, 4)) return MOE_ERR_MISALIGNED;
  if ((st = check_device()) != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(
      launch_grouped_projection(x, offsets, w, w_layout == MOE_W_OUT_IN, cap_rows, d_in, d_out, E, y, stream));
}

moe_status moe_swiglu_backward(const uint16_t* dh, const uint16_t* u, const int32_t* offsets, int32_t E,
                               int64_t cap_rows, int64_t h, uint16_t* du, hipStream_t stream) {
  if (cap_rows < 0 || cap_rows > kMaxSlots || bad_width(h) || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_BAD_SHAPE;
  if (missing(dh, cap_rows * h) || missing(u, cap_rows * 2 * h) || missing(offsets, E + 1) ||
      missing(du, cap_rows * 2 * h))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(dh, 16) || misaligned(u, 16) || misaligned(du, 16) || misaligned(offsets, 4)) return MOE_ERR_MISALIGNED;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_swiglu_backward(dh, u, offsets, E, cap_rows, h, du, stream));
}

moe_status moe_grouped_dgrad(const uint16_t* dy, const int32_t* offsets, const uint16_t* w, int32_t w_layout,
                             int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dx,
                             hipStream_t stream) {
  if (w_layout != MOE_W_IN_OUT && w_layout != MOE_W_OUT_IN) return MOE_ERR_BAD_SHAPE;
  moe_status st = check_gemm_shape(cap_rows, d_in, d_out, E);
  if (st != MOE_OK) return st;
  if (missing(dy, cap_rows * d_out) || missing(offsets, E + 1) || missing(w, (int64_t)E * d_in * d_out) ||
      missing(dx, cap_rows * d_in))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(dy, 16) || misaligned(w, 16) || misaligned(dx, 16) || misaligned(offsets, 4)) return MOE_ERR_MISALIGNED;
  if ((st = check_device()) != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_grouped_dgrad(dy, offsets, w, w_layout == MOE_W_OUT_IN, cap_rows, d_in, d_out, E, dx, stream));
}

size_t moe_grouped_wgrad_workspace_bytes(int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E) {
  if (check_gemm_shape(cap_rows, d_in, d_out, E) != MOE_OK) return 0;
  return (size_t)wgrad_partial_slots(cap_rows) * (size_t)d_in * (size_t)d_out * sizeof(float);
}

moe_status moe_grouped_wgrad(const uint16_t* x, const uint16_t* dy, const int32_t* offsets, int32_t w_layout,
                             int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dw,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (w_layout != MOE_W_IN_OUT && w_layout != MOE_W_OUT_IN) return MOE_ERR_BAD_SHAPE;
  moe_status st = check_gemm_shape(cap_rows, d_in, d_out, E);
  if (st != MOE_OK) return st;
  const size_t need = moe_grouped_wgrad_workspace_bytes(cap_rows, d_in, d_out, E);
  if (missing(x, cap_rows * d_in) || missing(dy, cap_rows * d_out) || missing(offsets, E + 1) ||
      missing(dw, (int64_t)E * d_in * d_out) || missing(workspace, (int64_t)need))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(x, 16) || misaligned(dy, 16) || misaligned(dw, 16) || misaligned(offsets, 4) ||
      misaligned(workspace, 16))
    return MOE_ERR_MISALIGNED;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if ((st = check_device()) != MOE_OK) return st;
  (void)hipGetLastError();
  return launched(launch_grouped_wgrad(x, dy, offsets, w_layout == MOE_W_OUT_IN, cap_rows, d_in, d_out, E, dw,
                                       static_cast<float*>(workspace), stream));
}

moe_status moe_permute_backward(const uint16_t* dx_perm, const int32_t* inv_map, int64_t T, int32_t k, int64_t d,
                                uint16_t* dx, hipStream_t stream) {
  if (T < 0 || k < 1 || bad_width(d) || T > kMaxSlots / k) return MOE_ERR_BAD_SHAPE;
  const int64_t S = T * k;
  if (missing(dx_perm, S * d) || missing(inv_map, S) || missing(dx, T * d)) return MOE_ERR_NULL_POINTER;
  if (misaligned(dx_perm, 16) || misaligned(dx, 16) || misaligned(inv_map, 4)) return MOE_ERR_MISALIGNED;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_unpermute(dx_perm, inv_map, nullptr, T, k, d, dx, stream));
}

moe_status moe_unpermute_backward(const uint16_t* dy, const uint16_t* y_perm, const int32_t* inv_map,
                                  const float* routing_w, int64_t T, int32_t k, int64_t d, uint16_t* dy_perm,
                                  float* d_routing_w, hipStream_t stream) {
  if (T < 0 || k < 1 || bad_width(d) || T > kMaxSlots / k) return MOE_ERR_BAD_SHAPE;
  const int64_t S = T * k;
  if (missing(dy, T * d) || missing(y_perm, S * d) || missing(inv_map, S) || missing(routing_w, S) ||
      missing(dy_perm, S * d) || missing(d_routing_w, S))
    return MOE_ERR_NULL_POINTER;
  if (misaligned(dy, 16) || misaligned(y_perm, 16) || misaligned(dy_perm, 16) || misaligned(inv_map, 4) ||
      misaligned(routing_w, 4) || misaligned(d_routing_w, 4))
    return MOE_ERR_MISALIGNED;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  (void)hipGetLastError();
  return launched(launch_unpermute_backward(dy, y_perm, inv_map, routing_w, T, k, d, dy_perm, d_routing_w, stream));
}

static_assert(sizeof(moe_status) == sizeof(int), "moe_status travels as a C int");

const char* moe_status_string(moe_status s) {
  // A C caller may pass any int. In C++ an enum without a fixed underlying type only holds
  // the values of its enumerators' bit width, so the code is read as raw int bits.
  int code;
  std::memcpy(&code, &s, sizeof(code));
  switch (code) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL_POINTER: return "MOE_ERR_NULL_POINTER: a pointer is NULL while its tensor is non-empty";
    case MOE_ERR_BAD_SHAPE: return "MOE_ERR_BAD_SHAPE: a size is out of range (T, k, E, d, h or T*k)";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: a bf16 tensor is not 16-byte aligned or an int32/fp32 tensor not 4-byte aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than the call's *_workspace_bytes()";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "MOE_ERR_UNSUPPORTED_DEVICE: the current HIP device is not gfx950";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: a kernel launch reported a HIP error";
    case MOE_ERR_TOO_LARGE: return "MOE_ERR_TOO_LARGE: the call needs more than the fixed table of moe_permute_noalloc (E * ceil(T*k/256) > 2^20)";
  }
  return "unknown moe_status";
}

}  // extern "C"
