/*
 * moe_grouped.h -- C ABI of the routed MoE expert step on MI355X (gfx950).
 *
 * The library runs the forward expert step of a routed mixture-of-experts
 * layer on one GPU as three stream-ordered calls:
 *
 *   moe_permute            histogram of expert ids, exclusive scan into int32
 *                          offsets, drop of invalid ids, stable order, inverse
 *                          map and the permuted gather of token rows;
 *   grouped_swiglu_expert  one persistent grouped GEMM over the ragged
 *                          per-expert row blocks with SwiGLU fused into the
 *                          gate/up projection, then the grouped down projection;
 *   moe_unpermute          atomic-free gather + weighted reduction back to
 *                          token order through the inverse map.
 *
 * The grouped expert also comes as its two single-launch halves and with the
 * permuted gather fused into the gate/up projection's loads. The backward
 * (Eq 15) adds grouped Dgrad and Wgrad for either weight layout, a plain
 * grouped projection, the SwiGLU backward, the atomic-free backward of both
 * permutations and a gate/up launch that also keeps the pre-activation U for
 * the backward.
 *
 * Sources: "Section 09: Grouped GEMM" of the OLMo-core MoE report (Eq 13 for
 * the expert, Figs 35-37 and Secs 9.2-9.4 for device-side offsets, fixed
 * capacity buffers and unpadded compute, Sec 9.5 / Eq 15 / Table 15 for the
 * backward) and the halo toolkit's "Grouped GEMM" notes (dropping ids outside
 * [0, E) before the sort, int32 cumulative offsets, the sentinel-padded
 * inverse map used for an atomic-free scatter-back and permute backward,
 * gate-then-up weight chunks).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is a DEVICE pointer on the current HIP device. bf16
 *   values are passed as uint16_t bit patterns. Every tensor is dense and
 *   row-major with the shape given next to it.
 * - The caller allocates and frees every buffer, workspaces included. The
 *   library keeps no state between calls beyond per-device properties it
 *   caches on first use.
 * - Calls are asynchronous on `stream`: no call synchronises, copies a count
 *   to the host or allocates. Row counts exist only as device data.
 * - Shapes are capacity shapes: S = T*k dispatch slots; x_perm, h_buf and
 *   y_perm have S rows whatever the routing, and only their first
 *   M = offsets[E] rows are written (rows >= M and perm[M..S) are left as they
 *   were). Dispatch slot s = t*k + j is token t's j-th routed expert.
 * - A pointer may be NULL only when its tensor has zero elements.
 * - Return values are host-side validation and launch results. Nothing is
 *   ever reported from the device: invalid expert ids are data, and are
 *   dropped. Status codes are listed in moe_status.
 * - Calls on different streams are independent and thread-safe.
 */
#ifndef MOE_GROUPED_H_
#define MOE_GROUPED_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_EXPERTS 1024

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL_POINTER = 1,       /* a pointer is NULL while its tensor is non-empty           */
  MOE_ERR_BAD_SHAPE = 2,          /* T<0, k<1, E<1 or E>1024, d or h < 8 or not a multiple of 8,
                                     d or h > 2^24 (> 2^20 for the grouped GEMM calls),
                                     T*k >= 2^31, or cap_rows < 0                               */
  MOE_ERR_MISALIGNED = 3,         /* a bf16 tensor not 16-byte aligned, or an int32/float
                                     tensor not 4-byte aligned                                  */
  MOE_ERR_WORKSPACE = 4,          /* workspace_bytes below the call's *_workspace_bytes()       */
  MOE_ERR_UNSUPPORTED_DEVICE = 5, /* the current HIP device is not gfx950, or no device         */
  MOE_ERR_LAUNCH = 6,             /* a HIP error was reported while launching                    */
  MOE_ERR_TOO_LARGE = 7           /* moe_permute_noalloc only: E * ceil(T*k / 256) exceeds its
                                     fixed table of MOE_PERMUTE_NOALLOC_TABLE_ENTRIES            */
} moe_status;

/* Bytes of device workspace moe_permute needs for T tokens, k slots per token
 * and E experts (a per-chunk histogram table). Pure host arithmetic; returns 0
 * for invalid shapes. */
size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E);

/* Dispatch preparation (OLMo report Sec 9.2-9.3 and Fig 37; halo notes on the
 * expert step and on the inverse map).
 *
 *   x           bf16  [T, d]  token rows
 *   expert_ids  int32 [T, k]  routed expert of each slot; any id outside
 *                             [0, E) (such as the -1 padding of an expert-
 *                             parallel dispatch) marks a dropped slot
 *   x_perm      bf16  [T*k, d] out: rows [0, M) hold X[perm[p] / k]; may be NULL,
 *                             then no rows are copied (x is then not read and
 *                             may be NULL too) and a *_gather GEMM call reads
 *                             X through perm instead
 *   counts      int32 [E]     out: kept slots per expert
 *   offsets     int32 [E+1]   out: offsets[0] = 0, offsets[e+1] =
 *                             offsets[e] + counts[e]; expert e owns sorted
 *                             rows [offsets[e], offsets[e+1]); M = offsets[E]
 *   perm        int32 [T*k]   out: perm[p] = slot in sorted row p, p < M
 *   inv_map     int32 [T, k]  out: sorted row of each slot, -1 if dropped
 *   workspace   device scratch of at least moe_permute_workspace_bytes(T,k,E)
 *
 * Inside an expert's block, slots keep ascending slot order (the order of a
 * stable sort by expert id), so counts, offsets, perm[0, M) and inv_map are
 * fully determined by expert_ids. T = 0 is valid (counts and offsets become
 * zeros). */
moe_status moe_permute(const uint16_t* x, const int32_t* expert_ids, int64_t T, int32_t k, int64_t d,
                       int32_t E, uint16_t* x_perm, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv_map, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_permute for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, results and stream semantics as
 * moe_permute, without the workspace: the per-chunk histogram table lives in a
 * fixed array of MOE_PERMUTE_NOALLOC_TABLE_ENTRIES int32 (4 MiB) in the
 * library's own device memory, one per GPU, held until the process ends. Its
 * address is resolved on a device's first call (that device current); the call
 * never allocates, frees or synchronises.
 *
 * Limit: E * ceil(T*k / 256) <= MOE_PERMUTE_NOALLOC_TABLE_ENTRIES (for E = 64,
 * up to 4,194,304 slots; for E = 1024, up to 262,144), else MOE_ERR_TOO_LARGE
 * and nothing is launched. Every call on one GPU shares that GPU's table: calls
 * whose executions overlap on one GPU (concurrent streams, or graphs replayed
 * on several streams) race and give wrong results; calls ordered on one stream
 * are safe. The table's contents from the previous call are never read. */
#define MOE_PERMUTE_NOALLOC_TABLE_ENTRIES (1 << 20)
moe_status moe_permute_noalloc(const uint16_t* x, const int32_t* expert_ids, int64_t T, int32_t k, int64_t d,
                               int32_t E, uint16_t* x_perm, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv_map, hipStream_t stream);

/* Grouped SwiGLU expert (OLMo report Eq 13 and Sec 9.2's device-scheduled
 * grouped GEMM). For every expert e with rows [offsets[e], offsets[e+1]):
 *
 *   U_e = x_perm[rows] * W_ug[e]^T          bf16 inputs, fp32 accumulation,
 *                                           rounded to bf16 (round-to-nearest-even)
 *   H_e = bf16( SiLU(U_e[:, :h]) * U_e[:, h:] )      written to h_buf[rows]
 *   Y_e = bf16( H_e * W_down[e] )                    written to y_perm[rows]
 *
 *   x_perm   bf16  [cap_rows, d]
 *   offsets  int32 [E+1]       device offsets as written by moe_permute; each is
 *                              clamped into [0, cap_rows] on the device (an
 *                              expert whose end precedes its start is empty),
 *                              so no row outside the buffers is ever touched
 *   w_ug     bf16  [E, 2h, d]  gate rows [0, h), up rows [h, 2h)
 *   w_down   bf16  [E, h, d]
 *   h_buf    bf16  [cap_rows, h] out (the SwiGLU activations)
 *   y_perm   bf16  [cap_rows, d] out
 *
 * Empty experts cost nothing; K need not be a multiple of the K tile; rows
 * past M are never computed. Equivalent to moe_gemm_up_swiglu followed by
 * moe_gemm_down on the same stream. */
moe_status grouped_swiglu_expert(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                 const uint16_t* w_down, int64_t cap_rows, int64_t d, int64_t h, int32_t E,
                                 uint16_t* h_buf, uint16_t* y_perm, hipStream_t stream);

/* The first half of grouped_swiglu_expert alone: one kernel launch that
 * writes h_buf[rows] = bf16(SiLU(bf16(g)) * bf16(u)) with [g | u] =
 * x_perm[rows] * W_ug[e]^T. Arguments as above. */
moe_status moe_gemm_up_swiglu(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                              int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf,
                              hipStream_t stream);

/* The first half for a forward that keeps what its backward needs: as
 * moe_gemm_up_swiglu, and the same launch also stores the gate/up
 * pre-activation of Eq 13,
 *
 *   u_buf    bf16  [cap_rows, 2h]  out: u_buf[p] = bf16(x_perm[p] W_ug[e]^T),
 *                                  gate block (columns [0, h)) then up block
 *
 * the bf16 values the SwiGLU epilogue reads (rows past M untouched). The
 * SwiGLU backward needs U; with u_buf kept, the backward does not recompute
 * the gate/up projection (OLMo report Sec 9.5, Eq 15: the backward is two more
 * grouped problems per projection; recomputing U would add a third). h_buf is
 * bit for bit that of moe_gemm_up_swiglu, u_buf that of
 * moe_grouped_projection(x_perm, offsets, w_ug, MOE_W_OUT_IN, ...). */
moe_status moe_gemm_up_swiglu_u(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_ug,
                                int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* h_buf,
                                uint16_t* u_buf, hipStream_t stream);

/* The first half with the permuted gather fused into its loads (OLMo report
 * Sec 9.4: GEMM 1 takes its A rows straight from the dispatch order, with no
 * permuted copy in between). Sorted row p of expert e's block reads token row
 * x[perm[p] / k]; nothing else changes:
 *
 *   x        bf16  [T, d]    token rows
 *   perm     int32 [T*k]     as written by moe_permute (entries [0, M) are read;
 *                            out-of-range entries are clamped, never faulting)
 *   offsets  int32 [E+1]     as written by moe_permute
 *   w_ug     bf16  [E, 2h, d]
 *   h_buf    bf16  [T*k, h]  out
 *
 * One kernel launch; same results as moe_permute's x_perm followed by
 * moe_gemm_up_swiglu, bit for bit. */
moe_status moe_gemm_up_swiglu_gather(const uint16_t* x, const int32_t* perm, int64_t T, int32_t k,
                                     const int32_t* offsets, const uint16_t* w_ug, int64_t d, int64_t h, int32_t E,
                                     uint16_t* h_buf, hipStream_t stream);

/* moe_gemm_up_swiglu_gather followed by moe_gemm_down (cap_rows = T*k): the
 * grouped SwiGLU expert on token rows gathered through perm. */
moe_status grouped_swiglu_expert_gather(const uint16_t* x, const int32_t* perm, int64_t T, int32_t k,
                                        const int32_t* offsets, const uint16_t* w_ug, const uint16_t* w_down,
                                        int64_t d, int64_t h, int32_t E, uint16_t* h_buf, uint16_t* y_perm,
                                        hipStream_t stream);

/* The second half alone: one kernel launch that writes y_perm[rows] =
 * bf16(h_buf[rows] * W_down[e]). Arguments as above. */
moe_status moe_gemm_down(const uint16_t* h_buf, const int32_t* offsets, const uint16_t* w_down,
                         int64_t cap_rows, int64_t d, int64_t h, int32_t E, uint16_t* y_perm,
                         hipStream_t stream);

/* Atomic-free scatter-back (halo notes: the inverse map turns the scatter
 * into a gather plus a reduction; routing weights are applied here).
 *
 *   y_perm     bf16  [T*k, d]
 *   inv_map    int32 [T, k]   sorted row of each slot; entries outside
 *                             [0, T*k) (such as -1) are skipped
 *   routing_w  fp32  [T, k]
 *   y          bf16  [T, d]   out: y[t] = bf16( sum over kept j, ascending,
 *                             of routing_w[t,j] * y_perm[inv_map[t,j]] ),
 *                             accumulated in fp32; a token with no kept slot
 *                             gets a zero row
 *
 * Every row of y is written. Weights are not renormalised over kept slots. */
moe_status moe_unpermute(const uint16_t* y_perm, const int32_t* inv_map, const float* routing_w, int64_t T,
                         int32_t k, int64_t d, uint16_t* y, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward (OLMo report Sec 9.5, Eq 15 and Table 15; halo notes on the
 * atomic-free permute backward). For one grouped projection Y_e = X_e W_e with
 * X_e [M_e, d_in] and W_e [d_in, d_out], Dgrad dX_e = dY_e W_e^T keeps M_e as
 * its output rows and Wgrad dW_e = X_e^T dY_e contracts over M_e. Weights are
 * stored in one of two layouts:
 *   MOE_W_IN_OUT  [E, d_in, d_out]  (W_down [E, h, d]: d_in = h, d_out = d)
 *   MOE_W_OUT_IN  [E, d_out, d_in]  (W_ug [E, 2h, d]: d_in = d, d_out = 2h)
 * bf16 inputs, fp32 accumulation, bf16 outputs (round-to-nearest-even).
 * Offsets are clamped as in the forward.
 * ------------------------------------------------------------------------- */
typedef enum moe_weight_layout { MOE_W_IN_OUT = 0, MOE_W_OUT_IN = 1 } moe_weight_layout;

/* One grouped projection without activation: y[rows_e] = bf16(x[rows_e] * W_e)
 * (the forward of Eq 15's Y_e = X_e W_e).
 *
 *   x        bf16  [cap_rows, d_in]
 *   offsets  int32 [E+1]
 *   w        bf16  [E, d_in, d_out] or [E, d_out, d_in] per w_layout
 *   y        bf16  [cap_rows, d_out] out (rows past M untouched)
 *
 * With MOE_W_IN_OUT this is moe_gemm_down; with MOE_W_OUT_IN and W_ug it
 * recomputes the gate/up pre-activation U = [G | Up] that the SwiGLU backward
 * needs. */
moe_status moe_grouped_projection(const uint16_t* x, const int32_t* offsets, const uint16_t* w, int32_t w_layout,
                                  int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* y,
                                  hipStream_t stream);

/* SwiGLU backward over the sorted rows [0, offsets[E]) (clamped to cap_rows):
 * with [g | up] = u[row] and s = sigmoid(g), du[row] = [dG | dUp] where
 * dG = bf16(dh * up * s * (1 + g * (1 - s))) and dUp = bf16(dh * g * s),
 * evaluated in fp32 (the pages define the projections' backward, not the
 * activation's; the forward's bf16 roundings are taken as identities).
 *
 *   dh       bf16  [cap_rows, h]
 *   u        bf16  [cap_rows, 2h]   gate block then up block, as the forward's U
 *   offsets  int32 [E+1]
 *   du       bf16  [cap_rows, 2h]   out (rows past M untouched) */
moe_status moe_swiglu_backward(const uint16_t* dh, const uint16_t* u, const int32_t* offsets, int32_t E,
                               int64_t cap_rows, int64_t h, uint16_t* du, hipStream_t stream);

/* Dgrad: dx[rows_e] = bf16(dy[rows_e] * W_e^T) for every expert e.
 *
 *   dy       bf16  [cap_rows, d_out]
 *   offsets  int32 [E+1]
 *   w        bf16  [E, d_in, d_out] or [E, d_out, d_in] per w_layout
 *   dx       bf16  [cap_rows, d_in] out (rows past M untouched)
 *
 * A forward-shaped grouped GEMM (K = d_out, N = d_in): same kernels and tile
 * choice as the forward projections. An unknown w_layout is MOE_ERR_BAD_SHAPE. */
moe_status moe_grouped_dgrad(const uint16_t* dy, const int32_t* offsets, const uint16_t* w, int32_t w_layout,
                             int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dx,
                             hipStream_t stream);

/* Bytes of device workspace moe_grouped_wgrad needs (fp32 partial gradients
 * of experts whose rows are split; 0 when cap_rows <= 4096). Host arithmetic
 * only; 0 for invalid shapes. */
size_t moe_grouped_wgrad_workspace_bytes(int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E);

/* Wgrad: dW_e = bf16(x[rows_e]^T * dy[rows_e]), written [E, d_in, d_out]
 * (MOE_W_IN_OUT) or transposed [E, d_out, d_in] (MOE_W_OUT_IN), so the
 * gradient has the layout of the weight it belongs to.
 *
 *   x          bf16  [cap_rows, d_in]    the projection's input rows
 *   dy         bf16  [cap_rows, d_out]   the gradient of its output rows
 *   offsets    int32 [E+1]
 *   dw         bf16  [E * d_in * d_out]  out, every element written; an
 *                                       expert with no rows gets zeros
 *   workspace  at least moe_grouped_wgrad_workspace_bytes(...) bytes,
 *              16-byte aligned (may be NULL when that is 0)
 *
 * One persistent launch over 256 x 256 output tiles, largest experts first;
 * an expert with more than 4096 rows is split into row chunks whose fp32
 * partials a second launch sums in chunk order before the one rounding to
 * bf16, so the result is deterministic. */
moe_status moe_grouped_wgrad(const uint16_t* x, const uint16_t* dy, const int32_t* offsets, int32_t w_layout,
                             int64_t cap_rows, int64_t d_in, int64_t d_out, int32_t E, uint16_t* dw,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward of moe_permute's row gather (x_perm[p] = x[perm[p] / k]):
 * dx[t] = bf16(sum over kept j, ascending, of dx_perm[inv_map[t, j]]), fp32
 * accumulation; a gather through the inverse map, no atomics.
 *
 *   dx_perm  bf16  [T*k, d]
 *   inv_map  int32 [T, k]   entries outside [0, T*k) are skipped
 *   dx       bf16  [T, d]   out, every row written (zeros for a token with no
 *                           kept slot) */
moe_status moe_permute_backward(const uint16_t* dx_perm, const int32_t* inv_map, int64_t T, int32_t k, int64_t d,
                                uint16_t* dx, hipStream_t stream);

/* Backward of moe_unpermute (y[t] = sum_j w[t, j] * y_perm[inv_map[t, j]]):
 *
 *   dy           bf16  [T, d]
 *   y_perm       bf16  [T*k, d]  the forward's expert outputs
 *   inv_map      int32 [T, k]
 *   routing_w    fp32  [T, k]
 *   dy_perm      bf16  [T*k, d]  out: row inv_map[t, j] = bf16(w[t, j] * dy[t])
 *                                for kept slots; other rows untouched
 *   d_routing_w  fp32  [T, k]    out: sum_c dy[t, c] * y_perm[inv_map[t, j], c]
 *                                (fp32), 0 for dropped slots */
moe_status moe_unpermute_backward(const uint16_t* dy, const uint16_t* y_perm, const int32_t* inv_map,
                                  const float* routing_w, int64_t T, int32_t k, int64_t d, uint16_t* dy_perm,
                                  float* d_routing_w, hipStream_t stream);

/* A static, human-readable name for a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GROUPED_H_ */
