// Launchers of the mixture-of-experts routing kernels (moe.hip).  Expert
// rows are expert-major, each expert's block padded with zero rows to a
// multiple of 256; off[E + 1] (device) holds the blocks' first rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

// sel[T, k] = the k experts with the largest logits (ties to the lower
// index), gates[T, k] = softmax over those logits.  logits fp32 [T, ld].
hipError_t launch_moe_route(const float* logits, int64_t ld, int64_t T, int E, int k, int32_t* sel,
                            float* gates, hipStream_t s);
// off[E + 1], pos[T, k] (row of each token-slot pair) and rowtok[rows] (token
// of each row, -1 for padding); one workgroup, deterministic.
hipError_t launch_moe_plan(const int32_t* sel, int64_t T, int E, int k, int32_t* off, int32_t* pos,
                           int32_t* rowtok, hipStream_t s);
// X[row] = n2[rowtok[row]] or zeros, rows < off[E] (grid: `rows` = the maximum).
hipError_t launch_moe_gather(const uint16_t* n2, int h, const int32_t* rowtok, const int32_t* off,
                             int E, int64_t rows, uint16_t* X, hipStream_t s);
// y[t] = h1[t] + sum_j gates[t, j] Yo[pos[t, j]].
hipError_t launch_moe_combine(const float* h1, const float* Yo, const int32_t* pos,
                              const float* gates, int k, int h, int64_t T, float* y,
                              hipStream_t s);
// dout[pos[t, j]] = bf16(gates[t, j] dy[t]); dlog [T, ldl] bf16 = router-logit
// gradient (softmax over the selected logits), 0 at unselected experts.
hipError_t launch_moe_bwd_gates(const float* dy, const float* Yo, const int32_t* pos,
                                const int32_t* sel, const float* gates, int k, int E, int h,
                                int64_t T, uint16_t* dout, uint16_t* dlog, int64_t ldl,
                                hipStream_t s);
// Zero rows r < off[E] with rowtok[r] < 0 of a bf16 [rows, h] matrix.
hipError_t launch_moe_zero_pad(const int32_t* rowtok, const int32_t* off, int E, int h,
                               int64_t rows, uint16_t* X, hipStream_t s);
// dn[t] = sum_j dX[pos[t, j]].
hipError_t launch_moe_bwd_combine(const float* dX, const int32_t* pos, int k, int h, int64_t T,
                                  float* dn, hipStream_t s);

}  // namespace mt
