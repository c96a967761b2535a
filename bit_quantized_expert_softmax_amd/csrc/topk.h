// Block-wide top-k of a token's router logits, shared by the router and the
// expert kernels. Ties go to the lower expert id; the output is in rank
// order; the weights are a softmax over the selected logits.
#pragma once

#include "launch.h"

namespace moe {

__device__ __forceinline__ bool key_better(double v1, int e1, double v2, int e2) {
  return v1 > v2 || (v1 == v2 && e1 < e2);
}

// Top-k of E logits held in LDS (zs), by rank: an expert's rank is the number
// of experts with a larger (z, -id) key; ranks below k are the selection in
// rank order. Writes ids / w (and the optional copies). All block threads call.
__device__ inline void topk_block(const double* zs, int E, int k, double* sel_z, int* sel_e,
                           int32_t* ids, float* w, int32_t* ids2, float* w2) {
  // every rank slot starts with a valid id, so non-finite logits cannot
  // produce an out-of-range expert index downstream
  if (threadIdx.x < static_cast<unsigned>(k)) {
    sel_e[threadIdx.x] = threadIdx.x;
    sel_z[threadIdx.x] = 0.0;
  }
  __syncthreads();
  // P threads share one expert's comparisons (P = largest power of two with
  // P * E <= blockDim, at most 8); their partial ranks are summed in-wave
  int P = 1;
  while (P < 8 && 2 * P * E <= static_cast<int>(blockDim.x)) P *= 2;
  const int per = (E + P - 1) / P;
  for (int t0 = 0; t0 < E * P; t0 += blockDim.x) {
    const int t = t0 + threadIdx.x;
    const int e = t / P;
    const int part = t % P;
    const bool valid = e < E;
    const double v = zs[valid ? e : 0];
    int rank = 0;
    const int f0 = part * per;
    const int f1 = f0 + per < E ? f0 + per : E;
    // eight logits per batch, so that the batch's LDS reads are in flight
    // together instead of one read latency per comparison
    int f = f0;
    for (; f + 8 <= f1; f += 8) {
      double zf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) zf[i] = zs[f + i];
#pragma unroll
      for (int i = 0; i < 8; ++i) rank += key_better(zf[i], f + i, v, e) ? 1 : 0;
    }
    for (; f < f1; ++f) rank += key_better(zs[f], f, v, e) ? 1 : 0;
    for (int o = 1; o < P; o <<= 1) rank += __shfl_xor(rank, o, 64);
    if (valid && part == 0 && rank < k) {
      sel_z[rank] = v;
      sel_e[rank] = e;
    }
  }
  __syncthreads();
  if (threadIdx.x < static_cast<unsigned>(k)) {
    const int j = threadIdx.x;
    float tot = 0.f;
    for (int i = 0; i < k; ++i) tot += expf(static_cast<float>(sel_z[i] - sel_z[0]));
    const float wj = expf(static_cast<float>(sel_z[j] - sel_z[0])) / tot;
    if (ids) ids[j] = sel_e[j];
    if (w) w[j] = wj;
    if (ids2) ids2[j] = sel_e[j];
    if (w2) w2[j] = wj;
  }
  __syncthreads();
}

}  // namespace moe
