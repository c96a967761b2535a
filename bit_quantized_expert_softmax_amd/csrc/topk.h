// Block-wide top-k of a token's router logits, shared by the router and the
// expert kernels. Ties go to the lower expert id; the output is in rank
// order; the weights are a softmax over the selected logits.
#pragma once

#include "launch.h"

static_assert(moe::kMaxTopK <= 16, "the weights' sum runs over one 16-lane DPP row");

namespace moe {

// Order-preserving 64-bit key of an fp64 logit: the unsigned order of the
// keys is the numeric order of the logits (-0 is taken as +0; a NaN gets key
// 0, below every number), so the rank loop compares integers instead of fp64
// values (measured faster on gfx950).
__device__ __forceinline__ unsigned long long logit_key(double z) {
  if (z != z) return 0ull;
  const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(z + 0.0));
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ double key_logit(unsigned long long key) {
  const unsigned long long b = (key >> 63) ? (key & 0x7FFFFFFFFFFFFFFFull) : ~key;
  return __longlong_as_double(static_cast<long long>(b));
}

// (key f, expert f) ranks before (key e, expert e): a larger key, or the same
// key and a lower expert id. Keys as (low word, high word).
__device__ __forceinline__ bool key_better(uint2 kf, int f, uint2 ke, int e) {
  const unsigned long long a = static_cast<unsigned long long>(kf.y) << 32 | kf.x;
  const unsigned long long b = static_cast<unsigned long long>(ke.y) << 32 | ke.x;
  return a > b || (a == b && f < e);
}

// Top-k of E logits held in LDS (zs), by rank: an expert's rank is the number
// of experts ranking before it; ranks below k are the selection in rank order
// (sel_z, sel_e), visible to the whole block on return. zs is overwritten with
// the logits' keys. All block threads call.
__device__ inline void topk_select(double* zs, int E, int k, double* sel_z, int* sel_e) {
  // every rank slot starts with a valid id, so non-finite logits cannot
  // produce an out-of-range expert index downstream
  if (threadIdx.x < static_cast<unsigned>(k)) {
    sel_e[threadIdx.x] = threadIdx.x;
    sel_z[threadIdx.x] = 0.0;
  }
  // each thread converts the logits it reads back, so no barrier between
  unsigned long long* kz64 = reinterpret_cast<unsigned long long*>(zs);
  for (int e = threadIdx.x; e < E; e += blockDim.x) kz64[e] = logit_key(zs[e]);
  __syncthreads();
  const uint2* kz = reinterpret_cast<const uint2*>(zs);
  // P threads (adjacent lanes) share one expert's comparisons (P = largest
  // power of two with P * E <= blockDim, at most 8); part p takes the keys
  // p, p + P, ..., so at each step the parts of a wave read adjacent words
  // (no bank conflicts) and the experts of a part share one address
  int P = 1;
  while (P < 8 && 2 * P * E <= static_cast<int>(blockDim.x)) P *= 2;
  for (int t0 = 0; t0 < E * P; t0 += blockDim.x) {
    const int t = t0 + threadIdx.x;
    const int e = t / P;
    const int part = t % P;
    const bool valid = e < E;
    const uint2 ke = kz[valid ? e : 0];
    int rank = 0;
    // eight keys per batch, so that the batch's LDS reads are in flight together
    int f = part;
    for (; f + 7 * P < E; f += 8 * P) {
      uint2 kf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[i] = kz[f + i * P];
#pragma unroll
      for (int i = 0; i < 8; ++i) rank += key_better(kf[i], f + i * P, ke, e) ? 1 : 0;
    }
    for (; f < E; f += P) rank += key_better(kz[f], f, ke, e) ? 1 : 0;
    // partial ranks of the P lanes (an aligned group of 2, 4 or 8) by DPP:
    // lane ^ 1, lane ^ 2, then the mirrored quad
    if (P >= 2) rank += static_cast<int>(dpp<0xB1>(static_cast<uint32_t>(rank)));
    if (P >= 4) rank += static_cast<int>(dpp<0x4E>(static_cast<uint32_t>(rank)));
    if (P >= 8) rank += static_cast<int>(dpp<0x141>(static_cast<uint32_t>(rank)));
    if (valid && part == 0 && rank < k) {
      sel_z[rank] = key_logit(static_cast<unsigned long long>(ke.y) << 32 | ke.x);
      sel_e[rank] = e;
    }
  }
  __syncthreads();
}

// The selection's softmax weights w_j = exp(z_j - z_0) / sum_i exp(z_i - z_0)
// (one exp per lane, the sum over the k lanes by DPP in a fixed order) and
// the writes of ids / w and the optional copies, by the first 16 lanes of the
// block (k <= 16); nothing to write, nothing done. All block threads call;
// no barrier.
__device__ inline void topk_weights(const double* sel_z, const int* sel_e, int k, int32_t* ids, float* w,
                                    int32_t* ids2, float* w2) {
  if (!ids && !w && !ids2 && !w2) return;
  if (threadIdx.x < 16u) {
    const int j = threadIdx.x;
    const float ej = j < k ? expf(static_cast<float>(sel_z[j] - sel_z[0])) : 0.f;
    const float tot = dpp_sum<16>(ej);
    if (j < k) {
      const float wj = ej / tot;
      if (ids) ids[j] = sel_e[j];
      if (w) w[j] = wj;
      if (ids2) ids2[j] = sel_e[j];
      if (w2) w2[j] = wj;
    }
  }
}

// Both, with a barrier after the writes.
__device__ inline void topk_block(double* zs, int E, int k, double* sel_z, int* sel_e,
                                  int32_t* ids, float* w, int32_t* ids2, float* w2) {
  topk_select(zs, E, k, sel_z, sel_e);
  topk_weights(sel_z, sel_e, k, ids, w, ids2, w2);
  __syncthreads();
}

}  // namespace moe
