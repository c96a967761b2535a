// Router of one MoE layer: input preparation, fp64 logits, top-k + softmax.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", section "Qual é o principal truque da
// arquitetura": the router of every layer picks the 8 experts the current
// token needs. Selection is on the logits (softmax is monotone), ties go to
// the lower expert id, the weights are a softmax over the selected logits.
#include <float.h>
#include <math.h>

#include "launch.h"

namespace moe {
namespace {

constexpr int kPrepThreads = 256;

// One block per token. x' = x + add_in (fp32 add of the fp16 perturbation);
// u = x' * 1/sqrt(mean(x'^2) + 1e-6) when rmsnorm, else u = x'.
__global__ __launch_bounds__(kPrepThreads) void k_route_prep(const float* __restrict__ x,
                                                             const uint16_t* __restrict__ add_in,
                                                             int H, int rmsnorm,
                                                             float* __restrict__ u,
                                                             DigitGroup* __restrict__ udig,
                                                             float* __restrict__ usc) {
  const int b = blockIdx.x;
  const float* xb = x + static_cast<size_t>(b) * H;
  const uint16_t* ab = add_in ? add_in + static_cast<size_t>(b) * H : nullptr;
  __shared__ float red[kPrepThreads / kWave];
  __shared__ float s_scale;
  float r = 1.0f;
  if (rmsnorm) {
    float ss = 0.f;
    for (int h = threadIdx.x; h < H; h += kPrepThreads) {
      float v = xb[h] + (ab ? h2f(ab[h]) : 0.f);
      ss = fmaf(v, v, ss);
    }
    ss = seg_sum<kWave>(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
      for (int i = 0; i < kPrepThreads / kWave; ++i) t += red[i];
      s_scale = 1.0f / sqrtf(t / static_cast<float>(H) + 1e-6f);
    }
    __syncthreads();
    r = s_scale;
  }
  const int ng = H / kGroup;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  float* ub = u + static_cast<size_t>(b) * H;
  DigitGroup* db = udig + static_cast<size_t>(b) * ng;
  float* sb = usc + static_cast<size_t>(b) * ng;
  for (int g0 = 2 * wave; g0 < ng; g0 += 2 * (kPrepThreads / kWave)) {
    const int g = g0 + (lane >> 5);
    float v = 0.f;
    if (g < ng) {
      const int h = g * kGroup + (lane & 31);
      v = xb[h] + (ab ? h2f(ab[h]) : 0.f);
      if (rmsnorm) v *= r;
      ub[h] = v;
    }
    quant_pair_of_groups(v, g0, ng, db, sb);
  }
}

constexpr int kLogitWaves = 4;

// One wave per expert row; fp64 accumulation of exact fp32 x fp16 products.
__global__ __launch_bounds__(kLogitWaves* kWave) void k_route_logits(
    const float* __restrict__ u, int B, int H, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int E, double* __restrict__ z) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * kLogitWaves + wave;
  if (e >= E) return;
  const uint16_t* row = wr + static_cast<size_t>(e) * H;
  const int nc = H / 8;  // 16-byte chunks of 8 fp16
  for (int b = 0; b < B; ++b) {
    const float* ub = u + static_cast<size_t>(b) * H;
    double acc = 0.0;
    for (int c = lane; c < nc; c += kWave) {
      const uint4 wv = *reinterpret_cast<const uint4*>(row + 8 * c);
      const float4 u0 = *reinterpret_cast<const float4*>(ub + 8 * c);
      const float4 u1 = *reinterpret_cast<const float4*>(ub + 8 * c + 4);
      const uint32_t wp[4] = {wv.x, wv.y, wv.z, wv.w};
      const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double w_lo = static_cast<double>(h2f(static_cast<uint16_t>(wp[i] & 0xFFFFu)));
        const double w_hi = static_cast<double>(h2f(static_cast<uint16_t>(wp[i] >> 16)));
        acc = fma(static_cast<double>(uv[2 * i]), w_lo, acc);
        acc = fma(static_cast<double>(uv[2 * i + 1]), w_hi, acc);
      }
    }
    acc = seg_sum_f64<kWave>(acc);
    if (lane == 0) z[static_cast<size_t>(b) * E + e] = acc + (bias ? static_cast<double>(bias[e]) : 0.0);
  }
}

constexpr int kMaxPerLane = 1024 / kWave;  // E <= 1024

__device__ __forceinline__ bool key_better(double v1, int e1, double v2, int e2) {
  return v1 > v2 || (v1 == v2 && e1 < e2);
}

// One wave per token: k rounds of a wave-wide argmax on (z, -id).
__global__ __launch_bounds__(kWave) void k_route_topk(const double* __restrict__ z64,
                                                      const float* __restrict__ z32, int E, int k,
                                                      int32_t* __restrict__ ids,
                                                      float* __restrict__ w,
                                                      int32_t* __restrict__ ids2,
                                                      float* __restrict__ w2) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  double v[kMaxPerLane];
  const int per = (E + kWave - 1) / kWave;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int e = lane + kWave * j;
    double t = -DBL_MAX;
    if (j < per && e < E)
      t = z64 ? z64[static_cast<size_t>(b) * E + e]
              : static_cast<double>(z32[static_cast<size_t>(b) * E + e]);
    v[j] = t;
  }
  uint32_t taken = 0;  // bit j: candidate j of this lane already selected
  double sel_v = 0.0, v0 = 0.0;
  int sel_e = 0;
  for (int r = 0; r < k; ++r) {
    double bv = -DBL_MAX;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + kWave * j;
      if (j < per && e < E && !((taken >> j) & 1u) && key_better(v[j], e, bv, be)) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      if (key_better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    if (r == 0) v0 = bv;
    if (lane == r) {
      sel_v = bv;
      sel_e = be;
    }
  }
  // softmax over the k selected logits, max-subtracted (v0 is the largest)
  double ex = lane < k ? exp(sel_v - v0) : 0.0;
  double tot = seg_sum_f64<kWave>(ex);
  if (lane < k) {
    const float wv = static_cast<float>(ex / tot);
    ids[static_cast<size_t>(b) * k + lane] = sel_e;
    w[static_cast<size_t>(b) * k + lane] = wv;
    if (ids2) ids2[static_cast<size_t>(b) * k + lane] = sel_e;
    if (w2) w2[static_cast<size_t>(b) * k + lane] = wv;
  }
}

}  // namespace

hipError_t launch_route_prep(const float* x, const uint16_t* add_in, int B, int H, bool rmsnorm,
                             float* u, DigitGroup* udig, float* usc, hipStream_t s) {
  hipLaunchKernelGGL(k_route_prep, dim3(B), dim3(kPrepThreads), 0, s, x, add_in, H,
                     rmsnorm ? 1 : 0, u, udig, usc);
  return hipGetLastError();
}

hipError_t launch_route_logits(const float* u, int B, int H, const uint16_t* wr, const float* bias,
                               int E, double* z, hipStream_t s) {
  const int blocks = (E + kLogitWaves - 1) / kLogitWaves;
  hipLaunchKernelGGL(k_route_logits, dim3(blocks), dim3(kLogitWaves * kWave), 0, s, u, B, H, wr,
                     bias, E, z);
  return hipGetLastError();
}

hipError_t launch_route_topk(const double* z64, const float* z32, int B, int E, int k, int32_t* ids,
                             float* w, int32_t* ids2, float* w2, hipStream_t s) {
  hipLaunchKernelGGL(k_route_topk, dim3(B), dim3(kWave), 0, s, z64, z32, E, k, ids, w, ids2, w2);
  return hipGetLastError();
}

}  // namespace moe
