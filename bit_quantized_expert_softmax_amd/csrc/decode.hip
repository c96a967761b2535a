// B=1 decode FFN of one MoE layer: routed experts + shared expert.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", sections "Qual é o principal truque da
// arquitetura" (8 routed experts and a shared-expert branch per token) and
// "Sem dependências do llama.cpp e MLX" (4-bit quantisation, GEMV and MoE
// kernels). Each expert is a GeGLU FFN, o = Wd (gelu_tanh(Wg u) * (Wu u)),
// and the layer output is o_shared + sum_j w_j o_j.
//
// Work split (HBM-bound GEMVs, ~3.5 flop per weight byte):
//   gate/up kernel: every (gate row i, up row i) pair of every source is one
//     unit; a wave takes 4 pairs, 8 lanes per row, each lane streaming 16-byte
//     chunks (one quantisation group) with the activation's digit planes in
//     LDS. The GeGLU epilogue writes a[i]; the wave that completes a group of
//     32 activations quantises it to digit planes for the down projection.
//   down kernel: output n gathers the down rows of all k+1 sources as one
//     virtual row of (k*I + I_s)/32 chunks, one wave per output, the routing
//     weight folded into each group's scale; a fixed-order wave reduction
//     gives the weighted combine without atomics.
#include "launch.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kLanesPerRow = 8;
constexpr int kPairsPerWave = kWave / kLanesPerRow / 2;  // 4

__device__ __forceinline__ const uint8_t* source_base(const SourceSet& S, int j) {
  if (j >= S.k) return S.shared;
  const int e = S.ids ? S.ids[j] : S.slot.v[j];
  return S.experts + static_cast<size_t>(e) * S.blob_e;
}

__global__ __launch_bounds__(kThreads) void k_ffn_gateup(SourceSet S, int item_lo, int n_items,
                                                         const DigitGroup* __restrict__ udig,
                                                         const float* __restrict__ usc,
                                                         float* __restrict__ a,
                                                         DigitGroup* __restrict__ adig,
                                                         float* __restrict__ asc,
                                                         int32_t* __restrict__ cnt) {
  extern __shared__ uint4 lds_raw[];
  const int ngu = S.H / kGroup;
  DigitGroup* xd = reinterpret_cast<DigitGroup*>(lds_raw);
  float* xs = reinterpret_cast<float*>(xd + ngu);
  for (int i = threadIdx.x; i < ngu * 4; i += kThreads)
    reinterpret_cast<uint4*>(xd)[i] = reinterpret_cast<const uint4*>(udig)[i];
  for (int i = threadIdx.x; i < ngu; i += kThreads) xs[i] = usc[i];
  __syncthreads();

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int row = lane / kLanesPerRow;  // 0..7
  const int pair = row >> 1;
  const bool is_up = row & 1;
  const int ln = lane & (kLanesPerRow - 1);
  const int routed_items = S.k * (S.I / (2 * kPairsPerWave)) * 2;  // k * I/4
  const size_t hq = static_cast<size_t>(S.H) / 2;
  const size_t hs = static_cast<size_t>(ngu);  // scales per row

  for (int it = blockIdx.x * kWaves + wave; it < n_items; it += gridDim.x * kWaves) {
    const int item = item_lo + it;
    int src, i0, inter, aoff;
    if (item < routed_items) {
      const int per = S.I / kPairsPerWave;
      src = item / per;
      i0 = (item % per) * kPairsPerWave;
      inter = S.I;
      aoff = src * S.I;
    } else {
      src = S.k;
      i0 = (item - routed_items) * kPairsPerWave;
      inter = S.Is;
      aoff = S.k * S.I;
    }
    const BlobOffsets o = blob_offsets(S.H, inter);
    const uint8_t* base = source_base(S, src);
    const int i = i0 + pair;
    const uint8_t* q = base + (is_up ? o.up_q : o.gate_q) + static_cast<size_t>(i) * hq;
    const uint16_t* sc =
        reinterpret_cast<const uint16_t*>(base + (is_up ? o.up_s : o.gate_s)) + static_cast<size_t>(i) * hs;

    float acc = 0.f;
    constexpr int U = 4;
    for (int c0 = ln; c0 < ngu; c0 += kLanesPerRow * U) {
      uint4 wv[U];
      float sw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kLanesPerRow;
        if (c < ngu) {
          wv[u] = load_w16(q + 16 * static_cast<size_t>(c));
          sw[u] = h2f(sc[c]);
        } else {
          wv[u] = make_uint4(0, 0, 0, 0);
          sw[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kLanesPerRow;
        if (c < ngu) {
          const int t = chunk_dot(wv[u], xd[c]);
          acc = fmaf(static_cast<float>(t), sw[u] * xs[c], acc);
        }
      }
    }
    acc = seg_sum<kLanesPerRow>(acc);
    const float up = __shfl_down(acc, kLanesPerRow, kWave);
    if ((lane & (2 * kLanesPerRow - 1)) == 0) a[aoff + i] = gelu_tanh(acc) * up;

    // the wave completing a group of 32 activations quantises it
    __threadfence();
    const int grp = (aoff + i0) / kGroup;
    int old = 0;
    if (lane == 0) old = atomicAdd(&cnt[grp], 1);
    old = __shfl(old, 0, kWave);
    if (old == kGroup / kPairsPerWave - 1) {
      __threadfence();
      float v = 0.f;
      if (lane < kGroup)
        v = __hip_atomic_load(a + grp * kGroup + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      quant_pair_of_groups(v, grp, grp + 1, adig, asc);
      if (lane == 0) __hip_atomic_store(&cnt[grp], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

constexpr int kDownMaxIt = 8;  // chunks per lane: (k*I + I_s)/32 <= 512

__global__ __launch_bounds__(kThreads) void k_ffn_down(SourceSet S, const float* __restrict__ w,
                                                       const DigitGroup* __restrict__ adig,
                                                       const float* __restrict__ asc,
                                                       const float* __restrict__ x,
                                                       const uint16_t* __restrict__ add_in,
                                                       int residual, float* __restrict__ y) {
  extern __shared__ uint4 lds_raw[];
  const int gi = S.I / kGroup;
  const int gs = S.Is / kGroup;
  const int nga = S.k * gi + gs;
  DigitGroup* xd = reinterpret_cast<DigitGroup*>(lds_raw);
  float* xs = reinterpret_cast<float*>(xd + nga);
  for (int i = threadIdx.x; i < nga * 4; i += kThreads)
    reinterpret_cast<uint4*>(xd)[i] = reinterpret_cast<const uint4*>(adig)[i];
  for (int g = threadIdx.x; g < nga; g += kThreads)
    xs[g] = asc[g] * (g < S.k * gi ? w[g / gi] : 1.0f);
  __syncthreads();

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  // this lane's chunks of the virtual row: (source, chunk) resolved once
  const uint8_t* qb[kDownMaxIt];
  const uint16_t* sb[kDownMaxIt];
  size_t qstride[kDownMaxIt];
  int sstride[kDownMaxIt];
  int nit = 0;
#pragma unroll
  for (int t = 0; t < kDownMaxIt; ++t) {
    const int c = lane + kWave * t;
    qb[t] = nullptr;
    sb[t] = nullptr;
    qstride[t] = 0;
    sstride[t] = 0;
    if (c < nga) {
      int src, cc, inter;
      if (c < S.k * gi) {
        src = c / gi;
        cc = c % gi;
        inter = S.I;
      } else {
        src = S.k;
        cc = c - S.k * gi;
        inter = S.Is;
      }
      const BlobOffsets o = blob_offsets(S.H, inter);
      const uint8_t* base = source_base(S, src);
      qb[t] = base + o.down_q + 16 * static_cast<size_t>(cc);
      sb[t] = reinterpret_cast<const uint16_t*>(base + o.down_s) + cc;
      qstride[t] = static_cast<size_t>(inter) / 2;
      sstride[t] = inter / kGroup;
      nit = t + 1;
    }
  }
  for (int n = blockIdx.x * kWaves + wave; n < S.H; n += gridDim.x * kWaves) {
    uint4 wv[kDownMaxIt];
    float sw[kDownMaxIt];
#pragma unroll
    for (int t = 0; t < kDownMaxIt; ++t) {
      if (qb[t]) {
        wv[t] = load_w16(qb[t] + static_cast<size_t>(n) * qstride[t]);
        sw[t] = h2f(sb[t][static_cast<size_t>(n) * sstride[t]]);
      } else {
        wv[t] = make_uint4(0, 0, 0, 0);
        sw[t] = 0.f;
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < kDownMaxIt; ++t) {
      if (qb[t]) {
        const int c = lane + kWave * t;
        const int d = chunk_dot(wv[t], xd[c]);
        acc = fmaf(static_cast<float>(d), sw[t] * xs[c], acc);
      }
    }
    (void)nit;
    acc = seg_sum<kWave>(acc);
    if (lane == 0) {
      float r = 0.f;
      if (residual) r = x[n] + (add_in ? h2f(add_in[n]) : 0.f);
      y[n] = r + acc;
    }
  }
}

}  // namespace

hipError_t launch_ffn_gateup(const SourceSet& src, bool do_routed, bool do_shared,
                             const DigitGroup* udig, const float* usc, float* a, DigitGroup* adig,
                             float* asc, int32_t* cnt, hipStream_t s) {
  const int routed = src.k * (src.I / kPairsPerWave);
  const int shared = src.Is / kPairsPerWave;
  const int lo = do_routed ? 0 : routed;
  const int n = (do_routed ? routed : 0) + (do_shared ? shared : 0);
  if (n == 0) return hipSuccess;
  const int ngu = src.H / kGroup;
  const size_t lds = static_cast<size_t>(ngu) * (sizeof(DigitGroup) + sizeof(float));
  const int blocks = (n + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(k_ffn_gateup, dim3(blocks), dim3(kThreads), lds, s, src, lo, n, udig, usc, a,
                     adig, asc, cnt);
  return hipGetLastError();
}

hipError_t launch_ffn_down(const SourceSet& src, const float* w, const DigitGroup* adig,
                           const float* asc, const float* x, const uint16_t* add_in, bool residual,
                           float* y, hipStream_t s) {
  const int nga = src.k * (src.I / kGroup) + src.Is / kGroup;
  const size_t lds = static_cast<size_t>(nga) * (sizeof(DigitGroup) + sizeof(float));
  const int blocks = (src.H + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(k_ffn_down, dim3(blocks), dim3(kThreads), lds, s, src, w, adig, asc, x,
                     add_in, residual ? 1 : 0, y);
  return hipGetLastError();
}

}  // namespace moe
