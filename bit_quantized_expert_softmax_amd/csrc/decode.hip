// Decode FFN of one MoE layer for one token: routed experts + shared expert.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", sections "Qual é o principal truque da
// arquitetura" (8 routed experts and a shared-expert branch per token) and
// "Sem dependências do llama.cpp e MLX" (4-bit quantisation, GEMV and MoE
// kernels). Each expert is a GeGLU FFN, o = Wd (gelu_tanh(Wg u) * (Wu u)),
// and the layer output is o_shared + sum_j w_j o_j.
//
// The work is HBM-bound (~3.5 flop per weight byte), so both kernels are
// shaped for streaming: every lane keeps all of its 16-byte weight loads in
// flight before consuming any, and nothing waits on another block.
//
// gate/up kernel: a wave owns 8 (gate row i, up row i) pairs of one source,
//   4 lanes per row. The GeGLU epilogue produces 8 consecutive activations,
//   which the same wave quantises to one digit word per digit (a "position"
//   of 8 values with its own scale), so the down projection can run on the
//   dot8 path with no cross-block reduction or synchronisation.
// down kernel: output n gathers the down rows of all k+1 sources as one
//   virtual row of (k*I + I_s)/32 chunks, half a wave (32 lanes) per output;
//   the routing weight is folded into each position's scale and a fixed-order
//   lane reduction gives the weighted combine without atomics.
#include "launch.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kLanesPerRow = 8;                     // one row pair per 8 lanes
constexpr int kPairsPerItem = kWave / kLanesPerRow;  // 8

__device__ __forceinline__ const uint8_t* source_base(const SourceSet& S, int j) {
  if (j >= S.k) return S.shared;
  const int e = S.ids ? S.ids[j] : S.slot.v[j];
  return S.experts + static_cast<size_t>(e) * S.blob_e;
}

// Copies n16 uint4 and nf floats from global memory to LDS with every load of
// a thread issued before its first store (the trip counts are small).
__device__ __forceinline__ void stage_to_lds(const uint4* __restrict__ g16, uint4* l16, int n16,
                                             const float* __restrict__ gf, float* lf, int nf) {
  constexpr int U = 8;
  for (int i0 = 0; i0 < n16; i0 += kThreads * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int i = i0 + threadIdx.x + kThreads * u;
      v[u] = g16[i < n16 ? i : n16 - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    // unconditional stores (clamped index) keep the loads ahead of the first
    // wait; lanes past the end rewrite the last element with its own value
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + threadIdx.x + kThreads * u;
      l16[i < n16 ? i : n16 - 1] = v[u];
    }
  }
  for (int i0 = 0; i0 < nf; i0 += kThreads * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int i = i0 + threadIdx.x + kThreads * u;
      v[u] = gf[i < nf ? i : nf - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + threadIdx.x + kThreads * u;
      lf[i < nf ? i : nf - 1] = v[u];
    }
  }
}

// Quantises one value per 8-lane segment head (lanes 0, 8, ..., 56) as one
// "position" of 8 activations and writes its 4 digit words and scale.
__device__ __forceinline__ void quant_position(float a, uint4* dst, float* dsc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int p = lane >> 3;  // position slot of this segment
  float m = (lane & 7) == 0 ? fabsf(a) : 0.f;
  m = fmaxf(m, __shfl_xor(m, 8, kWave));
  m = fmaxf(m, __shfl_xor(m, 16, kWave));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  const float inv = m > 0.f ? static_cast<float>(kQmax) / m : 0.f;
  int q = static_cast<int>(rintf(a * inv));
  q = q > kQmax ? kQmax : (q < -kQmax ? -kQmax : q);
  const int d0 = ((q + 8) & 15) - 8;
  q = (q - d0) / 16;
  const int d1 = ((q + 8) & 15) - 8;
  q = (q - d1) / 16;
  const int d2 = ((q + 8) & 15) - 8;
  const int d3 = (q - d2) / 16;
  const bool head = (lane & 7) == 0;
  uint32_t w0 = head ? static_cast<uint32_t>(d0 & 15) << (4 * p) : 0u;
  uint32_t w1 = head ? static_cast<uint32_t>(d1 & 15) << (4 * p) : 0u;
  uint32_t w2 = head ? static_cast<uint32_t>(d2 & 15) << (4 * p) : 0u;
  uint32_t w3 = head ? static_cast<uint32_t>(d3 & 15) << (4 * p) : 0u;
#pragma unroll
  for (int o = 8; o < kWave; o <<= 1) {
    w0 |= __shfl_xor(w0, o, kWave);
    w1 |= __shfl_xor(w1, o, kWave);
    w2 |= __shfl_xor(w2, o, kWave);
    w3 |= __shfl_xor(w3, o, kWave);
  }
  if (lane == 0 && dst) {
    *dst = make_uint4(w0, w1, w2, w3);
    *dsc = m / static_cast<float>(kQmax);
  }
}

template <int NT>
__global__ __launch_bounds__(kThreads) void k_gateup(SourceSet S, int item_lo, int n_items,
                                                     const DigitGroup* __restrict__ udig,
                                                     const float* __restrict__ usc,
                                                     uint4* __restrict__ adig,
                                                     float* __restrict__ asc) {
  extern __shared__ uint4 lds_raw[];
  __shared__ double sel_z[kMaxTopK];
  __shared__ int sel_e[kMaxTopK];
  const int ngu = S.H / kGroup;
  DigitGroup* xd = reinterpret_cast<DigitGroup*>(lds_raw);
  float* xs = reinterpret_cast<float*>(xd + ngu);
  double* zs = reinterpret_cast<double*>(lds_raw + ngu * 4 + (ngu + 3) / 4);

  // in-kernel routing: every block derives the token's top-k from the logits
  if (S.z) {
    for (int f = threadIdx.x; f < S.E; f += kThreads) zs[f] = S.z[f];
    __syncthreads();
    const bool first = blockIdx.x == 0;
    topk_block(zs, S.E, S.k, sel_z, sel_e, first ? S.ids_g : nullptr, first ? S.w_g : nullptr,
               first ? S.ids2 : nullptr, first ? S.w2 : nullptr);
  }

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int pair = lane / kLanesPerRow;  // 0..7: gate row i and up row i
  const int ln = lane & (kLanesPerRow - 1);
  const int per_routed = S.I / kPairsPerItem;
  const int routed_items = S.k * per_routed;
  const size_t hq = static_cast<size_t>(S.H) / 2;
  const int stride = gridDim.x * kWaves;
  bool staged = false;

  // every wave runs the same number of item rounds so that the block-wide
  // staging barrier below is reached by all of them
  const int rounds = (n_items + stride - 1) / stride;
  for (int rd = 0; rd < rounds; ++rd) {
    const int it_raw = blockIdx.x * kWaves + wave + rd * stride;
    const bool live = it_raw < n_items;
    const int item = item_lo + (live ? it_raw : n_items - 1);
    int src, i0, inter, aoff;
    if (item < routed_items) {
      src = item / per_routed;
      i0 = (item % per_routed) * kPairsPerItem;
      inter = S.I;
      aoff = src * S.I;
    } else {
      src = S.k;
      i0 = (item - routed_items) * kPairsPerItem;
      inter = S.Is;
      aoff = S.k * S.I;
    }
    const BlobOffsets o = blob_offsets(S.H, inter);
    const uint8_t* base;
    if (src >= S.k) base = S.shared;
    else if (S.z) base = S.experts + static_cast<size_t>(sel_e[src]) * S.blob_e;
    else base = source_base(S, src);
    const int i = i0 + pair;
    const uint8_t* qg = base + o.gate_q + static_cast<size_t>(i) * hq;
    const uint8_t* qu = base + o.up_q + static_cast<size_t>(i) * hq;
    const uint16_t* sg = reinterpret_cast<const uint16_t*>(base + o.gate_s) + static_cast<size_t>(i) * ngu;
    const uint16_t* su = reinterpret_cast<const uint16_t*>(base + o.up_s) + static_cast<size_t>(i) * ngu;

    float acc_g = 0.f, acc_u = 0.f;
    for (int c0 = 0; c0 < ngu; c0 += kLanesPerRow * NT) {
      // all loads of the batch are issued before any is consumed; chunks past
      // the row end re-read its last chunk and are masked out. A wave
      // instruction covers 8 rows x 128 contiguous bytes.
      uint4 wg[NT], wu[NT];
      uint16_t fg[NT], fu[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        int c = c0 + ln + kLanesPerRow * t;
        c = c < ngu ? c : ngu - 1;
        wg[t] = load_w16(qg + 16 * static_cast<size_t>(c));
        wu[t] = load_w16(qu + 16 * static_cast<size_t>(c));
        fg[t] = sg[c];
        fu[t] = su[c];
      }
      // the activation digits are staged while the weight loads are in flight
      if (!staged) {
        stage_to_lds(reinterpret_cast<const uint4*>(udig), reinterpret_cast<uint4*>(xd), ngu * 4, usc,
                     xs, ngu);
        __syncthreads();
        staged = true;
      }
      // keep every load of the batch ahead of the first use
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int c = c0 + ln + kLanesPerRow * t;
        const int cc = c < ngu ? c : ngu - 1;
        const DigitGroup xv = xd[cc];
        const float m = xs[cc] * static_cast<float>(c < ngu);
        acc_g = fmaf(static_cast<float>(chunk_dot(wg[t], xv)), h2f(fg[t]) * m, acc_g);
        acc_u = fmaf(static_cast<float>(chunk_dot(wu[t], xv)), h2f(fu[t]) * m, acc_u);
      }
    }
    acc_g = seg_sum<kLanesPerRow>(acc_g);
    acc_u = seg_sum<kLanesPerRow>(acc_u);
    const float a = gelu_tanh(acc_g) * acc_u;  // same on all 8 lanes of a pair
    const int pos = (aoff + i0) / kPairsPerItem;
    quant_position(a, live ? adig + pos : nullptr, live ? asc + pos : nullptr);
  }
}

constexpr int kOutLanes = 32;                   // lanes per output row
constexpr int kOutPerWave = kWave / kOutLanes;  // 2

template <int NT>
__global__ __launch_bounds__(kThreads) void k_down(SourceSet S, const float* __restrict__ w,
                                                   const uint4* __restrict__ adig,
                                                   const float* __restrict__ asc,
                                                   const float* __restrict__ x,
                                                   const uint16_t* __restrict__ add_in,
                                                   int residual, float* __restrict__ y) {
  extern __shared__ uint4 lds_raw[];
  __shared__ float wsh[kMaxTopK + 1];
  const int gi = S.I / kGroup;
  const int gs = S.Is / kGroup;
  const int nga = S.k * gi + gs;  // chunks of the virtual row
  const int npos = nga * 4;       // positions of 8 activations
  uint4* xd = lds_raw;
  float* xs = reinterpret_cast<float*>(xd + npos);

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int half = lane / kOutLanes;
  const int l = lane & (kOutLanes - 1);
  // this lane's chunks of the virtual row, resolved once; chunks past the end
  // alias the last one and are masked out
  const uint8_t* qb[NT];
  const uint16_t* sb[NT];
  int qstride[NT], sstride[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int c = l + kOutLanes * t;
    c = c < nga ? c : nga - 1;
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
    qstride[t] = inter / 2;
    sstride[t] = inter / kGroup;
  }
  const int stride = gridDim.x * kWaves * kOutPerWave;
  const int rounds = (S.H + stride - 1) / stride;
  for (int rd = 0; rd < rounds; ++rd) {
    const int n_raw = (blockIdx.x * kWaves + wave) * kOutPerWave + rd * stride + half;
    const int n = n_raw < S.H ? n_raw : S.H - 1;
    uint4 wv[NT];
    uint16_t sw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      wv[t] = load_w16(qb[t] + static_cast<size_t>(n) * qstride[t]);
      sw[t] = sb[t][static_cast<size_t>(n) * sstride[t]];
    }
    if (rd == 0) {
      // activations and routing weights are staged while the weights stream in
      if (threadIdx.x <= static_cast<unsigned>(S.k))
        wsh[threadIdx.x] = threadIdx.x < static_cast<unsigned>(S.k) ? w[threadIdx.x] : 1.0f;
      stage_to_lds(adig, xd, npos, asc, xs, npos);
      __syncthreads();
      // fold the routing weight of each source into its positions' scales
      for (int i = threadIdx.x; i < npos; i += kThreads) {
        const int g = i / 4;
        xs[i] *= wsh[g < S.k * gi ? g / gi : S.k];
      }
      __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = l + kOutLanes * t;
      const int cc = c < nga ? c : nga - 1;
      const uint32_t wq[4] = {wv[t].x, wv[t].y, wv[t].z, wv[t].w};
      float part = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 xv = xd[4 * cc + p];
        const int d0 = sdot8(wq[p], xv.x, 0);
        const int d1 = sdot8(wq[p], xv.y, 0);
        const int d2 = sdot8(wq[p], xv.z, 0);
        const int d3 = sdot8(wq[p], xv.w, 0);
        const int tq = d0 + 16 * d1 + 256 * d2 + 4096 * d3;
        part = fmaf(static_cast<float>(tq), xs[4 * cc + p], part);
      }
      acc = fmaf(part, h2f(sw[t]) * static_cast<float>(c < nga), acc);
    }
    acc = seg_sum<kOutLanes>(acc);
    if (l == 0 && n_raw < S.H) {
      float r = 0.f;
      if (residual) r = x[n] + (add_in ? h2f(add_in[n]) : 0.f);
      y[n] = r + acc;
    }
  }
}

}  // namespace

hipError_t launch_ffn_gateup(const SourceSet& src, bool do_routed, bool do_shared,
                             const DigitGroup* udig, const float* usc, uint4* adig, float* asc,
                             hipStream_t s) {
  const int routed = src.k * (src.I / kPairsPerItem);
  const int shared = src.Is / kPairsPerItem;
  const int lo = do_routed ? 0 : routed;
  const int n = (do_routed ? routed : 0) + (do_shared ? shared : 0);
  if (n == 0) return hipSuccess;
  const int ngu = src.H / kGroup;
  // digit groups, their scales (padded to 16 bytes) and the logits for in-kernel top-k
  const size_t lds = static_cast<size_t>(ngu) * sizeof(DigitGroup) + ((ngu + 3) / 4) * 16 +
                     (src.z ? sizeof(double) * src.E : 0);
  const int blocks = (n + kWaves - 1) / kWaves;
  const int need = (ngu + kLanesPerRow - 1) / kLanesPerRow;  // chunks per lane and row
#define MOE_GATEUP(NT) hipLaunchKernelGGL(k_gateup<NT>, dim3(blocks), dim3(kThreads), lds, s, src, lo, n, udig, usc, adig, asc)
  if (need <= 2) MOE_GATEUP(2);
  else if (need <= 4) MOE_GATEUP(4);
  else if (need <= 6) MOE_GATEUP(6);
  else if (need <= 8) MOE_GATEUP(8);
  else if (need <= 11) MOE_GATEUP(11);
  else if (need <= 12) MOE_GATEUP(12);
  else MOE_GATEUP(16);
#undef MOE_GATEUP
  return hipGetLastError();
}

hipError_t launch_ffn_down(const SourceSet& src, const float* w, const uint4* adig, const float* asc,
                           const float* x, const uint16_t* add_in, bool residual, float* y,
                           hipStream_t s) {
  const int nga = src.k * (src.I / kGroup) + src.Is / kGroup;
  const size_t lds = static_cast<size_t>(nga) * 4 * (sizeof(uint4) + sizeof(float));
  const int per_block = kWaves * kOutPerWave;
  const int blocks = (src.H + per_block - 1) / per_block;
  const int need = (nga + kOutLanes - 1) / kOutLanes;
#define MOE_DOWN(NT) hipLaunchKernelGGL(k_down<NT>, dim3(blocks), dim3(kThreads), lds, s, src, w, adig, asc, x, add_in, residual ? 1 : 0, y)
  if (need <= 2) MOE_DOWN(2);
  else if (need <= 4) MOE_DOWN(4);
  else if (need <= 8) MOE_DOWN(8);
  else MOE_DOWN(16);
#undef MOE_DOWN
  return hipGetLastError();
}

}  // namespace moe
