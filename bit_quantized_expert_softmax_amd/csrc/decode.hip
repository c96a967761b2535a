// Decode FFN of one MoE layer for one token: routed experts + shared expert.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", sections "Qual é o principal truque da
// arquitetura" (8 routed experts and a shared-expert branch per token) and
// "Sem dependências do llama.cpp e MLX" (4-bit quantisation, GEMV and MoE
// kernels). Each expert is a GeGLU FFN, o = Wd (gelu_tanh(Wg u) * (Wu u)),
// and the layer output is o_shared + sum_j w_j o_j.
//
// The work is HBM-bound (~3.5 flop per weight byte) and short (tens of MB per
// token), so both kernels are shaped for latency: 1024-thread blocks (16 waves
// per CU); every lane owns one 16-byte chunk column and a few rows of it,
// loads that chunk's activation digits once into registers and issues all of
// its loads before any is consumed; per-chunk partial products are reduced in
// LDS in a fixed order; the two kernels do not synchronise across blocks.
//
// gate/up kernel: one block per group of 32 activations of one source: the 32
//   gate rows and 32 up rows (contiguous in the blob) are streamed as one
//   span; after the row sums, the GeGLU values of the group are quantised to
//   digit planes for the down projection.
// down kernel: one block per 11 outputs; an output gathers the down rows of
//   all k+1 sources as one virtual row of (k*I + I_s)/32 chunks, the routing
//   weight folded into each group's scale; the row sum is the weighted
//   combine, in a fixed order, without atomics.
#include <hip/hip_ext.h>

#include "launch.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kGroupRows = 32;  // activations per gate/up block

__device__ __forceinline__ const uint8_t* source_base(const SourceSet& S, int j) {
  if (j >= S.k) return S.shared;
  const int e = S.ids ? S.ids[j] : S.slot.v[j];
  return S.experts + static_cast<size_t>(e) * S.blob_e;
}

// Gate/up of one group of 32 (gate row i, up row i) pairs; NT tasks per lane.
// PUB: block 0 takes the token's top-k and publishes it (P), the other blocks
// shift down by one (a separate instantiation, so that the code of the
// launches without it stays as it is).
template <int NT, bool PUB>
__global__ __launch_bounds__(kThreads) void k_gateup(SourceSet S, int n_routed_blocks,
                                                     const DigitGroup* __restrict__ udig,
                                                     const float* __restrict__ usc,
                                                     DigitGroup* __restrict__ adig,
                                                     float* __restrict__ asc, FillList F, TopkPublish P) {
  extern __shared__ uint4 lds_raw[];
  __shared__ double sel_z[kMaxTopK];
  __shared__ int sel_e[kMaxTopK];
  const int ngu = S.H / kGroup;
  int bx = blockIdx.x;
  if constexpr (PUB) {
    // the token's top-k and its publication to the host, ahead of the rest
    if (bx == 0) {
      double* zs = reinterpret_cast<double*>(reinterpret_cast<float*>(lds_raw) + 2 * kGroupRows * ngu + 2);
      for (int f = threadIdx.x; f < P.E; f += kThreads) zs[f] = P.z[f];
      __syncthreads();
      topk_block(zs, P.E, P.k, sel_z, sel_e, P.ids, P.w, P.ids2, P.w2);
      if (threadIdx.x == 0) {
        // the release store orders the id stores before the sequence number
        for (int j = 0; j < P.k; ++j)
          __hip_atomic_store(P.ids_host + j, sel_e[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(P.seq_host, P.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      return;
    }
    bx -= 1;
  }
  // fill blocks first (cache mode, fill-kernel option): block f copies its
  // share of blob f / blocks_per_blob from the pinned host store to the slot,
  // while the compute blocks of the same launch run
  const int nfill = F.n * F.blocks_per_blob;
  if (bx < nfill) {
    const int m = bx / F.blocks_per_blob;
    const size_t n16 = F.bytes / 16;
    const size_t per = (n16 + F.blocks_per_blob - 1) / F.blocks_per_blob;
    const size_t lo = (bx % F.blocks_per_blob) * per;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    const uint4* __restrict__ src;
    uint4* __restrict__ dst;
    if (F.dlist) {
      // miss list from the device-side cache step: blobs past its count leave
      if (m >= F.dlist[0]) return;
      src = reinterpret_cast<const uint4*>(F.src_base + static_cast<size_t>(F.dlist[1 + m]) * F.bytes);
      dst = reinterpret_cast<uint4*>(F.dst_base + static_cast<size_t>(F.dlist[1 + F.n + m]) * F.bytes);
    } else {
      src = reinterpret_cast<const uint4*>(F.src[m]);
      dst = reinterpret_cast<uint4*>(F.dst[m]);
    }
    constexpr int U = 4;
    for (size_t i0 = lo; i0 < hi; i0 += static_cast<size_t>(kThreads) * U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = i0 + threadIdx.x + static_cast<size_t>(kThreads) * u;
        v[u] = src[i < hi ? i : hi - 1];
      }
      __builtin_amdgcn_sched_barrier(0);
      // streaming stores: the blob is read next from memory by the expert
      // kernels, so it need not stay in (and be written back from) the L2
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = i0 + threadIdx.x + static_cast<size_t>(kThreads) * u;
        if (i < hi) store_nt16(dst + i, v[u]);
      }
    }
    return;
  }
  const int bid = bx - nfill;
  __shared__ float rowsum[2 * kGroupRows];
  float* part = reinterpret_cast<float*>(lds_raw);                          // [64][ngu]
  double* zs = reinterpret_cast<double*>(part + 2 * kGroupRows * ngu + 2);  // [E]

  // blocks [0, n_routed_blocks): groups of the routed ranks (all k, or the
  // selected ones); the rest: groups of the shared expert
  const int gpr = S.I / kGroupRows;
  const int routed_groups = S.k * gpr;
  int grp;  // group of 32 activations in [0, (k*I + I_s)/32)
  if (bid < n_routed_blocks) {
    const int ls = bid / gpr;
    grp = (S.nsel > 0 ? S.rsel.v[ls] : ls) * gpr + bid % gpr;
  } else {
    grp = routed_groups + (bid - n_routed_blocks);
  }
  int src, i0, inter;
  if (grp < routed_groups) {
    src = grp / (S.I / kGroupRows);
    i0 = (grp % (S.I / kGroupRows)) * kGroupRows;
    inter = S.I;
  } else {
    src = S.k;
    i0 = (grp - routed_groups) * kGroupRows;
    inter = S.Is;
  }
  // in-kernel routing (resident mode): a routed block derives the token's top-k
  // from the logits; the first block publishes ids and weights for the down kernel
  const uint8_t* base;
  if (src < S.k && S.z) {
    for (int f = threadIdx.x; f < S.E; f += kThreads) zs[f] = S.z[f];
    __syncthreads();
    const bool first = grp == 0;
    topk_block(zs, S.E, S.k, sel_z, sel_e, first ? S.ids_g : nullptr, first ? S.w_g : nullptr,
               first ? S.ids2 : nullptr, first ? S.w2 : nullptr);
    base = S.experts + static_cast<size_t>(sel_e[src]) * S.blob_e;
  } else {
    base = source_base(S, src);
  }
  const BlobOffsets o = blob_offsets(S.H, inter);
  const size_t rowb = static_cast<size_t>(S.H) / 2;
  // Lane (r0, c) = (threadIdx / ngu, threadIdx % ngu) owns chunk column c of
  // rows r0, r0 + R, ... (R = kThreads / ngu; rows 0..31 gate, 32..63 up).
  // It loads that chunk's activation digits once into registers, next to its
  // weights, so no staging pass and no per-chunk LDS reads are needed;
  // consecutive lanes read consecutive 16-byte chunks of a row.
  const int R = kThreads / ngu;
  const int c = threadIdx.x % ngu;
  const int r0 = threadIdx.x / ngu;
  const uint8_t* gq = base + o.gate_q + static_cast<size_t>(i0) * rowb + 16 * static_cast<size_t>(c);
  const uint8_t* uq = base + o.up_q + static_cast<size_t>(i0) * rowb + 16 * static_cast<size_t>(c);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(base + o.gate_s) + static_cast<size_t>(i0) * ngu + c;
  const uint16_t* us = reinterpret_cast<const uint16_t*>(base + o.up_s) + static_cast<size_t>(i0) * ngu + c;
  // the activation digits first: loads retire in order, so chunk t can be
  // consumed as soon as its own bytes are in while later chunks still stream
  const DigitGroup xd = udig[c];
  const float xs = usc[c];
  uint4 wv[NT];
  uint16_t sw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int r = r0 + R * t;
    r = r < 2 * kGroupRows ? r : 2 * kGroupRows - 1;  // clamped: loaded, not stored
    const bool up = r >= kGroupRows;
    const int rr = up ? r - kGroupRows : r;
    wv[t] = load_w16((up ? uq : gq) + static_cast<size_t>(rr) * rowb);
    sw[t] = (up ? us : gs)[static_cast<size_t>(rr) * ngu];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = r0 + R * t;
    const float p = static_cast<float>(chunk_dot(wv[t], xd)) * (h2f(sw[t]) * xs);
    if (r < 2 * kGroupRows) part[r * ngu + c] = p;
  }
  __syncthreads();
  // 64 row sums: 16 lanes per row, 4 rows per wave, fixed order
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  {
    const int r = 4 * wave + (lane >> 4);
    const int l = lane & 15;
    float acc = 0.f;
    for (int c = l; c < ngu; c += 16) acc += part[r * ngu + c];
    acc = dpp_sum<16>(acc);
    if (l == 0) rowsum[r] = acc;
  }
  __syncthreads();
  if (wave == 0) {
    // GeGLU of the 32 activations of this group, then their digit planes
    float a = 0.f;
    if (lane < kGroupRows) a = gelu_tanh(rowsum[lane]) * rowsum[kGroupRows + lane];
    quant_pair_of_groups(a, grp, grp + 1, adig, asc);
  }
}

constexpr int kOutPerBlock = 11;

// Down projections of kOutPerBlock outputs of all k+1 sources and the combine.
template <int NT>
__global__ __launch_bounds__(kThreads) void k_down(SourceSet S, const float* __restrict__ w,
                                                   const DigitGroup* __restrict__ adig,
                                                   const float* __restrict__ asc,
                                                   const float* __restrict__ x,
                                                   const uint16_t* __restrict__ add_in,
                                                   int residual, float* __restrict__ y) {
  extern __shared__ uint4 lds_raw[];
  const int gi = S.I / kGroup;
  const int gsh = S.Is / kGroup;
  const int nga = S.k * gi + gsh;  // chunks of the virtual row
  float* part = reinterpret_cast<float*>(lds_raw);  // [kOutPerBlock][nga]
  const int n0 = blockIdx.x * kOutPerBlock;
  const int nout = S.H - n0 < kOutPerBlock ? S.H - n0 : kOutPerBlock;
  // Lane (o0, c) = (threadIdx / nga, threadIdx % nga) owns chunk c of the
  // virtual row for outputs o0, o0 + R, ... (R = kThreads / nga); it loads
  // that chunk's activation digits once, with the routing weight of the
  // chunk's source folded into the scale. Each lane finds its source's
  // address itself, so no barrier and no routing-weight load stands before
  // the weight loads (the weight only scales the sum).
  const int R = kThreads / nga;
  const int c = threadIdx.x % nga;
  const int o0 = threadIdx.x / nga;
  const bool on = o0 < R;
  int j, cc, inter;
  if (c < S.k * gi) {
    j = c / gi;
    cc = c - j * gi;
    inter = S.I;
  } else {
    j = S.k;
    cc = c - S.k * gi;
    inter = S.Is;
  }
  const BlobOffsets o = blob_offsets(S.H, inter);
  const uint8_t* srcj = source_base(S, j);
  const uint8_t* qb = srcj + o.down_q + 16 * static_cast<size_t>(cc);
  const uint16_t* sb = reinterpret_cast<const uint16_t*>(srcj + o.down_s) + cc;
  const DigitGroup xd = adig[c];  // first, as in the gate/up kernel
  const float xsa = asc[c];
  const float wj = j < S.k ? w[j] : 1.0f;
  uint4 wv[NT];
  uint16_t sw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int ob = o0 + R * t;
    ob = ob < nout ? ob : nout - 1;  // clamped: loaded, not stored
    const size_t n = static_cast<size_t>(n0 + ob);
    wv[t] = load_w16(qb + n * (inter / 2));
    sw[t] = sb[n * (inter / kGroup)];
  }
  __builtin_amdgcn_sched_barrier(0);
  const float xs = xsa * wj;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int ob = o0 + R * t;
    const float p = static_cast<float>(chunk_dot(wv[t], xd)) * (h2f(sw[t]) * xs);
    if (on && ob < nout) part[ob * nga + c] = p;
  }
  __syncthreads();
  // one wave per output: fixed-order sum of its nga partials
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (wave < nout) {
    float acc = 0.f;
    for (int c = lane; c < nga; c += kWave) acc += part[wave * nga + c];
    // row sums by DPP, then the four rows through scalar reads (lane 0 writes)
    acc = dpp_sum<16>(acc);
    acc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 16)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 48));
    if (lane == 0) {
      const int n = n0 + wave;
      float r = 0.f;
      if (residual) r = x[n] + (add_in ? h2f(add_in[n]) : 0.f);
      y[n] = r + acc;
    }
  }
}

}  // namespace

size_t decode_lds_bytes(int H, int E, int k, int I, int Is) {
  const size_t ngu = H / kGroup, nga = (static_cast<size_t>(k) * I + Is) / kGroup;
  const size_t gu = (2 * kGroupRows * ngu + 2) * 4 + sizeof(double) * E;
  const size_t dn = static_cast<size_t>(kOutPerBlock) * nga * 4;
  return gu > dn ? gu : dn;
}

hipError_t launch_ffn_gateup(const SourceSet& src, bool do_routed, bool do_shared,
                             const DigitGroup* udig, const float* usc, DigitGroup* adig, float* asc,
                             hipStream_t s, hipEvent_t t0, hipEvent_t t1, const FillList* fill,
                             const TopkPublish* topk) {
  FillList F{};
  if (fill && fill->n > 0) {
    if (fill->n > kMaxTopK || fill->blocks_per_blob < 1 || fill->bytes % 16) return hipErrorInvalidValue;
    F = *fill;
  }
  TopkPublish P{};
  if (topk) {
    if (!topk->z || !topk->ids || !topk->w || !topk->ids_host || !topk->seq_host || topk->k < 1 ||
        topk->k > kMaxTopK || topk->k > topk->E)
      return hipErrorInvalidValue;
    P = *topk;
  }
  const int nr = do_routed ? (src.nsel > 0 ? src.nsel : src.k) * (src.I / kGroupRows) : 0;
  const int shared = src.Is / kGroupRows;
  const int n = (topk ? 1 : 0) + F.n * F.blocks_per_blob + nr + (do_shared ? shared : 0);
  if (n == 0) return hipSuccess;
  const int ngu = src.H / kGroup;
  const int Ez = src.z ? src.E : (topk ? topk->E : 0);
  const size_t lds = static_cast<size_t>(2 * kGroupRows * ngu + 2) * 4 + sizeof(double) * Ez;
  if (ngu > kThreads) return hipErrorInvalidValue;
  const int rows_per_pass = kThreads / ngu;
  const int need = (2 * kGroupRows + rows_per_pass - 1) / rows_per_pass;
#define MOE_GATEUP_PUB(NT, PUB)                                                                          \
  do {                                                                                                   \
    if (t0) hipExtLaunchKernelGGL((k_gateup<NT, PUB>), dim3(n), dim3(kThreads), lds, s, t0, t1, 0, src, nr, udig, usc, adig, asc, F, P); \
    else hipLaunchKernelGGL((k_gateup<NT, PUB>), dim3(n), dim3(kThreads), lds, s, src, nr, udig, usc, adig, asc, F, P);               \
  } while (0)
#define MOE_GATEUP(NT)                        \
  do {                                        \
    if (topk) MOE_GATEUP_PUB(NT, true);       \
    else MOE_GATEUP_PUB(NT, false);           \
  } while (0)
  if (need <= 1) MOE_GATEUP(1);
  else if (need <= 2) MOE_GATEUP(2);
  else if (need <= 4) MOE_GATEUP(4);
  else if (need <= 6) MOE_GATEUP(6);
  else if (need <= 8) MOE_GATEUP(8);
  else if (need <= 12) MOE_GATEUP(12);
  else if (need <= 16) MOE_GATEUP(16);
  else return hipErrorInvalidValue;  // H beyond what the LDS budget admits
#undef MOE_GATEUP
#undef MOE_GATEUP_PUB
  return hipGetLastError();
}

hipError_t launch_ffn_down(const SourceSet& src, const float* w, const DigitGroup* adig, const float* asc,
                           const float* x, const uint16_t* add_in, bool residual, float* y,
                           hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const int nga = src.k * (src.I / kGroup) + src.Is / kGroup;
  const size_t lds = static_cast<size_t>(kOutPerBlock) * nga * 4;
  if (nga > kThreads) return hipErrorInvalidValue;
  const int blocks = (src.H + kOutPerBlock - 1) / kOutPerBlock;
  const int outs_per_pass = kThreads / nga;
  const int need = (kOutPerBlock + outs_per_pass - 1) / outs_per_pass;
#define MOE_DOWN(NT)                                                                                     \
  do {                                                                                                   \
    if (t0) hipExtLaunchKernelGGL(k_down<NT>, dim3(blocks), dim3(kThreads), lds, s, t0, t1, 0, src, w, adig, asc, x, add_in, residual ? 1 : 0, y); \
    else hipLaunchKernelGGL(k_down<NT>, dim3(blocks), dim3(kThreads), lds, s, src, w, adig, asc, x, add_in, residual ? 1 : 0, y);               \
  } while (0)
  if (need <= 1) MOE_DOWN(1);
  else if (need <= 2) MOE_DOWN(2);
  else if (need <= 3) MOE_DOWN(3);
  else if (need <= 4) MOE_DOWN(4);
  else if (need <= 6) MOE_DOWN(6);
  else if (need <= 12) MOE_DOWN(12);
  else return hipErrorInvalidValue;
#undef MOE_DOWN
  return hipGetLastError();
}

}  // namespace moe
