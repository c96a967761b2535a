// Router of one MoE layer: input preparation, fp64 logits, top-k + softmax.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", section "Qual é o principal truque da
// arquitetura": the router of every layer picks the 8 experts the current
// token needs. Selection is on the logits (softmax is monotone), ties go to
// the lower expert id, the weights are a softmax over the selected logits.
//
// Layer path (k_route_fused): one launch per call. Every block recomputes the
// (cheap) RMSNorm of the token; the logit blocks compute the logits of 2
// experts each (one per wave) in fp64, and blocks of their own after them
// quantise the normalised input to digit planes for the expert GEMVs. Where
// the launch also takes the top-k, the logits are written with agent-scope
// (L2-bypassing) stores; after its stores have completed each block bumps its
// token's counter, and the block that arrives last takes that token's top-k.
// No block waits for another and no cache writeback is needed. Otherwise (one
// token) the logits cross the kernel boundary and the top-k runs in a later
// launch: in every routed gate/up block (resident), in the first block of the
// shared-expert launch (cache mode, copy engine) or in a one-block selection
// launch (cache mode with fill blocks or a device-stepped cache). The batched
// router (k_route_tok) is described below.
#include <float.h>
#include <math.h>

#include "launch.h"
#include "moedecode.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kThreads = 128;  // 2 waves (2 experts) per block: 64 blocks at E = 128
constexpr int kWaves = kThreads / kWave;

struct RouteArgs {
  const float* x;
  const uint16_t* add_in;
  int B, H, rmsnorm;
  const uint16_t* wr;
  const float* bias;
  int E, k;
  float* u_out;       // optional [B][H]
  DigitGroup* udig;   // optional [B][H/32] digit planes of u
  float* usc;         // [B][H/32]
  uint16_t* u16;      // optional [B][H] fp16 of u / tsc, each 8-block in the
                      // order (0,4,1,5,2,6,3,7) of the matrix-core kernels
  float* tsc;         // [B] power of two with ||u||_2 / tsc < 16
  double* z;          // [B][E]
  int32_t* cnt;       // arrival counter, zero between calls
  int32_t *ids, *ids2;
  float *w, *w2;
  // optional (selection launch, one token): the ids also go to host-coherent
  // memory, then seq_host is set to seq with a system-scope release store
  int32_t* ids_host;
  int32_t* seq_host;
  int32_t seq;
  // optional (selection launch, one token): the layer's expert-slot cache is
  // stepped right after the top-k
  DevCache dc;
  int use_dc;
};

// Per wave: one expert's router row and the whole token input x' are loaded
// in a single batch (8 consecutive inputs per lane and step); the wave
// derives the RMSNorm factor from the same registers, so no block reduction
// and no second pass over x' is needed. A lane's 8 inputs are exactly one
// "position" of a quantisation group, so a wave that owns a group writes its
// digit planes straight from registers.
constexpr int kMaxSteps = 8;  // H <= 8 * 64 * 8 = 4096 in one batch

// One step of the layer's expert-slot cache for the token's ids (sel_e, rank
// order), by the whole block, on an LDS copy of the state: hits first (in
// parallel, the ids are distinct), then the misses in rank order, each
// taking the victim a wave finds by a (key, slot) minimum: empty slots key
// on their index alone, so the lowest empty slot wins; the others (those
// holding none of the token's ids) key on (frequency, last use) for LFU or
// last use for LRU, ties to the lower slot. The same rule as the host cache.
__device__ void dcache_step(const DevCache& C, const int* sel_e, int k, int E, int32_t* lds) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int S = C.n_slots;
  int32_t* lexp = lds;           // [S]
  int32_t* lfreq = lexp + S;     // [S]
  int32_t* llast = lfreq + S;    // [S]
  int32_t* lwhere = llast + S;   // [E]
  int32_t* lseen = lwhere + E;   // [E]
  __shared__ int32_t hit[kMaxTopK], nm_sh, victim_sh;
  const int nt = blockDim.x;
  for (int i = tid; i < S; i += nt) {
    lexp[i] = C.expert[i];
    lfreq[i] = C.freq[i];
    llast[i] = C.last[i];
  }
  for (int e = tid; e < E; e += nt) {
    lwhere[e] = C.where[e];
    lseen[e] = 0;
  }
  const int32_t tick = static_cast<int32_t>(C.counters[0]);
  __syncthreads();
  if (tid < k) {
    const int e = sel_e[tid];
    lseen[e] = 1;
    const int sl = lwhere[e];
    hit[tid] = sl >= 0;
    if (sl >= 0) {
      lfreq[sl] += 1;
      llast[sl] = tick;
      C.slot_of_rank[tid] = sl;
      int32_t* ev = C.ev + 4 * tid;
      ev[0] = e;
      ev[1] = sl;
      ev[2] = 1;
      ev[3] = -1;
    }
  }
  if (tid == 0) nm_sh = 0;
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    if (hit[j]) continue;  // uniform: every thread reads the same LDS word
    if (tid < kWave) {
      unsigned long long best = ~0ull;
      int bs = S;
      for (int sl = lane; sl < S; sl += kWave) {
        const int ex = lexp[sl];
        unsigned long long key;
        if (ex < 0) key = static_cast<unsigned long long>(sl);
        else if (lseen[ex]) key = ~0ull;
        else if (C.policy == MOE_POLICY_LRU) key = (1ull << 62) | static_cast<unsigned int>(llast[sl] + 1);
        else
          key = (1ull << 62) | (static_cast<unsigned long long>(lfreq[sl]) << 31) |
                static_cast<unsigned int>(llast[sl] + 1);
        if (key < best) {  // slots in increasing order: the first minimum stays
          best = key;
          bs = sl;
        }
      }
#pragma unroll
      for (int o = kWave / 2; o >= 1; o >>= 1) {
        const unsigned long long ob = static_cast<unsigned long long>(
            __shfl_xor(static_cast<long long>(best), o, kWave));
        const int os = __shfl_xor(bs, o, kWave);
        if (ob < best || (ob == best && os < bs)) {
          best = ob;
          bs = os;
        }
      }
      // a victim always exists (n_slots >= k, and fewer than k slots hold the
      // token's ids while a miss is placed); the clamp only keeps every index
      // inside the pool whatever the state
      bs = bs < S ? bs : S - 1;
      if (lane == 0) {
        const int e = sel_e[j];
        const int old = lexp[bs];
        if (old >= 0) lwhere[old] = -1;
        lexp[bs] = e;
        lfreq[bs] = 1;
        llast[bs] = tick;
        lwhere[e] = bs;
        C.slot_of_rank[j] = bs;
        int32_t* ev = C.ev + 4 * j;
        ev[0] = e;
        ev[1] = bs;
        ev[2] = 0;
        ev[3] = old;
        const int m = nm_sh;
        C.miss[1 + m] = e;
        C.miss[1 + k + m] = bs;
        nm_sh = m + 1;
      }
    }
    __syncthreads();
  }
  for (int i = tid; i < S; i += nt) {
    C.expert[i] = lexp[i];
    C.freq[i] = lfreq[i];
    C.last[i] = llast[i];
  }
  for (int e = tid; e < E; e += nt) C.where[e] = lwhere[e];
  if (tid == 0) {
    const int nm = nm_sh;
    C.miss[0] = nm;
    C.counters[0] += 1;
    C.counters[1] += k - nm;
    C.counters[2] += nm;
  }
}

// Top-k variant, after the block's logit stores (agent scope): the block
// bumps its token's counter; the last of the token's gridDim.x blocks takes
// the token's top-k. All threads call.
__device__ void route_tail(const RouteArgs& A, double* zs, double* sel_z, int* sel_e, int* is_last_p) {
  int& is_last = *is_last_p;
  const int nb = gridDim.x;
  // Every logit store of this block has completed before the block arrives:
  // the stores are agent-scope atomics (written through to the device-coherent
  // level, not held in this XCD's L2), s_waitcnt(0) waits for their
  // completion, and the last block reads the logits with agent-scope atomic
  // loads. A release/acquire arrival would add an L2 write-back (buffer_wbl2)
  // per block for data that is already coherent: measured 15.1 -> 23.6 us for
  // the batched router at B = 64 (512 blocks), so the arrival stays relaxed.
  const int tok = blockIdx.y;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(A.cnt + tok, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = old == nb - 1;
    if (is_last) __hip_atomic_store(A.cnt + tok, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!is_last) return;
  for (int f = threadIdx.x; f < A.E; f += blockDim.x)
    zs[f] = __hip_atomic_load(A.z + static_cast<size_t>(tok) * A.E + f, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const size_t o = static_cast<size_t>(tok) * A.k;
  topk_block(zs, A.E, A.k, sel_z, sel_e, A.ids + o, A.w + o, A.ids2 ? A.ids2 + o : nullptr,
             A.w2 ? A.w2 + o : nullptr);
}

template <bool HAS_ADD, bool RMS, bool TOPK>
__global__ __launch_bounds__(kThreads) void k_route_fused(RouteArgs A) {
  extern __shared__ double zs[];  // [E] for the top-k of the last block
  __shared__ double sel_z[kMaxTopK];
  __shared__ int sel_e[kMaxTopK];
  __shared__ int is_last;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int H = A.H, ngu = H / kGroup, n8 = H / 8;
  const int gw = blockIdx.x * kWaves + wave;        // global wave index
  const int e = gw < A.E ? gw : A.E - 1;            // expert row of this wave
  // blocks past the logit blocks quantise: wave qw takes steps qw, qw + nqw,
  // ... of the token (64 x 8 inputs each, 16 groups, every lane); the logit
  // waves skip the quantisation, the quantising waves the dot products
  const int nlog = (A.E + kWaves - 1) / kWaves;
  const bool qblk = static_cast<int>(blockIdx.x) >= nlog;
  const int qw = (static_cast<int>(blockIdx.x) - nlog) * kWaves + wave;
  const int nqw = (static_cast<int>(gridDim.x) - nlog) * kWaves;
  const uint16_t* row = A.wr + static_cast<size_t>(e) * H;

  {
    const int b = blockIdx.y;  // one token per grid row
    const float* xb = A.x + static_cast<size_t>(b) * H;
    const uint16_t* ab = HAS_ADD ? A.add_in + static_cast<size_t>(b) * H : nullptr;
    // inputs wider than one batch: the RMSNorm factor needs a pass of its own
    float r_all = 1.0f, ss_all = 0.f;
    const bool multi = n8 > kWave * kMaxSteps;
    if ((RMS || A.u16) && multi) {
      float ss = 0.f;
      for (int c = lane; c < n8; c += kWave) {
        const float4 x0 = *reinterpret_cast<const float4*>(xb + 8 * c);
        const float4 x1 = *reinterpret_cast<const float4*>(xb + 8 * c + 4);
        const uint4 av = HAS_ADD ? *reinterpret_cast<const uint4*>(ab + 8 * c) : make_uint4(0, 0, 0, 0);
        const uint32_t ap[4] = {av.x, av.y, av.z, av.w};
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v0 = xv[2 * i] + h2f(static_cast<uint16_t>(ap[i] & 0xFFFFu));
          const float v1 = xv[2 * i + 1] + h2f(static_cast<uint16_t>(ap[i] >> 16));
          ss = fmaf(v0, v0, ss);
          ss = fmaf(v1, v1, ss);
        }
      }
      ss_all = wave_sum(ss);
      if (RMS) r_all = 1.0f / sqrtf(ss_all / static_cast<float>(H) + 1e-6f);
    }
    double acc = 0.0;
    for (int c0 = 0; c0 < n8; c0 += kWave * kMaxSteps) {
      uint4 wv[kMaxSteps], av[kMaxSteps];
      float4 x0[kMaxSteps], x1[kMaxSteps];
#pragma unroll
      for (int t = 0; t < kMaxSteps; ++t) {
        int c = c0 + lane + kWave * t;
        c = c < n8 ? c : n8 - 1;
        wv[t] = *reinterpret_cast<const uint4*>(row + 8 * c);
        x0[t] = *reinterpret_cast<const float4*>(xb + 8 * c);
        x1[t] = *reinterpret_cast<const float4*>(xb + 8 * c + 4);
        av[t] = HAS_ADD ? *reinterpret_cast<const uint4*>(ab + 8 * c) : make_uint4(0, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      float u[kMaxSteps][8];
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < kMaxSteps; ++t) {
        const int c = c0 + lane + kWave * t;
        const uint32_t ap[4] = {av[t].x, av[t].y, av[t].z, av[t].w};
        const float xv[8] = {x0[t].x, x0[t].y, x0[t].z, x0[t].w, x1[t].x, x1[t].y, x1[t].z, x1[t].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u[t][2 * i] = xv[2 * i] + h2f(static_cast<uint16_t>(ap[i] & 0xFFFFu));
          u[t][2 * i + 1] = xv[2 * i + 1] + h2f(static_cast<uint16_t>(ap[i] >> 16));
        }
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) part = fmaf(u[t][i], u[t][i], part);
        ss += c < n8 ? part : 0.f;
      }
      float r = r_all;
      if ((RMS || A.u16) && !multi) {
        ss = wave_sum(ss);
        if (RMS) r = 1.0f / sqrtf(ss / static_cast<float>(H) + 1e-6f);
      } else {
        ss = ss_all;
      }
      // token scale of the fp16 copy: a power of two, so scaling is exact
      float tsc = 1.0f;
      if (A.u16) {
        const float nrm = sqrtf(ss) * r;
        if (nrm > 0.f && nrm <= FLT_MAX) {
          int ex;
          frexpf(nrm, &ex);
          tsc = ldexpf(1.0f, ex - 4);
        }
        if (blockIdx.x == 0 && threadIdx.x == 0 && c0 == 0) A.tsc[b] = tsc;
      }
#pragma unroll
      for (int t = 0; t < kMaxSteps; ++t) {
        const int c = c0 + lane + kWave * t;
        const uint32_t wp[4] = {wv[t].x, wv[t].y, wv[t].z, wv[t].w};
        if (RMS) {
#pragma unroll
          for (int i = 0; i < 8; ++i) u[t][i] *= r;
        }
        if (!qblk) {
          double part = 0.0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            part = fma(static_cast<double>(u[t][2 * i]), static_cast<double>(h2f(static_cast<uint16_t>(wp[i] & 0xFFFFu))), part);
            part = fma(static_cast<double>(u[t][2 * i + 1]), static_cast<double>(h2f(static_cast<uint16_t>(wp[i] >> 16))), part);
          }
          acc += c < n8 ? part : 0.0;
          continue;
        }
        // a quantising wave's step: group g = c / 4, its 4 positions of 8
        // values in an aligned lane quad (uniform test: whole steps)
        const int g = c / 4;
        const int st = c0 / kWave + t;
        if (st % nqw != qw || c0 + kWave * t >= n8) continue;
        const bool own = c < n8;
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(u[t][i]));
        m = fmaxf(m, dpp<0xB1>(m));  // the group's 4 lanes (an aligned quad)
        m = fmaxf(m, dpp<0x4E>(m));
        if (own) {
          const float inv = m > 0.f ? static_cast<float>(kQmax) / m : 0.f;
          uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            int q = static_cast<int>(rintf(u[t][i] * inv));
            q = q > kQmax ? kQmax : (q < -kQmax ? -kQmax : q);
            const uint32_t nb = digit_nibbles(q);
#pragma unroll
            for (int d = 0; d < 4; ++d) wd[d] |= ((nb >> (4 * d)) & 15u) << (4 * i);
          }
          if (A.udig) {
            DigitGroup* dg = A.udig + static_cast<size_t>(b) * ngu + g;
            dg->p[c & 3] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            if ((c & 3) == 0) A.usc[static_cast<size_t>(b) * ngu + g] = m / static_cast<float>(kQmax);
          }
          if (A.u16) {
            const float inv_t = 1.0f / tsc;
            uint32_t hw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const _Float16 lo = static_cast<_Float16>(u[t][i] * inv_t);
              const _Float16 hi = static_cast<_Float16>(u[t][i + 4] * inv_t);
              hw[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
            }
            *reinterpret_cast<uint4*>(A.u16 + static_cast<size_t>(b) * H + 8 * c) =
                make_uint4(hw[0], hw[1], hw[2], hw[3]);
          }
          if (A.u_out) {
            float* uo = A.u_out + static_cast<size_t>(b) * H + 8 * c;
            *reinterpret_cast<float4*>(uo) = make_float4(u[t][0], u[t][1], u[t][2], u[t][3]);
            *reinterpret_cast<float4*>(uo + 4) = make_float4(u[t][4], u[t][5], u[t][6], u[t][7]);
          }
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0 && gw < A.E) {
      const double zv = acc + (A.bias ? static_cast<double>(A.bias[e]) : 0.0);
      if (TOPK)
        __hip_atomic_store(A.z + static_cast<size_t>(b) * A.E + e, zv, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        A.z[static_cast<size_t>(b) * A.E + e] = zv;  // read after the kernel boundary
    }
  }
  if (!TOPK) return;
  route_tail(A, zs, sel_z, sel_e, &is_last);
}

// Batched router (B > 1, matrix-core path: fp16 inputs, no digit planes).
// A wave holds one token's whole input in registers (STEPS steps of 8
// consecutive values per lane) and computes kEW experts' logits from it, so
// a token's input is read E / kEW times instead of E times and a token takes
// E / (4 kEW) blocks. Per expert the fp64 products and their order are those
// of k_route_fused, so the logits (and the ids) are the same bits.
constexpr int kEW = 4;

// 4 waves per block (more blocks per token only add arrivals and input loads)
constexpr int kTokWaves = 4;
constexpr int kTokThreads = kTokWaves * kWave;

template <bool HAS_ADD, bool RMS, int STEPS>
__global__ __launch_bounds__(kTokThreads) void k_route_tok(RouteArgs A) {
  extern __shared__ double zs[];  // [E] for the top-k of the last block
  __shared__ double sel_z[kMaxTopK];
  __shared__ int sel_e[kMaxTopK];
  __shared__ int is_last;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int H = A.H, n8 = H / 8;
  const int b = blockIdx.y;
  const int e0 = (blockIdx.x * kTokWaves + wave) * kEW;
  const float* xb = A.x + static_cast<size_t>(b) * H;
  const uint16_t* ab = HAS_ADD ? A.add_in + static_cast<size_t>(b) * H : nullptr;

  // the rows of the wave's kEW experts first, all in one batch of loads with
  // the token's input below (issued per expert next to its products, the
  // compiler serialised the later experts' loads, one round trip each)
  uint4 wv[kEW][STEPS];
#pragma unroll
  for (int j = 0; j < kEW; ++j) {
    const int e = e0 + j < A.E ? e0 + j : A.E - 1;
    const uint16_t* row = A.wr + static_cast<size_t>(e) * H;
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      int c = lane + kWave * t;
      c = c < n8 ? c : n8 - 1;
      wv[j][t] = *reinterpret_cast<const uint4*>(row + 8 * c);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float u[STEPS][8];
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < STEPS; ++t) {
    int c = lane + kWave * t;
    const bool valid = c < n8;
    c = valid ? c : n8 - 1;
    const float4 x0 = *reinterpret_cast<const float4*>(xb + 8 * c);
    const float4 x1 = *reinterpret_cast<const float4*>(xb + 8 * c + 4);
    const uint4 av = HAS_ADD ? *reinterpret_cast<const uint4*>(ab + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint32_t ap[4] = {av.x, av.y, av.z, av.w};
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u[t][2 * i] = xv[2 * i] + h2f(static_cast<uint16_t>(ap[i] & 0xFFFFu));
      u[t][2 * i + 1] = xv[2 * i + 1] + h2f(static_cast<uint16_t>(ap[i] >> 16));
    }
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part = fmaf(u[t][i], u[t][i], part);
    ss += valid ? part : 0.f;
  }
  ss = wave_sum(ss);
  const float r = RMS ? 1.0f / sqrtf(ss / static_cast<float>(H) + 1e-6f) : 1.0f;
  // token scale of the fp16 copy: a power of two, so scaling is exact
  float tsc = 1.0f;
  {
    const float nrm = sqrtf(ss) * r;
    if (nrm > 0.f && nrm <= FLT_MAX) {
      int ex;
      frexpf(nrm, &ex);
      tsc = ldexpf(1.0f, ex - 4);
    }
  }
  if (RMS) {
#pragma unroll
    for (int t = 0; t < STEPS; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) u[t][i] *= r;
  }
  if (blockIdx.x == 0) {
    // the token's fp16 copy (and u), one step per wave
    if (threadIdx.x == 0) A.tsc[b] = tsc;
    const float inv_t = 1.0f / tsc;
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const int c = lane + kWave * t;
      if (t % kTokWaves != wave || c >= n8) continue;
      uint32_t hw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 lo = static_cast<_Float16>(u[t][i] * inv_t);
        const _Float16 hi = static_cast<_Float16>(u[t][i + 4] * inv_t);
        hw[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
      }
      *reinterpret_cast<uint4*>(A.u16 + static_cast<size_t>(b) * H + 8 * c) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if (A.u_out) {
        float* uo = A.u_out + static_cast<size_t>(b) * H + 8 * c;
        *reinterpret_cast<float4*>(uo) = make_float4(u[t][0], u[t][1], u[t][2], u[t][3]);
        *reinterpret_cast<float4*>(uo + 4) = make_float4(u[t][4], u[t][5], u[t][6], u[t][7]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kEW; ++j) {
    const int e = e0 + j < A.E ? e0 + j : A.E - 1;
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const bool valid = lane + kWave * t < n8;
      const uint32_t wp[4] = {wv[j][t].x, wv[j][t].y, wv[j][t].z, wv[j][t].w};
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part = fma(static_cast<double>(u[t][2 * i]), static_cast<double>(h2f(static_cast<uint16_t>(wp[i] & 0xFFFFu))), part);
        part = fma(static_cast<double>(u[t][2 * i + 1]), static_cast<double>(h2f(static_cast<uint16_t>(wp[i] >> 16))), part);
      }
      acc += valid ? part : 0.0;
    }
    acc = wave_sum(acc);
    if (lane == 0 && e0 + j < A.E) {
      const double zv = acc + (A.bias ? static_cast<double>(A.bias[e]) : 0.0);
      __hip_atomic_store(A.z + static_cast<size_t>(b) * A.E + e, zv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  route_tail(A, zs, sel_z, sel_e, &is_last);
}

constexpr int kLogitWaves = 4;

// Standalone router: one wave per expert row, fp64 accumulation of exact
// fp32 x fp16 products.
__global__ __launch_bounds__(kLogitWaves* kWave) void k_route_logits(
    const float* __restrict__ u, int B, int H, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int E, double* __restrict__ z) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * kLogitWaves + wave;
  if (e >= E) return;
  const uint16_t* row = wr + static_cast<size_t>(e) * H;
  for (int b = 0; b < B; ++b) {
    const float* ub = u + static_cast<size_t>(b) * H;
    double acc = 0.0;
    for (int c = lane; c < H / 8; c += kWave) {
      const uint4 wv = *reinterpret_cast<const uint4*>(row + 8 * c);
      const float4 u0 = *reinterpret_cast<const float4*>(ub + 8 * c);
      const float4 u1 = *reinterpret_cast<const float4*>(ub + 8 * c + 4);
      const uint32_t wp[4] = {wv.x, wv.y, wv.z, wv.w};
      const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fma(static_cast<double>(uv[2 * i]), static_cast<double>(h2f(static_cast<uint16_t>(wp[i] & 0xFFFFu))), acc);
        acc = fma(static_cast<double>(uv[2 * i + 1]), static_cast<double>(h2f(static_cast<uint16_t>(wp[i] >> 16))), acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) z[static_cast<size_t>(b) * E + e] = acc + (bias ? static_cast<double>(bias[e]) : 0.0);
  }
}

// Standalone top-k: one block per token, logits from fp64 z64 or fp32 z32.
__global__ __launch_bounds__(kThreads) void k_route_topk(const double* __restrict__ z64,
                                                         const float* __restrict__ z32, int E, int k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w,
                                                         int32_t* __restrict__ ids2,
                                                         float* __restrict__ w2) {
  extern __shared__ double zs[];
  __shared__ double sel_z[kMaxTopK];
  __shared__ int sel_e[kMaxTopK];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kThreads)
    zs[e] = z64 ? z64[static_cast<size_t>(b) * E + e] : static_cast<double>(z32[static_cast<size_t>(b) * E + e]);
  __syncthreads();
  const size_t o = static_cast<size_t>(b) * k;
  topk_block(zs, E, k, sel_z, sel_e, ids + o, w + o, ids2 ? ids2 + o : nullptr, w2 ? w2 + o : nullptr);
}

// Selection step of one token (a block of kSelThreads): top-k of the logits,
// then the device-side cache step and / or the publication of the ids.
constexpr int kSelThreads = 1024;
__global__ __launch_bounds__(kSelThreads) void k_route_select(RouteArgs A) {
  extern __shared__ double zs[];  // [E], then the cache state
  __shared__ double sel_z[kMaxTopK];
  __shared__ int sel_e[kMaxTopK];
  for (int f = threadIdx.x; f < A.E; f += kSelThreads) zs[f] = A.z[f];
  __syncthreads();
  topk_select(zs, A.E, A.k, sel_z, sel_e);
  if (A.seq_host && threadIdx.x == 0) {
    // one thread writes the ids and then publishes them (the host waits for
    // them, so before the weights): the release store orders its own earlier
    // stores before the sequence number
    for (int j = 0; j < A.k; ++j)
      __hip_atomic_store(A.ids_host + j, sel_e[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(A.seq_host, A.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  topk_weights(sel_z, sel_e, A.k, A.ids, A.w, A.ids2, A.w2);
  if (A.use_dc) dcache_step(A.dc, sel_e, A.k, A.E, reinterpret_cast<int32_t*>(zs + A.E));
}

}  // namespace

hipError_t launch_route_select(const double* z, int E, int k, int32_t* ids, float* w, int32_t* ids2, float* w2,
                               int32_t* ids_host, int32_t* seq_host, int32_t seq, const DevCache* dcache,
                               hipStream_t s) {
  if (!z || !ids || !w || k < 1 || k > kMaxTopK || k > E || (seq_host && !ids_host)) return hipErrorInvalidValue;
  RouteArgs A{};
  A.z = const_cast<double*>(z);  // read only by the selection kernel
  A.E = E;
  A.k = k;
  A.ids = ids;
  A.w = w;
  A.ids2 = ids2;
  A.w2 = w2;
  A.ids_host = ids_host;
  A.seq_host = seq_host;
  A.seq = seq;
  if (dcache) {
    A.dc = *dcache;
    A.use_dc = 1;
  }
  const size_t lds = sizeof(double) * E + (dcache ? dcache_lds_bytes(dcache->n_slots, E) : 0);
  hipLaunchKernelGGL(k_route_select, dim3(1), dim3(kSelThreads), lds, s, A);
  return hipGetLastError();
}

hipError_t launch_route_layer(const float* x, const uint16_t* add_in, int B, int H, bool rmsnorm,
                              const uint16_t* wr, const float* bias, int E, int k, float* u_out,
                              DigitGroup* udig, float* usc, uint16_t* u16, float* tsc, double* z,
                              int32_t* cnt, int32_t* ids, float* w, int32_t* ids2, float* w2,
                              hipStream_t s) {
  RouteArgs A{x, add_in, B, H, rmsnorm ? 1 : 0, wr, bias, E, k, u_out, udig, usc, u16, tsc, z, cnt,
              ids, ids2, w, w2, nullptr, nullptr, 0, DevCache{}, 0};
  const int blocks = (E + kWaves - 1) / kWaves;
  // one token's logits, for the top-k
  const size_t lds = sizeof(double) * E;
  // a batch with its top-k, for the matrix-core path (no digit planes): the
  // batched router, a token's input held in registers (H <= 4096)
  const int steps = (H / 8 + kWave - 1) / kWave;
  if (B > 1 && ids && !udig && u16 && tsc && steps <= kMaxSteps) {
    const dim3 grid((E + kTokWaves * kEW - 1) / (kTokWaves * kEW), B);
#define MOE_ROUTE_TOK(A_, R_)                                                                        \
  do {                                                                                             \
    if (steps <= 2) hipLaunchKernelGGL((k_route_tok<A_, R_, 2>), grid, dim3(kTokThreads), lds, s, A); \
    else if (steps <= 4) hipLaunchKernelGGL((k_route_tok<A_, R_, 4>), grid, dim3(kTokThreads), lds, s, A); \
    else if (steps <= 6) hipLaunchKernelGGL((k_route_tok<A_, R_, 6>), grid, dim3(kTokThreads), lds, s, A); \
    else hipLaunchKernelGGL((k_route_tok<A_, R_, 8>), grid, dim3(kTokThreads), lds, s, A);             \
  } while (0)
    if (add_in && rmsnorm) MOE_ROUTE_TOK(true, true);
    else if (add_in) MOE_ROUTE_TOK(true, false);
    else if (rmsnorm) MOE_ROUTE_TOK(false, true);
    else MOE_ROUTE_TOK(false, false);
#undef MOE_ROUTE_TOK
    return hipGetLastError();
  }
  const bool topk = ids != nullptr;
  // blocks that quantise u (one wave per 64 x 8 inputs), after the logit blocks
  const int qblocks = (udig || u16 || u_out) ? (steps + kWaves - 1) / kWaves : 0;
#define MOE_ROUTE(A_, R_, T_) hipLaunchKernelGGL((k_route_fused<A_, R_, T_>), dim3(blocks + qblocks, B), dim3(kThreads), lds, s, A)
  if (topk) {
    if (add_in && rmsnorm) MOE_ROUTE(true, true, true);
    else if (add_in) MOE_ROUTE(true, false, true);
    else if (rmsnorm) MOE_ROUTE(false, true, true);
    else MOE_ROUTE(false, false, true);
  } else {
    if (add_in && rmsnorm) MOE_ROUTE(true, true, false);
    else if (add_in) MOE_ROUTE(true, false, false);
    else if (rmsnorm) MOE_ROUTE(false, true, false);
    else MOE_ROUTE(false, false, false);
  }
#undef MOE_ROUTE
  return hipGetLastError();
}

size_t dcache_lds_bytes(int n_slots, int E) { return sizeof(int32_t) * (3 * static_cast<size_t>(n_slots) + 2 * E); }

hipError_t launch_route_logits(const float* u, int B, int H, const uint16_t* wr, const float* bias,
                               int E, double* z, hipStream_t s) {
  const int blocks = (E + kLogitWaves - 1) / kLogitWaves;
  hipLaunchKernelGGL(k_route_logits, dim3(blocks), dim3(kLogitWaves * kWave), 0, s, u, B, H, wr,
                     bias, E, z);
  return hipGetLastError();
}

hipError_t launch_route_topk(const double* z64, const float* z32, int B, int E, int k, int32_t* ids,
                             float* w, int32_t* ids2, float* w2, hipStream_t s) {
  hipLaunchKernelGGL(k_route_topk, dim3(B), dim3(kThreads), sizeof(double) * E, s, z64, z32, E, k,
                     ids, w, ids2, w2);
  return hipGetLastError();
}

}  // namespace moe
