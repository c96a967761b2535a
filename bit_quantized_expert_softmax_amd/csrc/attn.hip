// Attention step of one decoder layer, one token (decode): RMSNorm with a
// learned weight, the fused q/k/v projection, rotate-half RoPE, the append of
// the token's key and value to the fp16 KV cache, grouped-query attention over
// the cached positions, the output projection and the residual add.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum": section "Sem dependências do llama.cpp e MLX"
// names hand-written attention, RMSNorm and RoPE kernels; section "Qual é o
// principal truque da arquitetura" keeps the KV cache for the context resident
// in FP16.
//
// Three launches:
//  1. k_attn_gemv<kQkv>: every block quantises x * w into digit planes (LDS),
//     takes its rows of the int4 projection with v_dot8 (as the expert GEMVs)
//     and scales the row sums by the RMSNorm factor. A block's rows are pairs
//     (i, i + d/2) of one head, so its epilogue applies RoPE to q and k itself,
//     writes q (fp32) and appends k and v to the cache (fp16, nearest even).
//  2. k_attn_split: block (split, kv head) streams the K and V rows of its
//     positions once for all query heads of the group: scores, a softmax over
//     the split, the value sum. With one split it writes the attention output
//     as digit planes per group of 32; with more, its partial results, and
//  2b. k_attn_combine merges them in split order (a last-block combine inside
//     k_attn_split, behind an arrival counter, measured 7 us slower at 4096
//     positions: its store drain, counter round trip and L2-bypassing loads
//     are serial).
//  3. k_attn_gemv<kOut>: output projection of those digit planes (each lane
//     loads its column's group next to its weights) plus the residual.
#include <hip/hip_fp16.h>

#include <cmath>

#include "launch.h"

namespace moe {
namespace {

constexpr int kAThreads = 1024;
constexpr int kAWaves = kAThreads / kWave;
constexpr int kSplitThreads = 512;
constexpr int kSplitSteps = 4;  // position steps per split block

enum { kQkv = 0, kOut = 1 };
// passes of two groups per wave that cover the largest input (K = 4096:
// 128 groups over 16 waves)
constexpr int kMaxPairPasses = 4;

__device__ __forceinline__ uint16_t f2h_bits(float v) {
  return __half_as_ushort(__float2half_rn(v));
}

__device__ __forceinline__ float h_lo(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<uint16_t>(w & 0xFFFFu)));
}
__device__ __forceinline__ float h_hi(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16)));
}

// GEMV y = W x over rows of an int4 g32 matrix with K = 32 * ng columns, the
// input as digit planes per group of 32 (kQkv: the normed input, quantised by
// every block into LDS; kOut: read from global memory). Lane (r0, c) = (tid / ng, tid % ng)
// owns chunk column c of local rows r0, r0 + R, ... (R = 1024 / ng); the block
// owns RB local rows.
template <int MODE, int NT>
__global__ __launch_bounds__(kAThreads) void k_attn_gemv(AttnGemvArgs A) {
  extern __shared__ uint4 lds_raw[];
  __shared__ float red[kAWaves];
  __shared__ float rowsum[64];
  const int ng = A.K / kGroup;
  const int RB = A.RB;
  float* part = reinterpret_cast<float*>(lds_raw);                                // [RB][ng]
  DigitGroup* xd = reinterpret_cast<DigitGroup*>(part + static_cast<size_t>(RB) * ng);  // [ng]
  float* xs = reinterpret_cast<float*>(xd + ng);                                   // [ng]
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const int R = kAThreads / ng;
  const int c = tid % ng, r0 = tid / ng;
  const bool lane_on = r0 < R;
  const int half = RB / 2;
  const int d = A.d;

  // global row of local row r
  auto row_of = [&](int r) -> int {
    if (MODE == kQkv) {
      // pairs (i, i + d/2) of one head: local rows [0, half) are the first
      // halves, [half, RB) the second halves
      const int p = blockIdx.x * half + (r < half ? r : r - half);
      const int hh = p / (d / 2), i = p % (d / 2);
      return hh * d + i + (r < half ? 0 : d / 2);
    } else {
      const int n = blockIdx.x * RB + r;
      return n < A.N ? n : A.N - 1;  // rows past the end re-read the last row
    }
  };

  // the output projection's input digits first (loads retire in order, so a
  // weight chunk is consumed as soon as it is in); then the weights, whose
  // addresses do not depend on the input
  DigitGroup xc;
  float xsc;
  if (MODE == kOut) {
    xc = A.adig[c];
    xsc = A.asc[c];
  }
  const size_t rowb = static_cast<size_t>(A.K) / 2;
  uint4 wv[NT];
  uint16_t sw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int r = r0 + R * t;
    r = r < RB ? r : RB - 1;  // clamped: loaded, not stored
    const size_t n = static_cast<size_t>(row_of(r));
    wv[t] = load_w16(A.wq + n * rowb + 16 * static_cast<size_t>(c));
    sw[t] = A.ws[n * ng + c];
  }
  __builtin_amdgcn_sched_barrier(0);

  float inv = 1.0f;
  if (MODE == kQkv) {
    // The projection is linear, so the RMSNorm factor multiplies the row sums
    // at the end: the digit planes are those of x * w (two groups per wave
    // pass, every pass's loads issued first), and the sum of squares of x is
    // reduced alongside, in a fixed order.
    float xv[kMaxPairPasses], wv_n[kMaxPairPasses];
#pragma unroll
    for (int j = 0; j < kMaxPairPasses; ++j) {
      const int g = 2 * (wave + kAWaves * j) + (lane >> 5);
      const int i = kGroup * (g < ng ? g : ng - 1) + (lane & 31);
      xv[j] = A.x[i];
      wv_n[j] = A.norm_w[i];
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPairPasses; ++j) {
      const int g0 = 2 * (wave + kAWaves * j);
      if (g0 < ng) {  // uniform over the wave
        const bool on = g0 + (lane >> 5) < ng;
        ss = on ? fmaf(xv[j], xv[j], ss) : ss;
        quant_pair_of_groups(on ? xv[j] * wv_n[j] : 0.f, g0, ng, xd, xs);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    xc = xd[c];
    xsc = xs[c];
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kAWaves; ++w) tot += red[w];
    inv = 1.0f / sqrtf(tot / static_cast<float>(A.K) + A.eps);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = r0 + R * t;
    const float p = static_cast<float>(chunk_dot(wv[t], xc)) * (h2f(sw[t]) * xsc);
    if (lane_on && r < RB) part[r * ng + c] = p;
  }
  __syncthreads();
  {
    // row sums: 16 lanes per row, 4 rows per wave, fixed order
    const int r = 4 * wave + (lane >> 4);
    const int l = lane & 15;
    if (r < RB) {
      float acc = 0.f;
      for (int cc = l; cc < ng; cc += 16) acc += part[r * ng + cc];
      acc = dpp_sum<16>(acc);
      if (l == 0) rowsum[r] = acc;
    }
  }
  __syncthreads();
  if (MODE == kQkv) {
    if (tid < half) {
      const int p = blockIdx.x * half + tid;
      const int hh = p / (d / 2), i = p % (d / 2);
      float v0 = rowsum[tid] * inv, v1 = rowsum[tid + half] * inv;
      if (hh < A.nh + A.nkv) {
        // angle pos * theta^(-2i/d) and its reduction to [-pi, pi] in fp64
        // (|angle| < 2^14, so the reduction loses nothing), then sin and cos
        // of the reduced angle and the rotation in fp32
        const double ang = static_cast<double>(A.pos) * exp2(-2.0 * i / d * A.log2_theta);
        const double twopi = 6.283185307179586476925286766559;
        const float r = static_cast<float>(ang - twopi * rint(ang / twopi));
        float sf, cf;
        sincosf(r, &sf, &cf);
        const float r0v = v0 * cf - v1 * sf;
        const float r1v = v1 * cf + v0 * sf;
        v0 = r0v;
        v1 = r1v;
      }
      if (hh < A.nh) {
        A.q[hh * d + i] = v0;
        A.q[hh * d + i + d / 2] = v1;
      } else {
        const bool is_k = hh < A.nh + A.nkv;
        const int g = is_k ? hh - A.nh : hh - A.nh - A.nkv;
        uint16_t* cache = is_k ? A.kc : A.vc;
        const size_t base = (static_cast<size_t>(g) * A.max_ctx + A.pos) * d;
        cache[base + i] = f2h_bits(v0);
        cache[base + i + d / 2] = f2h_bits(v1);
      }
    }
  } else {
    if (tid < RB) {
      const int n = blockIdx.x * RB + tid;
      if (n < A.N) A.y[n] = A.x[n] + rowsum[tid];
    }
  }
}

// One split of the context for one key/value head and its G query heads. A
// position's d values are spread over LP = d / 16 lanes: lane j of a position
// takes elements [8j, 8j + 8) and [d/2 + 8j, d/2 + 8j + 8), so each of its two
// 16-byte loads of a K (or V) row makes, with the other LP - 1 lanes, one
// contiguous half row. A step covers 256 / LP positions, a split kSplitSteps
// steps. Every K and V load of the block is issued before any is used. The
// attention output is written as digit planes per group of 32 (the input
// format of the output projection).
template <int D, int G>
__global__ __launch_bounds__(kSplitThreads) void k_attn_split(AttnSplitArgs A) {
  constexpr int LP = D / 16;
  constexpr int PPS = kSplitThreads / LP;
  constexpr int P = kSplitSteps * PPS;
  __shared__ float sc[G][P];
  __shared__ float red[kSplitThreads / kWave][G][D];
  __shared__ float mh[G], lh[G];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int g = blockIdx.y, sp = blockIdx.x;
  const int slot = tid / LP, e0 = (tid % LP) * 8;  // elements [e0, e0 + 8) and [D/2 + e0, D/2 + e0 + 8)
  const int n = A.n, lo = sp * P;

  // loads in the order of use (q, every K row, every V row): loads retire in
  // order, so the scores of step s wait only for K row s while the later rows
  // and all V rows are still in flight
  float4 qraw[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = A.q + static_cast<size_t>(g * G + h) * D + e0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qraw[h][j] = *reinterpret_cast<const float4*>(qh + (j < 2 ? 4 * j : D / 2 + 4 * (j - 2)));
  }
  size_t base[kSplitSteps];
#pragma unroll
  for (int s = 0; s < kSplitSteps; ++s) {
    int t = lo + s * PPS + slot;
    t = t < n ? t : n - 1;  // clamped: loaded, masked below
    base[s] = (static_cast<size_t>(g) * A.max_ctx + t) * D + e0;
  }
  uint4 kr[kSplitSteps][2], vr[kSplitSteps][2];
#pragma unroll
  for (int s = 0; s < kSplitSteps; ++s) {
    kr[s][0] = *reinterpret_cast<const uint4*>(A.kc + base[s]);
    kr[s][1] = *reinterpret_cast<const uint4*>(A.kc + base[s] + D / 2);
  }
#pragma unroll
  for (int s = 0; s < kSplitSteps; ++s) {
    vr[s][0] = *reinterpret_cast<const uint4*>(A.vc + base[s]);
    vr[s][1] = *reinterpret_cast<const uint4*>(A.vc + base[s] + D / 2);
  }
  __builtin_amdgcn_sched_barrier(0);
  float qv[G][16];
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qv[h][4 * j] = qraw[h][j].x * scale;
      qv[h][4 * j + 1] = qraw[h][j].y * scale;
      qv[h][4 * j + 2] = qraw[h][j].z * scale;
      qv[h][4 * j + 3] = qraw[h][j].w * scale;
    }

  // scores q . k / sqrt(d): 16 products per lane, then a sum over the LP lanes
#pragma unroll
  for (int s = 0; s < kSplitSteps; ++s) {
    const uint32_t kw[8] = {kr[s][0].x, kr[s][0].y, kr[s][0].z, kr[s][0].w,
                            kr[s][1].x, kr[s][1].y, kr[s][1].z, kr[s][1].w};
    float kf[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kf[2 * j] = h_lo(kw[j]);
      kf[2 * j + 1] = h_hi(kw[j]);
    }
    const int t = lo + s * PPS + slot;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float dsum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) dsum = fmaf(qv[h][e], kf[e], dsum);
      dsum = dpp_sum<LP>(dsum);
      if (tid % LP == 0) sc[h][s * PPS + slot] = t < n ? dsum : -INFINITY;
    }
  }
  __syncthreads();
  // softmax over the split: wave h takes query head h
  if (wave < G) {
    const int h = wave;
    float m = -INFINITY;
    for (int j = lane; j < P; j += kWave) m = fmaxf(m, sc[h][j]);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float l = 0.f;
    for (int j = lane; j < P; j += kWave) {
      const float sv = sc[h][j];
      const float e = sv == -INFINITY ? 0.f : expf(sv - m);
      sc[h][j] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      mh[h] = m;
      lh[h] = l;
    }
  }
  __syncthreads();
  // value sum: each lane its 16 elements over its positions
  float acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int s = 0; s < kSplitSteps; ++s) {
    const uint32_t vw[8] = {vr[s][0].x, vr[s][0].y, vr[s][0].z, vr[s][0].w,
                            vr[s][1].x, vr[s][1].y, vr[s][1].z, vr[s][1].w};
    float vf[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      vf[2 * j] = h_lo(vw[j]);
      vf[2 * j + 1] = h_hi(vw[j]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = sc[h][s * PPS + slot];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
    }
  }
  // sum over the positions of the wave (lanes with the same elements), then
  // over the waves through LDS
#pragma unroll
  for (int o = LP; o < kWave; o <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] += __shfl_xor(acc[h][e], o, kWave);
  if (lane < LP) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[wave][h][(e < 8 ? 0 : D / 2 - 8) + e0 + e] = acc[h][e];
  }
  __syncthreads();
  const int nsplit = gridDim.x;
  // G * D is a multiple of 64, so every wave of the loop is whole (the
  // digit-plane writer needs all 64 lanes)
  for (int idx = tid; idx < G * D; idx += kSplitThreads) {
    const int h = idx / D, e = idx % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitThreads / kWave; ++w) o += red[w][h][e];
    const int qh = g * G + h;
    if (nsplit == 1) {
      const int g0 = (g * G * D + idx - lane) / kGroup;
      quant_pair_of_groups(o / lh[h], g0, g0 + 2, A.adig, A.asc);
    } else {
      // read by the combine kernel, after the kernel boundary
      A.po[(static_cast<size_t>(qh) * nsplit + sp) * D + e] = o;
      if (e == 0) {
        A.pm[static_cast<size_t>(qh) * nsplit + sp] = mh[h];
        A.pl[static_cast<size_t>(qh) * nsplit + sp] = lh[h];
      }
    }
  }
}

// Combine of the splits (more than one): block h takes query head h, thread
// e its element e. The block stages the splits' maxima and sums in LDS while
// every thread's value loads (up to 32 splits per batch) are already in
// flight; wave 0 forms M = max m_s, the weights exp(m_s - M) and
// L = sum of weight * l_s; each thread then sums weight * o_s in split order.
// Writes digit planes per group of 32.
__global__ __launch_bounds__(256) void k_attn_combine(AttnSplitArgs A, int nsplit) {
  extern __shared__ float cmb[];  // [2][nsplit]: maxima -> weights, sums
  __shared__ float Lsh;
  const int D = blockDim.x;
  const int h = blockIdx.x, e = threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const float* po = A.po + static_cast<size_t>(h) * nsplit * D + e;
  float* wm = cmb;
  float* wl = cmb + nsplit;
  constexpr int B = 32;
  float ov[B];
#pragma unroll
  for (int j = 0; j < B; ++j) ov[j] = po[static_cast<size_t>(j < nsplit ? j : nsplit - 1) * D];
  for (int s = e; s < nsplit; s += D) {
    wm[s] = A.pm[static_cast<size_t>(h) * nsplit + s];
    wl[s] = A.pl[static_cast<size_t>(h) * nsplit + s];
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    float m = -INFINITY;
    for (int s = lane; s < nsplit; s += kWave) m = fmaxf(m, wm[s]);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float l = 0.f;
    for (int s = lane; s < nsplit; s += kWave) {
      const float w = expf(wm[s] - m);
      wm[s] = w;
      l = fmaf(w, wl[s], l);
    }
    l = wave_sum(l);
    if (lane == 0) Lsh = l;
  }
  __syncthreads();
  float O = 0.f;
#pragma unroll
  for (int j = 0; j < B; ++j)
    if (j < nsplit) O = fmaf(wm[j], ov[j], O);
  for (int s0 = B; s0 < nsplit; s0 += B) {
#pragma unroll
    for (int j = 0; j < B; ++j) ov[j] = po[static_cast<size_t>(s0 + j < nsplit ? s0 + j : nsplit - 1) * D];
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (s0 + j < nsplit) O = fmaf(wm[s0 + j], ov[j], O);
  }
  const int g0 = (h * D + e - lane) / kGroup;
  quant_pair_of_groups(O / Lsh, g0, g0 + 2, A.adig, A.asc);
}

// rows per block of the projection: pairs of one head (a power of two that
// divides d), at most 6 passes of R rows, and about 256 blocks where the
// matrix has enough rows
int qkv_rows_per_block(int K, int rows, int d) {
  const int R = kAThreads / (K / kGroup);
  int RB = 64;
  while (RB > 2 && (RB > 6 * R || d % RB)) RB /= 2;
  int rmin = 2;
  while (rmin * 2 <= R && rmin * 2 <= RB) rmin *= 2;
  while (RB > rmin && rows / RB < 256) RB /= 2;
  return RB;
}

size_t gemv_lds(int K, int RB, bool staged_input) {
  const int ng = K / kGroup;
  return static_cast<size_t>(RB) * ng * sizeof(float) + (staged_input ? ng * (sizeof(DigitGroup) + sizeof(float)) : 0);
}

hipError_t launch_gemv(int mode, const AttnGemvArgs& A, int blocks, hipStream_t s) {
  const int R = kAThreads / (A.K / kGroup);
  const int NT = (A.RB + R - 1) / R;
  const size_t lds = gemv_lds(A.K, A.RB, mode == kQkv);
#define MOE_AG(M, T) hipLaunchKernelGGL((k_attn_gemv<M, T>), dim3(blocks), dim3(kAThreads), lds, s, A)
#define MOE_AG_NT(M)                  \
  switch (NT) {                       \
    case 1: MOE_AG(M, 1); break;      \
    case 2: MOE_AG(M, 2); break;      \
    case 3: MOE_AG(M, 3); break;      \
    case 4: MOE_AG(M, 4); break;      \
    case 5: MOE_AG(M, 5); break;      \
    case 6: MOE_AG(M, 6); break;      \
    default: return hipErrorInvalidValue; \
  }
  if (mode == kQkv) {
    MOE_AG_NT(kQkv)
  } else {
    MOE_AG_NT(kOut)
  }
#undef MOE_AG_NT
#undef MOE_AG
  return hipGetLastError();
}

}  // namespace

int attn_split_positions(int d) { return kSplitSteps * (kSplitThreads / (d / 16)); }

bool attn_lds_fits(int H, int nh, int nkv, int d) {
  const int rows = (nh + 2 * nkv) * d;
  const int RBq = qkv_rows_per_block(H, rows, d);
  const int Ko = nh * d;
  const int Ro = kAThreads / (Ko / kGroup);
  return gemv_lds(H, RBq, true) <= 65536 && gemv_lds(Ko, Ro, false) <= 65536;
}

AttnWorkspace attn_workspace(int nh, int d, int max_ctx) {
  const int max_split = (max_ctx + attn_split_positions(d) - 1) / attn_split_positions(d);
  AttnWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~static_cast<size_t>(255);
    return o;
  };
  w.q = take(static_cast<size_t>(nh) * d * sizeof(float));
  w.adig = take(static_cast<size_t>(nh) * d / kGroup * sizeof(DigitGroup));
  w.asc = take(static_cast<size_t>(nh) * d / kGroup * sizeof(float));
  w.pm = take(static_cast<size_t>(nh) * max_split * sizeof(float));
  w.pl = take(static_cast<size_t>(nh) * max_split * sizeof(float));
  w.po = take(static_cast<size_t>(nh) * max_split * d * sizeof(float));
  w.total = off;
  w.max_split = max_split;
  return w;
}

hipError_t launch_attn_decode(const AttnLaunch& L, hipStream_t s) {
  const int H = L.H, nh = L.nh, nkv = L.nkv, d = L.d;
  const AttnWorkspace W = attn_workspace(nh, d, L.max_ctx);
  uint8_t* ws = static_cast<uint8_t*>(L.workspace);
  float* q = reinterpret_cast<float*>(ws + W.q);
  DigitGroup* adig = reinterpret_cast<DigitGroup*>(ws + W.adig);
  float* asc = reinterpret_cast<float*>(ws + W.asc);

  // 1. RMSNorm + q/k/v projection + RoPE + cache append
  AttnGemvArgs a{};
  a.wq = L.qkv_q;
  a.ws = L.qkv_s;
  a.K = H;
  a.N = (nh + 2 * nkv) * d;
  a.RB = qkv_rows_per_block(H, a.N, d);
  a.x = L.x;
  a.norm_w = L.norm_w;
  a.eps = L.eps;
  a.d = d;
  a.nh = nh;
  a.nkv = nkv;
  a.pos = L.pos;
  a.log2_theta = std::log2(L.theta);
  a.max_ctx = L.max_ctx;
  a.q = q;
  a.kc = L.kc;
  a.vc = L.vc;
  hipError_t e = launch_gemv(kQkv, a, a.N / a.RB, s);
  if (e != hipSuccess) return e;

  // 2. attention over positions [0, pos]
  AttnSplitArgs b{};
  b.q = q;
  b.kc = L.kc;
  b.vc = L.vc;
  b.max_ctx = L.max_ctx;
  b.n = L.pos + 1;
  b.pm = reinterpret_cast<float*>(ws + W.pm);
  b.pl = reinterpret_cast<float*>(ws + W.pl);
  b.po = reinterpret_cast<float*>(ws + W.po);
  b.adig = adig;
  b.asc = asc;
  const int P = attn_split_positions(d);
  const dim3 grid((b.n + P - 1) / P, nkv);
  const int G = nh / nkv;
#define MOE_AS(DD, GG) hipLaunchKernelGGL((k_attn_split<DD, GG>), grid, dim3(kSplitThreads), 0, s, b)
#define MOE_AS_G(DD)                      \
  if (G == 1) MOE_AS(DD, 1);              \
  else if (G == 2) MOE_AS(DD, 2);         \
  else if (G == 4) MOE_AS(DD, 4);         \
  else return hipErrorInvalidValue;
  if (d == 64) {
    MOE_AS_G(64)
  } else if (d == 128) {
    MOE_AS_G(128)
  } else if (d == 256) {
    MOE_AS_G(256)
  } else {
    return hipErrorInvalidValue;
  }
#undef MOE_AS_G
#undef MOE_AS
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (grid.x > 1) {
    hipLaunchKernelGGL(k_attn_combine, dim3(nh), dim3(d), 2 * grid.x * sizeof(float), s, b,
                       static_cast<int>(grid.x));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // 3. output projection + residual
  AttnGemvArgs c{};
  c.wq = L.o_q;
  c.ws = L.o_s;
  c.K = nh * d;
  c.N = H;
  const int Ro = kAThreads / (c.K / kGroup);
  int nt = H / (Ro * 256);
  nt = nt < 1 ? 1 : (nt > 6 ? 6 : nt);
  c.RB = Ro * nt > 64 ? 64 : Ro * nt;
  c.adig = adig;
  c.asc = asc;
  c.x = L.x;
  c.y = L.y;
  return launch_gemv(kOut, c, (H + c.RB - 1) / c.RB, s);
}

}  // namespace moe
