// Batched decode (B tokens per call) of one MoE layer: tokens are grouped by
// expert so that every touched expert's int4 rows are read once per call.
//
// The layer is the one of "Como executar um modelo de 26 bilhões de
// parâmetros em dois gigabytes de memória em um Mac comum", section "Qual é
// o principal truque da arquitetura" (8 routed experts and a shared expert per
// token); grouping rows per loaded expert follows the same page's section
// "Desempenho no mundo real".
//
// After routing, the B*k assignments are sorted by expert (stable: expert,
// token, rank) and each expert becomes a segment of rows. A segment's
// gate/up rows are streamed once into registers and multiplied with the
// digit planes of every token of the segment (8 tokens per LDS tile); the
// GeGLU activations are quantised per 8 values in the wave, as in B=1 decode.
// The down kernel does the same per output row and writes one fp32 row per
// assignment; the combine adds, per token and in rank order, w_j times its
// routed rows to the shared expert's output (and the residual).
#include "launch.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kLanes = 8;                  // lanes per row (pair)
constexpr int kRowsPerWave = kWave / kLanes;  // 8
constexpr int kTT = 8;                     // tokens per LDS tile

// Segment s < E: routed expert s, rows = its assignments; s == E: shared
// expert, rows = all B tokens.
struct BatchArgs {
  const uint8_t* experts;
  const uint8_t* shared;
  size_t blob_e;
  int H, I, Is, E, k, B;
  const int32_t* seg;    // [E+1] segment starts in the sorted assignment list
  const int32_t* perm;   // sorted position -> assignment (token*k + rank)
  const DigitGroup* udig;  // [B][H/32]
  const float* usc;
  uint4* adig_r;  // [B*k][I/8]   routed activations by sorted position
  float* asc_r;
  uint4* adig_s;  // [B][Is/8]    shared activations by token
  float* asc_s;
  float* out_r;   // [B*k][H]
  float* out_s;   // [B][H]
};

__device__ __forceinline__ void segment_rows(const BatchArgs& A, int s, int& r0, int& nrows,
                                             const uint8_t*& blob, int& inter) {
  if (s < A.E) {
    r0 = A.seg[s];
    nrows = A.seg[s + 1] - r0;
    blob = A.experts + static_cast<size_t>(s) * A.blob_e;
    inter = A.I;
  } else {
    r0 = 0;
    nrows = A.B;
    blob = A.shared;
    inter = A.Is;
  }
}

__device__ __forceinline__ int token_of(const BatchArgs& A, int s, int row) {
  return s < A.E ? A.perm[row] / A.k : row;
}

// Quantises the activation of segment-head lanes (0, 8, ..., 56) as one
// position of 8 values (same encoding as the B=1 kernels).
__device__ __forceinline__ void quant_pos8(float a, uint4* dst, float* dsc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int p = lane >> 3;
  float m = (lane & 7) == 0 ? fabsf(a) : 0.f;
  m = fmaxf(m, __shfl_xor(m, 8, kWave));
  m = fmaxf(m, __shfl_xor(m, 16, kWave));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  const float inv = m > 0.f ? static_cast<float>(kQmax) / m : 0.f;
  int q = static_cast<int>(rintf(a * inv));
  q = q > kQmax ? kQmax : (q < -kQmax ? -kQmax : q);
  uint32_t wd[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int dg = d < 3 ? ((q + 8) & 15) - 8 : q;
    wd[d] = (lane & 7) == 0 ? static_cast<uint32_t>(dg & 15) << (4 * p) : 0u;
    q = (q - dg) / 16;
  }
#pragma unroll
  for (int o = 8; o < kWave; o <<= 1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) wd[d] |= __shfl_xor(wd[d], o, kWave);
  }
  if (lane == 0) {
    *dst = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    *dsc = m / static_cast<float>(kQmax);
  }
}

// Gate/up of one segment's 32-row-pair tile (4 waves x 8 pairs).
template <int NT>
__global__ __launch_bounds__(kThreads) void k_bgateup(BatchArgs A, int tiles_per_seg_max) {
  extern __shared__ uint4 lds_raw[];
  const int s = blockIdx.x / tiles_per_seg_max;
  const int tile = blockIdx.x % tiles_per_seg_max;
  int r0, nrows, inter;
  const uint8_t* blob;
  segment_rows(A, s, r0, nrows, blob, inter);
  if (nrows == 0 || tile * kWaves * kRowsPerWave >= inter) return;
  const int ngu = A.H / kGroup;
  DigitGroup* xd = reinterpret_cast<DigitGroup*>(lds_raw);            // [kTT][ngu]
  float* xs = reinterpret_cast<float*>(xd + static_cast<size_t>(kTT) * ngu);  // [kTT][ngu]
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int pair = lane / kLanes;
  const int ln = lane & (kLanes - 1);
  const int i0 = (tile * kWaves + wave) * kRowsPerWave;
  const bool live = i0 < inter;
  const int i = live ? i0 + pair : 0;
  const BlobOffsets o = blob_offsets(A.H, inter);
  const size_t hq = static_cast<size_t>(A.H) / 2;
  const uint8_t* qg = blob + o.gate_q + static_cast<size_t>(i) * hq;
  const uint8_t* qu = blob + o.up_q + static_cast<size_t>(i) * hq;
  const uint16_t* sg = reinterpret_cast<const uint16_t*>(blob + o.gate_s) + static_cast<size_t>(i) * ngu;
  const uint16_t* su = reinterpret_cast<const uint16_t*>(blob + o.up_s) + static_cast<size_t>(i) * ngu;
  // the rows stay in registers for every token tile
  uint4 wg[NT], wu[NT];
  float fg[NT], fu[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int c = ln + kLanes * t;
    c = c < ngu ? c : ngu - 1;
    wg[t] = load_w16(qg + 16 * static_cast<size_t>(c));
    wu[t] = load_w16(qu + 16 * static_cast<size_t>(c));
    fg[t] = h2f(sg[c]);
    fu[t] = h2f(su[c]);
  }
  for (int m0 = 0; m0 < nrows; m0 += kTT) {
    const int mt = nrows - m0 < kTT ? nrows - m0 : kTT;
    __syncthreads();
    // stage the digit planes of this tile's tokens
    for (int idx = threadIdx.x; idx < mt * ngu * 4; idx += kThreads) {
      const int m = idx / (ngu * 4);
      const int r = idx % (ngu * 4);
      const int tok = token_of(A, s, r0 + m0 + m);
      reinterpret_cast<uint4*>(xd + static_cast<size_t>(m) * ngu)[r] =
          reinterpret_cast<const uint4*>(A.udig + static_cast<size_t>(tok) * ngu)[r];
    }
    for (int idx = threadIdx.x; idx < mt * ngu; idx += kThreads) {
      const int m = idx / ngu;
      const int tok = token_of(A, s, r0 + m0 + m);
      xs[idx] = A.usc[static_cast<size_t>(tok) * ngu + idx % ngu];
    }
    __syncthreads();
    float ag[kTT], au[kTT];
#pragma unroll
    for (int m = 0; m < kTT; ++m) ag[m] = au[m] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = ln + kLanes * t;
      const int cc = c < ngu ? c : ngu - 1;
      const float mask = static_cast<float>(c < ngu);
#pragma unroll
      for (int m = 0; m < kTT; ++m) {
        if (m < mt) {
          const DigitGroup& xv = xd[static_cast<size_t>(m) * ngu + cc];
          const float f = xs[static_cast<size_t>(m) * ngu + cc] * mask;
          ag[m] = fmaf(static_cast<float>(chunk_dot(wg[t], xv)), fg[t] * f, ag[m]);
          au[m] = fmaf(static_cast<float>(chunk_dot(wu[t], xv)), fu[t] * f, au[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kTT; ++m) {
      const float g = seg_sum<kLanes>(ag[m]);
      const float v = seg_sum<kLanes>(au[m]);
      if (m < mt) {
        const float a = gelu_tanh(g) * v;
        const int row = r0 + m0 + m;  // sorted position (routed) or token (shared)
        uint4* dst;
        float* dsc;
        if (s < A.E) {
          dst = A.adig_r + static_cast<size_t>(row) * (A.I / 8) + i0 / 8;
          dsc = A.asc_r + static_cast<size_t>(row) * (A.I / 8) + i0 / 8;
        } else {
          dst = A.adig_s + static_cast<size_t>(row) * (A.Is / 8) + i0 / 8;
          dsc = A.asc_s + static_cast<size_t>(row) * (A.Is / 8) + i0 / 8;
        }
        quant_pos8(a, live ? dst : nullptr, live ? dsc : nullptr);
      }
    }
  }
}

// Down projection of one segment's 32-output-row tile.
template <int NT>
__global__ __launch_bounds__(kThreads) void k_bdown(BatchArgs A, int tiles_per_seg) {
  extern __shared__ uint4 lds_raw[];
  const int s = blockIdx.x / tiles_per_seg;
  const int tile = blockIdx.x % tiles_per_seg;
  int r0, nrows, inter;
  const uint8_t* blob;
  segment_rows(A, s, r0, nrows, blob, inter);
  if (nrows == 0) return;
  const int npos = inter / 8;
  const int ngk = inter / kGroup;
  uint4* xd = lds_raw;                                              // [kTT][npos]
  float* xs = reinterpret_cast<float*>(xd + static_cast<size_t>(kTT) * npos);  // [kTT][npos]
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int ln = lane & (kLanes - 1);
  const int n = (tile * kWaves + wave) * kRowsPerWave + lane / kLanes;  // output row
  const bool live = n < A.H;
  const int nn = live ? n : A.H - 1;
  const BlobOffsets o = blob_offsets(A.H, inter);
  const uint8_t* q = blob + o.down_q + static_cast<size_t>(nn) * (inter / 2);
  const uint16_t* sq = reinterpret_cast<const uint16_t*>(blob + o.down_s) + static_cast<size_t>(nn) * ngk;
  uint4 wv[NT];
  float fw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int c = ln + kLanes * t;
    c = c < ngk ? c : ngk - 1;
    wv[t] = load_w16(q + 16 * static_cast<size_t>(c));
    fw[t] = h2f(sq[c]);
  }
  const uint4* src_d = s < A.E ? A.adig_r : A.adig_s;
  const float* src_s = s < A.E ? A.asc_r : A.asc_s;
  for (int m0 = 0; m0 < nrows; m0 += kTT) {
    const int mt = nrows - m0 < kTT ? nrows - m0 : kTT;
    __syncthreads();
    for (int idx = threadIdx.x; idx < mt * npos; idx += kThreads) {
      const size_t g = static_cast<size_t>(r0 + m0 + idx / npos) * npos + idx % npos;
      xd[idx] = src_d[g];
      xs[idx] = src_s[g];
    }
    __syncthreads();
    float acc[kTT];
#pragma unroll
    for (int m = 0; m < kTT; ++m) acc[m] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = ln + kLanes * t;
      const int cc = c < ngk ? c : ngk - 1;
      const float mask = static_cast<float>(c < ngk);
      const uint32_t wq[4] = {wv[t].x, wv[t].y, wv[t].z, wv[t].w};
#pragma unroll
      for (int m = 0; m < kTT; ++m) {
        if (m < mt) {
          float part = 0.f;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint4 xv = xd[static_cast<size_t>(m) * npos + 4 * cc + p];
            const int tq = sdot8(wq[p], xv.x, 0) + 16 * sdot8(wq[p], xv.y, 0) +
                           256 * sdot8(wq[p], xv.z, 0) + 4096 * sdot8(wq[p], xv.w, 0);
            part = fmaf(static_cast<float>(tq), xs[static_cast<size_t>(m) * npos + 4 * cc + p], part);
          }
          acc[m] = fmaf(part, fw[t] * mask, acc[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kTT; ++m) {
      const float v = seg_sum<kLanes>(acc[m]);
      if (m < mt && ln == 0 && live) {
        const int row = r0 + m0 + m;
        if (s < A.E) A.out_r[static_cast<size_t>(row) * A.H + n] = v;
        else A.out_s[static_cast<size_t>(row) * A.H + n] = v;
      }
    }
  }
}

// y[t] = (x'[t] if residual) + out_s[t] + sum_j w[t][j] * out_r[pos_of[t*k + j]]
__global__ void k_bcombine(const float* __restrict__ out_s, const float* __restrict__ out_r,
                           const int32_t* __restrict__ pos_of, const float* __restrict__ w,
                           const float* __restrict__ x, const uint16_t* __restrict__ add_in,
                           int residual, int H, int k, float* __restrict__ y) {
  const int t = blockIdx.y;
  for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < H; n += gridDim.x * blockDim.x) {
    float v = out_s[static_cast<size_t>(t) * H + n];
    for (int j = 0; j < k; ++j)
      v = fmaf(w[t * k + j], out_r[static_cast<size_t>(pos_of[t * k + j]) * H + n], v);
    float r = 0.f;
    if (residual) r = x[static_cast<size_t>(t) * H + n] + (add_in ? h2f(add_in[static_cast<size_t>(t) * H + n]) : 0.f);
    y[static_cast<size_t>(t) * H + n] = r + v;
  }
}

}  // namespace

hipError_t launch_batched(const BatchedBuffers& bb, const uint8_t* experts, const uint8_t* shared,
                          size_t blob_e, int H, int I, int Is, int E, int k, int B,
                          const DigitGroup* udig, const float* usc, const float* w, const float* x,
                          const uint16_t* add_in, bool residual, float* y, hipStream_t s) {
  BatchArgs A{experts, shared, blob_e, H, I, Is, E, k, B, bb.seg, bb.perm, udig, usc,
              bb.adig_r, bb.asc_r, bb.adig_s, bb.asc_s, bb.out_r, bb.out_s};
  const int ngu = H / kGroup;
  // gate/up: (E + 1) segments x row tiles of 32 pairs (the longest segment sets the grid)
  const int inter_max = I > Is ? I : Is;
  const int tiles_gu = (inter_max + kWaves * kRowsPerWave - 1) / (kWaves * kRowsPerWave);
  const size_t lds_gu = static_cast<size_t>(kTT) * ngu * (sizeof(DigitGroup) + sizeof(float));
  const int need_gu = (ngu + kLanes - 1) / kLanes;
#define MOE_BGU(NT) hipLaunchKernelGGL(k_bgateup<NT>, dim3((E + 1) * tiles_gu), dim3(kThreads), lds_gu, s, A, tiles_gu)
  if (need_gu <= 2) MOE_BGU(2);
  else if (need_gu <= 4) MOE_BGU(4);
  else if (need_gu <= 8) MOE_BGU(8);
  else if (need_gu <= 11) MOE_BGU(11);
  else if (need_gu <= 16) MOE_BGU(16);
  else MOE_BGU(32);
#undef MOE_BGU
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // down: (E + 1) segments x 32-row output tiles; the K loop covers the longer segment
  const int tiles_dn = (H + kWaves * kRowsPerWave - 1) / (kWaves * kRowsPerWave);
  const int npos_max = inter_max / 8;
  const size_t lds_dn = static_cast<size_t>(kTT) * npos_max * (sizeof(uint4) + sizeof(float));
  const int need_dn = (inter_max / kGroup + kLanes - 1) / kLanes;
#define MOE_BDN(NT) hipLaunchKernelGGL(k_bdown<NT>, dim3((E + 1) * tiles_dn), dim3(kThreads), lds_dn, s, A, tiles_dn)
  if (need_dn <= 2) MOE_BDN(2);
  else if (need_dn <= 3) MOE_BDN(3);
  else if (need_dn <= 4) MOE_BDN(4);
  else if (need_dn <= 9) MOE_BDN(9);
  else if (need_dn <= 16) MOE_BDN(16);
  else MOE_BDN(32);
#undef MOE_BDN
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_bcombine, dim3((H + 255) / 256, B), dim3(256), 0, s, bb.out_s, bb.out_r, bb.pos_of, w,
                     x, add_in, residual ? 1 : 0, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
