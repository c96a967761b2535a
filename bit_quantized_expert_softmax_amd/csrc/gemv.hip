// Standalone int4 g32 GEMV for M token rows sharing one weight matrix, and
// the nibble unpack used for bit-exact checks.
//
// Weights are 4-bit with custom quantisation and GEMV kernels ("Como
// executar um modelo de 26 bilhões de parâmetros em dois gigabytes de memória
// em um Mac comum", section "Sem dependências do llama.cpp e MLX").
// y[m][n] = sum_k x[m][k] * nibble(n,k) * s[n][k/32].
#include "launch.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kLanesPerRow = 8;
constexpr int kRowsPerWave = kWave / kLanesPerRow;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
constexpr int kMaxTile = 8;  // token rows per pass

template <int NT>
__global__ __launch_bounds__(kThreads) void k_gemv_q4(const uint8_t* __restrict__ q,
                                                      const uint16_t* __restrict__ sc, int N, int K,
                                                      const float* __restrict__ x, int M, int tile,
                                                      float* __restrict__ y) {
  extern __shared__ uint4 lds_raw[];
  const int ng = K / kGroup;
  DigitGroup* xd = reinterpret_cast<DigitGroup*>(lds_raw);   // [tile][ng]
  float* xs = reinterpret_cast<float*>(xd + static_cast<size_t>(tile) * ng);  // [tile][ng]
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int n_raw = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave + lane / kLanesPerRow;
  const int n = n_raw < N ? n_raw : N - 1;  // rows past the end re-read the last row
  const int ln = lane & (kLanesPerRow - 1);
  const uint8_t* qrow = q + static_cast<size_t>(n) * (K / 2);
  const uint16_t* srow = sc + static_cast<size_t>(n) * ng;

  for (int m0 = 0; m0 < M; m0 += tile) {
    const int mt = (M - m0) < tile ? (M - m0) : tile;
    __syncthreads();  // previous tile's digits are no longer read
    const int half = (ng + 1) / 2;
    for (int p = wave; p < mt * half; p += kWaves) {
      const int m = p / half;
      const int g0 = 2 * (p % half);
      const int g = g0 + (lane >> 5);
      const float v = x[static_cast<size_t>(m0 + m) * K + (g < ng ? g : ng - 1) * kGroup + (lane & 31)];
      quant_pair_of_groups(g < ng ? v : 0.f, g0, ng, xd + static_cast<size_t>(m) * ng,
                           xs + static_cast<size_t>(m) * ng);
    }
    __syncthreads();
    float acc[kMaxTile];
#pragma unroll
    for (int m = 0; m < kMaxTile; ++m) acc[m] = 0.f;
    for (int c0 = 0; c0 < ng; c0 += kLanesPerRow * NT) {
      uint4 wv[NT];
      uint16_t sw[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        int c = c0 + ln + kLanesPerRow * t;
        c = c < ng ? c : ng - 1;
        wv[t] = load_w16(qrow + 16 * static_cast<size_t>(c));
        sw[t] = srow[c];
      }
      // keep every load of the batch ahead of the first use
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int c = c0 + ln + kLanesPerRow * t;
        const int cc = c < ng ? c : ng - 1;
        const float f = h2f(sw[t]) * static_cast<float>(c < ng);
#pragma unroll
        for (int m = 0; m < kMaxTile; ++m) {
          if (m < mt) {
            const int d = chunk_dot(wv[t], xd[static_cast<size_t>(m) * ng + cc]);
            acc[m] = fmaf(static_cast<float>(d), f * xs[static_cast<size_t>(m) * ng + cc], acc[m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kMaxTile; ++m) {
      const float v = seg_sum<kLanesPerRow>(acc[m]);
      if (m < mt && n_raw < N && ln == 0) y[static_cast<size_t>(m0 + m) * N + n] = v;
    }
  }
}

__global__ void k_unpack_q4(const uint8_t* __restrict__ q, size_t nbytes, int8_t* __restrict__ out) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < nbytes;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int b = q[i];
    const int lo = b & 15, hi = b >> 4;
    out[2 * i] = static_cast<int8_t>(lo >= 8 ? lo - 16 : lo);
    out[2 * i + 1] = static_cast<int8_t>(hi >= 8 ? hi - 16 : hi);
  }
}

}  // namespace

hipError_t launch_gemv_q4(const uint8_t* q, const uint16_t* sc, int N, int K, const float* x, int M,
                          float* y, hipStream_t s) {
  const int ng = K / kGroup;
  const size_t per_token = static_cast<size_t>(ng) * (sizeof(DigitGroup) + sizeof(float));
  int tile = static_cast<int>((64 * 1024) / per_token);
  tile = tile < 1 ? 1 : (tile > kMaxTile ? kMaxTile : tile);
  if (tile > M) tile = M;
  const int blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  const int need = (ng + kLanesPerRow - 1) / kLanesPerRow;
#define MOE_GEMV(NT) hipLaunchKernelGGL(k_gemv_q4<NT>, dim3(blocks), dim3(kThreads), per_token * tile, s, q, sc, N, K, x, M, tile, y)
  if (need <= 2) MOE_GEMV(2);
  else if (need <= 4) MOE_GEMV(4);
  else if (need <= 8) MOE_GEMV(8);
  else if (need <= 12) MOE_GEMV(12);
  else MOE_GEMV(16);
#undef MOE_GEMV
  return hipGetLastError();
}

hipError_t launch_unpack_q4(const uint8_t* q, int N, int K, int8_t* out, hipStream_t s) {
  const size_t nbytes = static_cast<size_t>(N) * (K / 2);
  size_t blocks = (nbytes + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_unpack_q4, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, q, nbytes, out);
  return hipGetLastError();
}

}  // namespace moe
