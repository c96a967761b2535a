// Standalone int4 g32 GEMV for M token rows sharing one weight matrix, the
// nibble unpack used for bit-exact checks, and a read-only stream that sets
// the floor one launch of a given size takes.
//
// Weights are 4-bit with custom quantisation and GEMV kernels ("Como
// executar um modelo de 26 bilhões de parâmetros em dois gigabytes de memória
// em um Mac comum", section "Sem dependências do llama.cpp e MLX").
// y[m][n] = sum_k x[m][k] * nibble(n,k) * s[n][k/32].
#include <hip/hip_ext.h>

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

// Read-only stream of n16 16-byte words: lane i of the grid loads words
// i, i + G, i + 2G, ... (G = grid threads; L of them, every load issued before
// any is used, the last word re-read where the range ends), folds them by XOR
// and the wave writes one word. It does no arithmetic on the data, so its
// duration is the floor for one launch that streams the same bytes on the same
// grid.
template <int L>
__global__ __launch_bounds__(1024) void k_read_floor(const uint8_t* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint4 v[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const int64_t i = i0 + j * stride;
    v[j] = load_w16(src + 16 * (i < n16 ? i : n16 - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < L; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  for (int o = kWave / 2; o >= 1; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o));
  if ((threadIdx.x & (kWave - 1)) == 0) out[blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave] = x;
}

}  // namespace

int read_floor_loads(int64_t bytes, int blocks) {
  const int64_t threads = static_cast<int64_t>(blocks) * 1024;
  return static_cast<int>((bytes / 16 + threads - 1) / threads);
}

hipError_t launch_read_floor(const uint8_t* src, int64_t bytes, int blocks, uint32_t* out, hipEvent_t t0,
                             hipEvent_t t1, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  switch (read_floor_loads(bytes, blocks)) {
#define MOE_FLOOR(L)                                                                                  \
  case L:                                                                                             \
    if (t0)                                                                                           \
      hipExtLaunchKernelGGL(k_read_floor<L>, dim3(blocks), dim3(1024), 0, s, t0, t1, 0, src, n16, out); \
    else                                                                                              \
      hipLaunchKernelGGL(k_read_floor<L>, dim3(blocks), dim3(1024), 0, s, src, n16, out);             \
    break;
    MOE_FLOOR(1) MOE_FLOOR(2) MOE_FLOOR(3) MOE_FLOOR(4) MOE_FLOOR(5) MOE_FLOOR(6) MOE_FLOOR(7) MOE_FLOOR(8)
    MOE_FLOOR(9) MOE_FLOOR(10) MOE_FLOOR(11) MOE_FLOOR(12) MOE_FLOOR(13) MOE_FLOOR(14) MOE_FLOOR(15)
    MOE_FLOOR(16)
#undef MOE_FLOOR
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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
