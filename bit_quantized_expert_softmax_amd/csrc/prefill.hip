// Prefill of T tokens through one MoE layer on the bf16 matrix cores.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", section "Desempenho no mundo real": prefill groups
// rows so that one loaded expert serves a group of token rows at once. Here
// the T*k (token, rank) assignments are sorted by expert (stable: expert,
// token, rank), each expert's rows form one GEMM against its int4 weights,
// which are dequantised tile by tile into bf16 in LDS; bf16 MFMA with fp32
// accumulation computes gate/up, the GeGLU activation is rounded to bf16,
// the down GEMM weights each row by its routing weight, and the shared
// expert's down GEMM adds the k routed rows of every token in rank order.
//
// Stages (one launch each): count per 256-assignment chunk, scan (expert
// offsets and the GEMM tile table), stable scatter, routed gate/up, shared
// gate/up, routed down, shared down + combine.
#include "launch.h"
#include "moedecode.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 256;   // assignments per counting chunk
constexpr int kTM = 64;       // GEMM tile rows
constexpr int kTK = 32;       // K step = one quantisation group
constexpr int kThreadsG = 256;
constexpr int kLdsRow = 40;   // bf16 per LDS tile row (32 + pad against bank conflicts)

// ---------------------------------------------------------------- permutation
__global__ __launch_bounds__(kChunk) void k_perm_count(const int32_t* __restrict__ ids, int n_asg, int E,
                                                       int32_t* __restrict__ hist,
                                                       int32_t* __restrict__ local_rank) {
  __shared__ int es[kChunk];
  const int c = blockIdx.x;
  const int a = c * kChunk + threadIdx.x;
  const int e = a < n_asg ? ids[a] : -1;
  es[threadIdx.x] = e;
  __syncthreads();
  if (a < n_asg) {
    int r = 0;
    for (int i = 0; i < static_cast<int>(threadIdx.x); ++i) r += es[i] == e ? 1 : 0;
    local_rank[a] = r;
  }
  for (int f = threadIdx.x; f < E; f += kChunk) {
    int n = 0;
    for (int i = 0; i < kChunk; ++i) n += es[i] == f ? 1 : 0;
    hist[static_cast<size_t>(c) * E + f] = n;
  }
}

// Single block: expert offsets (seg [E+1]), per-(chunk, expert) bases, and the
// routed tile table (expert, first row) with its length in *n_tiles.
__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ hist, int C, int E,
                                                    int32_t* __restrict__ base, int32_t* __restrict__ seg,
                                                    int2* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int tot[MOE_MAX_EXPERTS + 1];
  __shared__ int tstart[MOE_MAX_EXPERTS + 1];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int c = 0; c < C; ++c) s += hist[static_cast<size_t>(c) * E + e];
    tot[e] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0, t = 0;
    for (int e = 0; e < E; ++e) {
      const int n = tot[e];
      tot[e] = s;  // becomes the exclusive prefix
      tstart[e] = t;
      s += n;
      t += (n + kTM - 1) / kTM;
    }
    tot[E] = s;
    tstart[E] = t;
    *n_tiles = t;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) seg[e] = tot[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = tot[e];
    for (int c = 0; c < C; ++c) {
      base[static_cast<size_t>(c) * E + e] = s;
      s += hist[static_cast<size_t>(c) * E + e];
    }
    const int rows = tot[e + 1] - tot[e];
    for (int m = 0; m < rows; m += kTM) tiles[tstart[e] + m / kTM] = make_int2(e, tot[e] + m);
  }
}

__global__ __launch_bounds__(kChunk) void k_perm_scatter(const int32_t* __restrict__ ids, int n_asg, int E,
                                                         const int32_t* __restrict__ base,
                                                         const int32_t* __restrict__ local_rank,
                                                         int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ pos_of) {
  const int a = blockIdx.x * kChunk + threadIdx.x;
  if (a >= n_asg) return;
  const int p = base[static_cast<size_t>(blockIdx.x) * E + ids[a]] + local_rank[a];
  perm[p] = a;
  pos_of[a] = p;
}

// ---------------------------------------------------------------- grouped GEMM
__device__ __forceinline__ bf16x8 lds_frag(const __bf16* tile, int row, int lane) {
  return *reinterpret_cast<const bf16x8*>(tile + row * kLdsRow + 8 * (lane >> 4));
}

// Dequantises 16 consecutive K values (8 bytes of nibbles, one fp16 scale) of
// one weight row to bf16 and stores them to LDS.
__device__ __forceinline__ void dequant16(uint2 q, uint16_t s, __bf16* dst) {
  const float sc = h2f(s);
  __attribute__((aligned(16))) __bf16 v[16];
  const uint32_t w[2] = {q.x, q.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int nib = static_cast<int>((w[h] >> (4 * i)) & 15u);
      const int sv = nib >= 8 ? nib - 16 : nib;
      v[8 * h + i] = static_cast<__bf16>(static_cast<float>(sv) * sc);  // exact product, RNE to bf16
    }
  }
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(v);
  *reinterpret_cast<uint4*>(dst + 8) = *reinterpret_cast<const uint4*>(v + 8);
}

struct GemmArgs {
  // A rows: row r of a tile = A + row_index * lda (bf16), where row_index is
  // rmap[r_global] / rdiv when rmap is given, else r_global
  const __bf16* A;
  int lda;
  const int32_t* rmap;
  int rdiv;
  // weights: blob of one source (shared) or experts + e * blob_e (routed)
  const uint8_t* blob;
  const uint8_t* experts;
  size_t blob_e;
  int H, inter;
  // routed tiles from the table (tiles/n_tiles/seg), or a dense M x N job
  const int2* tiles;
  const int32_t* n_tiles;
  const int32_t* seg;
  int M_dense;
  // outputs
  __bf16* act;        // gate/up: activations [rows][inter] bf16
  float* out;         // down: [rows][H] fp32 (routed, weighted) or y [T][H] (shared)
  const float* wrow;  // routed down: routing weight per assignment (by perm[row])
  const int32_t* perm;
  // shared down: y[t] = o_shared[t] + sum_j out_r[pos_of[t*k + j]]
  const float* out_r;
  const int32_t* pos_of;
  int k;
};

// GATEUP: tile = 64 rows x (64 gate + 64 up) columns of one source; a wave
//   owns gate sub-tile w and the matching up sub-tile, so each lane holds g
//   and v of the same (row, column) and applies GeGLU in registers.
// DOWN:   tile = 64 rows x 128 output columns; a wave owns 2 column sub-tiles.
template <bool GATEUP, bool ROUTED>
__global__ __launch_bounds__(kThreadsG) void k_gemm(GemmArgs G) {
  __shared__ __attribute__((aligned(16))) __bf16 As[kTM * kLdsRow];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[128 * kLdsRow];
  const int n_tiles_n = GATEUP ? G.inter / 64 : G.H / 128;
  const int mt = blockIdx.x / n_tiles_n;
  const int nt = blockIdx.x % n_tiles_n;
  int r0, r_end;
  const uint8_t* blob;
  if (ROUTED) {
    if (mt >= *G.n_tiles) return;
    const int2 td = G.tiles[mt];
    r0 = td.y;
    r_end = G.seg[td.x + 1];
    blob = G.experts + static_cast<size_t>(td.x) * G.blob_e;
  } else {
    r0 = mt * kTM;
    r_end = G.M_dense;
    if (r0 >= r_end) return;
    blob = G.blob;
  }
  const BlobOffsets o = blob_offsets(G.H, G.inter);
  const int K = GATEUP ? G.H : G.inter;
  const int ngk = K / kGroup;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);

  // A loader: thread t loads row t/4, 8 bf16 at k offset 8*(t%4)
  const int ar = threadIdx.x >> 2;
  const int ak = 8 * (threadIdx.x & 3);
  const int arow_g = r0 + ar < r_end ? r0 + ar : r_end - 1;
  const int aidx = G.rmap ? G.rmap[arow_g] / G.rdiv : arow_g;
  const __bf16* arow = G.A + static_cast<size_t>(aidx) * G.lda + ak;
  // B loader: thread t dequantises column t/2 (of 128), K half t%2 (16 values)
  const int bc = threadIdx.x >> 1;
  const int bh = threadIdx.x & 1;
  const uint8_t* bq;
  const uint16_t* bs;
  if (GATEUP) {
    const int n = nt * 64 + (bc & 63);
    const bool up = bc >= 64;
    bq = blob + (up ? o.up_q : o.gate_q) + static_cast<size_t>(n) * (K / 2) + 8 * bh;
    bs = reinterpret_cast<const uint16_t*>(blob + (up ? o.up_s : o.gate_s)) + static_cast<size_t>(n) * ngk;
  } else {
    const int n = nt * 128 + bc;
    bq = blob + o.down_q + static_cast<size_t>(n) * (K / 2) + 8 * bh;
    bs = reinterpret_cast<const uint16_t*>(blob + o.down_s) + static_cast<size_t>(n) * ngk;
  }

  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < ngk; ++g) {
    const uint4 av = *reinterpret_cast<const uint4*>(arow + g * kTK);
    const uint2 qv = *reinterpret_cast<const uint2*>(bq + 16 * static_cast<size_t>(g));
    const uint16_t sv = bs[g];
    __syncthreads();  // previous step's fragments have been read
    *reinterpret_cast<uint4*>(As + ar * kLdsRow + ak) = av;
    dequant16(qv, sv, Bs + bc * kLdsRow + 16 * bh);
    __syncthreads();
    bf16x8 bfr[2];
    if (GATEUP) {
      bfr[0] = lds_frag(Bs, 16 * wave + (lane & 15), lane);
      bfr[1] = lds_frag(Bs, 64 + 16 * wave + (lane & 15), lane);
    } else {
      bfr[0] = lds_frag(Bs, 32 * wave + (lane & 15), lane);
      bfr[1] = lds_frag(Bs, 32 * wave + 16 + (lane & 15), lane);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 afr = lds_frag(As, 16 * i + (lane & 15), lane);
      acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[0], acc[i][0], 0, 0, 0);
      acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[1], acc[i][1], 0, 0, 0);
    }
  }

  // epilogue: lane holds rows 16i + 4*(lane/16) + r, column (lane % 16) of each sub-tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = r0 + 16 * i + 4 * (lane >> 4) + r;
      if (m >= r_end) continue;
      if (GATEUP) {
        const int n = nt * 64 + 16 * wave + (lane & 15);
        const float a = gelu_tanh(acc[i][0][r]) * acc[i][1][r];
        G.act[static_cast<size_t>(m) * G.inter + n] = static_cast<__bf16>(a);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = nt * 128 + 32 * wave + 16 * j + (lane & 15);
          float v = acc[i][j][r];
          if (ROUTED) {
            G.out[static_cast<size_t>(m) * G.H + n] = v * G.wrow[G.perm[m]];
          } else {
            // shared expert output plus the token's routed rows in rank order
            for (int jj = 0; jj < G.k; ++jj)
              v += G.out_r[static_cast<size_t>(G.pos_of[m * G.k + jj]) * G.H + n];
            G.out[static_cast<size_t>(m) * G.H + n] = v;
          }
        }
      }
    }
  }
}

__global__ void k_bf16_to_f32(const uint16_t* __restrict__ x, size_t n, float* __restrict__ y) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    y[i] = __uint_as_float(static_cast<uint32_t>(x[i]) << 16);
}

}  // namespace

int permute_chunks(int A) { return (A + kChunk - 1) / kChunk; }

hipError_t launch_permute(const int32_t* ids, int A, int E, int chunks, int32_t* hist, int32_t* lrank,
                          int32_t* base, int32_t* seg, int2* tiles, int32_t* n_tiles, int32_t* perm,
                          int32_t* pos_of, hipStream_t s) {
  hipLaunchKernelGGL(k_perm_count, dim3(chunks), dim3(kChunk), 0, s, ids, A, E, hist, lrank);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, hist, chunks, E, base, seg, tiles, n_tiles);
  hipLaunchKernelGGL(k_perm_scatter, dim3(chunks), dim3(kChunk), 0, s, ids, A, E, base, lrank, perm, pos_of);
  return hipGetLastError();
}

PrefillLayout prefill_layout(int T, int E, int k, int H, int I, int Is) {
  PrefillLayout L{};
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += (n + 255) & ~static_cast<size_t>(255);
    return o;
  };
  const size_t A = static_cast<size_t>(T) * k;
  const size_t C = (A + kChunk - 1) / kChunk;
  L.chunks = static_cast<int>(C);
  L.max_tiles = static_cast<int>((A + kTM - 1) / kTM + E);
  L.ids = take(A * 4);
  L.w = take(A * 4);
  L.hist = take(C * E * 4);
  L.base = take(C * E * 4);
  L.local_rank = take(A * 4);
  L.seg = take((E + 1) * 4);
  L.tiles = take(static_cast<size_t>(L.max_tiles) * 8);
  L.n_tiles = take(4);
  L.perm = take(A * 4);
  L.pos_of = take(A * 4);
  L.act_r = take(A * I * 2);
  L.act_s = take(static_cast<size_t>(T) * Is * 2);
  L.out_r = take(A * H * 4);
  L.xf = take(static_cast<size_t>(T) * H * 4);
  L.z = take(static_cast<size_t>(T) * E * 8);
  L.total = off;
  return L;
}

hipError_t launch_prefill(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16,
                          const float* logits_in, const uint16_t* router, const float* bias, int T,
                          int E, int k, int H, int I, int Is, const uint8_t* experts, size_t blob_e,
                          const uint8_t* shared, float* y, int32_t* ids_out, float* w_out,
                          hipStream_t s) {
  auto at = [&](size_t off) { return ws + off; };
  int32_t* ids = reinterpret_cast<int32_t*>(at(L.ids));
  float* w = reinterpret_cast<float*>(at(L.w));
  hipError_t e;
  if (logits_in) {
    e = launch_route_topk(nullptr, logits_in, T, E, k, ids, w, ids_out, w_out, s);
  } else {
    float* xf = reinterpret_cast<float*>(at(L.xf));
    const size_t n = static_cast<size_t>(T) * H;
    hipLaunchKernelGGL(k_bf16_to_f32, dim3(static_cast<unsigned>((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536)),
                       dim3(256), 0, s, x_bf16, n, xf);
    e = hipGetLastError();
    if (e == hipSuccess) e = launch_route_logits(xf, T, H, router, bias, E, reinterpret_cast<double*>(at(L.z)), s);
    if (e == hipSuccess)
      e = launch_route_topk(reinterpret_cast<double*>(at(L.z)), nullptr, T, E, k, ids, w, ids_out, w_out, s);
  }
  if (e != hipSuccess) return e;
  const int A = T * k;
  int32_t* hist = reinterpret_cast<int32_t*>(at(L.hist));
  int32_t* base = reinterpret_cast<int32_t*>(at(L.base));
  int32_t* lrank = reinterpret_cast<int32_t*>(at(L.local_rank));
  int32_t* seg = reinterpret_cast<int32_t*>(at(L.seg));
  int2* tiles = reinterpret_cast<int2*>(at(L.tiles));
  int32_t* n_tiles = reinterpret_cast<int32_t*>(at(L.n_tiles));
  int32_t* perm = reinterpret_cast<int32_t*>(at(L.perm));
  int32_t* pos_of = reinterpret_cast<int32_t*>(at(L.pos_of));
  if ((e = launch_permute(ids, A, E, L.chunks, hist, lrank, base, seg, tiles, n_tiles, perm, pos_of, s)) !=
      hipSuccess)
    return e;

  const __bf16* x = reinterpret_cast<const __bf16*>(x_bf16);
  __bf16* act_r = reinterpret_cast<__bf16*>(at(L.act_r));
  __bf16* act_s = reinterpret_cast<__bf16*>(at(L.act_s));
  float* out_r = reinterpret_cast<float*>(at(L.out_r));

  GemmArgs g{};
  g.H = H;
  g.k = k;
  // routed gate/up: rows are assignments in expert order, A row = token = perm / k
  g.A = x;
  g.lda = H;
  g.rmap = perm;
  g.rdiv = k;
  g.experts = experts;
  g.blob_e = blob_e;
  g.inter = I;
  g.tiles = tiles;
  g.n_tiles = n_tiles;
  g.seg = seg;
  g.act = act_r;
  hipLaunchKernelGGL((k_gemm<true, true>), dim3(L.max_tiles * (I / 64)), dim3(kThreadsG), 0, s, g);
  // shared gate/up: dense over tokens
  GemmArgs gs = g;
  gs.rmap = nullptr;
  gs.blob = shared;
  gs.inter = Is;
  gs.M_dense = T;
  gs.act = act_s;
  hipLaunchKernelGGL((k_gemm<true, false>), dim3(((T + kTM - 1) / kTM) * (Is / 64)), dim3(kThreadsG), 0, s, gs);
  // routed down: rows are the permuted activations, weighted by their routing weight
  GemmArgs d = g;
  d.A = act_r;
  d.lda = I;
  d.rmap = nullptr;
  d.out = out_r;
  d.wrow = w;
  d.perm = perm;
  hipLaunchKernelGGL((k_gemm<false, true>), dim3(L.max_tiles * (H / 128)), dim3(kThreadsG), 0, s, d);
  // shared down + combine into y
  GemmArgs ds = gs;
  ds.A = act_s;
  ds.lda = Is;
  ds.out = y;
  ds.out_r = out_r;
  ds.pos_of = pos_of;
  hipLaunchKernelGGL((k_gemm<false, false>), dim3(((T + kTM - 1) / kTM) * (H / 128)), dim3(kThreadsG), 0, s, ds);
  return hipGetLastError();
}

}  // namespace moe
