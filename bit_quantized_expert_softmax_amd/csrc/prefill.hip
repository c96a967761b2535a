// Prefill of T tokens through one MoE layer on the bf16 matrix cores.
//
// "Como executar um modelo de 26 bilhões de parâmetros em dois gigabytes de
// memória em um Mac comum", section "Desempenho no mundo real": prefill groups
// rows so that one loaded expert serves a group of token rows at once. Here
// the T*k (token, rank) assignments are sorted by expert (stable: expert,
// token, rank), each expert's rows form one GEMM against its int4 weights,
// which stream through registers and are dequantised there to bf16 (one
// rounding of the exact product); bf16 MFMA with fp32 accumulation computes
// gate/up against activation tiles staged in LDS, the GeGLU activation is
// rounded to bf16,
// the down GEMM weights each row by its routing weight, and the shared
// expert's down GEMM adds the k routed rows of every token in rank order.
//
// Stages (one launch each): count per 256-assignment chunk, scan (expert
// offsets and the GEMM tile table), stable scatter, routed gate/up, shared
// gate/up, routed down, shared down + combine.
#include <type_traits>

#include "launch.h"
#include "moedecode.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 256;   // assignments per counting chunk
constexpr int kTM = 128;      // GEMM tile rows (tokens)

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
// routed tile table (expert, first row) with its length in *n_tiles. P
// threads per expert (P = 1024 / E) each take a contiguous range of chunks;
// their partial counts meet in LDS, and the expert offsets and tile starts
// come from one block-wide scan (wave scans, then the waves' totals).
__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ hist, int C, int E,
                                                    int32_t* __restrict__ base, int32_t* __restrict__ seg,
                                                    int2* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  constexpr int kT = 1024;
  __shared__ int part[kT];
  __shared__ int tot[MOE_MAX_EXPERTS + 1];
  __shared__ int tst[MOE_MAX_EXPERTS + 1];
  __shared__ int wsum[kT / kWave][2];
  const int t = threadIdx.x;
  const int wave = t / kWave, lane = t % kWave;
  const int P = kT / E;  // E <= MOE_MAX_EXPERTS = 1024
  const int e = t / P, p = t % P;
  const bool on = e < E;
  const int per = (C + P - 1) / P;
  const int c0 = p * per;
  const int c1 = c0 + per < C ? c0 + per : C;
  int s = 0;
  if (on)
    for (int c = c0; c < c1; ++c) s += hist[static_cast<size_t>(c) * E + e];
  part[t] = s;
  __syncthreads();
  int off = 0;  // this thread's first row within its expert
  if (on)
    for (int q = 0; q < p; ++q) off += part[e * P + q];
  // expert t's rows and tiles, exclusive prefix over experts
  int n = 0;
  if (t < E)
    for (int q = 0; q < P; ++q) n += part[t * P + q];
  const int nt = (n + kTM - 1) / kTM;
  int a = n, b = nt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int ya = __shfl_up(a, d, kWave);
    const int yb = __shfl_up(b, d, kWave);
    if (lane >= d) {
      a += ya;
      b += yb;
    }
  }
  if (lane == kWave - 1) {
    wsum[wave][0] = a;
    wsum[wave][1] = b;
  }
  __syncthreads();
  int wa = 0, wb = 0;
  for (int w = 0; w < wave; ++w) {
    wa += wsum[w][0];
    wb += wsum[w][1];
  }
  if (t < E) {
    tot[t] = wa + a - n;
    tst[t] = wb + b - nt;
  }
  if (t == E - 1) {
    tot[E] = wa + a;
    tst[E] = wb + b;
    *n_tiles = wb + b;
  }
  __syncthreads();
  for (int f = t; f <= E; f += kT) seg[f] = tot[f];
  if (on) {
    int r = tot[e] + off;
    for (int c = c0; c < c1; ++c) {
      base[static_cast<size_t>(c) * E + e] = r;
      r += hist[static_cast<size_t>(c) * E + e];
    }
    const int rows = tot[e + 1] - tot[e];
    for (int m = p * kTM; m < rows; m += P * kTM) tiles[tst[e] + m / kTM] = make_int2(e, tot[e] + m);
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
// Weight rows stream from HBM into registers and are dequantised there; the
// block's 128 activation rows are staged in LDS per K step (double buffered)
// and shared by its 8 waves. A wave owns two 16-row weight tiles (GATEUP: 16
// gate rows and the matching 16 up rows; else 32 consecutive down rows) and
// all 8 16-row token tiles, so each dequantised weight feeds 8 MFMAs. (Four
// tiles per wave halve the LDS reads per flop but need one wave per SIMD;
// measured slower, 1.04 vs 0.83 ms, as dequant, LDS reads and MFMAs of one
// wave then overlap too little.)
//
// K step = 4 quant groups (128 values). The lane of 16-lane row q loads group
// 4*st + q of its weight row (16 bytes) and that group's scale; MFMA j of the
// step takes dword j (8 nibbles) of every lane's group, so one MFMA's K = 32
// spans the step's 4 groups, 8 values of each, and the activations are read
// at the same positions. Loads are issued kDepth steps ahead (activation
// slice first, then weights) into a register ring whose slots are
// compile-time indices, so every wait is for the oldest unit only.
constexpr int kTok = kTM / 16;            // 16-token tiles per block
constexpr int kWavesG = 8;               // waves per GEMM block
constexpr int kThreadsGemm = kWavesG * kWave;
constexpr int kStage = kTM * 16 / kThreadsGemm;  // 16-byte activation chunks per thread and step
constexpr int kStepK = 4 * kGroup;       // 128
constexpr int kBRow = kStepK * 2 + 16;   // LDS bytes per activation row of a step (padded)
constexpr int kDepth = 4;
constexpr int kMR = 2;                   // 16-row weight tiles per wave (GATEUP: half gate, half up)
constexpr int kHalf = kMR / 2;

// Byte B of x as a float (v_cvt_f32_ubyteB; written out because the compiler
// folds the surrounding masks and then loses the byte-select forms).
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
  float r;
  if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// bf16(n * s) for the 8 signed nibbles of w (k = 0..7 in bits 4k..4k+3), in
// k order: the product (n + 8) * s - 8 * s is exact in fp32 (at most 15
// significant bits), so the single rounding is the one to bf16.
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t w, float s) {
  const uint32_t x = w ^ 0x88888888u;          // nibble n -> n + 8
  const uint32_t lo = x & 0x0F0F0F0Fu;         // byte b: k = 2b
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // byte b: k = 2b + 1
  const float m8 = -8.0f * s;
  bf16x8 r;
  r[0] = static_cast<__bf16>(fmaf(ubyte_f32<0>(lo), s, m8));
  r[1] = static_cast<__bf16>(fmaf(ubyte_f32<0>(hi), s, m8));
  r[2] = static_cast<__bf16>(fmaf(ubyte_f32<1>(lo), s, m8));
  r[3] = static_cast<__bf16>(fmaf(ubyte_f32<1>(hi), s, m8));
  r[4] = static_cast<__bf16>(fmaf(ubyte_f32<2>(lo), s, m8));
  r[5] = static_cast<__bf16>(fmaf(ubyte_f32<2>(hi), s, m8));
  r[6] = static_cast<__bf16>(fmaf(ubyte_f32<3>(lo), s, m8));
  r[7] = static_cast<__bf16>(fmaf(ubyte_f32<3>(hi), s, m8));
  return r;
}

struct WStep {
  uint4 q[kMR];
  uint32_t s[kMR];
};

__device__ __forceinline__ void load_step(WStep& b, const uint8_t* const* qrow,
                                          const uint16_t* const* srow, int ngk, int st, int q) {
  int g = 4 * st + q;
  g = g < ngk ? g : ngk - 1;
#pragma unroll
  for (int m = 0; m < kMR; ++m) {
    b.q[m] = *reinterpret_cast<const uint4*>(qrow[m] + 16 * static_cast<size_t>(g));
    b.s[m] = srow[m][g];
  }
}

struct GemmArgs {
  // activation rows: row r of the tile = A + index * lda (bf16), where index
  // is rmap[r] / rdiv when rmap is given, else r
  const __bf16* A;
  int lda;
  const int32_t* rmap;
  int rdiv;
  // weights: blob of one source (shared) or experts + e * blob_e (routed)
  const uint8_t* blob;
  const uint8_t* experts;
  size_t blob_e;
  int H, inter;
  // routed tiles from the table (tiles/n_tiles/seg), or a dense job of M_dense rows
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
  // routed, slot pool: only the tiles of these experts run, each expert's
  // weights at experts + slot * blob_e (n_group == 0: every expert, at its id)
  SlotGroup group;
};

// One block's tile (block index bid of its job); lds_b: two activation slice
// buffers of kTM * kBRow bytes.
template <bool GATEUP, bool ROUTED>
__device__ __forceinline__ void gemm_tile(const GemmArgs& G, int bid, uint8_t (*lds_b)[kTM * kBRow]) {
  constexpr int rows_per_block = GATEUP ? kWavesG * kHalf * 16 : kWavesG * kMR * 16;
  const int nrows = GATEUP ? G.inter : G.H;
  const int n_tiles_n = (nrows + rows_per_block - 1) / rows_per_block;
  const int mt = bid / n_tiles_n;
  const int nt = bid % n_tiles_n;
  int r0, r_end;
  const uint8_t* blob;
  if (ROUTED) {
    if (mt >= *G.n_tiles) return;
    const int2 td = G.tiles[mt];
    int where = td.x;  // expert id (resident) or its slot (slot pool)
    if (G.group.n > 0) {
      where = -1;
      for (int i = 0; i < G.group.n; ++i)
        if (G.group.expert[i] == td.x) where = G.group.slot[i];
      if (where < 0) return;  // uniform over the block: not this group's expert
    }
    r0 = td.y;
    const int e_end = G.seg[td.x + 1];
    r_end = r0 + kTM < e_end ? r0 + kTM : e_end;
    blob = G.experts + static_cast<size_t>(where) * G.blob_e;
  } else {
    r0 = mt * kTM;
    if (r0 >= G.M_dense) return;
    r_end = r0 + kTM < G.M_dense ? r0 + kTM : G.M_dense;
    blob = G.blob;
  }
  const int mtok = r_end - r0;
  const BlobOffsets o = blob_offsets(G.H, G.inter);
  const int K = GATEUP ? G.H : G.inter;
  const int ngk = K / kGroup;
  const int nsteps = (ngk + 3) / 4;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int rbase = nt * rows_per_block + wave * (GATEUP ? kHalf * 16 : kMR * 16);
  const bool live = rbase < nrows;  // waves past the last row only stage and sync
  const uint8_t* qrow[kMR];
  const uint16_t* srow[kMR];
#pragma unroll
  for (int mr = 0; mr < kMR; ++mr) {
    int row = (GATEUP ? rbase + 16 * (mr % kHalf) : rbase + 16 * mr) + l16;
    row = live && row < nrows ? row : l16;
    const bool up = mr >= kHalf;
    const size_t qo = GATEUP ? (up ? o.up_q : o.gate_q) : o.down_q;
    const size_t so = GATEUP ? (up ? o.up_s : o.gate_s) : o.down_s;
    qrow[mr] = blob + qo + static_cast<size_t>(row) * (K / 2);
    srow[mr] = reinterpret_cast<const uint16_t*>(blob + so) + static_cast<size_t>(row) * ngk;
  }
  // this thread's 16-byte chunks of an activation slice (row = c / 16)
  const __bf16* brow[kStage];
  int boff[kStage], loff[kStage];
#pragma unroll
  for (int r = 0; r < kStage; ++r) {
    int c = threadIdx.x + kThreadsGemm * r;
    c = c < mtok * 16 ? c : mtok * 16 - 1;
    const int row = r0 + (c >> 4);
    const int idx = G.rmap ? G.rmap[row] / G.rdiv : row;
    brow[r] = G.A + static_cast<size_t>(idx) * G.lda;
    boff[r] = 8 * (c & 15);
    loff[r] = (c >> 4) * kBRow + 16 * (c & 15);
  }

  f32x4 acc[kMR][kTok];
#pragma unroll
  for (int mr = 0; mr < kMR; ++mr)
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) acc[mr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  WStep w[kDepth];
  u32x4 bs[kDepth][kStage];
  // st past the last step re-reads the last step: every step issues the same
  // loads, so the wait counts are the same on every path
  auto issue = [&](int st, WStep& wd, u32x4* bd) __attribute__((always_inline)) {
    st = st < nsteps ? st : nsteps - 1;
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      int kk = st * kStepK + boff[r];
      kk = kk < K ? kk : K - 8;  // past the end: any finite values (their weights are 0)
      bd[r] = *reinterpret_cast<const u32x4*>(brow[r] + kk);
    }
    load_step(wd, qrow, srow, ngk, st, q);
  };
  auto stage_store = [&](int bi, const u32x4* bd) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < kStage; ++r) *reinterpret_cast<u32x4*>(lds_b[bi] + loff[r]) = bd[r];
  };
  auto step = [&](auto slot, int s0, bool tail) __attribute__((always_inline)) {
    constexpr int D = decltype(slot)::value;
    const int st = s0 + D;
    if (tail && st >= nsteps) return;  // uniform over the block
    stage_store((st + 1) & 1, bs[(D + 1) % kDepth]);  // past the end: unused
    const uint8_t* lb = lds_b[st & 1];
    const bool gv = 4 * st + q < ngk;  // groups past K weigh 0
    bf16x8 a[kMR][4];
#pragma unroll
    for (int mr = 0; mr < kMR; ++mr) {
      const float sc = gv ? h2f(static_cast<uint16_t>(w[D].s[mr])) : 0.0f;
      a[mr][0] = dequant8_bf16(w[D].q[mr].x, sc);
      a[mr][1] = dequant8_bf16(w[D].q[mr].y, sc);
      a[mr][2] = dequant8_bf16(w[D].q[mr].z, sc);
      a[mr][3] = dequant8_bf16(w[D].q[mr].w, sc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // every token tile, also past mtok: an output column depends on its
      // own activation row only, and the columns of absent rows are dropped
#pragma unroll
      for (int tt = 0; tt < kTok; ++tt) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(lb + (tt * 16 + l16) * kBRow + 64 * q + 16 * j);
#pragma unroll
        for (int mr = 0; mr < kMR; ++mr)
          acc[mr][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mr][j], bv, acc[mr][tt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(st + kDepth, w[D], bs[D]);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  static_assert(kDepth == 3 || kDepth == 4, "the step sequence below is written out for 3 or 4 slots");
  constexpr int kD3 = kDepth > 3 ? 3 : 0;
  issue(0, w[0], bs[0]);
  issue(1, w[1], bs[1]);
  issue(2, w[2], bs[2]);
  if constexpr (kDepth > 3) issue(3, w[kD3], bs[kD3]);
  stage_store(0, bs[0]);
  __syncthreads();
  int s0 = 0;
  for (; s0 + kDepth <= nsteps; s0 += kDepth) {
    step(std::integral_constant<int, 0>{}, s0, false);
    step(std::integral_constant<int, 1>{}, s0, false);
    step(std::integral_constant<int, 2>{}, s0, false);
    if constexpr (kDepth > 3) step(std::integral_constant<int, kD3>{}, s0, false);
  }
  if (s0 < nsteps) {  // the last 1..kDepth-1 steps
    step(std::integral_constant<int, 0>{}, s0, true);
    step(std::integral_constant<int, 1>{}, s0, true);
    if constexpr (kDepth > 3) step(std::integral_constant<int, 2>{}, s0, true);
  }

  // epilogue: a lane holds rows 4q..4q+3 of each weight tile for token row
  // l16 of each token tile
#pragma unroll
  for (int tt = 0; tt < kTok; ++tt) {
    const int m = r0 + tt * 16 + l16;
    if (m >= r_end || !live) continue;
    if (GATEUP) {
#pragma unroll
      for (int mr = 0; mr < kHalf; ++mr) {
        __attribute__((aligned(8))) __bf16 av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[i] = static_cast<__bf16>(gelu_tanh(acc[mr][tt][i]) * acc[mr + kHalf][tt][i]);
        *reinterpret_cast<uint2*>(G.act + static_cast<size_t>(m) * G.inter + rbase + 16 * mr + 4 * q) =
            *reinterpret_cast<const uint2*>(av);
      }
    } else {
#pragma unroll
      for (int mr = 0; mr < kMR; ++mr) {
        const int n = rbase + 16 * mr + 4 * q;
        float4 v = make_float4(acc[mr][tt][0], acc[mr][tt][1], acc[mr][tt][2], acc[mr][tt][3]);
        if (ROUTED) {
          const float wr = G.wrow[G.perm[m]];
          v = make_float4(v.x * wr, v.y * wr, v.z * wr, v.w * wr);
        } else {
          // shared expert output plus the token's routed rows in rank order
          for (int jj = 0; jj < G.k; ++jj) {
            const float4 r = *reinterpret_cast<const float4*>(
                G.out_r + static_cast<size_t>(G.pos_of[m * G.k + jj]) * G.H + n);
            v = make_float4(v.x + r.x, v.y + r.y, v.z + r.z, v.w + r.w);
          }
        }
        *reinterpret_cast<float4*>(G.out + static_cast<size_t>(m) * G.H + n) = v;
      }
    }
  }
}

template <bool GATEUP, bool ROUTED>
__global__ __launch_bounds__(kThreadsGemm) void k_gemm(GemmArgs G) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kTM * kBRow];
  gemm_tile<GATEUP, ROUTED>(G, blockIdx.x, lds_b);
}

// The shared expert's gate/up (dense over the tokens, its n_shared blocks
// first) and the routed experts' gate/up in one launch: the two are
// independent, and the shared blocks, few and long, would otherwise form a
// launch of their own with a tail of one block per CU.
__global__ __launch_bounds__(kThreadsGemm) void k_gemm_gateup2(GemmArgs R, GemmArgs Sh, int n_shared) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kTM * kBRow];
  const int bid = blockIdx.x;
  if (bid < n_shared)
    gemm_tile<true, false>(Sh, bid, lds_b);
  else
    gemm_tile<true, true>(R, bid - n_shared, lds_b);
}

// Blocks along the weight rows of one GEMM (gate/up: row pairs; down: rows).
int gemm_row_tiles(bool gateup, int H, int inter) {
  const int rows = gateup ? inter : H;
  const int per = gateup ? kWavesG * kHalf * 16 : kWavesG * kMR * 16;
  return (rows + per - 1) / per;
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

hipError_t launch_prefill_route(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16,
                                const float* logits_in, const uint16_t* router, const float* bias, int T,
                                int E, int k, int H, int32_t* ids_out, float* w_out, hipStream_t s) {
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
  return launch_permute(ids, T * k, E, L.chunks, reinterpret_cast<int32_t*>(at(L.hist)),
                        reinterpret_cast<int32_t*>(at(L.local_rank)), reinterpret_cast<int32_t*>(at(L.base)),
                        reinterpret_cast<int32_t*>(at(L.seg)), reinterpret_cast<int2*>(at(L.tiles)),
                        reinterpret_cast<int32_t*>(at(L.n_tiles)), reinterpret_cast<int32_t*>(at(L.perm)),
                        reinterpret_cast<int32_t*>(at(L.pos_of)), s);
}

namespace {
GemmArgs routed_args(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16, int k, int H, int I,
                     const uint8_t* experts, size_t blob_e) {
  auto at = [&](size_t off) { return ws + off; };
  GemmArgs g{};
  g.H = H;
  g.k = k;
  // routed gate/up: rows are assignments in expert order, A row = token = perm / k
  g.A = reinterpret_cast<const __bf16*>(x_bf16);
  g.lda = H;
  g.rmap = reinterpret_cast<const int32_t*>(at(L.perm));
  g.rdiv = k;
  g.experts = experts;
  g.blob_e = blob_e;
  g.inter = I;
  g.tiles = reinterpret_cast<const int2*>(at(L.tiles));
  g.n_tiles = reinterpret_cast<const int32_t*>(at(L.n_tiles));
  g.seg = reinterpret_cast<const int32_t*>(at(L.seg));
  g.act = reinterpret_cast<__bf16*>(at(L.act_r));
  return g;
}
}  // namespace

namespace {
GemmArgs shared_gateup_args(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16, int T, int k, int H,
                            int Is, const uint8_t* shared) {
  GemmArgs gs{};
  gs.H = H;
  gs.k = k;
  gs.A = reinterpret_cast<const __bf16*>(x_bf16);
  gs.lda = H;
  gs.blob = shared;
  gs.inter = Is;
  gs.M_dense = T;
  gs.act = reinterpret_cast<__bf16*>(ws + L.act_s);
  return gs;
}
}  // namespace

hipError_t launch_prefill_routed(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16, int k, int H,
                                 int I, const uint8_t* experts, size_t blob_e, const SlotGroup* group,
                                 hipStream_t s, const SharedGateup* with_shared) {
  GemmArgs g = routed_args(L, ws, x_bf16, k, H, I, experts, blob_e);
  if (group) {
    if (group->n < 1 || group->n > kMaxGroup) return hipErrorInvalidValue;
    g.group = *group;
  }
  const int routed_blocks = L.max_tiles * gemm_row_tiles(true, H, I);
  if (with_shared) {
    const GemmArgs gs = shared_gateup_args(L, ws, x_bf16, with_shared->T, k, H, with_shared->Is, with_shared->shared);
    const int n_shared = ((with_shared->T + kTM - 1) / kTM) * gemm_row_tiles(true, H, with_shared->Is);
    hipLaunchKernelGGL(k_gemm_gateup2, dim3(n_shared + routed_blocks), dim3(kThreadsGemm), 0, s, g, gs, n_shared);
  } else {
    hipLaunchKernelGGL((k_gemm<true, true>), dim3(routed_blocks), dim3(kThreadsGemm), 0, s, g);
  }
  // routed down: rows are the permuted activations, weighted by their routing weight
  GemmArgs d = g;
  d.A = reinterpret_cast<const __bf16*>(ws + L.act_r);
  d.lda = I;
  d.rmap = nullptr;
  d.out = reinterpret_cast<float*>(ws + L.out_r);
  d.wrow = reinterpret_cast<const float*>(ws + L.w);
  d.perm = reinterpret_cast<const int32_t*>(ws + L.perm);
  hipLaunchKernelGGL((k_gemm<false, true>), dim3(L.max_tiles * gemm_row_tiles(false, H, I)), dim3(kThreadsGemm), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_prefill_shared(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16, int T, int k,
                                 int H, int Is, const uint8_t* shared, float* y, hipStream_t s, bool gateup_done) {
  const GemmArgs gs = shared_gateup_args(L, ws, x_bf16, T, k, H, Is, shared);
  // shared gate/up: dense over tokens (unless it ran with the routed one)
  if (!gateup_done)
    hipLaunchKernelGGL((k_gemm<true, false>), dim3(((T + kTM - 1) / kTM) * gemm_row_tiles(true, H, Is)), dim3(kThreadsGemm), 0, s, gs);
  // shared down + combine into y (each token's routed rows in rank order)
  GemmArgs ds = gs;
  ds.A = reinterpret_cast<const __bf16*>(ws + L.act_s);
  ds.lda = Is;
  ds.out = y;
  ds.out_r = reinterpret_cast<const float*>(ws + L.out_r);
  ds.pos_of = reinterpret_cast<const int32_t*>(ws + L.pos_of);
  hipLaunchKernelGGL((k_gemm<false, false>), dim3(((T + kTM - 1) / kTM) * gemm_row_tiles(false, H, Is)), dim3(kThreadsGemm), 0, s, ds);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16,
                          const float* logits_in, const uint16_t* router, const float* bias, int T,
                          int E, int k, int H, int I, int Is, const uint8_t* experts, size_t blob_e,
                          const uint8_t* shared, float* y, int32_t* ids_out, float* w_out,
                          hipStream_t s) {
  hipError_t e = launch_prefill_route(L, ws, x_bf16, logits_in, router, bias, T, E, k, H, ids_out, w_out, s);
  const SharedGateup sg{shared, T, Is};
  if (e == hipSuccess) e = launch_prefill_routed(L, ws, x_bf16, k, H, I, experts, blob_e, nullptr, s, &sg);
  if (e == hipSuccess) e = launch_prefill_shared(L, ws, x_bf16, T, k, H, Is, shared, y, s, true);
  return e;
}

}  // namespace moe
