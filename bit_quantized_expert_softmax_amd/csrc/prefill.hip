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
// the routed down GEMM weights each row by its routing weight, the shared
// expert's down GEMM writes y, and a combine adds the k routed rows of every
// token to it in rank order.
//
// Stages (one launch each): count per 256-assignment chunk, scan (expert
// offsets and the GEMM tile table), stable scatter, shared + routed gate/up,
// shared + routed down, combine (through the slot pool the routed GEMMs run
// per group of resident experts, and the shared expert's on their own).
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
// routed tile table (expert, first row, rows) with its length in *n_tiles:
// an expert's n rows form ceil(n / 128) tiles of equal size rounded up to 16
// rows (the last one shorter), so no tile carries a mostly empty 128-row
// remainder (with 2048 tokens the mean expert has exactly 128 rows). P
// threads per expert (P = 1024 / E) each take a contiguous range of chunks;
// their partial counts meet in LDS, and the expert offsets and tile starts
// come from one block-wide scan (wave scans, then the waves' totals).
__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ hist, int C, int E,
                                                    int32_t* __restrict__ base, int32_t* __restrict__ seg,
                                                    int4* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
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
    const int ntl = (rows + kTM - 1) / kTM;
    const int size = ntl > 0 ? ((rows + ntl - 1) / ntl + 15) / 16 * 16 : 0;
    for (int m = p; m < ntl; m += P) {
      const int r0 = m * size;
      tiles[tst[e] + m] = make_int4(e, tot[e] + r0, rows - r0 < size ? rows - r0 : size, 0);
    }
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
// block's token rows are loaded per K step straight into LDS (global_load_lds,
// 16 bytes per lane, no registers on the way) into a ring of kBufs slices
// shared by its 4 waves. A wave owns two 32-row weight tiles (GATEUP: 32 gate
// rows and the matching 32 up rows; else 64 consecutive down rows) and all of
// the block's 32-token tiles (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
// each dequantised weight feeds up to 4 MFMAs and each activation operand
// read from LDS feeds 2, half the LDS bytes per flop of 16-row tiles.
//
// K step = 2 quant groups (64 values). The lane of 32-lane half h loads
// group 2*st + h of its weight row (16 bytes) and that group's scale; MFMA i
// of the step takes dword i (8 nibbles) of every lane's group, so one MFMA's
// K = 16 spans the step's 2 groups, 8 values of each, and the activations
// are read at the same positions (16-byte chunk 4h + i of the token's
// 128-byte step row).
//
// Pipeline: the loads of step s + kDepth (activation slice and weights) are
// issued at the start of step s, into the slice the previous step read; one
// barrier per step both frees the slice just read and publishes the next one
// (each wave has waited for its own loads of it). Within a step the weights
// of MFMA i + 1 are dequantised while the MFMAs of i run. The slice rows are
// 128-byte rows whose 8 chunks are stored XOR-swizzled (chunk c of token row
// t at position c ^ swz(t), swz(t) = (t & 7) ^ ((t >> 3) & 1)): the operand
// reads of 16 consecutive token rows at one chunk then fall on 16 different
// 16-byte bank groups over a 256-byte bank cycle, and on 8 over a 128-byte
// one.
constexpr int kWavesG = 4;               // waves per GEMM block
constexpr int kThreadsGemm = kWavesG * kWave;
constexpr int kStepK = 2 * kGroup;       // 64
constexpr int kRowB = kStepK * 2;        // LDS bytes per token row of a slice
constexpr int kSlice = kTM * kRowB;      // 16 KB
constexpr int kDepth = 3;                // steps loaded ahead of the one computed
constexpr int kBufs = kDepth + 1;        // slices in LDS (64 KB: two blocks per CU)
constexpr int kMR = 2;                   // 32-row weight tiles per wave (GATEUP: half gate, half up)
constexpr int kHalf = kMR / 2;
constexpr int kXcds = 8;                 // accelerator complex dies of an MI355X, each with its own L2

__device__ __forceinline__ int slice_swz(int t) { return (t & 7) ^ ((t >> 3) & 1); }

// s_waitcnt with vmcnt <= n and no wait on the other counters (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// bf16(n * s) for the 8 signed nibbles of w (k = 0..7 in bits 4k..4k+3), in
// k order. One and-xor (v_bitop3) per pair of nibbles at bits 4i and 16 + 4i
// puts them in fp16 mantissas with the offset n + 8: at bits 0-3 under the
// exponent of 1024 (fp16 1032 + n), at bits 4-7 under that of 64 (the
// mantissa is then 16 (n + 8): fp16 72 + n); w >> 8 brings i = 2, 3 to the
// same places. Each weight is then one mixed-precision fma (fp16 operand, fp32
// arithmetic): (1032 + n) s - 1032 s, with 1032 s and 72 s exact in fp32 (two
// set bits times an 11-bit scale), so the fma returns n s exactly (15
// significant bits at most) and the single rounding is the one to bf16.
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t w, float s, float c_lo, float c_hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t w8 = w >> 8;
  const h2 p0 = __builtin_bit_cast(h2, (w & 0x000F000Fu) ^ 0x64086408u);   // k = 0, 4
  const h2 p1 = __builtin_bit_cast(h2, (w & 0x00F000F0u) ^ 0x54805480u);   // k = 1, 5
  const h2 p2 = __builtin_bit_cast(h2, (w8 & 0x000F000Fu) ^ 0x64086408u);  // k = 2, 6
  const h2 p3 = __builtin_bit_cast(h2, (w8 & 0x00F000F0u) ^ 0x54805480u);  // k = 3, 7
  bf16x8 r;
  r[0] = static_cast<__bf16>(fmaf(static_cast<float>(p0.x), s, c_lo));
  r[1] = static_cast<__bf16>(fmaf(static_cast<float>(p1.x), s, c_hi));
  r[2] = static_cast<__bf16>(fmaf(static_cast<float>(p2.x), s, c_lo));
  r[3] = static_cast<__bf16>(fmaf(static_cast<float>(p3.x), s, c_hi));
  r[4] = static_cast<__bf16>(fmaf(static_cast<float>(p0.y), s, c_lo));
  r[5] = static_cast<__bf16>(fmaf(static_cast<float>(p1.y), s, c_hi));
  r[6] = static_cast<__bf16>(fmaf(static_cast<float>(p2.y), s, c_lo));
  r[7] = static_cast<__bf16>(fmaf(static_cast<float>(p3.y), s, c_hi));
  return r;
}

struct WStep {
  uint4 q[kMR];
  uint32_t s[kMR];
};

__device__ __forceinline__ void load_step(WStep& b, const uint8_t* const* qrow,
                                          const uint16_t* const* srow, int ngk, int st, int h) {
  int g = 2 * st + h;
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
  // routed tiles from the table (tiles/n_tiles), or a dense job of M_dense rows
  const int4* tiles;
  const int32_t* n_tiles;
  int M_dense;
  // outputs
  __bf16* act;        // gate/up: activations [rows][inter] bf16
  float* out;         // down: [rows][H] fp32 (routed, weighted) or y [T][H] (shared)
  const float* wrow;  // routed down: routing weight per assignment (by perm[row])
  const int32_t* perm;
  int k;
  // routed, slot pool: only the tiles of these experts run, each expert's
  // weights at experts + slot * blob_e (n_group == 0: every expert, at its id)
  SlotGroup group;
};

// The GEMM of one block: token rows [r0, r_end) (at most NTT 32-row tiles)
// against row tile nt of the weights in blob; lds: kBufs activation slices.
template <bool GATEUP, bool ROUTED, int NTT>
__device__ __forceinline__ void gemm_core(const GemmArgs& G, int nt, int r0, int r_end, const uint8_t* blob,
                                          uint8_t* lds) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int kRows = NTT * 32;                         // slice rows
  constexpr int kStage = kRows * (kRowB / 16) / kThreadsGemm;  // slice loads per thread and step
  static_assert(kStage * kThreadsGemm == kRows * (kRowB / 16), "whole slice loads per thread");
  constexpr int kLoads = kStage + 2 * kMR;                // vector loads per step
  constexpr int rows_per_block = GATEUP ? kWavesG * kHalf * 32 : kWavesG * kMR * 32;
  const int nrows = GATEUP ? G.inter : G.H;
  const int mtok = r_end - r0;
  const BlobOffsets o = blob_offsets(G.H, G.inter);
  const int K = GATEUP ? G.H : G.inter;
  const int ngk = K / kGroup;
  const int nsteps = (ngk + 1) / 2;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar registers
  const int lane = threadIdx.x & (kWave - 1);
  const int h = lane >> 5;     // K half of the MFMA operands
  const int l32 = lane & 31;   // weight row / token of the tiles
  const int rbase = nt * rows_per_block + wave * (GATEUP ? kHalf * 32 : kMR * 32);
  const bool live = rbase < nrows;  // waves past the last row only load and sync
  const uint8_t* qrow[kMR];
  const uint16_t* srow[kMR];
#pragma unroll
  for (int mr = 0; mr < kMR; ++mr) {
    int row = (GATEUP ? rbase + 32 * (mr % kHalf) : rbase + 32 * mr) + l32;
    row = live && row < nrows ? row : l32;
    const bool up = mr >= kHalf;
    const size_t qo = GATEUP ? (up ? o.up_q : o.gate_q) : o.down_q;
    const size_t so = GATEUP ? (up ? o.up_s : o.gate_s) : o.down_s;
    qrow[mr] = blob + qo + static_cast<size_t>(row) * (K / 2);
    srow[mr] = reinterpret_cast<const uint16_t*>(blob + so) + static_cast<size_t>(row) * ngk;
  }
  // This lane's part of the slice loads: load u of the wave writes slice
  // positions P = 64 (wave + 4u) + lane (16 bytes each), i.e. row P / 8 at
  // position P % 8, which holds the token's chunk (P % 8) ^ swz(row). Rows
  // past the tile repeat its last token (their outputs are dropped).
  const __bf16* arow[kStage];
  int achunk[kStage];
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int P = kWave * (wave + kWavesG * u) + lane;
    const int r = P >> 3;
    achunk[u] = (P & 7) ^ slice_swz(r);
    const int row = r0 + (r < mtok ? r : mtok - 1);
    const int idx = G.rmap ? G.rmap[row] / G.rdiv : row;
    arow[u] = G.A + static_cast<size_t>(idx) * G.lda;
  }

  f32x16 acc[kMR][NTT];
#pragma unroll
  for (int mr = 0; mr < kMR; ++mr)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mr][tt][v] = 0.f;

  WStep w[kBufs];
  // the loads of step st into slot sl (st past the last step re-loads the
  // last one: every step issues the same loads, so the wait counts hold on
  // every path)
  auto issue = [&](int st, int sl, WStep& wd) __attribute__((always_inline)) {
    st = st < nsteps ? st : nsteps - 1;
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      int kk = st * kStepK + 8 * achunk[u];
      kk = kk < K ? kk : K - 8;  // past the end: any finite values (their weights are 0)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(arow[u] + kk),
                                       (__attribute__((address_space(3))) void*)(lds + sl * kSlice +
                                                                                 kWave * 16 * (wave + kWavesG * u)),
                                       16, 0, 0);
    }
    load_step(wd, qrow, srow, ngk, st, h);
  };
  // MFMA operand i (dword i of each weight tile's group) of step st
  auto dequant = [&](int st, const WStep& wd, int i, bf16x8* a) __attribute__((always_inline)) {
    const bool gv = 2 * st + h < ngk;  // groups past K weigh 0
#pragma unroll
    for (int mr = 0; mr < kMR; ++mr) {
      const float sc = gv ? h2f(static_cast<uint16_t>(wd.s[mr])) : 0.0f;
      const uint32_t wi = i == 0 ? wd.q[mr].x : (i == 1 ? wd.q[mr].y : (i == 2 ? wd.q[mr].z : wd.q[mr].w));
      a[mr] = dequant8_bf16(wi, sc, -1032.0f * sc, -72.0f * sc);
    }
  };
  bf16x8 acur[kMR];
  // the activation operands of MFMA i of the slice in slot D (every token
  // tile, also past mtok: an output column depends on its own activation row
  // only, and the columns of absent rows are dropped)
  auto read_b = [&](int D, int i, bf16x8* b) __attribute__((always_inline)) {
    const uint8_t* lb = lds + D * kSlice;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int t = tt * 32 + l32;
      b[tt] = *reinterpret_cast<const bf16x8*>(lb + t * kRowB + 16 * ((4 * h + i) ^ slice_swz(t)));
    }
  };
  auto step = [&](auto slot, int s0, bool tail) __attribute__((always_inline)) {
    constexpr int D = decltype(slot)::value;  // slot of this step (step % kBufs)
    const int st = s0 + D;
    if (tail && st >= nsteps) return;  // uniform over the block
    // the first operands' LDS reads ahead of this step's loads (step st + 3)
    bf16x8 bcur[NTT];
    read_b(D, 0, bcur);
    __builtin_amdgcn_sched_barrier(0);
    issue(st + kDepth, (D + kDepth) % kBufs, w[(D + kDepth) % kBufs]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the next operands' LDS reads, and the weights of MFMA i + 1 of this
      // step (or 0 of the next), while the matrix cores work through i
      bf16x8 bnext[NTT];
      if (i < 3) read_b(D, i + 1, bnext);
      bf16x8 anext[kMR];
      if (i < 3) {
        dequant(st, w[D], i + 1, anext);
      } else {
        // this wave's loads of step st + 1 are in (those of st + 2, st + 3
        // may not be): its weights for the dequantisation below, its part of
        // the slice that the barrier publishes
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(kDepth - 1) * kLoads>();
        __builtin_amdgcn_sched_barrier(0);
        dequant(st + 1, w[(D + 1) % kBufs], 0, anext);
      }
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int mr = 0; mr < kMR; ++mr)
          acc[mr][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[mr], bcur[tt], acc[mr][tt], 0, 0, 0);
#pragma unroll
      for (int mr = 0; mr < kMR; ++mr) acur[mr] = anext[mr];
      if (i < 3)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) bcur[tt] = bnext[tt];
    }
    // every wave is done with slot D (the next step's loads may refill it),
    // and every wave's loads of step st + 1 have landed
    block_sync();
  };
  static_assert(kBufs == 4, "the step sequence below is written out for 4 slots");
  issue(0, 0, w[0]);
  issue(1, 1, w[1]);
  issue(2, 2, w[2]);
  wait_vmcnt<(kDepth - 1) * kLoads>();
  block_sync();
  dequant(0, w[0], 0, acur);
  int s0 = 0;
  for (; s0 + kBufs <= nsteps; s0 += kBufs) {
    step(std::integral_constant<int, 0>{}, s0, false);
    step(std::integral_constant<int, 1>{}, s0, false);
    step(std::integral_constant<int, 2>{}, s0, false);
    step(std::integral_constant<int, 3>{}, s0, false);
  }
  if (s0 < nsteps) {  // the last 1..3 steps
    step(std::integral_constant<int, 0>{}, s0, true);
    step(std::integral_constant<int, 1>{}, s0, true);
    step(std::integral_constant<int, 2>{}, s0, true);
  }
  // the loads still in flight (past the last step) complete before the
  // block ends: LDS is released with the block
  wait_vmcnt<0>();

  // epilogue: for token column l32 of each token tile, a lane holds rows
  // 8a + 4h + b (a, b = 0..3) of each 32-row weight tile in element 4a + b
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int m = r0 + tt * 32 + l32;
    if (m >= r_end || !live) continue;
    if (GATEUP) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        __attribute__((aligned(8))) __bf16 av[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
          av[b] = static_cast<__bf16>(gelu_tanh(acc[0][tt][4 * a + b]) * acc[1][tt][4 * a + b]);
        *reinterpret_cast<uint2*>(G.act + static_cast<size_t>(m) * G.inter + rbase + 8 * a + 4 * h) =
            *reinterpret_cast<const uint2*>(av);
      }
    } else {
      const float wr = ROUTED ? G.wrow[G.perm[m]] : 1.0f;
#pragma unroll
      for (int mr = 0; mr < kMR; ++mr) {
        if (rbase + 32 * mr >= nrows) continue;  // H a multiple of 32, not of 64: the wave's second tile is past it
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int n = rbase + 32 * mr + 8 * a + 4 * h;
          float4 v = make_float4(acc[mr][tt][4 * a], acc[mr][tt][4 * a + 1], acc[mr][tt][4 * a + 2],
                                 acc[mr][tt][4 * a + 3]);
          if (ROUTED) v = make_float4(v.x * wr, v.y * wr, v.z * wr, v.w * wr);
          *reinterpret_cast<float4*>(G.out + static_cast<size_t>(m) * G.H + n) = v;
        }
      }
    }
  }
}

// One block's tile (block index bid of its job): the token rows of its tile
// and its weight row tile, then the GEMM for the tile's number of 32-row
// token tiles (block-uniform, so each count runs its own unrolled code).
template <bool GATEUP, bool ROUTED>
__device__ __forceinline__ void gemm_tile(const GemmArgs& G, int bid, uint8_t* lds_b) {
  constexpr int rows_per_block = GATEUP ? kWavesG * kHalf * 32 : kWavesG * kMR * 32;
  const int nrows = GATEUP ? G.inter : G.H;
  const int n_tiles_n = (nrows + rows_per_block - 1) / rows_per_block;
  // XCD-aware order: blocks are dealt to the 8 XCDs in turn (block b to XCD
  // b % 8), so all row tiles of token tile mt get block ids congruent to mt
  // mod 8: they run on one XCD, and the token rows that the first of them
  // brings into that XCD's L2 serve the others
  const int xcd = bid % kXcds, jx = bid / kXcds;
  const int mt = xcd + kXcds * (jx / n_tiles_n);
  const int nt = jx % n_tiles_n;
  int r0, r_end;
  const uint8_t* blob;
  if (ROUTED) {
    if (mt >= *G.n_tiles) return;
    const int4 td = G.tiles[mt];
    int where = td.x;  // expert id (resident) or its slot (slot pool)
    if (G.group.n > 0) {
      where = -1;
      for (int i = 0; i < G.group.n; ++i)
        if (G.group.expert[i] == td.x) where = G.group.slot[i];
      if (where < 0) return;  // uniform over the block: not this group's expert
    }
    r0 = td.y;
    r_end = r0 + td.z;
    blob = G.experts + static_cast<size_t>(where) * G.blob_e;
  } else {
    r0 = mt * kTM;
    if (r0 >= G.M_dense) return;
    r_end = r0 + kTM < G.M_dense ? r0 + kTM : G.M_dense;
    blob = G.blob;
  }
  if (r_end <= r0) return;
  switch ((r_end - r0 + 31) / 32) {
    case 1: gemm_core<GATEUP, ROUTED, 1>(G, nt, r0, r_end, blob, lds_b); break;
    case 2: gemm_core<GATEUP, ROUTED, 2>(G, nt, r0, r_end, blob, lds_b); break;
    case 3: gemm_core<GATEUP, ROUTED, 3>(G, nt, r0, r_end, blob, lds_b); break;
    default: gemm_core<GATEUP, ROUTED, 4>(G, nt, r0, r_end, blob, lds_b); break;
  }
}

// y[t] += sum over j of the routed rows out_r[pos_of[t*k + j]], in rank
// order, after the shared expert's output o_shared[t] that y holds: the same
// additions in the same order as a combine inside the shared down GEMM, as a
// streaming pass over all blocks of the GPU (each token's k rows are read
// once, 16 bytes per lane). KMAX >= k: every lane issues KMAX loads (past k
// they repeat the last row) before the first add, and adds the first k.
template <int KMAX>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ out_r,
                                                 const int32_t* __restrict__ pos_of, int k, int H,
                                                 float* __restrict__ y) {
  const int t = blockIdx.y;
  int n = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  const bool on = n < H;
  n = on ? n : H - 4;
  float4 r[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int p = pos_of[static_cast<size_t>(t) * k + (j < k ? j : k - 1)];
    r[j] = *reinterpret_cast<const float4*>(out_r + static_cast<size_t>(p) * H + n);
  }
  const float4 y0 = *reinterpret_cast<const float4*>(y + static_cast<size_t>(t) * H + n);
  float vx = y0.x, vy = y0.y, vz = y0.z, vw = y0.w;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool add = j < k;  // per-component selects (a select of a float4 goes through memory)
    vx = add ? vx + r[j].x : vx;
    vy = add ? vy + r[j].y : vy;
    vz = add ? vz + r[j].z : vz;
    vw = add ? vw + r[j].w : vw;
  }
  if (on) *reinterpret_cast<float4*>(y + static_cast<size_t>(t) * H + n) = make_float4(vx, vy, vz, vw);
}

// Two waves per SIMD: the accumulation registers (128) and the rest within 256.
template <bool GATEUP, bool ROUTED>
__global__ __launch_bounds__(kThreadsGemm) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(GemmArgs G) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBufs * kSlice];
  gemm_tile<GATEUP, ROUTED>(G, blockIdx.x, lds_b);
}

// The shared expert's gate/up (dense over the tokens, its n_shared blocks
// first) and the routed experts' gate/up in one launch: the two are
// independent, and the shared blocks, few and long, would otherwise form a
// launch of their own with a tail of one block per CU.
__global__ __launch_bounds__(kThreadsGemm) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_gateup2(GemmArgs R, GemmArgs Sh, int n_shared) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBufs * kSlice];
  const int bid = blockIdx.x;
  if (bid < n_shared)
    gemm_tile<true, false>(Sh, bid, lds_b);
  else
    gemm_tile<true, true>(R, bid - n_shared, lds_b);
}

// The shared expert's down projection (its n_shared blocks first) and the
// routed experts' in one launch, for the same reason: alone, the shared
// expert's 176 blocks fill a third of the device's block slots.
__global__ __launch_bounds__(kThreadsGemm) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_down2(GemmArgs R, GemmArgs Sh, int n_shared) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBufs * kSlice];
  const int bid = blockIdx.x;
  if (bid < n_shared)
    gemm_tile<false, false>(Sh, bid, lds_b);
  else
    gemm_tile<false, true>(R, bid - n_shared, lds_b);
}

// Blocks along the weight rows of one GEMM (gate/up: row pairs; down: rows).
int gemm_row_tiles(bool gateup, int H, int inter) {
  const int rows = gateup ? inter : H;
  const int per = gateup ? kWavesG * kHalf * 32 : kWavesG * kMR * 32;
  return (rows + per - 1) / per;
}

// Grid of a GEMM of m_tiles token tiles (rounded up to whole XCD rounds, see
// gemm_tile; the blocks past the last tile exit).
int gemm_blocks(int m_tiles, bool gateup, int H, int inter) {
  return (m_tiles + kXcds - 1) / kXcds * kXcds * gemm_row_tiles(gateup, H, inter);
}

__global__ void k_bf16_to_f32(const uint16_t* __restrict__ x, size_t n, float* __restrict__ y) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    y[i] = __uint_as_float(static_cast<uint32_t>(x[i]) << 16);
}

}  // namespace

int permute_chunks(int A) { return (A + kChunk - 1) / kChunk; }

hipError_t launch_permute(const int32_t* ids, int A, int E, int chunks, int32_t* hist, int32_t* lrank,
                          int32_t* base, int32_t* seg, int4* tiles, int32_t* n_tiles, int32_t* perm,
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
  L.tiles = take(static_cast<size_t>(L.max_tiles) * 16);
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
                        reinterpret_cast<int32_t*>(at(L.seg)), reinterpret_cast<int4*>(at(L.tiles)),
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
  g.tiles = reinterpret_cast<const int4*>(at(L.tiles));
  g.n_tiles = reinterpret_cast<const int32_t*>(at(L.n_tiles));
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
  const int routed_blocks = gemm_blocks(L.max_tiles, true, H, I);
  if (with_shared) {
    const GemmArgs gs = shared_gateup_args(L, ws, x_bf16, with_shared->T, k, H, with_shared->Is, with_shared->shared);
    const int n_shared = gemm_blocks((with_shared->T + kTM - 1) / kTM, true, H, with_shared->Is);
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
  const int down_blocks = gemm_blocks(L.max_tiles, false, H, I);
  if (with_shared && with_shared->y) {
    // the shared expert's down into y in the same launch (its blocks first; a
    // multiple of 8 blocks, so the routed blocks keep their XCDs)
    GemmArgs ds = shared_gateup_args(L, ws, x_bf16, with_shared->T, k, H, with_shared->Is, with_shared->shared);
    ds.A = reinterpret_cast<const __bf16*>(ws + L.act_s);
    ds.lda = with_shared->Is;
    ds.out = with_shared->y;
    const int n_shared = gemm_blocks((with_shared->T + kTM - 1) / kTM, false, H, with_shared->Is);
    hipLaunchKernelGGL(k_gemm_down2, dim3(n_shared + down_blocks), dim3(kThreadsGemm), 0, s, d, ds, n_shared);
  } else {
    hipLaunchKernelGGL((k_gemm<false, true>), dim3(down_blocks), dim3(kThreadsGemm), 0, s, d);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_shared(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16, int T, int k,
                                 int H, int Is, const uint8_t* shared, float* y, hipStream_t s, bool gateup_done,
                                 bool down_done) {
  const GemmArgs gs = shared_gateup_args(L, ws, x_bf16, T, k, H, Is, shared);
  // shared gate/up: dense over tokens (unless it ran with the routed one)
  if (!gateup_done)
    hipLaunchKernelGGL((k_gemm<true, false>), dim3(gemm_blocks((T + kTM - 1) / kTM, true, H, Is)), dim3(kThreadsGemm), 0, s, gs);
  // shared down into y, then the combine (each token's routed rows in rank order)
  GemmArgs ds = gs;
  ds.A = reinterpret_cast<const __bf16*>(ws + L.act_s);
  ds.lda = Is;
  ds.out = y;
  if (!down_done)
    hipLaunchKernelGGL((k_gemm<false, false>), dim3(gemm_blocks((T + kTM - 1) / kTM, false, H, Is)), dim3(kThreadsGemm), 0, s, ds);
  const dim3 cg((H / 4 + 255) / 256, T);
  const float* out_r = reinterpret_cast<const float*>(ws + L.out_r);
  const int32_t* pos_of = reinterpret_cast<const int32_t*>(ws + L.pos_of);
  if (k <= 8) hipLaunchKernelGGL(k_combine<8>, cg, dim3(256), 0, s, out_r, pos_of, k, H, y);
  else hipLaunchKernelGGL(k_combine<kMaxTopK>, cg, dim3(256), 0, s, out_r, pos_of, k, H, y);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16,
                          const float* logits_in, const uint16_t* router, const float* bias, int T,
                          int E, int k, int H, int I, int Is, const uint8_t* experts, size_t blob_e,
                          const uint8_t* shared, float* y, int32_t* ids_out, float* w_out,
                          hipStream_t s) {
  hipError_t e = launch_prefill_route(L, ws, x_bf16, logits_in, router, bias, T, E, k, H, ids_out, w_out, s);
  const SharedGateup sg{shared, T, Is, y};
  if (e == hipSuccess) e = launch_prefill_routed(L, ws, x_bf16, k, H, I, experts, blob_e, nullptr, s, &sg);
  if (e == hipSuccess) e = launch_prefill_shared(L, ws, x_bf16, T, k, H, Is, shared, y, s, true, true);
  return e;
}

}  // namespace moe
