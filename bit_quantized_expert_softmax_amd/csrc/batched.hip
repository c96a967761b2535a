// Batched decode (B tokens per call) of one MoE layer on the matrix cores:
// tokens are grouped by expert so that every touched expert's int4 rows are
// read once per call.
//
// The layer is the one of "Como executar um modelo de 26 bilhões de
// parâmetros em dois gigabytes de memória em um Mac comum", section "Qual é
// o principal truque da arquitetura" (8 routed experts and a shared expert per
// token); grouping rows per loaded expert follows the same page's section
// "Desempenho no mundo real".
//
// After routing, each expert's segment of rows is its assignments a =
// token*k + rank in increasing a (token order); a block finds them itself by
// scanning the B*k ids, so no sort and no permutation arrays are needed, and
// per-assignment rows are stored by a. The shared expert is one more segment
// holding every token. Per segment the projection is a small dense product
// W [rows x K] * X [K x m], so it runs on 16x16x32 fp16 MFMA:
//
//   * a wave streams 16 weight rows per tile, 4 quant groups (64 contiguous
//     bytes of each row) per K step, prefetched DEPTH steps ahead in
//     registers: the lane of 16-lane row q loads group 4*st + q of its row
//     (16 bytes) and that group's scale. MFMA j of the step takes dword j of
//     every lane's group, so one MFMA's K = 32 spans the step's 4 groups (8
//     values of each); as each lane dequantises with its own group's scale,
//     the sum is unchanged and no lane exchange is needed;
//   * nibbles become fp16 by the exponent trick (0x6400 | n is 1024 + n),
//     which yields k in the order (0,4,1,5,2,6,3,7) within each 8; the
//     activations are stored in that same order, so the dot products are
//     unchanged. A weight is rounded once, to fp16(n * scale);
//   * the segment's activation slice of a K step (m tokens x 128 values) is
//     loaded with the step's weights, staged in LDS (double buffered) one
//     step ahead, and shared by the block's 4 waves;
//   * activations are fp16 copies pre-scaled by a per-token power of two
//     (tsc, set by the router) so that they stay far inside the fp16 range;
//     the epilogues undo the scale exactly.
//
// gate/up: a wave owns 16 (gate row, up row) pairs; the epilogue applies
// GeGLU and stores the activations for down (fp16, same order, scaled by
// 1/tsc^2). down: a wave owns 32 output rows and writes one fp32 row per
// assignment; the combine adds, per token and in rank order, w_j times its
// routed rows to the shared expert's row (and the residual).
#include <atomic>
#include <type_traits>
#include <utility>

#include "launch.h"

namespace moe {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kTile = 16;               // MFMA tile edge: rows and tokens
constexpr int kStepK = 4 * kGroup;      // K per step: one group per 16-lane row
constexpr int kBRow = kStepK * 2 + 16;  // LDS bytes per token of a step slice (padded)
constexpr int kMR = 2;                  // 16-row weight tiles per wave
// 16-byte scale chunks per lane and tile staged in registers in one batch: a
// tile's 32 * K/32 scale bytes over a wave, up to K = kScaleIters * 64 * 16 =
// 4096; the chunks past that (K above 4096) follow one per lane at a time
constexpr int kScaleIters = 4;

struct MArgs {
  const uint8_t* experts;
  const uint8_t* shared;
  size_t blob_e;
  int H, I, Is, E, k, B;
  const int32_t* ids;   // [B][k] experts of each token, in rank order
  int nA;                // B*k assignments a = token*k + rank
  const uint16_t* u16;   // [B][H] fp16 inputs / tsc
  const float* tsc;      // [B]
  uint16_t* act_r;       // [B*k][I]  routed GeGLU activations by assignment
  uint16_t* act_s;       // [B][Is]   shared activations by token
  float* out_r;          // [B*k][H]
  float* out_s;          // [B][H]
  int tiles_r, tiles_s;  // blocks per routed / shared segment (row tiles x token groups)
  int s_groups;          // the shared segment's token passes, split over this many blocks per row tile
  int early_scales;      // issue the scale loads before the scan of the ids (nearly every expert touched)
};

// 8 signed nibbles (k = 0..7 in bits 4k..4k+3) times scale s, as fp16 in the
// order (0,4,1,5,2,6,3,7).
__device__ __forceinline__ f16x8 dequant8(uint32_t w, _Float16 s) {
  const f16x2 sc = {s, s};
  // The nibbles at bits 4i and 16 + 4i for i = 0, 1 sit in the fp16
  // mantissa in place; w >> 8 brings i = 2, 3 to the same places. (b & 0xF)
  // ^ 8 is n + 8 for the two's complement nibble n, and the same xor sets
  // the exponent: at bits 0-3 it gives fp16(1024 + n + 8) (exponent 0x6400),
  // at bits 4-7 the mantissa is 16 (n + 8), so exponent 0x5400 gives
  // fp16(64 + n + 8). One and-xor (v_bitop3) per pair, one shift per 8
  // nibbles; n itself is exact, so the one rounding is that of n * s.
  auto pair = [&](uint32_t v, uint32_t mask, uint32_t bits, float bias) __attribute__((always_inline)) {
    const f16x2 bb = {static_cast<_Float16>(bias), static_cast<_Float16>(bias)};
    return (__builtin_bit_cast(f16x2, (v & mask) ^ bits) - bb) * sc;
  };
  const uint32_t w8 = w >> 8;
  const f16x2 h0 = pair(w, 0x000F000Fu, 0x64086408u, 1032.0f);
  const f16x2 h1 = pair(w, 0x00F000F0u, 0x54805480u, 72.0f);
  const f16x2 h2 = pair(w8, 0x000F000Fu, 0x64086408u, 1032.0f);
  const f16x2 h3 = pair(w8, 0x00F000F0u, 0x54805480u, 72.0f);
  return f16x8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(lo))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(hi))) << 16);
}

struct WStep {
  u32x4 q[kMR];  // group 4*st + q (16-lane row q of the wave) of the lane's row
};

// Weights of K step st: group 4*st + q of the lane's row in each tile (16
// bytes; a 16-lane row of the wave reads 64 contiguous bytes of each of its 16
// weight rows). Groups past K are clamped to the last one (their scale is
// zeroed when used). No loaded value is used here, so the loads stay in
// flight. The scales come from LDS (staged once per block).
__device__ __forceinline__ void load_step(WStep& b, const uint8_t* const* qrow, int ngk, int st, int q) {
  int g = 4 * st + q;
  g = g < ngk ? g : ngk - 1;
#pragma unroll
  for (int m = 0; m < kMR; ++m)
    // cached load: the other half of each 128-byte line is read one step later
    b.q[m] = *reinterpret_cast<const u32x4*>(qrow[m] + 16 * static_cast<size_t>(g));
}

// f(integral_constant<int, D>) for D = 0, 1, ...: ring slots as compile-time
// constants, so the ring stays in registers
template <class F, int... D>
__device__ __forceinline__ void for_slots(std::integer_sequence<int, D...>, F&& f) {
  (f(std::integral_constant<int, D>{}), ...);
}

// The work of one block over segment s (an expert, or s == E: the shared
// expert) with NTT 16-token tiles per pass. GATEUP: a wave's weight tiles are
// 16 gate rows and the 16 matching up rows; else 32 consecutive down rows.
// lds_slices: the two activation slice buffers, NTT * kTile * kBRow bytes
// each; alist: NTT * kTile ints.
// Passes p0 = first, first + stride, ... (in tokens) of the segment.
template <bool GATEUP, int NTT, int DEPTH>
__device__ __forceinline__ void mfma_body(const MArgs& A, int s, int tile, int first, int stride,
                                          uint8_t* lds_slices, int* alist, int* wcnt) {
  static_assert(DEPTH >= 2 && DEPTH <= 8, "ring of 2..8 load units");
  uint8_t* const lds_b[2] = {lds_slices, lds_slices + NTT * kTile * kBRow};
  const bool routed = s < A.E;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  // A routed segment's rows are the assignments a with ids[a] == s, in
  // increasing a (so in token order: a token holds an expert at most once).
  // scan() counts them and puts those of rows [p0, p0 + cap) in alist: a
  // ballot per wave, the waves' counts through LDS, ids read in batches.
  auto scan = [&](int p0, int cap) __attribute__((always_inline)) {
    constexpr int kBatch = 4;
    int total = 0;
    for (int c0 = 0; c0 < A.nA; c0 += kBatch * kThreads) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int a = c0 + u * kThreads + threadIdx.x;
        v[u] = a < A.nA ? A.ids[a] : -1;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (c0 + u * kThreads >= A.nA) break;  // uniform
        const bool hit = v[u] == s;
        const unsigned long long bal = __ballot(hit);
        if (lane == 0) wcnt[wave] = __popcll(bal);
        __syncthreads();
        int base = total, chunk = 0;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) {
          base += w2 < wave ? wcnt[w2] : 0;
          chunk += wcnt[w2];
        }
        const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
        if (hit && pos >= p0 && pos < p0 + cap) alist[pos - p0] = c0 + u * kThreads + threadIdx.x;
        total += chunk;
        __syncthreads();  // wcnt is rewritten by the next batch
      }
    }
    return total;
  };
  const uint8_t* blob = routed ? A.experts + static_cast<size_t>(s) * A.blob_e : A.shared;
  const int inter = routed ? A.I : A.Is;
  const int K = GATEUP ? A.H : inter;
  const int nrows = GATEUP ? inter : A.H;
  const int ngk = K / kGroup;
  const int nsteps = (ngk + 3) / 4;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const BlobOffsets o = blob_offsets(A.H, inter);
  const int rbase = (tile * kWaves + wave) * (GATEUP ? kTile : kMR * kTile);
  const bool live = rbase < nrows;
  const uint8_t* qrow[kMR];
  // The wave's scales, [kMR][16 rows][ngk], staged once: a tile's 16 rows
  // are consecutive, so its scales are one contiguous run of 32*ngk bytes,
  // read in 16-byte chunks (per step, scattered 2-byte loads would touch 16
  // cache lines per instruction for 128 bytes). Chunks are clamped to the
  // matrix's scale array; rows past it (and idle waves, which take the first
  // tile) get finite scales of other rows, whose results are not stored.
  // With early_scales the scale loads are issued before the scan of the ids,
  // so that their round trip and the scan's overlap; a block of an untouched
  // expert then reads its scales for nothing, so small batches (many
  // untouched experts) scan first.
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_scales[];
  uint16_t* ssc = reinterpret_cast<uint16_t*>(lds_scales) + static_cast<size_t>(wave) * kMR * kTile * ngk;
  u32x4 sv[kMR][kScaleIters];
  const u32x4* ssrc[kMR];
  int scmax[kMR];
#pragma unroll
  for (int mr = 0; mr < kMR; ++mr) {
    const int t0r = GATEUP ? rbase : rbase + kTile * mr;  // first row of the tile
    const int t0 = live && t0r < nrows ? t0r : 0;
    int row = t0 + l16;
    row = live && row < nrows ? row : l16;
    const size_t qo = GATEUP ? (mr == 0 ? o.gate_q : o.up_q) : o.down_q;
    const size_t so = GATEUP ? (mr == 0 ? o.gate_s : o.up_s) : o.down_s;
    qrow[mr] = blob + qo + static_cast<size_t>(row) * (K / 2);
    const u32x4* src = reinterpret_cast<const u32x4*>(blob + so + static_cast<size_t>(t0) * ngk * 2);
    const int t_rows = nrows - t0 < kTile ? nrows - t0 : kTile;  // 16: nrows, t0 multiples of 16
    const int cmax = t_rows * ngk / 8 - 1;                       // last chunk inside the scale array
    ssrc[mr] = src;
    scmax[mr] = cmax;
  }
  auto load_scales = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mr = 0; mr < kMR; ++mr)
#pragma unroll
      for (int i = 0; i < kScaleIters; ++i) {
        const int c = lane + kWave * i;
        sv[mr][i] = ssrc[mr][c < scmax[mr] ? c : scmax[mr]];
      }
  };
  if (A.early_scales) load_scales();
  const int m = routed ? scan(0, NTT * kTile) : A.B;
  if (m <= first) return;  // uniform over the block
  if (!A.early_scales) load_scales();
#pragma unroll
  for (int mr = 0; mr < kMR; ++mr) {
    u32x4* dst = reinterpret_cast<u32x4*>(ssc + mr * kTile * ngk);
#pragma unroll
    for (int i = 0; i < kScaleIters; ++i) {
      const int c = lane + kWave * i;
      if (c < 2 * ngk) dst[c] = sv[mr][i];
    }
    // K above 4096 (wave-uniform; no iteration at smaller K)
    for (int c = lane + kWave * kScaleIters; c < 2 * ngk; c += kWave) dst[c] = ssrc[mr][c < scmax[mr] ? c : scmax[mr]];
  }

  for (int p0 = first; p0 < m; p0 += stride) {
    const int mt = m - p0 < NTT * kTile ? m - p0 : NTT * kTile;
    if (routed && p0 > 0) scan(p0, NTT * kTile);  // this pass's assignments
    // this thread's 16-byte chunks of a step slice (token = c / 16)
    const uint16_t* brow[NTT];
    int boff[NTT], loff[NTT];
#pragma unroll
    for (int r = 0; r < NTT; ++r) {
      int c = threadIdx.x + kThreads * r;
      c = c < mt * 16 ? c : mt * 16 - 1;
      const int row = p0 + (c >> 4);  // row of the segment
      boff[r] = 8 * (c & 15);
      loff[r] = (c >> 4) * kBRow + 16 * (c & 15);
      if (GATEUP) {
        const int t = routed ? alist[row - p0] / A.k : row;
        brow[r] = A.u16 + static_cast<size_t>(t) * A.H;
      } else {
        brow[r] = routed ? A.act_r + static_cast<size_t>(alist[row - p0]) * A.I
                         : A.act_s + static_cast<size_t>(row) * A.Is;
      }
    }

    f32x4 acc[kMR][NTT];
#pragma unroll
    for (int mr = 0; mr < kMR; ++mr)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) acc[mr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Load unit y = (activation slice of step y+1, weights of step y), issued
    // in that order DEPTH steps ahead into ring slot y % DEPTH. Step x needs
    // its weights and stores the slice of step x+1 to LDS, both from unit x:
    // as loads retire in issue order, a step waits for its own unit only and
    // the DEPTH-1 later units stay in flight. Every ring index below is a
    // compile-time constant, so the ring lives in registers.
    WStep w[DEPTH];
    u32x4 bs[DEPTH][NTT];
    auto load_slice = [&](int st, u32x4* bd) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < NTT; ++r) {
        int kk = st * kStepK + boff[r];
        kk = kk < K ? kk : K - 8;  // past the end: any finite values (their weights are 0)
        bd[r] = *reinterpret_cast<const u32x4*>(brow[r] + kk);
      }
    };
    // st past the last step re-reads the last step: every step issues the
    // same loads, so the wait counts are the same on every path
    auto issue = [&](int st, WStep& wd, u32x4* bd) __attribute__((always_inline)) {
      st = st < nsteps ? st : nsteps - 1;
      load_slice(st + 1 < nsteps ? st + 1 : nsteps - 1, bd);
      load_step(wd, qrow, ngk, st, q);
    };
    auto stage_store = [&](int bi, const u32x4* bd) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < NTT; ++r) *reinterpret_cast<u32x4*>(lds_b[bi] + loff[r]) = bd[r];
    };
    auto step = [&](auto slot, int s0, bool tail) __attribute__((always_inline)) {
      constexpr int D = decltype(slot)::value;
      const int st = s0 + D;
      if (tail && st >= nsteps) return;  // uniform over the block
      stage_store((st + 1) & 1, bs[D]);  // past the end: unused
      const uint8_t* lb = lds_b[st & 1];
      // MFMA j takes dword j (8 nibbles) of every lane's group: the 4
      // 16-lane rows contribute groups 4*st .. 4*st+3, each dequantised with
      // its own scale, and the activations at the same positions
      const bool gv = 4 * st + q < ngk;  // groups past K weigh 0
      const int gs = gv ? 4 * st + q : ngk - 1;
      _Float16 sc[kMR];
#pragma unroll
      for (int mr = 0; mr < kMR; ++mr)
        sc[mr] = gv ? __builtin_bit_cast(_Float16, ssc[(mr * kTile + l16) * ngk + gs]) : static_cast<_Float16>(0.0f);
      // dequantised one dword (K slice of the MFMA) at a time: few live
      // operand registers leave room for a deeper load ring
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f16x8 a[kMR];
#pragma unroll
        for (int mr = 0; mr < kMR; ++mr) a[mr] = dequant8(w[D].q[mr][j], sc[mr]);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          if (tt * kTile < mt) {
            const f16x8 bv = *reinterpret_cast<const f16x8*>(lb + (tt * kTile + l16) * kBRow + 64 * q + 16 * j);
#pragma unroll
            for (int mr = 0; mr < kMR; ++mr)
              acc[mr][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mr], bv, acc[mr][tt], 0, 0, 0);
          }
        }
      }
      // the slot's next loads go after its last use (no overlapping live
      // ranges, so the ring keeps its registers across the loop)
      __builtin_amdgcn_sched_barrier(0);
      issue(st + DEPTH, w[D], bs[D]);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };
    {
      u32x4 b0[NTT];  // the slice of step 0, ahead of the ring
      load_slice(0, b0);
      for_slots(std::make_integer_sequence<int, DEPTH>{}, [&](auto slot) __attribute__((always_inline)) {
        constexpr int D = decltype(slot)::value;
        issue(D, w[D], bs[D]);
      });
      stage_store(0, b0);
    }
    __syncthreads();
    // whole groups of DEPTH steps: straight-line code with the same loads on
    // every path, so each wait is only for the unit it needs
    int s0 = 0;
    for (; s0 + DEPTH <= nsteps; s0 += DEPTH)
      for_slots(std::make_integer_sequence<int, DEPTH>{},
                [&](auto slot) __attribute__((always_inline)) { step(slot, s0, false); });
    if (s0 < nsteps)  // the last 1..DEPTH-1 steps
      for_slots(std::make_integer_sequence<int, DEPTH - 1>{},
                [&](auto slot) __attribute__((always_inline)) { step(slot, s0, true); });

    // epilogue: a lane holds rows 4q..4q+3 of each weight tile for token
    // column l16 of each token tile (columns past mt hold garbage, unused)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      if (tt * kTile >= mt) continue;  // uniform
      const int col = tt * kTile + l16;
      const bool valid = live && col < mt;
      const int row = p0 + (col < mt ? col : mt - 1);  // row of the segment
      const int asg = routed ? alist[row - p0] : row;    // its assignment (routed) or token
      const int tok = routed ? asg / A.k : row;
      const float ts = A.tsc[tok];
      if (GATEUP) {
        float av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = gelu_tanh(acc[0][tt][i] * ts) * acc[1][tt][i] / ts;
        const uint32_t lo = pack_f16(av[0], av[1]);
        const uint32_t hi = pack_f16(av[2], av[3]);
        // 16-lane rows 2b and 2b+1 hold values 0..3 and 4..7 of one 8-block
        // of the activation row; each writes one half of the interleaved block
        const bool odd = q & 1;
        const uint32_t recv = static_cast<uint32_t>(__shfl_xor(static_cast<int>(odd ? lo : hi), 16, kWave));
        uint2 out;
        if (!odd) {
          out.x = (lo & 0xFFFFu) | (recv << 16);
          out.y = (lo >> 16) | (recv & 0xFFFF0000u);
        } else {
          out.x = (recv & 0xFFFFu) | (hi << 16);
          out.y = (recv >> 16) | (hi & 0xFFFF0000u);
        }
        if (valid) {
          uint16_t* dst = routed ? A.act_r + static_cast<size_t>(asg) * A.I
                                 : A.act_s + static_cast<size_t>(row) * A.Is;
          *reinterpret_cast<uint2*>(dst + rbase + 8 * (q >> 1) + 4 * (q & 1)) = out;
        }
      } else if (valid) {
        const float f = ts * ts;
        float* dst = routed ? A.out_r + static_cast<size_t>(asg) * A.H
                            : A.out_s + static_cast<size_t>(row) * A.H;
#pragma unroll
        for (int mr = 0; mr < kMR; ++mr)
          *reinterpret_cast<float4*>(dst + rbase + kTile * mr + 4 * q) =
              make_float4(acc[mr][tt][0] * f, acc[mr][tt][1] * f, acc[mr][tt][2] * f, acc[mr][tt][3] * f);
      }
    }
  }
}

// One launch covers all segments: tiles_s blocks of the shared expert, then
// tiles_r blocks per routed expert (blocks of untouched experts exit at
// once). The routed experts' blocks take NTT_R token tiles per pass (their
// segments are short: B * k / E tokens on average), the shared expert's
// blocks NTT_S (its segment holds all B tokens).
// Waves per SIMD the compiler must leave room for: 4 (at most 128 registers)
// for the one-tile kernels of B <= 64, whose gate/up otherwise takes 132
// registers and 3 waves; no constraint for the larger tiles.
template <int NTT_R, int NTT_S>
constexpr int kMfmaWaves = NTT_R == 1 && NTT_S == 1 ? 4 : 1;
template <bool GATEUP, int NTT_R, int DEPTH_R, int NTT_S, int DEPTH_S>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kMfmaWaves<NTT_R, NTT_S>))) void k_mfma(MArgs A) {
  constexpr int kNT = NTT_R > NTT_S ? NTT_R : NTT_S;
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * kNT * kTile * kBRow];
  __shared__ int alist[kNT * kTile];
  __shared__ int wcnt[kWaves];
  // the shared expert's blocks first: its segment is the longest (every
  // token), so it starts before the routed blocks fill the device
  const int bx = blockIdx.x;
  const bool sh = bx < A.tiles_s;
  const int s = sh ? A.E : (bx - A.tiles_s) / A.tiles_r;
  if (s < A.E) {
    mfma_body<GATEUP, NTT_R, DEPTH_R>(A, s, (bx - A.tiles_s) % A.tiles_r, 0, NTT_R * kTile, lds_b, alist, wcnt);
  } else {
    // row tile bx % rows, token group bx / rows of the shared segment
    const int rows = A.tiles_s / A.s_groups;
    mfma_body<GATEUP, NTT_S, DEPTH_S>(A, s, bx % rows, (bx / rows) * NTT_S * kTile,
                                      A.s_groups * NTT_S * kTile, lds_b, alist, wcnt);
  }
}

// y[t] = (x'[t] if residual) + out_s[t] + sum_j w[t][j] * out_r[t*k + j]
__global__ void k_bcombine(const float* __restrict__ out_s, const float* __restrict__ out_r,
                           const float* __restrict__ w,
                           const float* __restrict__ x, const uint16_t* __restrict__ add_in,
                           int residual, int H, int k, float* __restrict__ y) {
  const int t = blockIdx.y;
  for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < H; n += gridDim.x * blockDim.x) {
    float v = out_s[static_cast<size_t>(t) * H + n];
    for (int j = 0; j < k; ++j)
      v = fmaf(w[t * k + j], out_r[(static_cast<size_t>(t) * k + j) * H + n], v);
    float r = 0.f;
    if (residual) r = x[static_cast<size_t>(t) * H + n] + (add_in ? h2f(add_in[static_cast<size_t>(t) * H + n]) : 0.f);
    y[static_cast<size_t>(t) * H + n] = r + v;
  }
}

// LDS of one k_mfma block: the double-buffered activation slices (static)
// and the staged scales of its 4 waves (dynamic, 2 tiles x 16 rows x K/32).
size_t mfma_static_lds(int ntt) { return 2 * static_cast<size_t>(ntt) * kTile * kBRow; }
size_t mfma_scale_lds(int K) { return static_cast<size_t>(kWaves) * kMR * kTile * (K / kGroup) * 2; }
int tiles_per_pass(int B) { return B <= kTile ? 1 : (B <= 2 * kTile ? 2 : 4); }
constexpr bool kSharedSplit = true;

// LDS one block may use on the current device (160 KiB on gfx950), looked up
// once per device (threads that race on the first lookup store the same
// value); 64 KiB if the query fails.
size_t block_lds_limit() {
  constexpr int kDevs = 64;
  static std::atomic<size_t> cached[kDevs];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 65536;
  size_t v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int a = 0;
    v = hipDeviceGetAttribute(&a, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && a > 0
            ? static_cast<size_t>(a)
            : 65536;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// ntt_r: tiles per pass of the routed experts' blocks, ntt_s: of the shared
// expert's; the launch's static LDS is that of the larger.
template <bool GATEUP>
hipError_t launch_mfma(const MArgs& A, int ntt_r, int ntt_s, hipStream_t s) {
  const dim3 grid(A.E * A.tiles_r + A.tiles_s);
  const size_t lds = mfma_scale_lds(GATEUP ? A.H : (A.I > A.Is ? A.I : A.Is));
  if (mfma_static_lds(ntt_r > ntt_s ? ntt_r : ntt_s) + lds > block_lds_limit()) return hipErrorInvalidValue;
#define MOE_MF(R_, DR_, S_, DS_) hipLaunchKernelGGL((k_mfma<GATEUP, R_, DR_, S_, DS_>), grid, dim3(kThreads), lds, s, A)
  if (ntt_r <= 1 && ntt_s <= 1) MOE_MF(1, 4, 1, 4);
  else if (ntt_r <= 1 && ntt_s == 2) MOE_MF(1, 4, 2, 4);
  else if (ntt_r <= 1) MOE_MF(1, 4, 4, 3);
  else if (ntt_r == 2 && ntt_s <= 2) MOE_MF(2, 4, 2, 4);
  else if (ntt_r == 2) MOE_MF(2, 4, 4, 3);
  else MOE_MF(4, 3, 4, 3);
#undef MOE_MF
  return hipGetLastError();
}

}  // namespace

bool batched_lds_fits(int H, int I, int Is, int max_B) {
  const size_t st = mfma_static_lds(tiles_per_pass(max_B));
  const size_t lim = block_lds_limit();
  return st + mfma_scale_lds(H) <= lim && st + mfma_scale_lds(I > Is ? I : Is) <= lim;
}

hipError_t launch_batched(const BatchedBuffers& bb, const uint8_t* experts, const uint8_t* shared,
                          size_t blob_e, int H, int I, int Is, int E, int k, int B,
                          const uint16_t* u16, const float* tsc, const int32_t* ids, const float* w,
                          const float* x, const uint16_t* add_in, bool residual, float* y, hipStream_t s) {
  if (!batched_lds_fits(H, I, Is, B)) return hipErrorInvalidValue;
  MArgs A{experts, shared, blob_e, H, I, Is, E, k, B, ids, B * k, u16, tsc,
          bb.act_r, bb.act_s, bb.out_r, bb.out_s, 0, 0};
  // tokens per pass over a segment's weights: up to 64; a longer segment
  // takes more passes (the later ones read the weights from cache). An
  // expert's segment holds about B * k / E tokens, so its blocks are sized
  // for twice that; the shared expert's holds all B, and its blocks (issued
  // first, so their extra passes overlap the routed blocks) for B / 4, at
  // most 4 passes. Smaller tiles keep the registers, and so the waves per
  // SIMD, of the common case.
  const int ntt_s = tiles_per_pass((B + 3) / 4);
  const int ntt_r = tiles_per_pass(2 * ((B * k + E - 1) / E));
  // the shared segment's passes, each in blocks of its own
  A.s_groups = kSharedSplit ? (B + ntt_s * kTile - 1) / (ntt_s * kTile) : 1;
  // B*k assignments over E experts: at B*k >= 4E about 1 in 50 experts is
  // untouched (B = 64: 3 of 128), at B*k = E about 1 in 3 (B = 16: 46)
  A.early_scales = B * k >= 4 * E;
  // gate/up: 64 row pairs per block
  A.tiles_r = (I + kWaves * kTile - 1) / (kWaves * kTile);
  A.tiles_s = (Is + kWaves * kTile - 1) / (kWaves * kTile) * A.s_groups;
  hipError_t e = launch_mfma<true>(A, ntt_r, ntt_s, s);
  if (e != hipSuccess) return e;
  // down: 128 output rows per block
  A.tiles_r = (H + kWaves * kMR * kTile - 1) / (kWaves * kMR * kTile);
  A.tiles_s = A.tiles_r * A.s_groups;
  if ((e = launch_mfma<false>(A, ntt_r, ntt_s, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_bcombine, dim3((H + 255) / 256, B), dim3(256), 0, s, bb.out_s, bb.out_r, w,
                     x, add_in, residual ? 1 : 0, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
