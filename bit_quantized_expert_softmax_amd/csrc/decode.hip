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
// token), so both kernels are shaped for latency: every lane issues all of its
// loads before any is consumed, each block reads its kernel arguments in one
// batch, row sums are fixed-order DPP trees, and the two kernels do not
// synchronise across blocks.
//
// gate/up kernel: one block per group of 32 activations of one source (its 32
//   gate rows and 32 up rows); a 16-lane segment owns whole rows, so the row
//   sums stay in registers; the token's activation digits are staged in LDS;
//   after the row sums, the GeGLU values of the group are quantised to digit
//   planes for the down projection.
// down kernel: 1024-thread blocks, one per 11 outputs; an output gathers the
//   down rows of all k+1 sources as one virtual row of (k*I + I_s)/32 chunks,
//   the routing weight folded into each group's scale; a lane owns one chunk
//   column (its activation digits in registers) and a few outputs; the row
//   sum is the weighted combine, in a fixed order, without atomics.
#include <hip/hip_ext.h>

#include "launch.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;  // lanes of a down block (and the unit of fill-block lanes)
constexpr int kGroupRows = 32;  // activations per gate/up block

// Entry i of a kernel-argument list, by selects over its constant-offset
// words: scalar loads from the argument segment (indexing it at run time
// reads it through the vector memory path, one more round trip). The empty
// asm statements keep the compiler from folding the selects back into an
// indexed load.
__device__ __forceinline__ int list_at(const SlotList& L, int i) {
  int v = L.v[0];
  asm("" : "+s"(v));
#pragma unroll
  for (int t = 1; t < kMaxTopK; ++t) {
    int c = L.v[t];
    asm("" : "+s"(c));
    v = i == t ? c : v;
  }
  return v;
}

__device__ __forceinline__ const uint8_t* source_base(const SourceSet& S, int j) {
  if (j >= S.k) return S.shared;
  const int e = S.ids ? S.ids[j] : list_at(S.slot, j);
  return S.experts + static_cast<size_t>(e) * S.blob_e;
}

// Touches, in one batch of scalar loads with one wait, every kernel argument
// the compute blocks of the B = 1 FFN kernels read before their first weight
// load: the arguments span several scalar-cache lines, and a chain of first
// touches, each issued behind the last one's wait, costs a memory round trip
// apiece while the other blocks' loads already queue at the memory.
__device__ __forceinline__ void touch_args(const SourceSet& S) {
  asm volatile("" ::"s"(S.experts), "s"(S.ids), "s"(S.slot.v[0]), "s"(S.slot.v[kMaxTopK - 1]),
               "s"(S.rsel.v[0]), "s"(S.rsel.v[kMaxTopK - 1]), "s"(S.nsel), "s"(S.shared),
               "s"(S.blob_e), "s"(S.H), "s"(S.I), "s"(S.Is), "s"(S.k), "s"(S.z), "s"(S.E));
}

// LDS of a gate/up block (byte offsets): the logits for an in-kernel top-k
// [E] fp64, the token's activation digits [4][ngu] uint4 (plane-major, so
// that adjacent lanes read adjacent words) and their scales [ngu], the weight
// scales of each 16-lane segment's rows (rps rows of ngu fp16, from the
// 16-byte boundary at or below their first byte: seg_sc bytes a segment),
// the block's 64 row sums.
struct GuLds {
  size_t zs, dig, dsc, wsc, seg_sc, act, total;
};
__host__ __device__ inline GuLds gateup_lds(int ngu, int E, int rps) {
  GuLds L;
  L.zs = 0;
  L.dig = (sizeof(double) * E + 15) & ~static_cast<size_t>(15);
  L.dsc = L.dig + static_cast<size_t>(ngu) * sizeof(DigitGroup);
  L.wsc = (L.dsc + 4 * static_cast<size_t>(ngu) + 15) & ~static_cast<size_t>(15);
  L.seg_sc = (14 + 2 * static_cast<size_t>(rps) * ngu + 15) & ~static_cast<size_t>(15);
  L.act = L.wsc + (2 * kGroupRows / rps) * L.seg_sc;
  L.total = L.act + 4 * 2 * kGroupRows;
  return L;
}

// Gate/up rows per 16-lane segment: 2 (a block of 8 waves, 2 per SIMD);
// launches whose blocks also take a top-k keep 1024 lanes (1 row a segment),
// since the block top-k's compares are spread over all the block's lanes, and
// so do rows of more than 8 x 16 chunks, whose weights would not fit in
// registers. Fewer waves issue the dot products too slowly (one wave per SIMD
// issues a VALU instruction every 12 cycles, four every 3); more read the
// staged digits from LDS too often (once per column and lane, for RPS rows).
__host__ __device__ constexpr int gu_rows_per_seg(int nc, bool topk) { return topk || nc > 8 ? 1 : 2; }
__host__ __device__ constexpr int gu_threads(int rps) { return kWave * (kGroupRows / 2) / rps; }

// Gate/up of one group of 32 (gate row i, up row i) pairs; NC chunk columns
// per lane and row, RPS rows per 16-lane segment (a block of 16/RPS waves).
// PUB: block 0 takes the token's top-k and publishes it (P), the other
// blocks shift down by one (a separate instantiation, so that the code of
// the launches without it stays as it is).
template <int NC, int RPS, bool PUB>
__global__ __launch_bounds__(kWave * 16 / RPS) void k_gateup(SourceSet S, int n_routed_blocks,
                                                     const DigitGroup* __restrict__ udig,
                                                     const float* __restrict__ usc,
                                                     DigitGroup* __restrict__ adig,
                                                     float* __restrict__ asc, FillList F, TopkPublish P) {
  constexpr int BT = kWave * 16 / RPS;  // threads of the block
  extern __shared__ uint4 lds_raw[];
  __shared__ double sel_z[kMaxTopK];
  __shared__ int sel_e[kMaxTopK];
  touch_args(S);
  asm volatile("" ::"s"(n_routed_blocks), "s"(udig), "s"(usc), "s"(adig), "s"(asc), "s"(F.n),
               "s"(F.blocks_per_blob));
  const int ngu = S.H / kGroup;
  const GuLds lay = gateup_lds(ngu, S.z ? S.E : (PUB ? P.E : 0), RPS);
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds_raw);
  int bx = blockIdx.x;
  if constexpr (PUB) {
    // the token's top-k and its publication to the host, ahead of the rest
    if (bx == 0) {
      double* zs = reinterpret_cast<double*>(lds + lay.zs);
      for (int f = threadIdx.x; f < P.E; f += BT) zs[f] = P.z[f];
      __syncthreads();
      topk_select(zs, P.E, P.k, sel_z, sel_e);
      if (threadIdx.x == 0) {
        // the release store orders the id stores before the sequence number
        for (int j = 0; j < P.k; ++j)
          __hip_atomic_store(P.ids_host + j, sel_e[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(P.seq_host, P.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      // the weights (for the down kernel, a later launch) after the ids are out
      topk_weights(sel_z, sel_e, P.k, P.ids, P.w, P.ids2, P.w2);
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
    for (size_t i0 = lo; i0 < hi; i0 += static_cast<size_t>(BT) * U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = i0 + threadIdx.x + static_cast<size_t>(BT) * u;
        v[u] = src[i < hi ? i : hi - 1];
      }
      __builtin_amdgcn_sched_barrier(0);
      // streaming stores: the blob is read next from memory by the expert
      // kernels, so it need not stay in (and be written back from) the L2
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = i0 + threadIdx.x + static_cast<size_t>(BT) * u;
        if (i < hi) store_nt16(dst + i, v[u]);
      }
    }
    return;
  }
  const int bid = bx - nfill;
  double* zs = reinterpret_cast<double*>(lds + lay.zs);  // [E]

  // blocks [0, n_routed_blocks): groups of the routed ranks (all k, or the
  // selected ones); the rest: groups of the shared expert
  const int gpr = S.I / kGroupRows;
  const int routed_groups = S.k * gpr;
  int grp;  // group of 32 activations in [0, (k*I + I_s)/32)
  if (bid < n_routed_blocks) {
    const int ls = bid / gpr;
    grp = (S.nsel > 0 ? list_at(S.rsel, ls) : ls) * gpr + bid % gpr;
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
    for (int f = threadIdx.x; f < S.E; f += BT) zs[f] = S.z[f];
    __syncthreads();
    topk_select(zs, S.E, S.k, sel_z, sel_e);
    base = S.experts + static_cast<size_t>(sel_e[src]) * S.blob_e;
  } else {
    base = source_base(S, src);
  }
  const BlobOffsets o = blob_offsets(S.H, inter);
  const size_t rowb = static_cast<size_t>(S.H) / 2;
  // Wave w owns RPS gate rows and RPS up rows per pair of 16-lane segments:
  // segments 0 and 1 gate rows 2 RPS w + [0, RPS) and + [RPS, 2 RPS),
  // segments 2 and 3 the same up rows. Lane j of a segment takes chunk
  // columns j, j + 16, ... (NC of them; past ngu masked) of each of its rows,
  // so a row's sum stays in its segment's registers (DPP) and the GeGLU pairs
  // meet in one wave: no partial sums in LDS. The token's activation digits
  // and their scales (L2-resident: every block reads them) and the segment's
  // rows' weight scales are staged in LDS; the weight chunks go to registers.
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int seg = lane >> 4;
  const int j = lane & 15;
  const bool upr = seg >= 2;
  const int rb = 2 * RPS * wave + RPS * (seg & 1);  // first row of the segment, in its half
  const uint8_t* qrow = base + (upr ? o.up_q : o.gate_q) + static_cast<size_t>(i0 + rb) * rowb;
  // the segment's rows' weight scales, from the 16-byte boundary at or below
  // them (the blob and its scale arrays start on one, and the bytes after the
  // up scales are the down scales, so the vectors stay inside the blob)
  const uint8_t* sbeg = base + (upr ? o.up_s : o.gate_s) + static_cast<size_t>(i0 + rb) * ngu * 2;
  const int lead = static_cast<int>(reinterpret_cast<uintptr_t>(sbeg) & 15);
  const u32x4* svec = reinterpret_cast<const u32x4*>(sbeg - lead);
  uint4* sdig = reinterpret_cast<uint4*>(lds + lay.dig);    // [4][ngu]
  float* sdsc = reinterpret_cast<float*>(lds + lay.dsc);    // [ngu]
  uint8_t* sseg = lds + lay.wsc + (4 * wave + seg) * lay.seg_sc;
  const uint16_t* swsc = reinterpret_cast<const uint16_t*>(sseg + lead);  // [RPS][ngu]
  float* sact = reinterpret_cast<float*>(lds + lay.act);    // [64]: gate, then up row sums
  // staging loads, issued first (loads return in order): digit items
  // i = 4 c + q, digit scales and the segment's scale vectors, clamped (the
  // same bytes to the same place where repeated)
  constexpr int DI = (4 * 16 * NC + BT - 1) / BT;                    // digit items per lane
  constexpr int SI = (16 * NC + BT - 1) / BT;                        // digit scales per lane
  constexpr int WV = ((14 + 2 * RPS * 16 * NC + 15) / 16 + 15) / 16;  // scale vectors per lane
  const int nd = 4 * ngu;
  const int nv = (lead + 2 * RPS * ngu + 15) / 16;  // the segment's scale vectors
  // (16-byte values as vector types: arrays of them stay in registers)
  u32x4 dv[DI];
  float sv[SI];
#pragma unroll
  for (int u = 0; u < DI; ++u) {
    const int di = static_cast<int>(threadIdx.x) + BT * u;
    dv[u] = reinterpret_cast<const u32x4*>(udig)[di < nd ? di : nd - 1];
  }
#pragma unroll
  for (int u = 0; u < SI; ++u) {
    const int si = static_cast<int>(threadIdx.x) + BT * u;
    sv[u] = usc[si < ngu ? si : ngu - 1];
  }
  u32x4 wsv[WV];
#pragma unroll
  for (int u = 0; u < WV; ++u) {
    const int vi = j + 16 * u;
    wsv[u] = svec[vi < nv ? vi : nv - 1];
  }
  __builtin_amdgcn_sched_barrier(0);
  // issued in the order of use (column by column, the rows of a column together)
  uint4 wv[RPS][NC];
#pragma unroll
  for (int m = 0; m < NC; ++m) {
#pragma unroll
    for (int r = 0; r < RPS; ++r) {
      int cc = j + 16 * m;
      cc = cc < ngu ? cc : ngu - 1;  // clamped: loaded, not summed
      wv[r][m] = load_w16(qrow + static_cast<size_t>(r) * rowb + 16 * static_cast<size_t>(cc));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < DI; ++u) {
    int di = static_cast<int>(threadIdx.x) + BT * u;
    di = di < nd ? di : nd - 1;
    reinterpret_cast<u32x4*>(sdig)[(di & 3) * ngu + (di >> 2)] = dv[u];
  }
#pragma unroll
  for (int u = 0; u < SI; ++u) {
    const int si = static_cast<int>(threadIdx.x) + BT * u;
    sdsc[si < ngu ? si : ngu - 1] = sv[u];
  }
#pragma unroll
  for (int u = 0; u < WV; ++u) {
    const int vi = j + 16 * u;
    reinterpret_cast<u32x4*>(sseg)[vi < nv ? vi : nv - 1] = wsv[u];
  }
  block_sync();  // the weight loads stay in flight
  float acc[RPS];
#pragma unroll
  for (int r = 0; r < RPS; ++r) acc[r] = 0.f;
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    const int cc = j + 16 * m;
    const int cl = cc < ngu ? cc : ngu - 1;
    DigitGroup xd;
#pragma unroll
    for (int q = 0; q < 4; ++q) xd.p[q] = sdig[q * ngu + cl];
    const float xs = sdsc[cl];
#pragma unroll
    for (int r = 0; r < RPS; ++r) {
      const float p = static_cast<float>(chunk_dot(wv[r][m], xd)) * (h2f(swsc[r * ngu + cl]) * xs);
      acc[r] += cc < ngu ? p : 0.f;
    }
  }
  // row sums over the 16 lanes (the order: each lane's columns j, j + 16, ...
  // in turn, then the DPP tree), gate rows then up rows in LDS; wave 0 takes
  // the GeGLU of the 32 pairs and writes their digit planes
#pragma unroll
  for (int r = 0; r < RPS; ++r) {
    const float rs = dpp_sum<16>(acc[r]);
    if (j == 0) sact[(upr ? kGroupRows : 0) + rb + r] = rs;
  }
  __syncthreads();
  if (wave == 0) {
    const float a = lane < kGroupRows ? gelu_tanh(sact[lane]) * sact[kGroupRows + lane] : 0.f;
    quant_pair_of_groups(a, grp, grp + 1, adig, asc);
  }
  // in-kernel routing: the first routed block writes the token's ids and
  // weights for the down kernel, off the path to its weight loads
  if (src < S.k && S.z && grp == 0) topk_weights(sel_z, sel_e, S.k, S.ids_g, S.w_g, S.ids2, S.w2);
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
  touch_args(S);
  asm volatile("" ::"s"(w), "s"(adig), "s"(asc), "s"(x), "s"(add_in), "s"(residual), "s"(y));
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
  // the residual input of the output this wave sums at the end (wave w <
  // nout owns output n0 + w), loaded now, behind the weights, so that no
  // round trip follows the sums; branch-free (a wave-uniform address, add_in
  // replaced by x when absent and its value dropped)
  const int wv_out = static_cast<int>(threadIdx.x) / kWave;
  const int nres = n0 + (wv_out < nout ? wv_out : nout - 1);
  const float xres = x[nres];
  const uint16_t ares = (add_in ? add_in : reinterpret_cast<const uint16_t*>(x))[nres];
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
      if (residual) r = xres + (add_in ? h2f(ares) : 0.f);
      y[n] = r + acc;
    }
  }
}

}  // namespace

size_t decode_lds_bytes(int H, int E, int k, int I, int Is) {
  const size_t ngu = H / kGroup, nga = (static_cast<size_t>(k) * I + Is) / kGroup;
  // the largest over the row splits a launch may take (the staged scales'
  // padding grows as rows per segment shrink)
  size_t gu = 0;
  for (int rps : {1, 2}) {
    const size_t b = gateup_lds(static_cast<int>(ngu), E, rps).total;
    gu = b > gu ? b : gu;
  }
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
  const int ngu = src.H / kGroup;
  const int need = (ngu + 15) / 16;  // chunk columns per lane and row
  if (need > 16) return hipErrorInvalidValue;
  const int nc = need <= 4 ? need : (need <= 6 ? 6 : (need <= 8 ? 8 : (need <= 12 ? 12 : 16)));
  const bool with_topk = topk != nullptr || (do_routed && src.z != nullptr);
  const int rps = gu_rows_per_seg(nc, with_topk);
  F.blocks_per_blob *= kThreads / gu_threads(rps);  // the same lanes per blob
  const int nr = do_routed ? (src.nsel > 0 ? src.nsel : src.k) * (src.I / kGroupRows) : 0;
  const int shared = src.Is / kGroupRows;
  const int n = (topk ? 1 : 0) + F.n * F.blocks_per_blob + nr + (do_shared ? shared : 0);
  if (n == 0) return hipSuccess;
  const int Ez = src.z ? src.E : (topk ? topk->E : 0);
  const size_t lds = gateup_lds(ngu, Ez, rps).total;
#define MOE_GATEUP_RPS(NT, RPS, PUB)                                                                     \
  do {                                                                                                   \
    constexpr int BT_ = gu_threads(RPS);                                                                 \
    if (t0) hipExtLaunchKernelGGL((k_gateup<NT, RPS, PUB>), dim3(n), dim3(BT_), lds, s, t0, t1, 0, src, nr, udig, usc, adig, asc, F, P); \
    else hipLaunchKernelGGL((k_gateup<NT, RPS, PUB>), dim3(n), dim3(BT_), lds, s, src, nr, udig, usc, adig, asc, F, P);               \
  } while (0)
#define MOE_GATEUP(NT)                                               \
  do {                                                               \
    if (topk) MOE_GATEUP_RPS(NT, 1, true);                           \
    else if (with_topk) MOE_GATEUP_RPS(NT, 1, false);                \
    else MOE_GATEUP_RPS(NT, gu_rows_per_seg(NT, false), false);      \
  } while (0)
  switch (nc) {
    case 1: MOE_GATEUP(1); break;
    case 2: MOE_GATEUP(2); break;
    case 3: MOE_GATEUP(3); break;
    case 4: MOE_GATEUP(4); break;
    case 6: MOE_GATEUP(6); break;
    case 8: MOE_GATEUP(8); break;
    case 12: MOE_GATEUP(12); break;
    default: MOE_GATEUP(16); break;
  }
#undef MOE_GATEUP
#undef MOE_GATEUP_RPS
  return hipGetLastError();
}

hipError_t launch_ffn_down(const SourceSet& src, const float* w, const DigitGroup* adig, const float* asc,
                           const float* x, const uint16_t* add_in, bool residual, float* y,
                           hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const int nga = src.k * (src.I / kGroup) + src.Is / kGroup;
  const size_t lds = static_cast<size_t>(kOutPerBlock) * nga * 4;
  if (nga > kThreads || !x) return hipErrorInvalidValue;  // x: read for every output (residual or not)
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
