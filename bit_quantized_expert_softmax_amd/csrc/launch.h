// Kernel launchers used by the C-ABI layer. Each returns the HIP status of
// its launch; argument checking happens before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

constexpr int kMaxTopK = 16;

// Byte offsets inside one expert blob (gate.q | up.q | down.q | gate.s | up.s | down.s).
struct BlobOffsets {
  size_t gate_q, up_q, down_q, gate_s, up_s, down_s, total;
};
__host__ __device__ inline BlobOffsets blob_offsets(size_t H, size_t I) {
  BlobOffsets o;
  o.gate_q = 0;
  o.up_q = I * H / 2;
  o.down_q = I * H;
  o.gate_s = 3 * I * H / 2;
  o.up_s = o.gate_s + I * (H / kGroup) * 2;
  o.down_s = o.up_s + I * (H / kGroup) * 2;
  o.total = o.down_s + H * (I / kGroup) * 2;
  return o;
}

struct DevCache;  // device-stepped expert-slot cache (below)

// ---------------------------------------------------------------- routing
// Layer router, one launch: x' = x (+ add_in); u = x' or rmsnorm(x'); u's
// digit planes; fp64 logits (+ bias); top-k + softmax by the last block to
// finish. Grid: (E/4 blocks) x B tokens (with u16 and no digit planes, B > 1:
// E/16 blocks, four experts per wave). cnt holds B arrival counters, zero
// before the launch and after it.
// Top-k variant (ids != nullptr): the last block of each token's grid row
// takes that token's top-k.
hipError_t launch_route_layer(const float* x, const uint16_t* add_in, int B, int H, bool rmsnorm,
                              const uint16_t* wr, const float* bias, int E, int k, float* u_out,
                              DigitGroup* udig, float* usc, uint16_t* u16, float* tsc, double* z,
                              int32_t* cnt, int32_t* ids, float* w, int32_t* ids2, float* w2,
                              hipStream_t s);
// Selection step of a one-token cache-mode call, after a logits-only
// launch_route_layer: one block takes the top-k of z [E], writes ids / w (and
// the optional copies), then steps the device-side cache (dcache) or
// publishes the ids to host memory (ids_host, then seq to *seq_host with a
// system-scope release store), or both or neither.
hipError_t launch_route_select(const double* z, int E, int k, int32_t* ids, float* w, int32_t* ids2, float* w2,
                               int32_t* ids_host, int32_t* seq_host, int32_t seq, const DevCache* dcache,
                               hipStream_t s);
// Standalone router: z[b][e] = sum_h u[b][h] * wr[e][h] (+ bias[e]) in fp64.
hipError_t launch_route_logits(const float* u, int B, int H, const uint16_t* wr, const float* bias,
                               int E, double* z, hipStream_t s);
// top-k (ties to the lower id) and softmax over the selected; logits from z64
// (fp64) or z32 (fp32). ids2/w2 are optional second copies.
hipError_t launch_route_topk(const double* z64, const float* z32, int B, int E, int k, int32_t* ids,
                             float* w, int32_t* ids2, float* w2, hipStream_t s);

// ---------------------------------------------------------------- decode FFN
struct SlotList {
  int32_t v[kMaxTopK];
};

struct SourceSet {
  const uint8_t* experts;  // resident expert array or slot pool
  const int32_t* ids;      // device ids [k] of this token, or nullptr (slots / in-kernel top-k)
  SlotList slot;           // cache mode: slot of each rank
  SlotList rsel;           // gate/up: routed ranks to compute (rsel.v[0..nsel)); nsel 0 = all k
  int nsel;
  const uint8_t* shared;   // shared expert blob
  size_t blob_e, blob_s;
  int H, I, Is, k;
  // in-kernel routing (gate/up kernel, resident mode): top-k of the fp64
  // logits z [E]; the first block writes ids_g / w_g (and the optional copies)
  const double* z;
  int E;
  int32_t* ids_g;
  float* w_g;
  int32_t* ids2;
  float* w2;
};

// Misses to copy host -> slot by fill blocks (cache mode, fill-kernel option).
// With dlist, the list is in device memory (written by the device-side cache
// step): dlist[0] misses, experts dlist[1 .. k], slots dlist[1 + k .. 2k];
// blob m is read at src_base + expert * bytes and written at dst_base +
// slot * bytes, and n (= k) blobs' worth of fill blocks are launched, those
// past the miss count leaving at once.
struct FillList {
  const uint8_t* src[kMaxTopK];  // device-accessible pinned host blobs
  uint8_t* dst[kMaxTopK];        // slots in HBM
  int n;                         // number of blobs
  int blocks_per_blob;           // in units of 1024 lanes (the launch may split them)
  size_t bytes;                  // blob size, a multiple of 16
  const int32_t* dlist;
  const uint8_t* src_base;
  uint8_t* dst_base;
};

// LFU (or LRU) expert-slot cache of one layer kept in device memory and
// stepped by one block after the token's top-k, with the host cache's rule (lowest
// empty slot, else the smallest (frequency, last use, slot), or (last use,
// slot) for LRU, among slots holding none of the token's ids; hits first).
struct DevCache {
  int32_t* expert;    // [n_slots], -1 = empty
  int32_t* freq;      // [n_slots]
  int32_t* last;      // [n_slots], -1 = never
  int32_t* where;     // [E] expert -> slot, -1 = absent
  long long* counters;  // [3]: steps, hits, misses
  int32_t* slot_of_rank;  // [k]
  int32_t* miss;      // [1 + 2k], see FillList::dlist
  int32_t* ev;        // [k][4]: expert, slot, hit, evicted
  int n_slots, policy;
};
// LDS bytes the step needs beyond the router's own.
size_t dcache_lds_bytes(int n_slots, int E);

// Gate/up GEMVs with the GeGLU epilogue for routed ranks [0,k), or the ranks
// src.rsel selects (do_routed), and/or the shared expert (do_shared). The activations a [k*I + I_s] leave
// as digit planes, one DigitGroup and one scale per 32 activations.
// t0/t1 (optional, both or neither): events stamped by the dispatch itself at
// the kernel's start and end (kernel time without the cost of separate records).
// fill (optional): blobs copied by extra blocks of the same launch.
// topk (optional, one token): an extra first block takes the top-k of the
// logits z (written by the previous launch), writes ids / w (and the
// optional copies), then the ids to host-coherent memory and seq to
// *seq_host with a system-scope release store, while the other blocks run.
struct TopkPublish {
  const double* z;
  int E, k;
  int32_t* ids;
  float* w;
  int32_t* ids2;
  float* w2;
  int32_t* ids_host;
  int32_t* seq_host;
  int32_t seq;
};
hipError_t launch_ffn_gateup(const SourceSet& src, bool do_routed, bool do_shared,
                             const DigitGroup* udig, const float* usc, DigitGroup* adig, float* asc,
                             hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr,
                             const FillList* fill = nullptr, const TopkPublish* topk = nullptr);
// Down GEMVs of all k+1 sources, weighted combine (w [k], shared weight 1),
// optional residual x' = x + add_in, y [H].
hipError_t launch_ffn_down(const SourceSet& src, const float* w, const DigitGroup* adig,
                           const float* asc, const float* x, const uint16_t* add_in, bool residual,
                           float* y, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Largest LDS footprint of the one-token kernels for a shape (bytes).
size_t decode_lds_bytes(int H, int E, int k, int I, int Is);

// ---------------------------------------------------------------- prefill
// Workspace layout of a prefill of up to T tokens (byte offsets).
// Experts of one slot-pool group and their slots (prefill through the pool).
constexpr int kMaxGroup = 16;
struct SlotGroup {
  int32_t expert[kMaxGroup];
  int32_t slot[kMaxGroup];
  int32_t n;
};

struct PrefillLayout {
  size_t ids, w, hist, base, local_rank, seg, tiles, n_tiles, perm, pos_of, act_r, act_s, out_r, xf, z,
      total;
  int chunks, max_tiles;
};
PrefillLayout prefill_layout(int T, int E, int k, int H, int I, int Is);
// Routing (given logits, or x . router), stable sort of the T*k assignments
// by expert, bf16 MFMA grouped GEMMs (gate/up + GeGLU, down weighted by the
// routing weight), shared expert, and the combine into y [T][H] fp32.
hipError_t launch_prefill(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16,
                          const float* logits_in, const uint16_t* router, const float* bias, int T,
                          int E, int k, int H, int I, int Is, const uint8_t* experts, size_t blob_e,
                          const uint8_t* shared, float* y, int32_t* ids_out, float* w_out,
                          hipStream_t s);
// Its stages, for prefill through the slot pool: routing and the stable sort
// of the assignments (seg / tiles / perm / pos_of in the layout); the routed
// GEMMs (group == nullptr: every expert, experts + id * blob_e; else only the
// group's experts, experts + slot * blob_e; with_shared: the shared expert's
// gate/up runs in the same launch as the routed one, and with y its down
// projection into y in the same launch as the routed down); the shared expert
// (its gate/up unless gateup_done, its down unless down_done) and the combine
// into y.
struct SharedGateup {
  const uint8_t* shared;
  int T, Is;
  float* y;  // nullable
};
hipError_t launch_prefill_route(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16,
                                const float* logits_in, const uint16_t* router, const float* bias, int T,
                                int E, int k, int H, int32_t* ids_out, float* w_out, hipStream_t s);
hipError_t launch_prefill_routed(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16, int k, int H,
                                 int I, const uint8_t* experts, size_t blob_e, const SlotGroup* group,
                                 hipStream_t s, const SharedGateup* with_shared = nullptr);
hipError_t launch_prefill_shared(const PrefillLayout& L, uint8_t* ws, const uint16_t* x_bf16, int T, int k,
                                 int H, int Is, const uint8_t* shared, float* y, hipStream_t s,
                                 bool gateup_done = false, bool down_done = false);

// Stable sort of A assignments (token*k + rank, expert ids[a]) by expert:
// seg [E+1] segment starts, perm [A] sorted position -> assignment, pos_of [A]
// assignment -> sorted position, tiles/n_tiles the GEMM tile table
// (expert, first row, rows; at most 128 rows per tile).
hipError_t launch_permute(const int32_t* ids, int A, int E, int chunks, int32_t* hist, int32_t* lrank,
                          int32_t* base, int32_t* seg, int4* tiles, int32_t* n_tiles, int32_t* perm,
                          int32_t* pos_of, hipStream_t s);
int permute_chunks(int A);

// ---------------------------------------------------------------- batched decode

struct BatchedBuffers {
  uint16_t* act_r;  // [B*k][I] fp16 GeGLU activations by assignment token*k + rank
  uint16_t* act_s;  // [B][Is]
  float* out_r;     // [B*k][H]
  float* out_s;     // [B][H]
};
// Whether the matrix-core kernels' LDS (activation slices for up to max_B
// tokens per pass plus the staged scales of a block's rows) fits one block.
bool batched_lds_fits(int H, int I, int Is, int max_B);
// Grouped gate/up and down products per expert on the matrix cores (inputs:
// u16/tsc of launch_route_layer and the ids [B][k]; every block finds its
// expert's tokens in the ids), then the combine.
hipError_t launch_batched(const BatchedBuffers& bb, const uint8_t* experts, const uint8_t* shared,
                          size_t blob_e, int H, int I, int Is, int E, int k, int B,
                          const uint16_t* u16, const float* tsc, const int32_t* ids, const float* w,
                          const float* x, const uint16_t* add_in, bool residual, float* y, hipStream_t s);

// ---------------------------------------------------------------- standalone GEMV
hipError_t launch_gemv_q4(const uint8_t* q, const uint16_t* sc, int N, int K, const float* x, int M,
                          float* y, hipStream_t s);
hipError_t launch_unpack_q4(const uint8_t* q, int N, int K, int8_t* out, hipStream_t s);
// Read-only stream of `bytes` (a multiple of 16) on blocks x 1024 threads;
// loads per lane = read_floor_loads(bytes, blocks), at most 16. With t0/t1 the
// dispatch stamps the events at its start and end.
int read_floor_loads(int64_t bytes, int blocks);
hipError_t launch_read_floor(const uint8_t* src, int64_t bytes, int blocks, uint32_t* out, hipEvent_t t0,
                             hipEvent_t t1, hipStream_t s);

// ---------------------------------------------------------------- attention step
struct AttnGemvArgs {
  const uint8_t* wq;   // int4 rows [N][K/2]
  const uint16_t* ws;  // fp16 scales [N][K/32]
  int K, N, RB;        // columns, rows, rows per block
  const float* x;      // projection input (RMSNorm in) or residual (output projection)
  const float* norm_w;
  float eps;
  const DigitGroup* adig;  // output projection input [K / 32] as digit planes
  const float* asc;        // and their scales
  float* y;            // output projection: y = x + W a
  int d, nh, nkv, pos, max_ctx;
  double log2_theta;
  float* q;            // rotated queries [nh][d]
  uint16_t* kc;        // fp16 caches [nkv][max_ctx][d]
  uint16_t* vc;
};

struct AttnSplitArgs {
  const float* q;
  const uint16_t* kc;
  const uint16_t* vc;
  int max_ctx, n;      // n = positions attended (pos + 1)
  float* pm;           // per-split max [nh][nsplit]
  float* pl;           // per-split sum of exponentials
  float* po;           // per-split unnormalised value sums [nh][nsplit][d]
  DigitGroup* adig;    // attention output [nh * d / 32] as digit planes
  float* asc;
};

struct AttnWorkspace {
  size_t q, adig, asc, pm, pl, po, total;
  int max_split;
};

struct AttnLaunch {
  int H, nh, nkv, d, max_ctx, pos;
  double theta;
  float eps;
  const float* norm_w;
  const uint8_t* qkv_q;
  const uint16_t* qkv_s;
  const uint8_t* o_q;
  const uint16_t* o_s;
  uint16_t* kc;
  uint16_t* vc;
  const float* x;
  float* y;
  void* workspace;
};

// Positions per split block of the attention kernel for head width d.
int attn_split_positions(int d);
// The projection kernels' LDS fits one block at this shape.
bool attn_lds_fits(int H, int nh, int nkv, int d);
AttnWorkspace attn_workspace(int nh, int d, int max_ctx);
hipError_t launch_attn_decode(const AttnLaunch& L, hipStream_t s);

}  // namespace moe
