// C-ABI entry points that need no layer handle: blob layout, routing, the
// standalone int4 GEMV and the nibble unpack. Every argument is checked
// before anything is enqueued.
#include <hip/hip_runtime.h>

#include <vector>

#include "host_common.h"
#include "launch.h"

using moe::fail;

namespace moe {

moe_status check_shape(const moe_shape* sh, const char* fn) {
  if (!sh) return fail(MOE_EINVAL, "%s: shape is NULL", fn);
  if (sh->group != kGroup) return fail(MOE_ESHAPE, "%s: group must be 32 (got %d)", fn, sh->group);
  if (sh->hidden < kGroup || sh->hidden > MOE_MAX_DIM || sh->hidden % kGroup)
    return fail(MOE_ESHAPE, "%s: hidden %d must be a multiple of 32 in [32, %d]", fn, sh->hidden, MOE_MAX_DIM);
  if (sh->n_experts < 1 || sh->n_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ESHAPE, "%s: n_experts %d outside [1, %d]", fn, sh->n_experts, MOE_MAX_EXPERTS);
  if (sh->top_k < 1 || sh->top_k > sh->n_experts || sh->top_k > MOE_MAX_TOPK)
    return fail(MOE_ESHAPE, "%s: top_k %d outside [1, min(n_experts, %d)]", fn, sh->top_k, MOE_MAX_TOPK);
  if (sh->inter < kGroup || sh->inter > MOE_MAX_DIM || sh->inter % kGroup)
    return fail(MOE_ESHAPE, "%s: inter %d must be a multiple of 32 in [32, %d]", fn, sh->inter, MOE_MAX_DIM);
  if (sh->shared_inter < kGroup || sh->shared_inter > MOE_MAX_DIM || sh->shared_inter % kGroup)
    return fail(MOE_ESHAPE, "%s: shared_inter %d must be a multiple of 32 in [32, %d]", fn,
                sh->shared_inter, MOE_MAX_DIM);
  return MOE_OK;
}

size_t route_ws_bytes(const moe_shape* sh, int32_t B) {
  return (static_cast<size_t>(B) * sh->n_experts * sizeof(double) + 255) & ~static_cast<size_t>(255);
}

}  // namespace moe

#define HIP_OR_FAIL(expr, fn)                                                        \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e_)); \
  } while (0)

extern "C" {

size_t moe_expert_bytes(int32_t hidden, int32_t inter) {
  if (hidden <= 0 || inter <= 0 || hidden % moe::kGroup || inter % moe::kGroup) return 0;
  return moe::blob_offsets(hidden, inter).total;
}

moe_status moe_blob_layout_of(int32_t hidden, int32_t inter, moe_blob_layout* out) {
  moe::clear_error();
  if (!out) return fail(MOE_EINVAL, "moe_blob_layout_of: out is NULL");
  if (moe_expert_bytes(hidden, inter) == 0)
    return fail(MOE_ESHAPE, "moe_blob_layout_of: hidden %d / inter %d not positive multiples of 32", hidden, inter);
  const moe::BlobOffsets o = moe::blob_offsets(hidden, inter);
  *out = moe_blob_layout{o.gate_q, o.up_q, o.down_q, o.gate_s, o.up_s, o.down_s, o.total};
  return MOE_OK;
}

size_t moe_route_workspace_bytes(const moe_shape* sh, int32_t B) {
  if (!sh || B < 0 || sh->n_experts < 1) return 0;
  return moe::route_ws_bytes(sh, B);
}

moe_status moe_route(const moe_shape* sh, const float* x, const uint16_t* wr, const float* bias,
                     const float* logits_in, int32_t B, int32_t* ids, float* w, void* workspace,
                     size_t workspace_bytes, void* stream) {
  moe::clear_error();
  const char* fn = "moe_route";
  moe_status st = moe::check_shape(sh, fn);
  if (st) return st;
  if (B < 0) return fail(MOE_ESHAPE, "%s: B=%d is negative", fn, B);
  if (B == 0) return MOE_OK;
  if (!ids || !w) return fail(MOE_EINVAL, "%s: ids and w must not be NULL", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (logits_in) {
    HIP_OR_FAIL(moe::launch_route_topk(nullptr, logits_in, B, sh->n_experts, sh->top_k, ids, w,
                                       nullptr, nullptr, s), fn);
    return MOE_OK;
  }
  if (!x || !wr) return fail(MOE_EINVAL, "%s: x and wr must not be NULL without logits_in", fn);
  if (!workspace) return fail(MOE_EINVAL, "%s: workspace is NULL", fn);
  if (!moe::aligned16(x) || !moe::aligned16(wr) || !moe::aligned16(workspace))
    return fail(MOE_EALIGN, "%s: x, wr and workspace must be 16-byte aligned", fn);
  if (workspace_bytes < moe::route_ws_bytes(sh, B))
    return fail(MOE_ENOMEM, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes,
                moe::route_ws_bytes(sh, B));
  double* z = static_cast<double*>(workspace);
  HIP_OR_FAIL(moe::launch_route_logits(x, B, sh->hidden, wr, bias, sh->n_experts, z, s), fn);
  HIP_OR_FAIL(moe::launch_route_topk(z, nullptr, B, sh->n_experts, sh->top_k, ids, w, nullptr,
                                     nullptr, s), fn);
  return MOE_OK;
}

moe_status moe_expert_gemv_q4(const moe_q4* W, int32_t N, int32_t K, const float* x, int32_t M,
                              float* y, void* stream) {
  moe::clear_error();
  const char* fn = "moe_expert_gemv_q4";
  if (!W || !W->q || !W->s || !x || !y) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  if (K < moe::kGroup || K % moe::kGroup || K > MOE_MAX_DIM)
    return fail(MOE_ESHAPE, "%s: K=%d must be a multiple of 32 in [32, %d]", fn, K, MOE_MAX_DIM);
  if (N < 0 || M < 0 || M > 64) return fail(MOE_ESHAPE, "%s: N=%d, M=%d (need N >= 0, 0 <= M <= 64)", fn, N, M);
  if (!moe::aligned16(W->q) || !moe::aligned16(x))
    return fail(MOE_EALIGN, "%s: W.q and x must be 16-byte aligned", fn);
  if (N == 0 || M == 0) return MOE_OK;
  HIP_OR_FAIL(moe::launch_gemv_q4(W->q, W->s, N, K, x, M, y, static_cast<hipStream_t>(stream)), fn);
  return MOE_OK;
}

moe_status moe_debug_unpack_q4(const moe_q4* W, int32_t N, int32_t K, int8_t* out, void* stream) {
  moe::clear_error();
  const char* fn = "moe_debug_unpack_q4";
  if (!W || !W->q || !out) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  if (K < 2 || K % 2 || N < 0) return fail(MOE_ESHAPE, "%s: N=%d, K=%d", fn, N, K);
  if (N == 0) return MOE_OK;
  HIP_OR_FAIL(moe::launch_unpack_q4(W->q, N, K, out, static_cast<hipStream_t>(stream)), fn);
  return MOE_OK;
}

static moe_status check_attn_shape(const moe_attn_shape* sh, const char* fn) {
  if (!sh) return fail(MOE_EINVAL, "%s: shape is NULL", fn);
  if (sh->hidden < moe::kGroup || sh->hidden > 4096 || sh->hidden % moe::kGroup)
    return fail(MOE_ESHAPE, "%s: hidden %d must be a multiple of 32 in [32, 4096]", fn, sh->hidden);
  if (sh->head_dim != 64 && sh->head_dim != 128 && sh->head_dim != 256)
    return fail(MOE_ESHAPE, "%s: head_dim %d must be 64, 128 or 256", fn, sh->head_dim);
  if (sh->n_kv_heads < 1 || sh->n_heads < sh->n_kv_heads || sh->n_heads % sh->n_kv_heads)
    return fail(MOE_ESHAPE, "%s: n_heads %d must be a positive multiple of n_kv_heads %d", fn, sh->n_heads,
                sh->n_kv_heads);
  const int G = sh->n_heads / sh->n_kv_heads;
  if (G != 1 && G != 2 && G != 4)
    return fail(MOE_ESHAPE, "%s: %d query heads per key/value head (1, 2 or 4 supported)", fn, G);
  if (sh->n_heads * sh->head_dim > 8192)
    return fail(MOE_ESHAPE, "%s: n_heads * head_dim = %d above 8192", fn, sh->n_heads * sh->head_dim);
  const int P = moe::attn_split_positions(sh->head_dim);
  if (sh->max_ctx < 1 || sh->max_ctx > P * P)
    return fail(MOE_ESHAPE, "%s: max_ctx %d outside [1, %d]", fn, sh->max_ctx, P * P);
  if (!(sh->rope_theta > 0.f) || !(sh->eps >= 0.f))
    return fail(MOE_EINVAL, "%s: rope_theta must be > 0 and eps >= 0", fn);
  if (!moe::attn_lds_fits(sh->hidden, sh->n_heads, sh->n_kv_heads, sh->head_dim))
    return fail(MOE_ESHAPE, "%s: the projection blocks' LDS exceeds 64 KiB at this shape", fn);
  return MOE_OK;
}

moe_status moe_attn_workspace_bytes(const moe_attn_shape* sh, size_t* out) {
  moe::clear_error();
  const char* fn = "moe_attn_workspace_bytes";
  if (!out) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  const moe_status st = check_attn_shape(sh, fn);
  if (st != MOE_OK) return st;
  *out = moe::attn_workspace(sh->n_heads, sh->head_dim, sh->max_ctx).total;
  return MOE_OK;
}

moe_status moe_attn_decode(const moe_attn_shape* sh, const moe_attn_weights* W, uint16_t* k_cache,
                           uint16_t* v_cache, int32_t pos, const float* x, float* y, void* workspace,
                           size_t workspace_bytes, void* stream) {
  moe::clear_error();
  const char* fn = "moe_attn_decode";
  moe_status st = check_attn_shape(sh, fn);
  if (st != MOE_OK) return st;
  if (!W || !W->norm_w || !W->qkv_q || !W->qkv_s || !W->o_q || !W->o_s || !k_cache || !v_cache || !x || !y ||
      !workspace)
    return fail(MOE_EINVAL, "%s: NULL argument", fn);
  if (pos < 0 || pos >= sh->max_ctx) return fail(MOE_EINVAL, "%s: pos %d outside [0, %d)", fn, pos, sh->max_ctx);
  if (!moe::aligned16(W->qkv_q) || !moe::aligned16(W->o_q) || !moe::aligned16(k_cache) ||
      !moe::aligned16(v_cache) || !moe::aligned16(workspace))
    return fail(MOE_EALIGN, "%s: projections, caches and workspace must be 16-byte aligned", fn);
  const size_t need = moe::attn_workspace(sh->n_heads, sh->head_dim, sh->max_ctx).total;
  if (workspace_bytes < need)
    return fail(MOE_ENOMEM, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
  moe::AttnLaunch L{};
  L.H = sh->hidden;
  L.nh = sh->n_heads;
  L.nkv = sh->n_kv_heads;
  L.d = sh->head_dim;
  L.max_ctx = sh->max_ctx;
  L.pos = pos;
  L.theta = sh->rope_theta;
  L.eps = sh->eps;
  L.norm_w = W->norm_w;
  L.qkv_q = W->qkv_q;
  L.qkv_s = W->qkv_s;
  L.o_q = W->o_q;
  L.o_s = W->o_s;
  L.kc = k_cache;
  L.vc = v_cache;
  L.x = x;
  L.y = y;
  L.workspace = workspace;
  HIP_OR_FAIL(moe::launch_attn_decode(L, static_cast<hipStream_t>(stream)), fn);
  return MOE_OK;
}

moe_status moe_debug_read_floor(const void* src, int64_t bytes, int64_t region_stride, int32_t regions,
                                int32_t blocks, int32_t reps, uint32_t* out, double* mean_us, void* stream) {
  moe::clear_error();
  const char* fn = "moe_debug_read_floor";
  if (!src || !out) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  if (bytes < 16 || bytes % 16 || regions < 1 || reps < 1 || blocks < 1 || blocks > 65536)
    return fail(MOE_ESHAPE, "%s: bytes %lld, regions %d, blocks %d, reps %d out of range", fn,
                static_cast<long long>(bytes), regions, blocks, reps);
  if (regions > 1 && (region_stride < bytes || region_stride % 16))
    return fail(MOE_ESHAPE, "%s: region_stride %lld must be a multiple of 16 and >= bytes", fn,
                static_cast<long long>(region_stride));
  if (moe::read_floor_loads(bytes, blocks) > 16)
    return fail(MOE_ESHAPE, "%s: %lld bytes need more than 16 loads per lane on %d blocks", fn,
                static_cast<long long>(bytes), blocks);
  if (!moe::aligned16(src)) return fail(MOE_EALIGN, "%s: src must be 16-byte aligned", fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* base = static_cast<const uint8_t*>(src);
  std::vector<hipEvent_t> ev;
  if (mean_us) {
    ev.resize(2 * static_cast<size_t>(reps), nullptr);
    for (auto& e : ev) {
      if (hipEventCreate(&e) != hipSuccess) {
        for (auto& f : ev)
          if (f) (void)hipEventDestroy(f);
        return fail(MOE_EHIP, "%s: hipEventCreate failed", fn);
      }
    }
  }
  moe_status st = MOE_OK;
  for (int i = 0; i < reps && st == MOE_OK; ++i) {
    const uint8_t* p = base + static_cast<int64_t>(i % regions) * region_stride;
    const hipError_t e = moe::launch_read_floor(p, bytes, blocks, out, mean_us ? ev[2 * i] : nullptr,
                                                mean_us ? ev[2 * i + 1] : nullptr, s);
    if (e != hipSuccess) st = fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
  }
  if (mean_us && st == MOE_OK) {
    double tot = 0.0;
    for (int i = 0; i < reps && st == MOE_OK; ++i) {
      float ms = 0.f;
      hipError_t e = hipEventSynchronize(ev[2 * i + 1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]);
      if (e != hipSuccess) st = fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
      tot += ms;
    }
    *mean_us = 1000.0 * tot / reps;
  }
  for (auto& e : ev) (void)hipEventDestroy(e);
  return st;
}

}  // extern "C"
