// Layer handle: one MoE layer's weights, workspace, streams and LFU cache.
//
// Decode of one token ("Como executar um modelo de 26 bilhões de parâmetros
// em dois gigabytes de memória em um Mac comum", section "Qual é o principal
// truque da arquitetura"): the router picks 8 experts; the expert cache
// (16 slots, LFU) is checked; missing experts are loaded into GPU-visible
// buffers while the GPU computes the shared-expert branch; then the experts
// run and are combined.
//
// Cache mode on one GPU: the slot pool lives in HBM, the backing store is
// pinned host memory, and each miss is one host->HBM copy on a side stream.
// The ids must reach the host before any copy can be issued (the routing of
// a layer depends on the previous layer's output), so a cache-mode call
// waits once: a block takes the top-k of the router logits and writes the ids
// to host-coherent memory and then a sequence word (system-scope release), and
// the host spins on that word (bounded) instead of a device->host copy and an
// event. With copy-engine fills that block is the first of the shared-expert
// gate/up launch (the router launch then only writes logits, and the shared
// expert computes while the host waits and the copies run); with fill blocks
// it is a one-block launch after the router. A slot overwritten for token t was
// last read by the previous call's kernels, which precede this call's routing
// kernel on the same stream and so have finished when the ids are published.
#include <hip/hip_runtime.h>
#include <string.h>

#include <chrono>
#include <new>
#include <vector>

#include "host_common.h"
#include "launch.h"

using moe::fail;

namespace moe {
moe_status check_shape(const moe_shape* sh, const char* fn);

// Widest hidden size of the one-token gate/up: a lane takes at most 16
// chunks (quantisation groups) of a row, 16 lanes a row.
constexpr int kMaxDecodeHidden = 16 * 16 * kGroup;

namespace {

struct WsLayout {
  size_t u, udig, usc, z, ids, w, adig, asc, cnt, pre;
  // device-stepped slot cache: counters, per-slot and per-expert arrays, the
  // call's slot per rank, miss list and events
  size_t dc;
  // batched decode (max_B > 1): fp16 inputs and per-assignment outputs
  size_t out_r, out_s, u16, tsc, act;
  size_t total;
};

// [3] int64 counters, then int32: expert, freq, last [E] (n_slots <= E),
// where [E], slot of rank [kMaxTopK], miss list [1 + 2 kMaxTopK], events
// [kMaxTopK][4]
size_t dcache_region_bytes(int E) {
  return 32 + sizeof(int32_t) * (4 * static_cast<size_t>(E) + kMaxTopK + 1 + 2 * kMaxTopK + 4 * kMaxTopK);
}

DevCache dcache_at(uint8_t* base, int E, int n_slots, int policy) {
  DevCache c{};
  c.counters = reinterpret_cast<long long*>(base);
  int32_t* p = reinterpret_cast<int32_t*>(base + 32);
  c.expert = p;
  c.freq = p + E;
  c.last = p + 2 * E;
  c.where = p + 3 * E;
  c.slot_of_rank = p + 4 * E;
  c.miss = c.slot_of_rank + kMaxTopK;
  c.ev = c.miss + 1 + 2 * kMaxTopK;
  c.n_slots = n_slots;
  c.policy = policy;
  return c;
}

WsLayout ws_layout(const moe_shape& sh, int maxB, int maxT) {
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += (n + 255) & ~static_cast<size_t>(255);
    return o;
  };
  const size_t H = sh.hidden, E = sh.n_experts, k = sh.top_k, I = sh.inter, Is = sh.shared_inter;
  const size_t ngu = H / kGroup, npos = (k * I + Is) / 8;
  const size_t B = maxB;
  WsLayout L;
  L.u = take(B * H * 4);
  L.udig = take(B * ngu * sizeof(DigitGroup));
  L.usc = take(B * ngu * 4);
  L.z = take(B * E * 8);
  L.ids = take(B * k * 4);
  L.w = take(B * k * 4);
  L.adig = take(B * npos * 16);
  L.asc = take(B * npos * 4);
  L.cnt = take(B * 4);  // router arrival counters, one per token
  L.dc = take(dcache_region_bytes(static_cast<int>(E)));
  L.pre = take(maxT > 0 ? prefill_layout(maxT, sh.n_experts, sh.top_k, sh.hidden, sh.inter,
                                         sh.shared_inter).total
                        : 0);
  const size_t A = B > 1 ? B * k : 0;
  L.out_r = take(A * H * 4);
  L.out_s = take(B > 1 ? B * H * 4 : 0);
  L.u16 = take(B > 1 ? B * H * 2 : 0);
  L.tsc = take(B > 1 ? B * 4 : 0);
  L.act = take(B > 1 ? (A * I + B * Is) * 2 : 0);
  L.total = off;
  return L;
}

}  // namespace
}  // namespace moe

// profiling kinds: 0 routing, 1 shared-expert gate/up (cache mode), 2 gate/up of
// the routed experts (plus the shared expert in resident mode), 3 down + combine,
// 4 prefill
constexpr int kProfKinds = 5;

struct moe_layer {
  moe_shape sh{};
  moe_layer_desc d{};
  bool cache_mode = false;
  bool dcache = false;     // the slot cache is stepped on the device
  moe::DevCache dc{};
  int max_B = 0, max_T = 0;
  moe_cache* cache = nullptr;
  moe_cache* cache_backup = nullptr;
  size_t blob_e = 0, blob_s = 0;
  moe::WsLayout ws{};
  uint8_t* wsb = nullptr;
  int32_t* ids_host = nullptr;  // host-coherent, [kMaxTopK] ids then the sequence word
  int32_t* seq_host = nullptr;
  int32_t seq = 0;              // sequence number of the last routing published
  const uint8_t* host_dev = nullptr;  // device address of experts_host (fill-kernel option)
  hipEvent_t ev_fill = nullptr;
  // a second copy stream of the handle's own: misses alternate between the
  // caller's copy stream and this one, so two copy engines overlap each
  // copy's fixed cost (ev_fill2: its copies of the last call)
  hipStream_t copy2 = nullptr;
  hipEvent_t ev_fill2 = nullptr;
  bool fill2_pending = false;
  // file store (cache mode): the misses are read into pinned staging first
  uint8_t* staging = nullptr;            // [kMaxTopK][stride]
  const uint8_t* staging_dev = nullptr;  // its device address (fill-kernel option)
  int64_t stride = 0;
  bool staging_busy = false;  // copies out of the staging may still run (ev_fill)
  // prefill through the slot pool (cache mode)
  int32_t* seg_host = nullptr;    // pinned, the chunk's expert offsets [E+1]
  int32_t prefill_chunk = 128;    // tokens per chunk (the pages' value), at most max_T
  hipEvent_t ev_pool = nullptr;   // the pool's readers (kernels on the call's stream) are done
  // test support: the fail_copy_in-th miss copy from now on fails before it
  // is issued, as if the runtime had refused it (0 = off)
  int32_t fail_copy_in = 0;
  // stage times (MOE_F_STAGE_TIMES): start of the call on the stream, the two
  // copy streams' first and last copy, the stream's wait for them, the end
  hipEvent_t st_t0 = nullptr, st_c0 = nullptr, st_c1 = nullptr, st_d0 = nullptr, st_d1 = nullptr;
  hipEvent_t st_w0 = nullptr, st_w1 = nullptr, st_end = nullptr;
  // profiling
  bool prof = false;
  uint32_t prof_mask = 0;  // kinds recorded while profiling (bit i = kind i)
  uint32_t prof_every = 1; // record one call in prof_every
  uint32_t prof_calls = 0;
  bool prof_now = false;   // this call is recorded
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[kProfKinds];
  std::vector<hipEvent_t> pool;
  int64_t prof_launches[kProfKinds] = {};
  double prof_ms[kProfKinds] = {};

  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(wsb + off); }
};

namespace {

hipEvent_t pool_get(moe_layer* L) {
  if (!L->pool.empty()) {
    hipEvent_t e = L->pool.back();
    L->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records an event before a launch when profiling; returns it (or nullptr).
hipEvent_t prof_begin(moe_layer* L, int kind, hipStream_t s) {
  if (!L->prof_now || !(L->prof_mask & (1u << kind))) return nullptr;
  hipEvent_t e = pool_get(L);
  if (e && hipEventRecord(e, s) != hipSuccess) {
    L->pool.push_back(e);
    return nullptr;
  }
  return e;
}

void prof_end(moe_layer* L, int kind, hipEvent_t b, hipStream_t s) {
  if (!b) return;
  hipEvent_t e = pool_get(L);
  if (!e || hipEventRecord(e, s) != hipSuccess) {
    L->pool.push_back(b);
    if (e) L->pool.push_back(e);
    return;
  }
  L->rec[kind].emplace_back(b, e);
}

// Events for a single-kernel stage, stamped by the kernel's own dispatch
// (start and end of the kernel), so the figure is the kernel's duration.
struct ProfPair {
  hipEvent_t a = nullptr, b = nullptr;
};

ProfPair prof_pair(moe_layer* L, int kind) {
  if (!L->prof_now || !(L->prof_mask & (1u << kind))) return {};
  hipEvent_t a = pool_get(L);
  hipEvent_t b = a ? pool_get(L) : nullptr;
  if (!b) {
    if (a) L->pool.push_back(a);
    return {};
  }
  return {a, b};
}

void prof_add(moe_layer* L, int kind, ProfPair p) {
  if (p.a) L->rec[kind].emplace_back(p.a, p.b);
}

// Waits until the routing kernel has published the ids of call L->seq (it
// writes them to host-coherent memory, then the sequence word with release
// semantics). Bounded: false after 10 s without it (a failed or stalled launch).
bool wait_routing(moe_layer* L) {
  const auto t0 = std::chrono::steady_clock::now();
  for (uint32_t spin = 0;; ++spin) {
    if (__atomic_load_n(L->seq_host, __ATOMIC_ACQUIRE) == L->seq) return true;
    if ((spin & 1023u) == 1023u &&
        std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10))
      return false;
#if defined(__x86_64__)
    __builtin_ia32_pause();
#endif
  }
}

moe::SourceSet make_sources(const moe_layer* L) {
  moe::SourceSet S{};
  S.shared = L->d.shared_blob;
  S.blob_e = L->blob_e;
  S.blob_s = L->blob_s;
  S.H = L->sh.hidden;
  S.I = L->sh.inter;
  S.Is = L->sh.shared_inter;
  S.k = L->sh.top_k;
  return S;
}

// One miss copy host -> slot on copy stream cs, unless the test hook says
// that this one fails first.
hipError_t enqueue_miss_copy(moe_layer* L, uint8_t* dst, const uint8_t* src, hipStream_t cs, bool* injected) {
  if (L->fail_copy_in > 0 && --L->fail_copy_in == 0) {
    *injected = true;
    return hipErrorUnknown;
  }
  return hipMemcpyAsync(dst, src, L->blob_e, hipMemcpyHostToDevice, cs);
}

// A step of the miss fill failed after n_enq copies (or fill blocks) into
// the slots enq_slot[] had been enqueued. Those copies still run: wait for
// them (so that none writes a slot after this returns and no later copy into
// the same slot can race with it), restore the cache's state from before the
// call's step, and mark each of those slots empty, since its bytes are no
// longer its old expert's and may not yet be the new one's. A later call
// then refills them like any other miss.
moe_status undo_fill(moe_layer* L, const int32_t* enq_slot, int n_enq, bool kernel_fill, hipStream_t s,
                     const char* fn, const char* what, hipError_t cause, bool injected) {
  if (n_enq > 0) {
    if (kernel_fill) (void)hipStreamSynchronize(s);
    if (L->d.copy_stream) (void)hipStreamSynchronize(static_cast<hipStream_t>(L->d.copy_stream));
    if (L->copy2) (void)hipStreamSynchronize(L->copy2);
    (void)hipGetLastError();
  }
  moe::cache_assign(L->cache, L->cache_backup);
  for (int i = 0; i < n_enq; ++i) moe::cache_clear_slot(L->cache, enq_slot[i]);
  if (n_enq > 0) {
    L->staging_busy = false;
    L->fill2_pending = false;
  }
  return fail(MOE_EHIP, "%s: %s: %s", fn, what,
              injected ? "failure injected by moe_debug_fail_copy" : hipGetErrorString(cause));
}

float elapsed_ms(hipEvent_t a, hipEvent_t b) {
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return -1.f;
  return ms;
}

}  // namespace

#define HIP_OR_FAIL(expr, fn)                                                        \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e_)); \
  } while (0)

extern "C" {

moe_status moe_layer_workspace_bytes(const moe_shape* sh, int32_t max_B, int32_t max_T, size_t* out) {
  moe::clear_error();
  moe_status st = moe::check_shape(sh, "moe_layer_workspace_bytes");
  if (st) return st;
  if (!out) return fail(MOE_EINVAL, "moe_layer_workspace_bytes: out is NULL");
  if (max_B < 1 || max_B > 4096 || max_T < 0 || max_T > 65536)
    return fail(MOE_ESHAPE, "moe_layer_workspace_bytes: max_B %d / max_T %d out of range", max_B, max_T);
  *out = moe::ws_layout(*sh, max_B, max_T).total;
  return MOE_OK;
}

moe_status moe_layer_create(const moe_shape* sh, const moe_layer_desc* d, int32_t max_B,
                            int32_t max_T, moe_layer** out) {
  moe::clear_error();
  const char* fn = "moe_layer_create";
  moe_status st = moe::check_shape(sh, fn);
  if (st) return st;
  if (!d || !out) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  if (max_B < 1 || max_B > 4096 || max_T < 0 || max_T > 65536)
    return fail(MOE_ESHAPE, "%s: max_B %d / max_T %d out of range", fn, max_B, max_T);
  if (sh->hidden > moe::kMaxDecodeHidden)
    return fail(MOE_ESHAPE, "%s: hidden %d above %d (the one-token gate/up takes at most 16 chunks of a row per lane)",
                fn, sh->hidden, moe::kMaxDecodeHidden);
  const int nga = (sh->top_k * sh->inter + sh->shared_inter) / moe::kGroup;
  if (nga > 512)
    return fail(MOE_ESHAPE, "%s: (top_k*inter + shared_inter)/32 = %d exceeds 512", fn, nga);
  const size_t lds = moe::decode_lds_bytes(sh->hidden, sh->n_experts, sh->top_k, sh->inter, sh->shared_inter);
  if (lds > 65536)
    return fail(MOE_ESHAPE, "%s: shape needs %zu bytes of LDS per decode block (limit 65536)", fn, lds);
  if (max_B > 1 && !moe::batched_lds_fits(sh->hidden, sh->inter, sh->shared_inter, max_B))
    return fail(MOE_ESHAPE, "%s: batched decode of this shape needs more LDS per block than the device has", fn);
  if (!d->router || !d->shared_blob || !d->workspace)
    return fail(MOE_EINVAL, "%s: router, shared_blob and workspace are required", fn);
  const bool cache_mode = d->experts_dev == nullptr;
  if (cache_mode) {
    if (!d->slot_pool || (!d->experts_host) == (!d->store))
      return fail(MOE_EINVAL, "%s: cache mode needs slot_pool and exactly one of experts_host and store", fn);
    if (d->store &&
        !moe::store_fits(d->store, d->store_layer, sh->n_experts, moe_expert_bytes(sh->hidden, sh->inter)))
      return fail(MOE_ESHAPE, "%s: the store has no layer %d of %d blobs of this shape", fn, d->store_layer,
                  sh->n_experts);
    if (d->cache_policy != MOE_POLICY_LFU && d->cache_policy != MOE_POLICY_LRU)
      return fail(MOE_EINVAL, "%s: unknown cache_policy %d", fn, d->cache_policy);
    if (d->n_slots < sh->top_k || d->n_slots > sh->n_experts)
      return fail(MOE_ESHAPE, "%s: n_slots %d outside [top_k=%d, n_experts=%d]", fn, d->n_slots,
                  sh->top_k, sh->n_experts);
    if (!moe::aligned16(d->slot_pool)) return fail(MOE_EALIGN, "%s: slot_pool not 16-byte aligned", fn);
    if (d->cache_on_device && d->store)
      return fail(MOE_EINVAL, "%s: a device-stepped cache fills from experts_host, not from a store", fn);
    if (d->cache_on_device &&
        sizeof(double) * sh->n_experts + moe::dcache_lds_bytes(d->n_slots, sh->n_experts) > 65536)
      return fail(MOE_ESHAPE, "%s: the device-stepped cache of %d slots and %d experts exceeds 64 KiB of LDS", fn,
                  d->n_slots, sh->n_experts);
  } else if (d->cache_on_device) {
    return fail(MOE_EINVAL, "%s: cache_on_device needs a cache-mode handle", fn);
  } else if (!moe::aligned16(d->experts_dev)) {
    return fail(MOE_EALIGN, "%s: experts_dev not 16-byte aligned", fn);
  }
  if (!moe::aligned16(d->router) || !moe::aligned16(d->shared_blob) || !moe::aligned16(d->workspace))
    return fail(MOE_EALIGN, "%s: router, shared_blob and workspace must be 16-byte aligned", fn);
  const moe::WsLayout ws = moe::ws_layout(*sh, max_B, max_T);
  if (d->workspace_bytes < ws.total)
    return fail(MOE_ENOMEM, "%s: workspace %zu bytes < %zu needed", fn, d->workspace_bytes, ws.total);

  moe_layer* L = new (std::nothrow) moe_layer;
  if (!L) return fail(MOE_ENOMEM, "%s: out of host memory", fn);
  L->sh = *sh;
  L->d = *d;
  L->cache_mode = cache_mode;
  L->max_B = max_B;
  L->max_T = max_T;
  L->blob_e = moe_expert_bytes(sh->hidden, sh->inter);
  L->blob_s = moe_expert_bytes(sh->hidden, sh->shared_inter);
  L->ws = ws;
  L->wsb = static_cast<uint8_t*>(d->workspace);
  auto cleanup = [&](moe_status code, const char* what, hipError_t e) {
    moe_layer_destroy(L);
    return fail(code, "%s: %s: %s", fn, what, hipGetErrorString(e));
  };
  hipError_t e = hipMemset(L->wsb + ws.cnt, 0, static_cast<size_t>(max_B) * 4);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return cleanup(MOE_EHIP, "clearing the workspace counters", e);
  if (cache_mode) {
    // the routing kernel writes the ids here and then bumps the sequence word
    // with a system-scope release store; coherent memory makes both visible
    // to the host without a copy
    e = hipHostMalloc(reinterpret_cast<void**>(&L->ids_host), sizeof(int32_t) * (moe::kMaxTopK + 16),
                      hipHostMallocCoherent | hipHostMallocMapped);
    if (e != hipSuccess) return cleanup(MOE_EHIP, "host-coherent ids buffer", e);
    L->seq_host = L->ids_host + moe::kMaxTopK;
    *L->seq_host = 0;
    // the fill-kernel option reads the store from the device; pinned memory
    // from hipHostMalloc has a device address, other memory has none
    if (d->store) {
      // staging for one token's misses, page aligned (unbuffered reads)
      L->stride = moe_store_stride(static_cast<int64_t>(L->blob_e));
      e = hipHostMalloc(reinterpret_cast<void**>(&L->staging), static_cast<size_t>(L->stride) * moe::kMaxTopK,
                        hipHostMallocDefault);
      if (e != hipSuccess) return cleanup(MOE_EHIP, "pinned staging for the store", e);
      void* dp = nullptr;
      if (hipHostGetDevicePointer(&dp, L->staging, 0) == hipSuccess) L->staging_dev = static_cast<const uint8_t*>(dp);
      (void)hipGetLastError();
    } else {
      hipPointerAttribute_t pa{};
      if (hipPointerGetAttributes(&pa, d->experts_host) == hipSuccess && pa.type == hipMemoryTypeHost &&
          pa.devicePointer)
        L->host_dev = static_cast<const uint8_t*>(pa.devicePointer);
      (void)hipGetLastError();  // a failed query leaves the option unavailable, not an error
    }
    e = hipEventCreateWithFlags(&L->ev_fill, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&L->ev_fill2, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&L->copy2, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&L->ev_pool, hipEventDisableTiming);
    for (hipEvent_t* t : {&L->st_t0, &L->st_c0, &L->st_c1, &L->st_d0, &L->st_d1, &L->st_w0, &L->st_w1, &L->st_end})
      if (e == hipSuccess) e = hipEventCreate(t);
    if (e != hipSuccess) return cleanup(MOE_EHIP, "events", e);
    if (max_T > 0) {
      e = hipHostMalloc(reinterpret_cast<void**>(&L->seg_host), sizeof(int32_t) * (sh->n_experts + 1),
                        hipHostMallocDefault);
      if (e != hipSuccess) return cleanup(MOE_EHIP, "pinned expert offsets", e);
    }
    if (d->cache_on_device) {
      // the fill blocks read the misses from experts_host through its device address
      if (!L->host_dev) {
        moe_layer_destroy(L);
        return fail(MOE_EINVAL, "%s: cache_on_device needs experts_host in device-accessible pinned memory", fn);
      }
      const int E = sh->n_experts;
      std::vector<uint8_t> init(moe::dcache_region_bytes(E), 0);
      int32_t* p = reinterpret_cast<int32_t*>(init.data() + 32);
      for (int i = 0; i < 4 * E; ++i) p[i] = (i < E || i >= 2 * E) ? -1 : 0;  // expert, last, where: -1
      e = hipMemcpy(L->wsb + ws.dc, init.data(), init.size(), hipMemcpyHostToDevice);
      if (e != hipSuccess) return cleanup(MOE_EHIP, "device cache state", e);
      L->dcache = true;
      L->dc = moe::dcache_at(L->wsb + ws.dc, E, d->n_slots, d->cache_policy);
    }
    moe_status cs = moe_cache_create_policy(d->n_slots, sh->n_experts, d->cache_policy, &L->cache);
    if (!cs) cs = moe_cache_create_policy(d->n_slots, sh->n_experts, d->cache_policy, &L->cache_backup);
    if (cs) {
      moe_layer_destroy(L);
      return cs;
    }
  }
  *out = L;
  return MOE_OK;
}

void moe_layer_destroy(moe_layer* L) {
  if (!L) return;
  if (L->ids_host) (void)hipHostFree(L->ids_host);
  if (L->staging) (void)hipHostFree(L->staging);
  if (L->seg_host) (void)hipHostFree(L->seg_host);
  if (L->ev_pool) (void)hipEventDestroy(L->ev_pool);
  if (L->ev_fill) (void)hipEventDestroy(L->ev_fill);
  if (L->ev_fill2) (void)hipEventDestroy(L->ev_fill2);
  if (L->copy2) (void)hipStreamDestroy(L->copy2);
  for (hipEvent_t t : {L->st_t0, L->st_c0, L->st_c1, L->st_d0, L->st_d1, L->st_w0, L->st_w1, L->st_end})
    if (t) (void)hipEventDestroy(t);
  for (auto& v : L->rec)
    for (auto& p : v) {
      (void)hipEventDestroy(p.first);
      (void)hipEventDestroy(p.second);
    }
  for (hipEvent_t e : L->pool) (void)hipEventDestroy(e);
  moe_cache_destroy(L->cache);
  moe_cache_destroy(L->cache_backup);
  delete L;
}

moe_status moe_layer_set_experts(moe_layer* L, const uint8_t* experts_dev) {
  moe::clear_error();
  if (!L || !experts_dev) return fail(MOE_EINVAL, "moe_layer_set_experts: NULL argument");
  if (L->cache_mode) return fail(MOE_ESTATE, "moe_layer_set_experts: handle is in cache mode");
  if (!moe::aligned16(experts_dev)) return fail(MOE_EALIGN, "moe_layer_set_experts: not 16-byte aligned");
  L->d.experts_dev = experts_dev;
  return MOE_OK;
}

moe_cache* moe_layer_cache(moe_layer* L) { return L && !L->dcache ? L->cache : nullptr; }

moe_status moe_layer_cache_state(moe_layer* L, int32_t* expert, int32_t* freq, int64_t* last, int32_t n,
                                 int64_t* hits, int64_t* misses, int64_t* steps, void* stream) {
  moe::clear_error();
  const char* fn = "moe_layer_cache_state";
  if (!L) return fail(MOE_EINVAL, "%s: NULL handle", fn);
  if (!L->cache_mode) return fail(MOE_ESTATE, "%s: resident handle has no slot cache", fn);
  if ((expert || freq || last) && n != L->d.n_slots)
    return fail(MOE_ESHAPE, "%s: n=%d but n_slots=%d", fn, n, L->d.n_slots);
  if (!L->dcache) {
    moe_status st = moe_cache_slots(L->cache, expert, freq, last, (expert || freq || last) ? n : L->d.n_slots);
    if (st) return st;
    return moe_cache_counters(L->cache, hits, misses, steps);
  }
  const int S = L->d.n_slots;
  std::vector<int32_t> ex(S), fr(S), la(S);
  long long cnt[3];
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipMemcpy(cnt, L->dc.counters, sizeof(cnt), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(ex.data(), L->dc.expert, sizeof(int32_t) * S, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(fr.data(), L->dc.freq, sizeof(int32_t) * S, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(la.data(), L->dc.last, sizeof(int32_t) * S, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
  for (int s = 0; s < S; ++s) {
    if (expert) expert[s] = ex[s];
    if (freq) freq[s] = fr[s];
    if (last) last[s] = la[s];
  }
  if (steps) *steps = cnt[0];
  if (hits) *hits = cnt[1];
  if (misses) *misses = cnt[2];
  return MOE_OK;
}

moe_status moe_layer_decode(moe_layer* L, const float* x, const uint16_t* add_in, int32_t B,
                            uint32_t flags, float* y, int32_t* ids_out, float* w_out, float* u_out,
                            moe_cache_event* trace, moe_decode_stats* stats, void* stream) {
  moe::clear_error();
  const char* fn = "moe_layer_decode";
  if (!L) return fail(MOE_EINVAL, "%s: NULL handle", fn);
  if (flags & ~(MOE_F_RMSNORM_IN | MOE_F_RESIDUAL | MOE_F_FILL_KERNEL | MOE_F_STAGE_TIMES))
    return fail(MOE_EINVAL, "%s: unknown flags 0x%x", fn, flags);
  const bool timed = flags & MOE_F_STAGE_TIMES;
  if (timed && (!L->cache_mode || L->dcache || !stats))
    return fail(MOE_EINVAL, "%s: MOE_F_STAGE_TIMES needs a host-stepped cache-mode handle and stats", fn);
  const bool fill_kernel = flags & MOE_F_FILL_KERNEL;
  if (fill_kernel && !L->cache_mode) return fail(MOE_EINVAL, "%s: MOE_F_FILL_KERNEL needs a cache-mode handle", fn);
  if (fill_kernel && !(L->d.store ? L->staging_dev : L->host_dev))
    return fail(MOE_EINVAL, "%s: MOE_F_FILL_KERNEL needs experts_host in device-accessible pinned memory", fn);
  if (B < 0 || B > L->max_B) return fail(MOE_ESHAPE, "%s: B=%d outside [0, max_B=%d]", fn, B, L->max_B);
  if (B == 0) return MOE_OK;
  if (!x || !y) return fail(MOE_EINVAL, "%s: x and y are required", fn);
  L->prof_now = L->prof && (L->prof_calls++ % L->prof_every) == 0;
  if (x == y) return fail(MOE_EINVAL, "%s: y must not alias x", fn);
  if (!moe::aligned16(x) || (add_in && !moe::aligned16(add_in)))
    return fail(MOE_EALIGN, "%s: x and add_in must be 16-byte aligned", fn);
  if (L->cache_mode && B != 1) return fail(MOE_ESHAPE, "%s: cache mode decodes one token per call", fn);
  const moe_shape& sh = L->sh;
  const int H = sh.hidden, E = sh.n_experts, k = sh.top_k;
  const int ngu = H / moe::kGroup;
  const int npos = (k * sh.inter + sh.shared_inter) / 8;
  hipStream_t s = static_cast<hipStream_t>(stream);

  auto* udig = L->at<moe::DigitGroup>(L->ws.udig);
  float* usc = L->at<float>(L->ws.usc);
  double* z = L->at<double>(L->ws.z);
  int32_t* ids = L->at<int32_t>(L->ws.ids);
  float* w = L->at<float>(L->ws.w);
  uint4* adig = L->at<uint4>(L->ws.adig);
  float* asc = L->at<float>(L->ws.asc);
  int32_t* cnt = L->at<int32_t>(L->ws.cnt);
  const bool rms = flags & MOE_F_RMSNORM_IN;
  const bool res = flags & MOE_F_RESIDUAL;

  const auto t_host0 = std::chrono::steady_clock::now();
  float ms_route = 0.f;
  if (timed) HIP_OR_FAIL(hipEventRecord(L->st_t0, s), fn);
  hipEvent_t pb = prof_begin(L, 0, s);
  // grouped path (B > 1, all experts resident): every touched expert is read
  // once per call by the matrix-core kernels, which take fp16 inputs and
  // find each expert's tokens in the ids; the router also takes each token's
  // top-k
  const bool grouped = !L->cache_mode && B > 1;
  // one token, resident: the router only produces logits; each gate/up block
  // takes the top-k itself (no cross-block handshake on the critical path)
  const bool in_kernel_topk = !L->cache_mode && !grouped;
  // one token, host-stepped cache with copy-engine fills: the router only
  // produces logits too; an extra first block of the shared-expert gate/up
  // launch takes the top-k and publishes the ids to the host, so the router
  // launch ends sooner and the host's wait overlaps the shared expert
  const bool deferred_topk = L->cache_mode && !L->dcache && !fill_kernel;
  // one token, cache mode otherwise (device-stepped cache, or fill blocks that
  // need the misses before their launch): the logits-only router is followed
  // by a one-block selection launch that takes the top-k and steps the cache
  // or publishes the ids (shorter than a last-arriving block of the router)
  const bool select_launch = L->cache_mode && !deferred_topk;
  const bool router_topk = !in_kernel_topk && !deferred_topk && !select_launch;
  uint16_t* u16 = grouped ? L->at<uint16_t>(L->ws.u16) : nullptr;
  float* tsc = grouped ? L->at<float>(L->ws.tsc) : nullptr;
  const int32_t seq = L->cache_mode ? L->seq + 1 : 0;
  HIP_OR_FAIL(moe::launch_route_layer(x, add_in, B, H, rms, L->d.router, L->d.bias, E, k, u_out,
                                      grouped ? nullptr : udig, usc, u16, tsc, z, cnt,
                                      router_topk ? ids : nullptr, router_topk ? w : nullptr,
                                      router_topk ? ids_out : nullptr, router_topk ? w_out : nullptr, s),
              fn);
  if (select_launch)
    HIP_OR_FAIL(moe::launch_route_select(z, E, k, ids, w, ids_out, w_out, L->dcache ? nullptr : L->ids_host,
                                         L->dcache ? nullptr : L->seq_host, seq, L->dcache ? &L->dc : nullptr, s),
                fn);
  if (L->cache_mode && !L->dcache) L->seq = seq;
  prof_end(L, 0, pb, s);

  moe::SourceSet S = make_sources(L);
  if (grouped) {
    // batched: grouped GEMVs that read each touched expert once, ordered combine
    const int A = B * k;
    uint16_t* act = L->at<uint16_t>(L->ws.act);
    moe::BatchedBuffers bb{act, act + static_cast<size_t>(A) * sh.inter, L->at<float>(L->ws.out_r),
                           L->at<float>(L->ws.out_s)};
    hipEvent_t p1 = prof_begin(L, 2, s);
    HIP_OR_FAIL(moe::launch_batched(bb, L->d.experts_dev, L->d.shared_blob, L->blob_e, H, sh.inter,
                                    sh.shared_inter, E, k, B, u16, tsc, ids, w, x, add_in, res, y, s), fn);
    prof_end(L, 2, p1, s);
    if (stats) stats->calls += 1;
    return MOE_OK;
  }
  if (!L->cache_mode) {
    // token by token: routed + shared gate/up (with the in-kernel top-k), then down
    S.experts = L->d.experts_dev;
    S.E = E;
    for (int b = 0; b < B; ++b) {
      const size_t ko = static_cast<size_t>(b) * k;
      moe::SourceSet G = S;
      G.ids = nullptr;
      G.z = z + static_cast<size_t>(b) * E;
      G.ids_g = ids + ko;
      G.w_g = w + ko;
      G.ids2 = ids_out ? ids_out + ko : nullptr;
      G.w2 = w_out ? w_out + ko : nullptr;
      auto* adb = reinterpret_cast<moe::DigitGroup*>(adig + static_cast<size_t>(b) * npos);
      float* asb = asc + static_cast<size_t>(b) * npos;
      const ProfPair p1 = prof_pair(L, 2);
      HIP_OR_FAIL(moe::launch_ffn_gateup(G, true, true, udig + static_cast<size_t>(b) * ngu,
                                         usc + static_cast<size_t>(b) * ngu, adb, asb, s, p1.a, p1.b), fn);
      prof_add(L, 2, p1);
      S.ids = ids + ko;
      const ProfPair p2 = prof_pair(L, 3);
      HIP_OR_FAIL(moe::launch_ffn_down(S, w + ko, adb, asb, x + static_cast<size_t>(b) * H,
                                       add_in ? add_in + static_cast<size_t>(b) * H : nullptr, res,
                                       y + static_cast<size_t>(b) * H, s, p2.a, p2.b), fn);
      prof_add(L, 3, p2);
    }
    if (stats) stats->calls += 1;
    return MOE_OK;
  }

  // ---- cache mode, one token
  S.experts = L->d.slot_pool;
  S.ids = nullptr;
  auto* adg = reinterpret_cast<moe::DigitGroup*>(adig);
  if (L->dcache) {
    // the routing kernel has stepped the cache: the fill blocks take the miss
    // list and the expert kernels each rank's slot from device memory
    moe::FillList F{};
    F.n = k;
    F.blocks_per_blob = 16;
    F.bytes = L->blob_e;
    F.dlist = L->dc.miss;
    F.src_base = L->host_dev;
    F.dst_base = L->d.slot_pool;
    const ProfPair p1 = prof_pair(L, 1);
    HIP_OR_FAIL(moe::launch_ffn_gateup(S, false, true, udig, usc, adg, asc, s, p1.a, p1.b, &F), fn);
    prof_add(L, 1, p1);
    S.ids = L->dc.slot_of_rank;
    {
      const ProfPair p2 = prof_pair(L, 2);
      HIP_OR_FAIL(moe::launch_ffn_gateup(S, true, false, udig, usc, adg, asc, s, p2.a, p2.b), fn);
      prof_add(L, 2, p2);
      const ProfPair p3 = prof_pair(L, 3);
      HIP_OR_FAIL(moe::launch_ffn_down(S, w, adg, asc, x, add_in, res, y, s, p3.a, p3.b), fn);
      prof_add(L, 3, p3);
    }
    if (trace) {
      int32_t evd[4 * moe::kMaxTopK];
      hipError_t te = hipMemcpyAsync(evd, L->dc.ev, sizeof(int32_t) * 4 * k, hipMemcpyDeviceToHost, s);
      if (te == hipSuccess) te = hipStreamSynchronize(s);
      if (te != hipSuccess) return fail(MOE_EHIP, "%s: reading the cache events: %s", fn, hipGetErrorString(te));
      for (int j = 0; j < k; ++j) trace[j] = moe_cache_event{evd[4 * j], evd[4 * j + 1], evd[4 * j + 2], evd[4 * j + 3]};
    }
    if (stats) stats->calls += 1;
    return MOE_OK;
  }
  if (!fill_kernel) {
    // the shared-expert gate/up runs while the host waits for the ids and
    // while the copy engine fills the misses
    const moe::TopkPublish P{z, E, k, ids, w, ids_out, w_out, L->ids_host, L->seq_host, seq};
    const ProfPair p1 = prof_pair(L, 1);
    HIP_OR_FAIL(moe::launch_ffn_gateup(S, false, true, udig, usc, adg, asc, s, p1.a, p1.b, nullptr, &P), fn);
    prof_add(L, 1, p1);
  }
  if (!wait_routing(L)) return fail(MOE_EHIP, "%s: timed out waiting for the routing kernel", fn);
  if (timed) ms_route = std::chrono::duration<float, std::milli>(std::chrono::steady_clock::now() - t_host0).count();

  // LFU step; the pre-step state is kept so that a failed fill can restore it
  moe_cache_event ev[moe::kMaxTopK];
  int32_t n_miss = 0;
  moe::cache_assign(L->cache_backup, L->cache);
  moe_status cs = moe_cache_step(L->cache, L->ids_host, k, ev, &n_miss);
  if (cs) return cs;
  // where each miss's bytes come from (host and device addresses): the host
  // store, or the staging that the file store reads them into
  const uint8_t* src_h[moe::kMaxTopK];
  const uint8_t* src_d[moe::kMaxTopK];
  std::chrono::steady_clock::time_point t_read0;
  float ms_read = 0.f;
  if (L->d.store && n_miss > 0) {
    // the staging's previous copies (this handle's last call) must be done
    if (L->staging_busy) {
      hipError_t se = hipEventSynchronize(L->ev_fill);
      if (se == hipSuccess && L->fill2_pending) se = hipEventSynchronize(L->ev_fill2);
      if (se != hipSuccess) {
        moe::cache_assign(L->cache, L->cache_backup);
        return fail(MOE_EHIP, "%s: waiting for the staging: %s", fn, hipGetErrorString(se));
      }
      L->staging_busy = false;
      L->fill2_pending = false;
    }
    int32_t mexp[moe::kMaxTopK];
    void* mdst[moe::kMaxTopK];
    int nm = 0;
    for (int j = 0; j < k; ++j)
      if (!ev[j].hit) {
        mexp[nm] = ev[j].expert;
        mdst[nm] = L->staging + static_cast<size_t>(nm) * L->stride;
        ++nm;
      }
    if (timed) t_read0 = std::chrono::steady_clock::now();
    const moe_status rs = moe_store_read(L->d.store, L->d.store_layer, mexp, nm, mdst);
    if (rs) {
      moe::cache_assign(L->cache, L->cache_backup);
      return rs;
    }
    if (timed) ms_read = std::chrono::duration<float, std::milli>(std::chrono::steady_clock::now() - t_read0).count();
  }
  for (int j = 0, m = 0; j < k; ++j) {
    if (ev[j].hit) continue;
    if (L->d.store) {
      src_h[j] = L->staging + static_cast<size_t>(m) * L->stride;
      src_d[j] = L->staging_dev ? L->staging_dev + static_cast<size_t>(m) * L->stride : nullptr;
      ++m;
    } else {
      src_h[j] = L->d.experts_host + static_cast<size_t>(ev[j].expert) * L->blob_e;
      src_d[j] = L->host_dev ? L->host_dev + static_cast<size_t>(ev[j].expert) * L->blob_e : nullptr;
    }
  }
  for (int j = 0; j < k; ++j) S.slot.v[j] = ev[j].slot;
  // the ranks whose experts were resident need not wait for the copies: their
  // gate/up runs while the misses are copied, the missed ranks' after them
  const bool split = n_miss > 0 && n_miss < k;
  moe::SourceSet S_hit = S, S_miss = S;
  if (split)
    for (int j = 0; j < k; ++j) {
      moe::SourceSet& T = ev[j].hit ? S_hit : S_miss;
      T.rsel.v[T.nsel++] = j;
    }
  // slots that enqueued work writes (for undo_fill if a later step fails)
  int32_t enq_slot[moe::kMaxTopK];
  int n_enq = 0;
  bool injected = false;
  hipError_t ce = hipSuccess;
  bool used2 = false;
  if (fill_kernel) {
    // the misses are copied by fill blocks of the shared-expert gate/up launch
    // (with the hit ranks' gate/up blocks when split)
    moe::FillList F{};
    F.blocks_per_blob = 16;
    F.bytes = L->blob_e;
    for (int j = 0; j < k; ++j) {
      if (ev[j].hit) continue;
      F.src[F.n] = src_d[j];
      F.dst[F.n] = L->d.slot_pool + static_cast<size_t>(ev[j].slot) * L->blob_e;
      ++F.n;
    }
    if (timed) ce = hipEventRecord(L->st_c0, s);
    const ProfPair p1 = split ? ProfPair{} : prof_pair(L, 1);
    if (ce == hipSuccess)
      ce = moe::launch_ffn_gateup(split ? S_hit : S, split, true, udig, usc, adg, asc, s, p1.a, p1.b, &F);
    if (ce == hipSuccess) {
      prof_add(L, 1, p1);
      for (int j = 0; j < k; ++j)
        if (!ev[j].hit) enq_slot[n_enq++] = ev[j].slot;
    }
    if (ce == hipSuccess && timed) ce = hipEventRecord(L->st_c1, s);
    if (ce == hipSuccess && L->d.store && n_miss > 0) {
      ce = hipEventRecord(L->ev_fill, s);
      L->staging_busy = ce == hipSuccess;
    }
  } else {
    hipStream_t cp = static_cast<hipStream_t>(L->d.copy_stream);
    if (timed && n_miss > 0) {
      ce = hipEventRecord(L->st_c0, cp);
      if (ce == hipSuccess && n_miss > 1) ce = hipEventRecord(L->st_d0, L->copy2);
    }
    for (int j = 0, m = 0; j < k && ce == hipSuccess; ++j) {
      if (ev[j].hit) continue;
      const bool second = (m++ & 1) != 0;  // every other miss on the second copy stream
      ce = enqueue_miss_copy(L, L->d.slot_pool + static_cast<size_t>(ev[j].slot) * L->blob_e, src_h[j],
                             second ? L->copy2 : cp, &injected);
      if (ce == hipSuccess) {
        used2 = used2 || second;
        enq_slot[n_enq++] = ev[j].slot;
      }
    }
    if (ce == hipSuccess && n_miss > 0) {
      ce = hipEventRecord(L->ev_fill, cp);
      if (ce == hipSuccess && used2) ce = hipEventRecord(L->ev_fill2, L->copy2);
      if (ce == hipSuccess && timed) ce = hipEventRecord(L->st_c1, cp);
      if (ce == hipSuccess && timed && used2) ce = hipEventRecord(L->st_d1, L->copy2);
      if (ce == hipSuccess && split) ce = moe::launch_ffn_gateup(S_hit, true, false, udig, usc, adg, asc, s);
      if (ce == hipSuccess && timed) ce = hipEventRecord(L->st_w0, s);
      if (ce == hipSuccess) ce = hipStreamWaitEvent(s, L->ev_fill, 0);
      if (ce == hipSuccess && used2) ce = hipStreamWaitEvent(s, L->ev_fill2, 0);
      if (ce == hipSuccess && timed) ce = hipEventRecord(L->st_w1, s);
      L->staging_busy = ce == hipSuccess && L->d.store;
      L->fill2_pending = L->staging_busy && used2;
    }
  }
  if (ce != hipSuccess) return undo_fill(L, enq_slot, n_enq, fill_kernel, s, fn, "miss fill", ce, injected);
  {
    // profiled only where the launch covers all k ranks
    const ProfPair p2 = split ? ProfPair{} : prof_pair(L, 2);
    ce = moe::launch_ffn_gateup(split ? S_miss : S, true, false, udig, usc, adg, asc, s, p2.a, p2.b);
    if (ce != hipSuccess) return undo_fill(L, enq_slot, n_enq, fill_kernel, s, fn, "expert gate/up", ce, false);
    prof_add(L, 2, p2);
    const ProfPair p3 = prof_pair(L, 3);
    ce = moe::launch_ffn_down(S, w, adg, asc, x, add_in, res, y, s, p3.a, p3.b);
    if (ce != hipSuccess) return undo_fill(L, enq_slot, n_enq, fill_kernel, s, fn, "expert down", ce, false);
    prof_add(L, 3, p3);
  }
  if (trace) memcpy(trace, ev, sizeof(moe_cache_event) * k);
  if (stats) {
    stats->hits += k - n_miss;
    stats->misses += n_miss;
    stats->h2d_bytes += static_cast<int64_t>(n_miss) * static_cast<int64_t>(L->blob_e);
    stats->calls += 1;
  }
  if (timed) {
    // wait for this call's work and read its stage times
    HIP_OR_FAIL(hipEventRecord(L->st_end, s), fn);
    HIP_OR_FAIL(hipEventSynchronize(L->st_end), fn);
    float ms_fill = 0.f, ms_wait = 0.f;
    if (n_miss > 0) {
      HIP_OR_FAIL(hipEventSynchronize(L->st_c1), fn);
      ms_fill = elapsed_ms(L->st_c0, L->st_c1);
      if (used2) {
        HIP_OR_FAIL(hipEventSynchronize(L->st_d1), fn);
        const float m2 = elapsed_ms(L->st_d0, L->st_d1);
        ms_fill = m2 > ms_fill ? m2 : ms_fill;
      }
      if (!fill_kernel) ms_wait = elapsed_ms(L->st_w0, L->st_w1);
    }
    stats->ms_route = ms_route;
    stats->ms_fill = ms_read + ms_fill;
    stats->ms_wait_fill = ms_wait;
    stats->ms_total = elapsed_ms(L->st_t0, L->st_end);
  }
  return MOE_OK;
}

namespace {

// Prefill through the slot pool (cache mode). "Como executar um modelo de 26
// bilhões de parâmetros em dois gigabytes de memória em um Mac comum",
// section "Desempenho no mundo real": prompt processing in chunks of 128
// tokens, so that one loaded expert serves a group of rows at once (the chunk
// is settable; a longer chunk loads each expert for more rows). Per chunk:
// routing and the stable sort of its assignments; the chunk's experts (from
// the sorted offsets, read back to the host) in groups of up to
// min(n_slots, 16), each an LFU step whose misses are copied into their slots
// after the previous group's kernels, then the group's routed GEMMs on the
// slots; last the shared expert and the combine. Each output row is the same
// sum as in the resident prefill, so the result is the same bits.
moe_status prefill_pool(moe_layer* L, const uint16_t* x_bf16, const float* logits_in, int T, float* y,
                        int32_t* ids_out, float* w_out, hipStream_t s, const char* fn) {
  const moe_shape& sh = L->sh;
  const int E = sh.n_experts, k = sh.top_k, H = sh.hidden;
  const int chunk = L->max_T < L->prefill_chunk ? L->max_T : L->prefill_chunk;
  const moe::PrefillLayout P = moe::prefill_layout(chunk, E, k, H, sh.inter, sh.shared_inter);
  uint8_t* pw = L->wsb + L->ws.pre;
  hipStream_t cp = static_cast<hipStream_t>(L->d.copy_stream);
  const int gmax = L->d.n_slots < moe::kMaxGroup ? L->d.n_slots : moe::kMaxGroup;
  for (int c0 = 0; c0 < T; c0 += chunk) {
    const int Tc = T - c0 < chunk ? T - c0 : chunk;
    const uint16_t* xc = x_bf16 + static_cast<size_t>(c0) * H;
    HIP_OR_FAIL(moe::launch_prefill_route(P, pw, xc, logits_in ? logits_in + static_cast<size_t>(c0) * E : nullptr,
                                          L->d.router, L->d.bias, Tc, E, k, H,
                                          ids_out ? ids_out + static_cast<size_t>(c0) * k : nullptr,
                                          w_out ? w_out + static_cast<size_t>(c0) * k : nullptr, s), fn);
    HIP_OR_FAIL(hipMemcpyAsync(L->seg_host, pw + P.seg, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost, s), fn);
    HIP_OR_FAIL(hipStreamSynchronize(s), fn);
    int32_t experts[MOE_MAX_EXPERTS];
    int nx = 0;
    for (int e = 0; e < E; ++e)
      if (L->seg_host[e + 1] > L->seg_host[e]) experts[nx++] = e;
    for (int g0 = 0; g0 < nx; g0 += gmax) {
      const int n = nx - g0 < gmax ? nx - g0 : gmax;
      moe_cache_event ev[moe::kMaxGroup];
      int32_t n_miss = 0;
      moe::cache_assign(L->cache_backup, L->cache);
      moe_status cs = moe_cache_step(L->cache, experts + g0, n, ev, &n_miss);
      if (cs) return cs;
      int32_t enq_slot[moe::kMaxGroup];
      int n_enq = 0;
      bool injected = false;
      if (n_miss > 0) {
        // a miss may evict a slot that earlier kernels on s still read
        hipError_t ce = hipEventRecord(L->ev_pool, s);
        if (ce == hipSuccess) ce = hipStreamWaitEvent(cp, L->ev_pool, 0);
        const uint8_t* src[moe::kMaxGroup];
        if (ce == hipSuccess && L->d.store) {
          if (L->staging_busy) {
            ce = hipEventSynchronize(L->ev_fill);
            if (ce == hipSuccess && L->fill2_pending) ce = hipEventSynchronize(L->ev_fill2);
            L->staging_busy = false;
            L->fill2_pending = false;
          }
          int32_t mexp[moe::kMaxGroup];
          void* mdst[moe::kMaxGroup];
          int nm = 0;
          for (int j = 0; j < n; ++j)
            if (!ev[j].hit) {
              mexp[nm] = ev[j].expert;
              mdst[nm] = L->staging + static_cast<size_t>(nm) * L->stride;
              src[j] = static_cast<const uint8_t*>(mdst[nm]);
              ++nm;
            }
          if (ce == hipSuccess) {
            const moe_status rs = moe_store_read(L->d.store, L->d.store_layer, mexp, nm, mdst);
            if (rs) {
              moe::cache_assign(L->cache, L->cache_backup);
              return rs;
            }
          }
        } else {
          for (int j = 0; j < n; ++j)
            if (!ev[j].hit) src[j] = L->d.experts_host + static_cast<size_t>(ev[j].expert) * L->blob_e;
        }
        for (int j = 0; j < n && ce == hipSuccess; ++j)
          if (!ev[j].hit) {
            ce = enqueue_miss_copy(L, L->d.slot_pool + static_cast<size_t>(ev[j].slot) * L->blob_e, src[j], cp,
                                   &injected);
            if (ce == hipSuccess) enq_slot[n_enq++] = ev[j].slot;
          }
        if (ce == hipSuccess) ce = hipEventRecord(L->ev_fill, cp);
        if (ce == hipSuccess) ce = hipStreamWaitEvent(s, L->ev_fill, 0);
        if (ce != hipSuccess) return undo_fill(L, enq_slot, n_enq, false, s, fn, "miss copy", ce, injected);
        L->staging_busy = L->d.store != nullptr;
      }
      moe::SlotGroup grp{};
      grp.n = n;
      for (int j = 0; j < n; ++j) {
        grp.expert[j] = ev[j].expert;
        grp.slot[j] = ev[j].slot;
      }
      const hipError_t ge = moe::launch_prefill_routed(P, pw, xc, k, H, sh.inter, L->d.slot_pool, L->blob_e, &grp, s);
      if (ge != hipSuccess) return undo_fill(L, enq_slot, n_enq, false, s, fn, "routed GEMMs", ge, false);
    }
    HIP_OR_FAIL(moe::launch_prefill_shared(P, pw, xc, Tc, k, H, sh.shared_inter, L->d.shared_blob,
                                           y + static_cast<size_t>(c0) * H, s), fn);
  }
  return MOE_OK;
}

}  // namespace

moe_status moe_layer_prefill(moe_layer* L, const uint16_t* x_bf16, const float* logits_in, int32_t T,
                             float* y, int32_t* ids_out, float* w_out, void* stream) {
  moe::clear_error();
  const char* fn = "moe_layer_prefill";
  if (!L) return fail(MOE_EINVAL, "%s: NULL handle", fn);
  if (L->dcache) return fail(MOE_ESTATE, "%s: the handle's slot cache is stepped on the device (decode only)", fn);
  if (T < 0 || T > L->max_T) return fail(MOE_ESHAPE, "%s: T=%d outside [0, max_T=%d]", fn, T, L->max_T);
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !y) return fail(MOE_EINVAL, "%s: x_bf16 and y are required", fn);
  L->prof_now = L->prof && (L->prof_calls++ % L->prof_every) == 0;
  if (!moe::aligned16(x_bf16)) return fail(MOE_EALIGN, "%s: x_bf16 must be 16-byte aligned", fn);
  const moe_shape& sh = L->sh;
  // the GEMMs take any K and row count in whole groups (32-row tiles; groups
  // past K of a step weigh 0, a wave's second 32-row tile past H is not stored)
  if (sh.inter % moe::kGroup || sh.shared_inter % moe::kGroup || sh.hidden % moe::kGroup)
    return fail(MOE_ESHAPE, "%s: needs hidden, inter and shared_inter multiples of %d", fn, moe::kGroup);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe::PrefillLayout P = moe::prefill_layout(L->max_T, sh.n_experts, sh.top_k, sh.hidden, sh.inter,
                                                   sh.shared_inter);
  hipEvent_t pb = prof_begin(L, 4, s);
  if (L->cache_mode) {
    const moe_status ps = prefill_pool(L, x_bf16, logits_in, T, y, ids_out, w_out, s, fn);
    if (ps) return ps;
    prof_end(L, 4, pb, s);
    return MOE_OK;
  }
  HIP_OR_FAIL(moe::launch_prefill(P, L->wsb + L->ws.pre, x_bf16, logits_in, L->d.router, L->d.bias, T,
                                  sh.n_experts, sh.top_k, sh.hidden, sh.inter, sh.shared_inter,
                                  L->d.experts_dev, L->blob_e, L->d.shared_blob, y, ids_out, w_out, s),
              fn);
  prof_end(L, 4, pb, s);
  return MOE_OK;
}

moe_status moe_layer_prefill_chunk(moe_layer* L, int32_t tokens) {
  moe::clear_error();
  const char* fn = "moe_layer_prefill_chunk";
  if (!L) return fail(MOE_EINVAL, "%s: NULL handle", fn);
  if (tokens < 1 || tokens > L->max_T)
    return fail(MOE_ESHAPE, "%s: %d tokens outside [1, max_T=%d]", fn, tokens, L->max_T);
  L->prefill_chunk = tokens;
  return MOE_OK;
}

moe_status moe_debug_fail_copy(moe_layer* L, int32_t nth) {
  moe::clear_error();
  const char* fn = "moe_debug_fail_copy";
  if (!L) return fail(MOE_EINVAL, "%s: NULL handle", fn);
  if (!L->cache_mode || L->dcache) return fail(MOE_ESTATE, "%s: needs a host-stepped cache-mode handle", fn);
  if (nth < 0) return fail(MOE_EINVAL, "%s: nth = %d is negative", fn, nth);
  L->fail_copy_in = nth;
  return MOE_OK;
}

moe_status moe_layer_profile(moe_layer* L, int32_t enable) {
  moe::clear_error();
  if (!L) return fail(MOE_EINVAL, "moe_layer_profile: NULL handle");
  L->prof = enable != 0;
  L->prof_mask = (1u << kProfKinds) - 1;
  L->prof_every = 1;
  return MOE_OK;
}

moe_status moe_layer_profile_kinds(moe_layer* L, uint32_t mask, int32_t every, int32_t reserve_events) {
  moe::clear_error();
  const char* fn = "moe_layer_profile_kinds";
  if (!L) return fail(MOE_EINVAL, "%s: NULL handle", fn);
  if (every < 1) return fail(MOE_EINVAL, "%s: every = %d, must be >= 1", fn, every);
  if (mask >> kProfKinds) return fail(MOE_EINVAL, "%s: mask 0x%x has kinds beyond %d", fn, mask, kProfKinds - 1);
  if (reserve_events < 0 || reserve_events > (1 << 20))
    return fail(MOE_EINVAL, "%s: reserve_events %d outside [0, 2^20]", fn, reserve_events);
  while (static_cast<int32_t>(L->pool.size()) < reserve_events) {
    hipEvent_t e = nullptr;
    HIP_OR_FAIL(hipEventCreate(&e), fn);
    L->pool.push_back(e);
  }
  L->prof_mask = mask;
  L->prof_every = static_cast<uint32_t>(every);
  L->prof_calls = 0;
  L->prof = mask != 0;
  return MOE_OK;
}

moe_status moe_layer_profile_read(moe_layer* L, int32_t kind, moe_kernel_time* out) {
  moe::clear_error();
  const char* fn = "moe_layer_profile_read";
  if (!L || !out) return fail(MOE_EINVAL, "%s: NULL argument", fn);
  if (kind < 0 || kind >= kProfKinds) return fail(MOE_EINVAL, "%s: kind %d outside [0, %d]", fn, kind, kProfKinds - 1);
  for (auto& v : L->rec) {
    for (auto& p : v) HIP_OR_FAIL(hipEventSynchronize(p.second), fn);
  }
  for (int kd = 0; kd < kProfKinds; ++kd) {
    for (auto& p : L->rec[kd]) {
      float ms = 0.f;
      HIP_OR_FAIL(hipEventElapsedTime(&ms, p.first, p.second), fn);
      L->prof_ms[kd] += ms;
      L->prof_launches[kd] += 1;
      L->pool.push_back(p.first);
      L->pool.push_back(p.second);
    }
    L->rec[kd].clear();
  }
  out->launches = L->prof_launches[kind];
  out->ms_total = L->prof_ms[kind];
  return MOE_OK;
}

}  // extern "C"
