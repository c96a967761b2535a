/*
 * libmoedecode -- decode-time Mixture-of-Experts FFN layer with 4-bit
 * group-quantised experts and an LFU expert-slot cache, for AMD MI355X
 * (gfx950).
 *
 * The operations follow the engine described on "Como executar um modelo de
 * 26 bilhões de parâmetros em dois gigabytes de memória em um Mac comum",
 * section "Qual é o principal truque da arquitetura" (German twin: "So führen
 * Sie ein 26-Milliarden-Parameter-Modell ...", section "Was ist der
 * Haupt-Architekturtrick?"):
 *   - the router of each layer picks the 8 experts of the current token
 *     (moe_route);
 *   - a local expert cache of 16 slots with an LFU policy is checked
 *     (moe_cache_step);
 *   - missing experts are loaded into GPU-visible buffers while the GPU runs
 *     the shared-expert branch (moe_layer_decode, cache mode);
 *   - 4-bit expert GEMVs (moe_expert_gemv_q4) and the MoE combine
 *     (moe_layer_decode);
 * and, from the same page's section "Desempenho no mundo real", prefill that
 * lets one loaded expert serve a group of token rows (moe_layer_prefill).
 *
 * ---------------------------------------------------------------- formats
 * int4 g32 matrix for y = W x, W with N outputs and K inputs (K % 32 == 0):
 *   q : uint8 [N][K/2]   byte j of row n holds input 2j in bits 0-3 and 2j+1
 *                        in bits 4-7; each nibble is 4-bit two's complement
 *                        (-8..7)
 *   s : fp16  [N][K/32]  scale of inputs [32g, 32g+32) of row n
 *   W[n][k] = nibble(n,k) * s[n][k/32]
 * Expert blob (one contiguous run per expert, moe_expert_bytes bytes):
 *   gate.q [I][H/2] | up.q [I][H/2] | down.q [H][I/2] |
 *   gate.s [I][H/32] | up.s [I][H/32] | down.s [H][I/32]
 * Expert FFN (GeGLU): o = Wd (gelu_tanh(Wg u) * (Wu u)),
 *   gelu_tanh(z) = z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
 * Layer: z = Wr u (+ bias); ids = top-k of z (ties to the lower id, rank
 * order); w = softmax of z over ids; y = o_shared + sum_j w_j o_{ids_j}
 * (+ the layer input with MOE_F_RESIDUAL).
 *
 * ---------------------------------------------------------------- conventions
 *  - Every call returns a moe_status; nothing throws or aborts. On an error
 *    return nothing was enqueued and no state changed; the text is in
 *    moe_last_error() (thread-local, valid until the next call on the thread).
 *  - "dev" pointers are device (HBM) pointers, "host" pointers are host memory;
 *    "pinned" means host memory allocated pinned (hipHostMalloc or torch
 *    pin_memory). The library never takes ownership of caller memory.
 *  - Device buffers must be 16-byte aligned (MOE_EALIGN otherwise).
 *  - stream is a hipStream_t (NULL = the null stream). Calls documented as
 *    asynchronous only enqueue work.
 *  - Floating-point results are deterministic: the same inputs give the same
 *    bits (no floating-point atomics).
 */
#ifndef MOEDECODE_H
#define MOEDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_EINVAL -1 /* null pointer, id out of range, duplicate id, bad flag  */
#define MOE_ESHAPE -2 /* K % 32 != 0, k > E, k > n_slots, size above a limit    */
#define MOE_EALIGN -3 /* device pointer not 16-byte aligned                      */
#define MOE_EHIP -4   /* HIP runtime error; text in moe_last_error()             */
#define MOE_ENOMEM -5 /* workspace too small                                     */
#define MOE_ESTATE -6 /* call not valid for this handle's mode                  */

/* Limits checked by every entry point. */
#define MOE_MAX_TOPK 16
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_DIM 16384

const char* moe_last_error(void);
int32_t moe_abi_version(void);

typedef struct moe_shape {
  int32_t hidden;       /* H                                   */
  int32_t n_experts;    /* E                                   */
  int32_t top_k;        /* k                                   */
  int32_t inter;        /* I, routed expert intermediate width */
  int32_t shared_inter; /* I_s, shared expert intermediate     */
  int32_t group;        /* quantisation group; must be 32      */
} moe_shape;

typedef struct moe_q4 {
  const uint8_t* q;  /* dev [N][K/2] */
  const uint16_t* s; /* dev [N][K/32] fp16 bits */
} moe_q4;

/* Byte offsets of the six arrays inside one expert blob, and its size. */
typedef struct moe_blob_layout {
  size_t gate_q, up_q, down_q, gate_s, up_s, down_s, total;
} moe_blob_layout;

/* Blob size 27*H*I/16 (0 when H or I is not a positive multiple of 32). */
size_t moe_expert_bytes(int32_t hidden, int32_t inter);
moe_status moe_blob_layout_of(int32_t hidden, int32_t inter, moe_blob_layout* out);

/* ---------------------------------------------------------------- 1. routing
 * Router of one layer for B tokens: z[b][e] = sum_h x[b][h] * wr[e][h]
 * (+ bias[e]) accumulated in fp64 (every fp32 x fp16 product is exact in
 * fp64), or z = logits_in when logits_in != NULL (x and wr are then unused
 * and may be NULL). ids[b][0..k) are the k largest z in rank order, ties to
 * the lower expert id; w[b][j] = exp(z_j - z_0) / sum over the k selected.
 *   x         dev fp32 [B][H]           wr   dev fp16 [E][H]
 *   bias      dev fp32 [E] or NULL      logits_in dev fp32 [B][E] or NULL
 *   ids       dev int32 [B][k] (out)    w    dev fp32 [B][k] (out)
 *   workspace dev, at least moe_route_workspace_bytes(sh, B) bytes (holds the
 *             fp64 logits); may be NULL when logits_in != NULL.
 * Asynchronous on stream. */
size_t moe_route_workspace_bytes(const moe_shape* sh, int32_t B);
moe_status moe_route(const moe_shape* sh, const float* x, const uint16_t* wr, const float* bias,
                     const float* logits_in, int32_t B, int32_t* ids, float* w, void* workspace,
                     size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_route
 * without the workspace argument. The fp64 logits live in a device array of
 * the library's own (MOE_ROUTE_NOALLOC_MAX doubles = 1 MiB per GPU, held
 * until the process ends); the call allocates nothing. Same kernels, same
 * results as moe_route. MOE_ESHAPE when B * n_experts exceeds
 * MOE_ROUTE_NOALLOC_MAX (only without logits_in, which needs no scratch).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams or threads) race. Asynchronous on stream. */
#define MOE_ROUTE_NOALLOC_MAX 131072
moe_status moe_route_noalloc(const moe_shape* sh, const float* x, const uint16_t* wr, const float* bias,
                             const float* logits_in, int32_t B, int32_t* ids, float* w, void* stream);

/* ---------------------------------------------------------------- 2. LFU cache
 * Host-only, synchronous, deterministic. One cache per layer, n_slots slots.
 * moe_cache_step looks up one token's k ids (host, rank order, distinct):
 *   - a resident id is a hit: its frequency grows by one, its last-use tick
 *     becomes the current step;
 *   - a missing id takes the lowest-index empty slot, else the slot with the
 *     smallest (frequency, last use, slot index) among slots holding none of
 *     this token's ids; it starts at frequency 1;
 *   - ev[j] (host, k entries, out) describes ids[j]: expert, slot, hit (1/0),
 *     evicted expert or -1; *n_miss (out, may be NULL) counts misses.
 * The step counter advances by one per successful call. Errors (k > n_slots,
 * id out of range, duplicate id) leave the cache unchanged.
 * Replacement policy variant (not the pages' policy; for comparisons):
 * MOE_POLICY_LRU takes the slot with the smallest (last use, slot index)
 * instead; everything else is the same (frequencies are still counted). */
#define MOE_POLICY_LFU 0
#define MOE_POLICY_LRU 1
typedef struct moe_cache moe_cache;
typedef struct moe_cache_event {
  int32_t expert, slot, hit, evicted;
} moe_cache_event;
/* An LFU cache (the pages' policy). */
moe_status moe_cache_create(int32_t n_slots, int32_t n_experts, moe_cache** out);
/* A cache with the given policy (MOE_POLICY_*); MOE_EINVAL for others. */
moe_status moe_cache_create_policy(int32_t n_slots, int32_t n_experts, int32_t policy, moe_cache** out);
void moe_cache_destroy(moe_cache* c);
moe_status moe_cache_step(moe_cache* c, const int32_t* ids, int32_t k, moe_cache_event* ev,
                          int32_t* n_miss);
moe_status moe_cache_reset(moe_cache* c);
/* Copies the slot table (host arrays of n entries each, any may be NULL):
 * expert (-1 = empty), frequency, last-use step. n must equal n_slots. */
moe_status moe_cache_slots(const moe_cache* c, int32_t* expert, int32_t* freq, int64_t* last,
                           int32_t n);
moe_status moe_cache_counters(const moe_cache* c, int64_t* hits, int64_t* misses, int64_t* steps);

/* ---------------------------------------------------------------- 3. GEMV
 * y[m][n] = sum_k x[m][k] * W[n][k] for M token rows sharing one int4 g32
 * matrix W (N outputs, K inputs, K % 32 == 0). fp32 accumulation; each
 * activation group of 32 is carried as a 16-bit fixed-point value with its
 * own scale (relative error below 2e-5 of the group's largest magnitude).
 *   W dev (q, s as above)    x dev fp32 [M][K]    y dev fp32 [M][N] (out)
 *   1 <= M <= 64. x must be finite.
 * Asynchronous on stream. */
moe_status moe_expert_gemv_q4(const moe_q4* W, int32_t N, int32_t K, const float* x, int32_t M,
                              float* y, void* stream);

/* ---------------------------------------------------------------- 4./5. layer
 * A layer handle binds one layer's weights and a workspace.
 * Resident mode: experts_dev != NULL, every expert blob in HBM.
 * Cache mode:    experts_dev == NULL, experts_host (pinned [E][blob]) holds
 *                the experts, slot_pool (dev [n_slots][blob]) is the expert
 *                slot cache, copy_stream carries the host->HBM miss copies.
 * All pointers are borrowed and must stay valid and unmodified until
 * moe_layer_destroy. */
typedef struct moe_layer moe_layer;
/* ---------------------------------------------------------------- expert file store
 * Source: "Show HN: mecanismo de código aberto executando Gemma 4 26B em 2 GB
 * de RAM em qualquer Mac com série M", section "Abordagem técnica (MoE +
 * streaming por SSD)": experts are streamed from the SSD with parallel pread.
 * The file holds expert blobs in the order [layer][expert], each padded to
 * moe_store_stride(blob) bytes (a whole number of 16 KiB pages; the padding is
 * not read into the slot). */
typedef struct moe_store moe_store;
int64_t moe_store_stride(int64_t blob_bytes);
/* Opens path with `threads` reader threads (1..64). direct != 0 asks for
 * unbuffered reads (O_DIRECT); where the file system refuses them the store
 * reads through the page cache (moe_store_is_direct tells which). The file
 * must hold n_layers * n_experts strides: MOE_ESHAPE otherwise, MOE_EINVAL if
 * it cannot be opened. */
moe_status moe_store_open(const char* path, int32_t n_layers, int32_t n_experts, int64_t blob_bytes,
                          int32_t threads, int32_t direct, moe_store** out);
int32_t moe_store_is_direct(const moe_store* s);
/* Joins the readers and closes the file (NULL: no-op). */
void moe_store_close(moe_store* s);
/* Reads the padded blobs of experts[0..n) of one layer into dst[i] (host
 * memory of at least one stride each; 4096-byte aligned for unbuffered
 * reads, MOE_EALIGN otherwise). Each blob is split into one page-aligned part
 * per reader; returns when every part is in. Calls on one store are
 * serialised. Errors: MOE_EINVAL (bad layer, expert or pointer, read error),
 * MOE_ESHAPE (file shorter than a blob). */
moe_status moe_store_read(moe_store* s, int32_t layer, const int32_t* experts, int32_t n, void* const* dst);

typedef struct moe_layer_desc {
  const uint16_t* router;       /* dev fp16 [E][H]                               */
  const float* bias;            /* dev fp32 [E] added to the logits, or NULL     */
  const uint8_t* shared_blob;   /* dev, moe_expert_bytes(H, I_s) bytes           */
  const uint8_t* experts_dev;   /* resident mode: dev [E][blob]; else NULL       */
  const uint8_t* experts_host;  /* cache mode: pinned host [E][blob]; else NULL  */
  uint8_t* slot_pool;           /* cache mode: dev [n_slots][blob]; else NULL    */
  int32_t n_slots;              /* cache mode: k <= n_slots <= E                 */
  void* copy_stream;            /* cache mode: hipStream_t for the miss copies
                                   (decode alternates the misses between it and a
                                   second copy stream the handle creates)        */
  void* workspace;              /* dev, moe_layer_workspace_bytes bytes          */
  size_t workspace_bytes;
  /* cache mode, instead of experts_host: the misses are read from this store
   * (layer store_layer) into pinned staging owned by the handle, then copied
   * to their slots like host-memory misses. Not owned by the handle. */
  moe_store* store;
  int32_t store_layer;
  int32_t cache_policy;         /* cache mode: MOE_POLICY_LFU (0) or MOE_POLICY_LRU */
  /* cache mode with experts_host in device-accessible pinned memory: 1 = the
   * cache lives in device memory (in the workspace) and a kernel after the
   * router steps it, so a decode call waits for nothing on the host and can be
   * captured in a graph; the misses are then always copied by fill blocks
   * (as with MOE_F_FILL_KERNEL). Same rule, same trace, same bits as the host
   * cache. 0 = the host steps the cache. */
  int32_t cache_on_device;
} moe_layer_desc;

/* Counters of decode calls (accumulated over the calls given the struct) and
 * the stage times of the last call made with MOE_F_STAGE_TIMES (left
 * unchanged by other calls), in milliseconds:
 *   ms_route      host clock, from the call's entry until the token's ids were
 *                 on the host (routing kernel, top-k and its publication)
 *   ms_fill       the misses' fill: with copy-engine fills the GPU time of the
 *                 longer of the two copy streams' runs of copies (first copy
 *                 start to last copy end), plus the host time of the expert
 *                 file reads when a store is the source; with fill blocks the
 *                 GPU time of the launch that holds them; 0 without misses.
 *                 Divided by the miss count it is the time per missed expert
 *                 ("Show HN: mecanismo de código aberto executando Gemma 4 26B
 *                 em 2 GB de RAM", section "Abordagem técnica": about 3 ms per
 *                 3.36 MB expert read from an SSD)
 *   ms_wait_fill  GPU time the call's stream waited for the copies after it
 *                 had run everything before them (copy-engine fills; 0 with
 *                 fill blocks, which the stream runs in order)
 *   ms_total      GPU time from the start of the call's first kernel to the
 *                 end of its last */
typedef struct moe_decode_stats {
  int64_t hits, misses, h2d_bytes; /* cache mode; accumulated over calls       */
  int64_t calls;
  float ms_route, ms_fill, ms_wait_fill, ms_total;
} moe_decode_stats;

#define MOE_F_RMSNORM_IN 1u /* u = x' / sqrt(mean(x'^2) + 1e-6) feeds router and FFN */
#define MOE_F_RESIDUAL 2u   /* y = x' + MoE(u) instead of y = MoE(u)                 */
/* Cache mode: the misses are copied from experts_host to their slots by fill
 * blocks that run in the same launch as the shared-expert gate/up, on the
 * call's stream, after the LFU step (no copy engine, no copy_stream, no
 * cross-stream event). experts_host must then be device-accessible pinned
 * memory (hipHostMalloc); copy_stream is unused. Same cache trace, same bits. */
#define MOE_F_FILL_KERNEL 4u
/* Host-stepped cache mode with stats != NULL: record events around the call's
 * stages, wait for the call's work before returning and write its stage times
 * into stats (a measurement mode: the events and the wait cost time). */
#define MOE_F_STAGE_TIMES 16u

/* Workspace for up to max_B decode tokens per call and max_T prefill tokens. */
moe_status moe_layer_workspace_bytes(const moe_shape* sh, int32_t max_B, int32_t max_T,
                                     size_t* out);
/* Validates, clears the workspace counters (synchronously) and returns a handle.
 * The one-token kernels take hidden up to 8192 (MOE_ESHAPE above).
 * max_B > 1 (batched decode, resident mode) also needs the batched kernels'
 * per-block LDS (the staged group scales of 128 weight rows of length K, i.e.
 * 8 K bytes for K = H and for K = max(inter, shared_inter), plus the
 * activation slices of up to 64 tokens, 8.5 / 17 / 34 KiB for max_B up to
 * 16 / 32 / above) to fit the device's LDS per block (160 KiB on gfx950:
 * every hidden up to 8192 at any max_B): MOE_ESHAPE if not. */
moe_status moe_layer_create(const moe_shape* sh, const moe_layer_desc* d, int32_t max_B,
                            int32_t max_T, moe_layer** out);
void moe_layer_destroy(moe_layer* L);
/* Resident mode only: point the handle at another resident expert array of the
 * same shape (e.g. a replica). Takes effect for calls enqueued afterwards. */
moe_status moe_layer_set_experts(moe_layer* L, const uint8_t* experts_dev);
/* The handle's LFU cache (cache mode, host-stepped), or NULL. Owned by the handle. */
moe_cache* moe_layer_cache(moe_layer* L);
/* State of the handle's expert-slot cache, host- or device-stepped: per slot
 * the expert (-1 empty), frequency and last use (n = n_slots), and the
 * counters. A device-stepped cache is read after synchronising stream (the
 * stream the decode calls run on). Any output may be NULL. MOE_ESTATE for a
 * resident handle. */
moe_status moe_layer_cache_state(moe_layer* L, int32_t* expert, int32_t* freq, int64_t* last, int32_t n,
                                 int64_t* hits, int64_t* misses, int64_t* steps, void* stream);

/* Decode B tokens through the layer.
 *   x       dev fp32 [B][H] layer input
 *   add_in  dev fp16 [B][H] added first, x' = x + add_in, or NULL (x' = x)
 *   flags   MOE_F_RMSNORM_IN | MOE_F_RESIDUAL (u = x' without RMSNORM_IN),
 *           MOE_F_FILL_KERNEL, MOE_F_STAGE_TIMES (cache mode only)
 *   y       dev fp32 [B][H] output; must not alias x
 *   ids_out dev int32 [B][k], w_out dev fp32 [B][k], u_out dev fp32 [B][H]:
 *           optional copies of the routing and of u (NULL to skip)
 *   trace   host [B][k] cache events (cache mode) or NULL; with a
 *           device-stepped cache the call then synchronises stream to read them
 *   stats   host, accumulated (cache mode counters) or NULL; a
 *           device-stepped cache counts on the device instead (only calls is
 *           accumulated here; moe_layer_cache_state reads the counters)
 * Resident mode is asynchronous on stream. With B > 1 (resident) the tokens
 * are grouped by expert: each touched expert's weights are read once per call
 * and multiplied on the matrix cores (fp16 weights and activations, fp32
 * accumulation); each token's result is its own B = 1 layer output within the
 * same tolerance, and its ids are the same. Cache mode requires B == 1 and
 * blocks the calling thread once, until the token's ids are on the host; it
 * returns with the miss copies and the expert kernels enqueued (the copies on
 * copy_stream and the handle's second copy stream, every other miss on each,
 * ordered before the expert kernels by events; with
 * MOE_F_FILL_KERNEL the copies are fill blocks of the shared-expert launch on
 * stream). */
moe_status moe_layer_decode(moe_layer* L, const float* x, const uint16_t* add_in, int32_t B,
                            uint32_t flags, float* y, int32_t* ids_out, float* w_out, float* u_out,
                            moe_cache_event* trace, moe_decode_stats* stats, void* stream);

/* Prefill T tokens (T <= max_T). x is bf16 [T][H]; routing uses
 * logits_in (dev fp32 [T][E]) when given, else x . router. Tokens are grouped
 * by expert; expert weights are dequantised to bf16 (one rounding of the
 * exact product) and multiplied on the matrix cores with fp32 accumulation; the GeGLU activation is rounded
 * to bf16 before the down projection. y dev fp32 [T][H]. ids_out / w_out
 * optional as in decode. Any shape the handle holds (hidden, inter and
 * shared_inter multiples of 32).
 * Resident mode: asynchronous on stream.
 * Cache mode (source: "Como executar um modelo de 26 bilhões de parâmetros em
 * dois gigabytes de memória em um Mac comum", section "Desempenho no mundo
 * real"): the tokens go through the slot pool in chunks of 128 tokens (see
 * moe_layer_prefill_chunk; at most max_T): per
 * chunk, its experts in groups of min(n_slots, 16), each an LFU step of the
 * handle's cache whose misses are copied (from experts_host or the store) on
 * copy_stream after the previous group's kernels, then the group's routed
 * products on the slots. The calling thread waits once per chunk (for the
 * chunk's expert list) and for store reads. Same bits as resident mode. */
moe_status moe_layer_prefill(moe_layer* L, const uint16_t* x_bf16, const float* logits_in,
                             int32_t T, float* y, int32_t* ids_out, float* w_out, void* stream);
/* Test support for the failure path of the miss fill (host-stepped cache
 * mode): the nth host->slot miss copy enqueued from now on, counted over this
 * handle's following decode and prefill calls, fails before it is issued, as
 * if the runtime had refused it (0 disarms; it fires once). The call then
 * returns MOE_EHIP after waiting for the copies it had already enqueued; its
 * cache step is undone, except that each slot one of those copies wrote is
 * left empty (expert -1, frequency 0, last use -1), since its bytes are no
 * longer those of the expert it held. Later calls refill such slots like any
 * other miss. */
moe_status moe_debug_fail_copy(moe_layer* L, int32_t nth);

/* Cache-mode prefill: tokens per chunk through the slot pool, 1..max_T
 * (default 128, the pages' value; a longer chunk loads each expert once for
 * more rows). MOE_ESHAPE outside that range. */
moe_status moe_layer_prefill_chunk(moe_layer* L, int32_t tokens);

/* Per-kernel GPU time of the handle's calls, measured with HIP events on the
 * launch stream while profiling is enabled: the one-kernel stages 1-3 of the
 * one-token paths take events stamped by the kernel's own dispatch (start and
 * end of the kernel); the other stages take events recorded around them.
 * The stamps bracket the dispatch, so a stage is charged a little more than
 * the kernel-execution time a kernel trace reports (about 1 us at B=1).
 * kind: 0 = routing (input prep, logits, top-k), 1 = shared-expert gate/up
 * launched ahead of the miss copies (cache mode), 2 = gate/up of the routed
 * experts (resident mode: together with the shared expert), 3 = down
 * projections + combine, 4 = prefill. Launch counts and times accumulate
 * over calls; reading synchronises with the recorded events. */
typedef struct moe_kernel_time {
  int64_t launches;
  double ms_total;
} moe_kernel_time;
moe_status moe_layer_profile(moe_layer* L, int32_t enable);
/* Profile only the kinds in mask (bit i = kind i; 0 turns profiling off), on
 * one call in `every` (>= 1), and pre-create reserve_events events (0..2^20),
 * so that a timed region pays neither for event creation (two events per
 * profiled stage and call) nor for timing every call. */
moe_status moe_layer_profile_kinds(moe_layer* L, uint32_t mask, int32_t every, int32_t reserve_events);
moe_status moe_layer_profile_read(moe_layer* L, int32_t kind, moe_kernel_time* out);

/* ---------------------------------------------------------------- attention step
 * The attention step of one decoder layer, next to the MoE FFN, for one
 * token ("Como executar um modelo de 26 bilhões de parâmetros em dois
 * gigabytes de memória em um Mac comum": section "Sem dependências do
 * llama.cpp e MLX" lists attention, RMSNorm and RoPE kernels; section "Qual
 * é o principal truque da arquitetura" keeps the KV cache for the context
 * resident in FP16). With a = the attention output:
 *   h = x / sqrt(mean(x^2) + eps) * norm_w
 *   [q | k | v] = Wqkv h                (int4 g32, q rows, then k rows, then v rows)
 *   q, k rotated by RoPE at pos: pairs (i, i + d/2), angle pos * theta^(-2i/d),
 *       (a, b) -> (a cos - b sin, b cos + a sin)
 *   K[g][pos] = fp16(k_g), V[g][pos] = fp16(v_g)   (round to nearest even)
 *   a_h = softmax over t in [0, pos] of q_h . K[g][t] / sqrt(d), applied to V[g],
 *       g = h / (n_heads / n_kv_heads)
 *   y = x + Wo a
 * The pages give no head counts; the Gemma-shaped configuration used with this
 * library is 16 query heads, 8 key/value heads, d = 256. */
typedef struct moe_attn_shape {
  int32_t hidden;      /* H: multiple of 32 in [32, 4096] */
  int32_t n_heads;     /* query heads; n_heads / n_kv_heads in {1, 2, 4}; n_heads * head_dim <= 8192 */
  int32_t n_kv_heads;  /* key/value heads */
  int32_t head_dim;    /* d: 64, 128 or 256 */
  int32_t max_ctx;     /* positions the caches hold: 1 .. (positions per split)^2 (16384 at d = 256) */
  float rope_theta;    /* > 0 */
  float eps;           /* RMSNorm epsilon, >= 0 */
} moe_attn_shape;

typedef struct moe_attn_weights {
  const float* norm_w;    /* dev fp32 [H] */
  const uint8_t* qkv_q;   /* dev int4 g32 [(n_heads + 2 n_kv_heads) d][H/2], 16-byte aligned */
  const uint16_t* qkv_s;  /* dev fp16 [(n_heads + 2 n_kv_heads) d][H/32] */
  const uint8_t* o_q;     /* dev int4 g32 [H][n_heads d / 2], 16-byte aligned */
  const uint16_t* o_s;    /* dev fp16 [H][n_heads d / 32] */
} moe_attn_weights;

/* Workspace of moe_attn_decode for this shape (queries, per-split partial
 * results, the attention output). MOE_ESHAPE for unsupported shapes. */
moe_status moe_attn_workspace_bytes(const moe_attn_shape* sh, size_t* out);
/* One token at position pos (0 <= pos < max_ctx) through the attention step,
 * asynchronous on stream. k_cache / v_cache: dev fp16 [n_kv_heads][max_ctx][d],
 * 16-byte aligned, owned by the caller; positions < pos hold the earlier
 * tokens, the call writes position pos and reads [0, pos]. x, y: dev fp32 [H]
 * (y may be x). workspace: dev, 16-byte aligned, at least
 * moe_attn_workspace_bytes (scratch, no contents kept between calls); calls
 * that share a workspace must be ordered on one stream. Checks every argument
 * before enqueueing anything. */
moe_status moe_attn_decode(const moe_attn_shape* sh, const moe_attn_weights* W, uint16_t* k_cache,
                           uint16_t* v_cache, int32_t pos, const float* x, float* y, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- test support
 * Unpacks the nibbles of W to int8 [N][K] (dev) for bit-exact comparison. */
moe_status moe_debug_unpack_q4(const moe_q4* W, int32_t N, int32_t K, int8_t* out, void* stream);

/* Measurement support: the floor of one launch that streams `bytes` from HBM
 * with no arithmetic, to set a GEMV launch of the same bytes against. Each of
 * reps launches (blocks x 1024 threads) reads `bytes` (a multiple of 16, at
 * most 16 x 16 B per lane) at src + (i % regions) * region_stride (dev,
 * 16-byte aligned; region_stride >= bytes when regions > 1, so that rotating
 * over a range larger than the last-level cache defeats it); every lane issues
 * all its 16-byte loads before using any, and each wave writes the XOR of its
 * words to out (dev uint32 [blocks * 16]). With mean_us non-NULL every launch
 * takes events stamped by its own dispatch, the call synchronises the stream
 * and *mean_us receives the mean duration; with NULL the launches are only
 * enqueued. MOE_ESHAPE for sizes out of range. */
moe_status moe_debug_read_floor(const void* src, int64_t bytes, int64_t region_stride, int32_t regions,
                                int32_t blocks, int32_t reps, uint32_t* out, double* mean_us, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEDECODE_H */
