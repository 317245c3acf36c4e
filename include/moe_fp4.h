/* moe_fp4.h - C ABI of the routed block-scaled MoE layer forward for MI355X (gfx950).
 *
 * The calls follow the layer as the FreeToken pages state the problem:
 *   - the gate is a linear layer followed by a softmax giving a selection
 *     probability per expert; the top-K experts are evaluated and their
 *     outputs mixed by a weighted sum; every expert is an independent FFN
 *     (page "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
 *     "混合专家架构（MoE）的天然稀疏性");
 *   - low-precision weights are dequantized at compute time (page
 *     "8GB显存跑35B MoE模型：FreeToken引擎本地部署实战", §2.1) and the formats
 *     are NVFP4 / MXFP4 / FP8 (page "8GB 笔记本 39.3 tok/s、单卡跑 753B：FreeToken
 *     把 frontier MoE 拉回本地", section "局限");
 *   - routed experts are looked up in a global LRU expert cache in VRAM, and
 *     misses become a GPU cache fill (same page, section "设计核心"), copied
 *     asynchronously on a stream, overlapped with compute (page "753B...",
 *     section "按带宽动态分配参数存储").
 *
 * Conventions
 *   - Pointers are DEVICE pointers unless marked [host] (ordinary or pinned
 *     host memory) or [pinned] (host memory from hipHostMalloc, which the GPU
 *     can also address).  bf16 values are uint16_t bit patterns.
 *   - moe_stream_t / moe_event_t are hipStream_t / hipEvent_t handles (NULL =
 *     the null stream / no event).
 *   - The caller owns and allocates every buffer (weights, slot pool, host
 *     pool, LRU state, outputs, workspaces), every stream and every event.
 *     The library allocates no memory and keeps no mutable global state
 *     except the per-thread error text and the static scratch array that
 *     moe_layer_forward_static uses in place of a caller workspace; calls are
 *     reentrant (that one only when serialised per GPU).
 *   - Every GPU call is stream-ordered: it validates its arguments on the
 *     host, enqueues its kernels and returns.  Errors are negative status
 *     codes; nothing aborts or throws across the ABI.  Shape/argument errors
 *     are detected before any HIP call.  A failed launch returns MOE_E_HIP
 *     with detail in moe_last_error().  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *
 * Weight formats (one matrix W[N][K]; blocks run along K, the reduction
 * dimension of each output row):
 *   NVFP4: W = e2m1(code) * e4m3(scale[n][k/16]) * tau   (tau: fp32 per matrix)
 *   MXFP4: W = e2m1(code) * 2^(scale[n][k/32] - 127)     (OCP MX v1.0)
 *   FP8  : W = e4m3(code) * sigma[n][k/128]              (sigma: fp32)
 * E2M1: 4-bit S.EE.M, bias 1 (magnitudes 0,0.5,1,1.5,2,3,4,6).  E4M3: OCP
 * "FN" (bias 7, max 448, S.1111.111 = NaN).  FP4 codes pack two elements per
 * byte, element 2i in the low nibble.
 *
 * Supported shapes: H and F in {256, 512, 1024, 2048, 4096, 6144, 8192};
 * 1 <= k <= min(E, 16), E <= 1024; T >= 0.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */
typedef void* moe_event_t;  /* hipEvent_t  */

enum moe_status {
  MOE_OK = 0,
  MOE_E_ARG = -1,       /* invalid argument, shape or alignment            */
  MOE_E_FORMAT = -2,    /* unknown weight format                           */
  MOE_E_CAPACITY = -3,  /* more distinct misses than evictable slots       */
  MOE_E_WORKSPACE = -4, /* workspace missing or too small                  */
  MOE_E_HIP = -5        /* a HIP runtime call failed (see moe_last_error)  */
};

enum moe_fmt { MOE_FMT_NVFP4 = 1, MOE_FMT_MXFP4 = 2, MOE_FMT_FP8_E4M3 = 3 };

/* moe_route flags */
#define MOE_ROUTE_RENORM 1u /* w /= sum of the selected probabilities (off by default) */
/* `router` points to a prepared router (moe_router_prepare): the fp32 [E][H]
 * router followed by its bf16 split, so that calls with many tokens do not
 * split the router again.  Accepted wherever route flags are. */
#define MOE_ROUTE_PREPARED 0x200u

/* moe_expert_ffn flags */
#define MOE_FFN_AUTO 0u
#define MOE_FFN_GEMV 1u    /* per-pair weight-streaming GEMV (batch-1 decode shape)  */
#define MOE_FFN_GROUPED 2u /* expert-grouped MFMA GEMM (prefill shape); needs pair_perm/expert_off */
/* OR-ed into moe_expert_ffn's flags (MOE_LAYER_MX_NATIVE into moe_layer_forward's
 * route_flags): MXFP4 on the grouped path runs the gfx950 scaled MFMA, which
 * takes the FP4 codes and E8M0 scales as stored and the bf16 activations as
 * two FP8 E4M3 terms with E8M0 scales per 32 elements (hi and the remainder
 * lo; exact for every value within 2^14 of its block's largest), instead of
 * dequantizing the weights in registers into bf16 MFMA operands.  Outputs
 * agree within the tolerance; without the flag the dequant path runs (as fast
 * or faster as the kernels stand: the scaled path's operands leave room for
 * 64-row tiles only, so an expert's weights stream once per 64 rows). */
#define MOE_FFN_MX_NATIVE 4u
#define MOE_LAYER_MX_NATIVE 0x100u

/* ------------------------------------------------------------------ misc */

/* Static text for a status code. */
const char* moe_status_str(int status);
/* Detail of the last error on the calling thread ("" if none).  Static per-thread storage. */
const char* moe_last_error(void);
/* ABI version: (major << 16) | minor. */
int moe_abi_version(void);

/* --------------------------------------------------------- expert blobs */

/* Bytes of one packed expert blob (gate, up, down with their scales and tensor
 * scales) for the given format and shape; 0 if the format or shape is invalid.
 * A blob holds, each section starting on a 256-byte boundary:
 *   gate codes, up codes, down codes, gate scales, up scales, down scales,
 *   tau[3] (fp32; 1.0 for MXFP4/FP8).
 * Each matrix [N][K] is pre-shuffled into fragments of 16 rows x 128 k
 * (N/16 row groups x K/128 steps, group-major).  Lane l of a wavefront owns row
 * 16g + l%16, elements 128s + 32(l/16) .. +31 of fragment (g, s):
 *   FP4 codes 1 KiB per fragment, lane l's 16 bytes at 16l (low nibble = lower k);
 *   FP8 codes 2 KiB, two pieces of 64 x 16 bytes (elements 0-15, 16-31 of a lane);
 *   NVFP4 scales 2 bytes per lane (128 B), MXFP4 1 byte (64 B), FP8 one float
 *   per row of the fragment (64 B).
 * Code and scale sections have the canonical sizes; use moe_pack_expert /
 * moe_unpack_expert to convert.
 * The slot pool and the host pool hold blobs at a caller-chosen stride that is
 * >= moe_expert_bytes and a multiple of 256. */
size_t moe_expert_bytes(int fmt, int H, int F);

/* Canonical arrays of one expert, 9 pointers in this order:
 *   [0] gate codes  uint8 [F][H/2] (FP4) or [F][H] (FP8)
 *   [1] up codes    same shape
 *   [2] down codes  uint8 [H][F/2] or [H][F]
 *   [3] gate scales NVFP4 uint8 [F][H/16]; MXFP4 uint8 [F][H/32]; FP8 float [F][H/128]
 *   [4] up scales   same
 *   [5] down scales NVFP4 [H][F/16]; MXFP4 [H][F/32]; FP8 float [H][F/128]
 *   [6] gate tau, [7] up tau, [8] down tau: one float each (ignored unless NVFP4;
 *       may be NULL for MXFP4/FP8).
 * moe_pack_expert: canonical [host] -> blob [host] (moe_expert_bytes bytes).
 * moe_unpack_expert: blob [host] -> canonical [host]; the exact inverse.
 * Both are pure host functions; MOE_E_ARG on NULL pointers or a bad shape. */
int moe_pack_expert(int fmt, int H, int F, const void* const canon[9], void* blob);
int moe_unpack_expert(int fmt, int H, int F, const void* blob, void* const canon[9]);

/* ------------------------------------------------------------- routing */

/* Workspace bytes for moe_route (device memory, 256-byte aligned, no
 * initialisation needed). */
size_t moe_route_workspace(int T, int H, int E, int k);

/* Router, softmax and top-k for T tokens (page "753B...", section
 * "混合专家架构（MoE）的天然稀疏性").
 *   x        bf16  [T][H]   token activations
 *   router   float [E][H]   gate weights
 *   topk_idx int32 [T][k]   out: experts by (fp32 logit desc, index asc)
 *   topk_w   float [T][k]   out: softmax probability (over all E experts) of
 *                           each selected expert; renormalised over the k
 *                           selected when flags has MOE_ROUTE_RENORM
 *   pair_perm  int32 [T*k]  out, optional (NULL): pairs q = t*k+j sorted stably
 *                           by expert
 *   expert_off int32 [E+1]  out, optional (NULL together with pair_perm):
 *                           exclusive prefix sum of the pairs per expert
 * Logits are fp32 sums of bf16*fp32 products. */
int moe_route(const uint16_t* x, const float* router, int T, int H, int E, int k, unsigned flags,
              int32_t* topk_idx, float* topk_w, int32_t* pair_perm, int32_t* expert_off,
              void* ws, size_t ws_bytes, moe_stream_t stream);

/* Bytes of a prepared router (device memory, 256-byte aligned): the fp32
 * router [E][H] as given, then at byte align256(E*H*4) three bf16 planes
 * [3][E][H] with hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid)
 * (round to nearest even).  bf16 carries 8 of fp32's 24 significand bits, so
 * hi + mid + lo = w exactly for every zero and every |w| in [2^-100, 3.3e38];
 * smaller weights lose the bits below bf16's smallest subnormal (2^-133) and
 * larger ones round to infinity.  The planes are the operand of the many-token
 * router GEMM (the same split that calls without a prepared router make on
 * every call); the fp32 copy serves the few-token GEMV. */
size_t moe_router_prepared_bytes(int E, int H);

/* Write a prepared router from an fp32 router [E][H] (16-byte aligned) into
 * `prepared` (device, 256-byte aligned, moe_router_prepared_bytes); once per
 * weight set.  Pass it as `router` with MOE_ROUTE_PREPARED in the route flags.
 * The logits are the same as from the plain router, bit for bit. */
int moe_router_prepare(const float* router, int E, int H, void* prepared, moe_stream_t stream);

/* --------------------------------------------------------------- cache */

/* LRU state of a VRAM expert cache, caller-owned device memory (page "8GB 笔记本
 * 39.3 tok/s...", section "设计核心": a global LRU expert cache in VRAM).  The
 * state is keyed: a lookup's expert e is key key_base + e.  A per-layer cache
 * has E keys = the layer's experts and key_base 0.  Layers that share one state
 * and one slot pool (the cross-layer form of the global cache) each pass a
 * moe_lru with the same arrays and their own key_base, e.g. layer j of a group
 * at j * experts, with E = the keys of the whole group.
 *   slot_expert int32 [S]  key held by each slot, -1 = empty
 *   expert_slot int32 [E]  slot holding each key, -1 = not resident
 *   slot_stamp  int64 [S]  clock value of the slot's last access (0 = never)
 *   clock       int64 [1]  accesses so far
 *   key_base    key of this lookup's expert 0 (0 <= key_base < E; every routed
 *               expert e must have key_base + e < E) */
typedef struct moe_lru {
  int32_t E, S;
  int32_t* slot_expert;
  int32_t* expert_slot;
  int64_t* slot_stamp;
  int64_t* clock;
  int32_t key_base;
} moe_lru;

/* Set the state to a cold cache (all slots empty, clock 0).  Stream-ordered. */
int moe_lru_reset(const moe_lru* lru, moe_stream_t stream);

/* Elastic slot cache: resize one layer's cache to another slot count and
 * rebuild it, keeping the host pool as it is (page "8GB 笔记本 39.3 tok/s、单卡跑
 * 753B：FreeToken 把 frontier MoE 拉回本地", section "设计核心", the third
 * mechanism: at a scheduler safe point the GPU expert cache is resized to the
 * memory at hand and rebuilt, with no restart and no reload of the
 * host-resident expert pool).  The pages fix no rule for what survives; this
 * call keeps the min(to->S, resident) experts with the latest stamps (equal
 * stamps, which lookups never produce, keep the lower slot first); a kept
 * expert whose slot is below to->S keeps it, the others take the lowest free
 * slots below to->S in ascending order of their old slot.  Stamps and the
 * clock carry over; slots added by growing start empty.
 *   from, from_pool  the current state and its pool (from->S blobs at `stride`)
 *   to, to_pool      the state and pool after the call (to->S slots, to->E ==
 *                    from->E).  to's arrays may be from's own memory (every old
 *                    value is read before any is written).  to_pool is either
 *                    from_pool itself (rebuilt in place: only the blobs that
 *                    change slot are copied, from slots >= to->S into free
 *                    slots below it; the allocation must hold to->S blobs) or
 *                    memory that does not overlap from_pool (every kept blob is
 *                    copied).
 *   ws               moe_lru_resize_workspace(to->S) bytes (the copy plan)
 * Call it between steps: no lookup, fill or FFN of this layer may be in flight
 * on another stream.  Two kernels on `stream`; nothing is allocated.  Errors:
 * MOE_E_ARG (NULL state or pool, E or S outside [1, 1024], E changed,
 * expert_bytes or stride not a multiple of 256, stride < expert_bytes, pools
 * not 16-byte aligned or partly overlapping), MOE_E_WORKSPACE, MOE_E_HIP. */
size_t moe_lru_resize_workspace(int S_new);
int moe_lru_resize(const moe_lru* from, const void* from_pool, const moe_lru* to, void* to_pool,
                   size_t expert_bytes, size_t stride, void* ws, size_t ws_bytes, moe_stream_t stream);

/* int32 words of a miss record for T*k accesses to a pool of S slots:
 *   [0] status (MOE_OK or MOE_E_CAPACITY)   [1] n_miss (distinct missed experts)
 *   [2] n_hit_pairs (pairs whose expert was resident at the start of the step)
 *   [3] n_hits (accesses minus n_miss)      [4] n_max = min(T*k, S)
 *   [5 .. 5+n_max)          missed experts in order of first appearance
 *   [5+n_max .. 5+2*n_max)  the victim slot assigned to each */
size_t moe_miss_record_words(int T, int k, int S);

/* One LRU step for the T*k accesses topk_idx (pair order q = t*k+j).
 * Hits are classified against the state at the start of the step.  Each distinct
 * missed expert takes a victim slot among slots whose expert is not requested
 * in this step: empty slots by ascending index first, then occupied slots by
 * ascending stamp.  Every access, in pair order, advances the clock and stamps
 * its slot.  With too few candidates the record says MOE_E_CAPACITY and the
 * state is left unchanged.
 *   pair_slot  int32 [T*k]  out: slot of each pair after the step
 *   pair_order int32 [T*k]  out: pairs resident at step start first, then the
 *                           rest, each in ascending q (for moe_expert_ffn's
 *                           pair_subset hit/miss split)
 *   miss_rec   int32 [moe_miss_record_words]  out, device or [pinned] memory;
 *                           valid on the host only after the caller has
 *                           synchronised with an event recorded after this call.
 * Limits: E <= 1024, S <= 1024.  The return value reports only argument and
 * launch errors; capacity is reported in miss_rec[0]. */
int moe_cache_lookup(const moe_lru* lru, const int32_t* topk_idx, int T, int k,
                     int32_t* pair_slot, int32_t* pair_order, int32_t* miss_rec,
                     moe_stream_t stream);

/* Enqueue the GPU cache fill for a completed miss record (read on the host)
 * (page "753B...", section "按带宽动态分配参数存储": asynchronous host->device
 * copies on their own stream; page "8GB 笔记本 39.3 tok/s...", section
 * "设计核心": the GPU fills the VRAM expert cache):  copy_stream first waits on slots_free (if not NULL; record it after the last
 * kernel that reads the victim slots), then one hipMemcpyAsync host->device of
 * expert_bytes per miss, from host_pool + expert*stride to slot_pool +
 * slot*stride, then fill_done is recorded (if not NULL).
 *   miss_rec   [host] complete record from moe_cache_lookup
 *   host_pool  [pinned] E blobs at `stride`
 *   slot_pool  device, S blobs at `stride` */
int moe_cache_fill(const int32_t* miss_rec, const void* host_pool, void* slot_pool,
                   size_t expert_bytes, size_t stride, moe_event_t slots_free,
                   moe_stream_t copy_stream, moe_event_t fill_done);

/* The same GPU cache fill with the miss record read on the device instead of
 * the host, so nothing waits on the host: copy_stream waits on record_ready
 * (if not NULL; recorded after moe_cache_lookup) and on slots_free (if not
 * NULL), then one kernel copies every missed blob from host_pool (pinned,
 * addressed by the GPU over PCIe) into its victim slot, then fill_done is
 * recorded (if not NULL).  Copies nothing when miss_rec[0] != MOE_OK.
 *   miss_rec  device or [pinned] record written by moe_cache_lookup
 *   host_pool [pinned] E blobs at `stride`; slot_pool device, S blobs at `stride`
 * expert_bytes must be a multiple of 256 (moe_expert_bytes is). */
int moe_cache_fill_device(const int32_t* miss_rec, const void* host_pool, void* slot_pool,
                          size_t expert_bytes, size_t stride, moe_event_t record_ready,
                          moe_event_t slots_free, moe_stream_t copy_stream, moe_event_t fill_done);

/* ----------------------------------------------------------- expert FFN */

/* Workspace bytes for moe_expert_ffn. */
size_t moe_ffn_workspace(int fmt, int T, int H, int F, int k, int E);

/* Expert FFNs of the routed pairs (page "753B...", section "混合专家架构（MoE）的
 * 天然稀疏性": each expert an independent FFN; page "8GB显存跑35B MoE模型...",
 * §2.1: weights dequantized at compute time):
 * for pair q = t*k+j with e = topk_idx[q]
 * and slot s = pair_slot ? pair_slot[q] : e,
 *     h = bf16( silu(G_s x_t) * (U_s x_t) ),   y_q = D_s h        (fp32 out)
 * with the weights of blob s dequantized in registers (never materialised).
 *   slot_pool   device, blobs at `stride` bytes
 *   x           bf16 [T][H]
 *   topk_idx    int32 [T][k] (from moe_route)
 *   pair_slot   int32 [T*k] or NULL (identity: slot = expert)
 *   pair_perm, expert_off: from moe_route; required by the grouped path
 *   pair_subset int32 [n_subset] or NULL (all pairs): compute only these pairs
 *               (GEMV path; e.g. the hits while the misses are being filled)
 *   topk_w, out: if out != NULL, also out[t] = bf16(sum_j w[t][j] * y[t][j])
 *               (the combine fused; requires pair_subset == NULL)
 *   y           float [T*k][H] pair-major, or NULL when out != NULL
 *   flags       MOE_FFN_AUTO / MOE_FFN_GEMV / MOE_FFN_GROUPED
 * AUTO picks the grouped MFMA path when pair_perm/expert_off are given, no
 * subset is requested and T*k >= 2*E; otherwise the GEMV path. */
int moe_expert_ffn(int fmt, const void* slot_pool, size_t stride, int H, int F, int E,
                   const uint16_t* x, int T, int k, const int32_t* topk_idx,
                   const int32_t* pair_slot, const int32_t* pair_perm, const int32_t* expert_off,
                   const int32_t* pair_subset, int n_subset, const float* topk_w, float* y,
                   uint16_t* out, unsigned flags, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Gate-weighted combine (page "753B...", section "混合专家架构（MoE）的天然稀疏性"):
 *   out[t][n] = bf16( sum_{j=0..k-1} topk_w[t][j] * y[t*k+j][n] ), fp32 sum in j order. */
int moe_combine(const float* y, const float* topk_w, int T, int H, int k, uint16_t* out,
                moe_stream_t stream);

/* -------------------------------------------------------- whole layer */

/* Workspace bytes for moe_layer_forward (device memory, 256-byte aligned, no
 * initialisation needed; one stream at a time). */
size_t moe_layer_workspace(int fmt, int T, int H, int F, int k, int E);

/* The whole layer for experts resident in `pool` (blob e at e*stride):
 * moe_route (router, softmax over all E, top-k), moe_expert_ffn and the
 * gate-weighted combine, with the same results as calling them in turn.
 * For T <= 4 (decode) it runs three kernels: the router GEMV, gate/up +
 * SwiGLU with the softmax/top-k evaluated inside each workgroup, and down +
 * combine.  Larger T routes with the permutation and uses moe_expert_ffn's
 * automatic path.
 *   x bf16 [T][H], router float [E][H]; out bf16 [T][H];
 *   topk_idx int32 [T][k], topk_w float [T][k] (outputs). */
int moe_layer_forward(int fmt, const void* pool, size_t stride, int H, int F, int E, int k,
                      unsigned route_flags, const uint16_t* x, int T, const float* router,
                      int32_t* topk_idx, float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                      moe_stream_t stream);

/* moe_layer_forward with a read-ahead hint for a stack of layers: while the
 * decode down + combine kernel runs (T <= 4), extra workgroups (as many as
 * its row groups leave compute units idle, at least 64) read the device
 * buffer `warm` (warm_bytes, the
 * multiple of 16 below it; contents unchanged) and discard it, so that the
 * kernel that reads it next (typically the next layer's router, a static
 * weight) finds it in the memory-side cache.  Parameters are fetched ahead of
 * use as the pages' bandwidth-aware parameter placement has it (page
 * "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
 * "按带宽动态分配参数存储").  Results are those of moe_layer_forward bit for
 * bit.  warm and warm_bytes are both NULL/0 (no hint) or both set; warm is
 * 16-byte aligned device memory (MOE_E_ARG otherwise).  Larger T ignores the
 * hint. */
int moe_layer_forward_prefetch(int fmt, const void* pool, size_t stride, int H, int F, int E, int k,
                               unsigned route_flags, const uint16_t* x, int T, const float* router,
                               int32_t* topk_idx, float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                               const void* warm, size_t warm_bytes, moe_stream_t stream);

/* moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The workspace is instead a static device array of
 * MOE_STATIC_SCRATCH_BYTES in the library, one per GPU it runs on, held until
 * the process ends; the caller still passes the inputs and outputs.  The call
 * allocates nothing (no hipMalloc/hipFree, no allocating library routine); the
 * array's device address is looked up once per device, on the first call made
 * with that device current.
 *   Limits: a call whose moe_layer_workspace(fmt, T, H, F, k, E) exceeds
 *   MOE_STATIC_SCRATCH_BYTES returns MOE_E_WORKSPACE and enqueues nothing
 *   (batch-1 decode needs well under 1 MiB at every supported shape; a
 *   2048-token prefill of the 35B-class layer needs about 155 MiB and must use
 *   moe_layer_forward).
 *   Sharing: every call on one GPU uses the same array, which keeps whatever
 *   the last call left (nothing in it needs to start at zero).  Calls that
 *   overlap on one GPU (other streams, other threads) race on it: serialise
 *   them, e.g. on one stream.
 * Results equal moe_layer_forward's bit for bit. */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)
int moe_layer_forward_static(int fmt, const void* pool, size_t stride, int H, int F, int E, int k,
                             unsigned route_flags, const uint16_t* x, int T, const float* router,
                             int32_t* topk_idx, float* topk_w, uint16_t* out, moe_stream_t stream);

/* ------------------------------------------- cached layer (host executor) */

/* One layer's VRAM expert cache, caller-owned: the router, the pinned host
 * pool holding all E blobs, the device slot pool of S blobs, the LRU state over
 * it, a [pinned] miss record (moe_miss_record_words(T, k, S) words) and three
 * events (created by the caller; slots_free may start unrecorded). */
typedef struct moe_cached_layer {
  const float* router;     /* float [E][H] */
  const void* host_pool;   /* [pinned] E blobs at stride */
  void* slot_pool;         /* S blobs at stride */
  moe_lru lru;             /* LRU state over the S slots (lru.S = S) */
  int32_t* miss_rec;       /* [pinned] miss record */
  moe_event_t lookup_done; /* recorded after the lookup; the host waits on it */
  moe_event_t slots_free;  /* recorded after the last kernel that reads the slots */
  moe_event_t fill_done;   /* recorded on copy_stream after the fill */
} moe_cached_layer;

/* Workspace bytes for moe_cached_layer_forward (device, 256-byte aligned). */
size_t moe_cached_layer_workspace(int fmt, int T, int H, int F, int k, int E);

/* The layer with its experts served from the layer's VRAM slot cache, misses
 * filled from pinned host memory on a side stream and overlapped with the
 * hits (page "8GB 笔记本 39.3 tok/s、单卡跑 753B：FreeToken 把 frontier MoE 拉回
 * 本地", section "设计核心"; page "753B...", section "按带宽动态分配参数存储").
 * It calls the entry points above in this order:
 *   moe_route (no permutation) -> moe_cache_lookup -> record lookup_done and
 *   wait for it on the host -> moe_cache_fill on copy_stream (waits
 *   slots_free, records fill_done) -> moe_expert_ffn on the pairs that hit
 *   (GEMV path, pair_subset = the first n_hit_pairs of pair_order) -> `stream`
 *   waits fill_done -> moe_expert_ffn on the remaining pairs -> slots_free
 *   recorded on `stream` -> moe_combine.
 * Every pair uses the same kernels as the all-resident path, so `out` equals
 * moe_expert_ffn + moe_combine on a pool holding every expert, bit for bit.
 *   x bf16 [T][H]; topk_idx int32 [T][k], topk_w float [T][k], pair_slot and
 *   pair_order int32 [T*k] (outputs, device); out bf16 [T][H].
 *   n_hits, n_miss: [host] optional, receive miss_rec[3] and miss_rec[1].
 * Blocks the calling thread until this layer's lookup has run.  Returns
 * MOE_E_CAPACITY (state unchanged, nothing computed after the lookup) when a
 * step needs more victims than evictable slots. */
int moe_cached_layer_forward(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                             const moe_cached_layer* layer, const uint16_t* x, int T,
                             int32_t* topk_idx, float* topk_w, int32_t* pair_slot, int32_t* pair_order,
                             uint16_t* out, void* ws, size_t ws_bytes, moe_stream_t stream,
                             moe_stream_t copy_stream, int32_t* n_hits, int32_t* n_miss);

/* The cached layer without any host wait, on one stream:
 *   moe_route -> moe_cache_lookup -> gate/up and down (GEMV) for every pair, the
 *   pairs that hit (first miss_rec[2] entries of pair_order) reading their slot,
 *   the missed pairs streaming their expert's blob straight from the pinned host
 *   pool over PCIe and writing it into their victim slot on the way (the GPU
 *   cache fill overlapped with the missed pairs' own compute) -> moe_combine.
 * For T <= 4 the router GEMV is followed by the lookup kernel, which selects
 * the experts itself (softmax + top-k), and down runs fused with the combine:
 * the arithmetic of moe_layer_forward's decode path, so topk_idx, topk_w and
 * `out` equal moe_layer_forward on an all-resident pool bit for bit (larger T:
 * moe_route, and equal up to fp32 summation order).  The slots end up holding
 * the same blobs as with moe_cache_fill.
 * layer->miss_rec may be device memory; the events and copy streams of the
 * layer are not used.  If the lookup reports MOE_E_CAPACITY (miss_rec[0]),
 * nothing after the lookup writes anything and `out` keeps its contents: check
 * miss_rec[0] after synchronising.  Stream-ordered, so a whole decode step of
 * such layers can be captured in one graph. */
int moe_cached_layer_enqueue(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                             const moe_cached_layer* layer, const uint16_t* x, int T,
                             int32_t* topk_idx, float* topk_w, int32_t* pair_slot, int32_t* pair_order,
                             uint16_t* out, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_cached_layer_enqueue with predictive prefetch (T = 1): the gate's
 * output names the experts that come next, and they are copied in ahead of use
 * while the current step computes (page "FreeToken：753B大模型塞进单卡的本地部署
 * 硬件账该怎么算", section "按带宽动态分配参数存储": routing-aware asynchronous
 * copies on streams; prefetch accuracy is one of the validation dimensions the
 * same page lists).  The pages give no predictor; this one takes the token's
 * runner-up experts, ranks k .. k+m-1 of the same logits.  After the layer's
 * lookup on `stream`, the call records layer->lookup_done there, makes
 * pf_stream wait on it and enqueues on pf_stream:
 *   - one more LRU step of the layer's cache over the token's top-(k+m)
 *     experts in rank order: the routed k are hits (restamped in that order),
 *     a runner-up that misses takes a victim by the usual rule (never a slot
 *     this step requested) and is stamped after them;
 *   - a device copy of those runner-ups' blobs from the host pool into their
 *     victim slots (a few workgroups, so that it overlaps `stream`'s work).
 * The routed work on `stream` is moe_cached_layer_enqueue's, so topk_idx,
 * topk_w and `out` are those of moe_layer_forward bit for bit.  The caller
 * must make `stream` wait for pf_stream before this layer's next call (e.g.
 * once per decode step) and must not run another call on this layer's cache
 * meanwhile.
 *   m       runner-ups per token, 1 <= m, k + m <= 16
 *   pf_buf  device, moe_prefetch_buffer_bytes(E, k, m, S) bytes, 256-aligned,
 *           one per layer: a copy of the step's logits, then at byte
 *           moe_prefetch_record_offset(E) the prefetch step's miss record
 *           (moe_miss_record_words(1, k+m, S) words; its misses are the
 *           prefetched experts), then scratch.
 * Errors as moe_cached_layer_enqueue, plus MOE_E_ARG for T != 1, a bad m, a
 * missing lookup_done event or pf_stream == stream, and MOE_E_WORKSPACE. */
size_t moe_prefetch_buffer_bytes(int E, int k, int m, int S);
size_t moe_prefetch_record_offset(int E);
int moe_cached_layer_enqueue_prefetch(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                                      const moe_cached_layer* layer, const uint16_t* x, int T, int32_t* topk_idx,
                                      float* topk_w, int32_t* pair_slot, int32_t* pair_order, uint16_t* out,
                                      void* ws, size_t ws_bytes, int m, void* pf_buf, size_t pf_bytes,
                                      moe_stream_t stream, moe_stream_t pf_stream);

/* ------------------------------------------- host (CPU) experts: the q split */

/* Expert FFNs computed on the host CPU from blobs in host memory, for the
 * decode scheduler's split of a step's cache misses between GPU cache fills and
 * CPU compute (page "8GB 笔记本 39.3 tok/s、单卡跑 753B：FreeToken 把 frontier
 * MoE 拉回本地", section "设计核心", bandwidth-adaptive execution: the split
 * follows the measured PCIe and host-memory bandwidths).  For pair i:
 *   h = bf16( silu(G x_i) * (U x_i) ),   ys[i] = D h     (fp32 accumulation)
 * with the weights of blobs[i] (one packed blob, the layout moe_expert_bytes
 * describes) decoded on the host.  Pure host code with OpenMP (n_threads
 * threads); no HIP call.
 *   blobs [host] n pointers to blobs; xs [host] n pointers to bf16 [H] rows;
 *   ys [host] n pointers to float [H] outputs;
 *   scratch [host] n * (H + F) floats.
 * MOE_E_FORMAT, MOE_E_ARG (a NULL pointer, a bad shape or n < 0). */
int moe_host_expert_ffn(int fmt, int H, int F, int n, const void* const* blobs, const uint16_t* const* xs,
                        float* const* ys, float* scratch, int n_threads);

/* moe_cached_layer_forward with a share q of each step's distinct misses
 * computed on the host CPU instead of waiting for their fill (the decode
 * scheduler's split, page "8GB 笔记本 39.3 tok/s、单卡跑 753B：FreeToken 把
 * frontier MoE 拉回本地", section "设计核心": bandwidth-adaptive execution; the
 * pages give no formula for the share, so the caller picks q, e.g. from the
 * two measured bandwidths as B_host / (B_host + B_pcie)).
 * Order: `stream` waits defer_done (the previous call's deferred fills) ->
 * moe_route -> topk_idx and x copied to host_ws -> moe_cache_lookup -> record
 * lookup_done and wait for it on the host.  Of the record's nm distinct
 * misses, the last floor(q * nm) are CPU-served.  copy_stream: wait
 * slots_free, one hipMemcpyAsync per GPU-served miss, record fill_done, then
 * one per CPU-served miss (those experts still enter the cache), record
 * defer_done.  `stream`: the hit pairs (GEMV), wait fill_done, the GPU-served
 * missed pairs, record slots_free.  Meanwhile this thread computes the
 * CPU-served pairs with moe_host_expert_ffn (n_threads threads) from the
 * pinned host pool and copies their y rows to the device; then moe_combine.
 * The LRU state follows moe_cache_lookup exactly (q never changes it).  The
 * CPU-served pairs' y are the host kernel's (fp32 on the CPU), so `out` agrees
 * with the resident layer within the output tolerance, bit for bit when no
 * pair is CPU-served.
 *   layer: needs lookup_done and fill_done events and a [pinned] miss record;
 *   host_ws: [pinned] moe_cached_layer_split_host_bytes(T, H, F, k) bytes,
 *            256-aligned; a later call may reuse it (each call waits for its own
 *            lookup, which follows this call's work on `stream`);
 *   defer_done: an event owned by the layer (recorded by each call).
 *   n_hits, n_miss, n_cpu: [host] optional, the step's hits, distinct misses
 *   and CPU-served misses.
 * Errors as moe_cached_layer_forward, MOE_E_ARG for q outside [0, 1], more
 * than 64 pairs (T * k), a missing event or stream == copy_stream,
 * MOE_E_WORKSPACE. */
size_t moe_cached_layer_split_host_bytes(int T, int H, int F, int k);
int moe_cached_layer_forward_split(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                                   const moe_cached_layer* layer, const uint16_t* x, int T, int32_t* topk_idx,
                                   float* topk_w, int32_t* pair_slot, int32_t* pair_order, uint16_t* out,
                                   void* ws, size_t ws_bytes, moe_stream_t stream, moe_stream_t copy_stream,
                                   float q, void* host_ws, size_t host_ws_bytes, int n_threads,
                                   moe_event_t defer_done, int32_t* n_hits, int32_t* n_miss, int32_t* n_cpu);

/* ------------------------------------------- prefill with streamed experts */

/* Workspace bytes for moe_prefill_streamed (device, 256-byte aligned): one
 * moe_layer_forward workspace, shared by the layers in turn. */
size_t moe_prefill_streamed_workspace(int fmt, int T, int H, int F, int k, int E);

/* A prefill of T tokens through n_layers MoE layers whose experts live in
 * pinned host memory, double-buffered over PCIe (page "8GB 笔记本 39.3 tok/s、
 * 单卡跑 753B：FreeToken 把 frontier MoE 拉回本地", section "设计核心", the
 * first execution principle: while the GPU computes one layer's experts, the
 * next layer's experts stream in from host memory).  Two VRAM pools
 * alternate; for layer l (pool p = l % 2):
 *   copy_stream: wait events[2+p] (layer l-2, the pool's last reader, has
 *     finished) -> one hipMemcpyAsync of the layer's E blobs host_pools[l] ->
 *     pools[p] -> record events[p];
 *   stream: wait events[p] -> moe_layer_forward(pools[p], routers[l], x) into
 *     outs[l], topk_idx + l*T*k, topk_w + l*T*k -> record events[2+p].
 * The copies of layers 0 and 1 are enqueued first and the copy of layer l+2
 * right after the compute of layer l, so the copy of layer l+1 runs under the
 * compute of layer l.  Each layer receives the same x (the layers are not
 * chained).  Every layer runs moe_layer_forward's kernels, so its outputs
 * equal moe_layer_forward on a resident pool bit for bit.
 *   host_pools [host] array of n_layers [pinned] pointers, E*stride bytes each
 *   routers    [host] array of n_layers device pointers, float [E][H]
 *   outs       [host] array of n_layers device pointers, bf16 [T][H]
 *   topk_idx, topk_w: device, [n_layers][T][k]
 *   pools      [host] array of 2 device pointers, E*stride bytes each
 *   events     [host] array of 4 events: copy_done[2], compute_done[2]
 * Enqueues only (no host wait); stream != copy_stream. */
int moe_prefill_streamed(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                         int n_layers, const void* const* host_pools, const float* const* routers,
                         const uint16_t* x, int T, uint16_t* const* outs, int32_t* topk_idx,
                         float* topk_w, void* const* pools, void* ws, size_t ws_bytes,
                         moe_stream_t stream, moe_stream_t copy_stream, const moe_event_t* events);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP4_H */
