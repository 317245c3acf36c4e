// Internal launcher interface between the C-ABI host code and the kernels.
#pragma once
#include "common.h"

struct FfnArgs {
  int fmt, H, F, E, T, k;
  const uint8_t* pool;
  size_t stride;
  BlobLayout L;
  const uint16_t* x;
  const int32_t* topk_idx;
  const int32_t* pair_slot;
  const int32_t* pair_perm;
  const int32_t* expert_off;
  const int32_t* pair_subset;
  int n_pairs;  // pairs to compute (n_subset, or T*k)
  // Device-side split of pair_subset (GEMV path): with subset_rec (a miss
  // record) the grid covers all n_pairs entries and mode 1 computes the first
  // rec[2] of them (hits), mode 2 the rest, mode 3 all with the rest streamed
  // from miss_src; nothing runs unless rec[0] == MOE_OK.
  const int32_t* subset_rec;
  int subset_mode;
  // mode 3: host pool (pinned) the missed pairs stream their blob from; their
  // slot in `pool` is filled on the way
  const uint8_t* miss_src;
  const float* topk_w;
  float* y;        // [T*k][H] or NULL
  uint16_t* out;   // [T][H] or NULL
  uint16_t* hbuf;  // workspace [T*k][F] bf16
  float* ybuf;     // workspace [T*k][H] fp32 (grouped path with fused combine)
  int32_t* tiles;  // workspace: grouped-path tile list (grouped_tiles_bytes)
  int tiles_ready;  // the tile list was written with the permutation
  // fused decode down + combine: bytes to read (and discard) on otherwise idle
  // compute units, so that a later kernel finds them in the memory-side cache
  const uint8_t* warm;
  size_t warm_bytes;
  // MXFP4 on the grouped path: 1 = the scaled MFMA on the FP4 codes and their
  // E8M0 scales as stored, the bf16 activations entering as two FP8 terms with
  // E8M0 scales per 32 elements; 0 = bf16 MFMA on weights dequantized in registers
  int mx_native;
  uint8_t* xq;  // workspace (native): x as FP8 terms, [2][T][H] (hi plane, then lo plane)
  uint8_t* xs;  // workspace (native): their scales, [T][H/32][2] (hi, lo)
  uint8_t* hs;  // workspace (native): scales of h's FP8 terms, [T*k][F/32][2]; h's codes
                // ([2][T*k][F]) take the place of the bf16 h rows in hbuf
};
// Expert-FFN workspace: its size and the carving of FfnArgs' scratch pointers
// (hbuf, ybuf, tiles and, for MXFP4, the FP8 activation terms) from it.
size_t ffn_ws_bytes(int fmt, int T, int H, int F, int k, int E);
void ffn_ws_carve(FfnArgs& a, uint8_t* ws);
size_t grouped_tiles_bytes(int T, int k, int E);
// Tile list geometry of the grouped path for a format: rows per tile and the
// list capacity (for the permutation kernel to write it).
int grouped_tile_rows(int fmt, int mx_native);
int grouped_max_tiles(int fmt, int mx_native, int n_pairs, int E);

// GEMV path: gate/up + SwiGLU into hbuf, then down (+ combine when out != NULL).
hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t s);
// The same with separate subset modes for the gate/up and the down kernel.
hipError_t launch_ffn_gemv_split(const FfnArgs& a, int gateup_mode, int down_mode, hipStream_t s);
// Decode layer: gate/up with the softmax/top-k of `logits` computed inside each
// workgroup (writes topk_idx/topk_w), then down + combine.  T*k pairs, T <= 4.
hipError_t launch_decode_layer(const FfnArgs& a, const float* logits, unsigned route_flags,
                               int32_t* topk_idx, float* topk_w, hipStream_t s);
// Grouped MFMA path (expert-sorted pairs).
hipError_t launch_ffn_grouped(const FfnArgs& a, hipStream_t s);

struct RouteArgs {
  const uint16_t* x;
  const float* router;
  int T, H, E, k;
  unsigned flags;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* pair_perm;
  int32_t* expert_off;
  // optional grouped-path tile list built with the permutation (tile_rows > 0):
  // tiles = [tile_e (max_tiles) | tile_m0 (max_tiles) | n_tiles]
  int32_t* tiles;
  int tile_rows, max_tiles;
  // prepared bf16 split of the router ([3][E][H], moe_router_prepare) or NULL
  const uint16_t* planes_ready;
  // workspace carve-up
  float* logits;       // [T][E]
  int32_t* counts;     // [64][E] pairs per expert in copies (permutation)
  uint16_t* planes;    // [3][E][H] bf16 split of the router (T > 4)
};
size_t route_ws_bytes(int T, int H, int E, int k);
void route_ws_carve(RouteArgs& a, void* ws);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// Router logits ([T][E] fp32): GEMV kernel for T <= 4 (launch_router_logits),
// bf16x3 MFMA GEMM otherwise (launch_router_gemm, planes = [3][E][H] bf16 scratch).
// counts (optional): [64][E] copies of the pairs per expert, zeroed by the router
// kernel, then one atomic increment per selected pair by the top-k kernel.
hipError_t launch_router_logits(const uint16_t* x, const float* R, int T, int H, int E, float* logits,
                                hipStream_t s, int32_t* counts = nullptr);
// The planes are split from R into `planes` first unless planes_ready is given.
hipError_t launch_router_gemm(const uint16_t* x, const float* R, int T, int H, int E, float* logits,
                              uint16_t* planes, hipStream_t s, const uint16_t* planes_ready = nullptr,
                              int32_t* counts = nullptr);
hipError_t launch_router_split(const float* R, int E, int H, uint16_t* planes, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, unsigned flags, int32_t* idx,
                       float* w, hipStream_t s, int nsplit = 1, int32_t* counts = nullptr);

hipError_t launch_combine(const float* y, const float* w, int T, int H, int k, uint16_t* out,
                          hipStream_t s);
// The same, skipped on the device unless rec[0] == MOE_OK (rec: a miss record).
hipError_t launch_combine_rec(const float* y, const float* w, int T, int H, int k, uint16_t* out,
                              const int32_t* rec, hipStream_t s);

hipError_t launch_lru_reset(const moe_lru& l, hipStream_t s);
// The same step with the routed experts selected inside the kernel from the
// router logits (softmax + top-k; T <= 4, k <= 16), writing topk_idx / topk_w.
// logit_out (optional): the kernel also stores the [T][E_route] logits it read.
hipError_t launch_lru_lookup_topk(const moe_lru& l, const float* logits, int E_route, int T, int k, unsigned flags,
                                  int32_t* topk_idx, float* topk_w, int32_t* pair_slot, int32_t* pair_order,
                                  int32_t* miss_rec, int n_max, hipStream_t s, float* logit_out = nullptr);
// Copy the blobs named by a miss record (read on the device) from the host
// pool (pinned, device-addressable) into their victim slots.
hipError_t launch_cache_fill(const int32_t* miss_rec, const uint8_t* host_pool, uint8_t* slot_pool,
                             size_t expert_bytes, size_t stride, hipStream_t s, int n_groups = 512);
// Rebuild a layer's slot cache for to.S slots (state and blobs; plan: 1 + 2 * to.S
// int32 of workspace).  from_pool == to_pool rebuilds the pool in place.
hipError_t launch_lru_resize(const moe_lru& from, const uint8_t* from_pool, const moe_lru& to, uint8_t* to_pool,
                             size_t expert_bytes, size_t stride, int32_t* plan, hipStream_t s);
hipError_t launch_lru_lookup(const moe_lru& l, const int32_t* topk_idx, int n_pairs,
                             int32_t* pair_slot, int32_t* pair_order, int32_t* miss_rec, int n_max,
                             hipStream_t s);
