// C-ABI entry points: argument validation, workspace carving and dispatch.
// Every check runs on the host before any HIP call; nothing throws across the
// ABI.  Semantics of each call are documented in include/moe_fp4.h.
#include <stdio.h>
#include <string.h>

#include <cstdarg>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MOE_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool valid_fmt(int fmt) {
  return fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_FP8_E4M3;
}

bool valid_dim(int v) {
  switch (v) {
    case 256: case 512: case 1024: case 2048: case 4096: case 6144: case 8192: return true;
    default: return false;
  }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int fmt, int H, int F) {
  if (!valid_fmt(fmt)) return fail(MOE_E_FORMAT, "unknown format %d", fmt);
  if (!valid_dim(H) || !valid_dim(F))
    return fail(MOE_E_ARG, "H=%d F=%d: each must be one of 256,512,1024,2048,4096,6144,8192", H, F);
  return MOE_OK;
}

int check_route_dims(int T, int H, int E, int k) {
  if (T < 0) return fail(MOE_E_ARG, "T=%d < 0", T);
  if (!valid_dim(H)) return fail(MOE_E_ARG, "H=%d unsupported", H);
  if (E < 1 || E > 1024) return fail(MOE_E_ARG, "E=%d outside [1, 1024]", E);
  if (k < 1 || k > E || k > 16) return fail(MOE_E_ARG, "k=%d outside [1, min(E, 16)]", k);
  return MOE_OK;
}

}  // namespace

size_t ffn_ws_bytes(int fmt, int T, int H, int F, int k, int E) {
  const size_t n = (size_t)T * k;
  size_t b = align256(n * F * 2) + align256(n * H * 4) + grouped_tiles_bytes(T, k, E) + 256;
  if (fmt == MOE_FMT_MXFP4)  // FP8 terms of x and the scales of x's and h's terms
    b += align256((size_t)T * H * 2) + align256((size_t)T * H / 16) + align256(n * F / 16);
  return b;
}

void ffn_ws_carve(FfnArgs& a, uint8_t* p) {
  const size_t n = (size_t)a.T * a.k;
  a.hbuf = reinterpret_cast<uint16_t*>(p);
  p += align256(n * a.F * 2);
  a.ybuf = reinterpret_cast<float*>(p);
  p += align256(n * a.H * 4);
  a.tiles = reinterpret_cast<int32_t*>(p);
  p += grouped_tiles_bytes(a.T, a.k, a.E) + 256;
  if (a.fmt == MOE_FMT_MXFP4) {
    a.xq = p;
    p += align256((size_t)a.T * a.H * 2);
    a.xs = p;
    p += align256((size_t)a.T * a.H / 16);
    a.hs = p;
  } else {
    a.xq = a.xs = a.hs = nullptr;
    a.mx_native = 0;
  }
}

extern "C" {

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_ARG: return "invalid argument";
    case MOE_E_FORMAT: return "unknown weight format";
    case MOE_E_CAPACITY: return "cache capacity exceeded";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_abi_version(void) { return (1 << 16) | 2; }

// ------------------------------------------------------------------ blobs

size_t moe_expert_bytes(int fmt, int H, int F) {
  if (!valid_fmt(fmt) || !valid_dim(H) || !valid_dim(F)) return 0;
  return blob_layout(fmt, H, F).total;
}

// Canonical row-major matrix <-> fragment order (the blob geometry in common.h).
// Every move is a whole 16-byte code chunk or a lane's scale bytes, so the two
// directions are exact inverses.
static void shuffle_matrix(int fmt, int N, int K, uint8_t* canon_codes, uint8_t* canon_scales,
                           uint8_t* codes, uint8_t* scales, bool to_blob) {
  const int S = K / kFragK;
  auto mv = [to_blob](uint8_t* blob_p, uint8_t* canon_p, size_t n) {
    if (to_blob) memcpy(blob_p, canon_p, n);
    else memcpy(canon_p, blob_p, n);
  };
  for (int n = 0; n < N; ++n) {
    const int g = n / kFragRows, r = n % kFragRows;
    for (int s = 0; s < S; ++s) {
      const size_t f = (size_t)g * S + s;
      for (int q = 0; q < 4; ++q) {
        const int l = q * 16 + r, k0 = s * kFragK + 32 * q;  // lane and its first element
        if (fmt == MOE_FMT_FP8_E4M3) {
          for (int p = 0; p < 2; ++p)
            mv(codes + f * 2048 + p * 1024 + l * 16, canon_codes + (size_t)n * K + k0 + 16 * p, 16);
        } else {
          mv(codes + f * 1024 + l * 16, canon_codes + (size_t)n * (K / 2) + k0 / 2, 16);
        }
        if (fmt == MOE_FMT_NVFP4) mv(scales + f * 128 + l * 2, canon_scales + (size_t)n * (K / 16) + k0 / 16, 2);
        if (fmt == MOE_FMT_MXFP4) mv(scales + f * 64 + l, canon_scales + (size_t)n * (K / 32) + k0 / 32, 1);
      }
      if (fmt == MOE_FMT_FP8_E4M3) mv(scales + f * 64 + r * 4, canon_scales + ((size_t)n * S + s) * 4, 4);
    }
  }
}

static void copy_sections(int fmt, int H, int F, const BlobLayout& L, uint8_t* blob,
                          void* const canon[9], bool to_blob) {
  auto c = [&](int i) { return static_cast<uint8_t*>(canon[i]); };
  shuffle_matrix(fmt, F, H, c(0), c(3), blob + L.cg, blob + L.sg, to_blob);
  shuffle_matrix(fmt, F, H, c(1), c(4), blob + L.cu, blob + L.su, to_blob);
  shuffle_matrix(fmt, H, F, c(2), c(5), blob + L.cd, blob + L.sd, to_blob);
  float* tau = reinterpret_cast<float*>(blob + L.tau);
  for (int i = 0; i < 3; ++i) {
    if (to_blob) {
      tau[i] = (fmt == MOE_FMT_NVFP4) ? *static_cast<const float*>(canon[6 + i]) : 1.0f;
    } else if (canon[6 + i]) {
      *static_cast<float*>(canon[6 + i]) = tau[i];
    }
  }
}

int moe_pack_expert(int fmt, int H, int F, const void* const canon[9], void* blob) {
  g_err[0] = 0;
  int st = check_shape(fmt, H, F);
  if (st) return st;
  if (!canon || !blob) return fail(MOE_E_ARG, "NULL canon or blob");
  const int need = fmt == MOE_FMT_NVFP4 ? 9 : 6;
  for (int i = 0; i < need; ++i)
    if (!canon[i]) return fail(MOE_E_ARG, "canon[%d] is NULL", i);
  const BlobLayout L = blob_layout(fmt, H, F);
  uint8_t* b = static_cast<uint8_t*>(blob);
  memset(b, 0, L.total);
  copy_sections(fmt, H, F, L, b, const_cast<void* const*>(canon), true);
  return MOE_OK;
}

int moe_unpack_expert(int fmt, int H, int F, const void* blob, void* const canon[9]) {
  g_err[0] = 0;
  int st = check_shape(fmt, H, F);
  if (st) return st;
  if (!canon || !blob) return fail(MOE_E_ARG, "NULL canon or blob");
  for (int i = 0; i < 6; ++i)
    if (!canon[i]) return fail(MOE_E_ARG, "canon[%d] is NULL", i);
  copy_sections(fmt, H, F, blob_layout(fmt, H, F),
                const_cast<uint8_t*>(static_cast<const uint8_t*>(blob)), canon, false);
  return MOE_OK;
}

// ---------------------------------------------------------------- routing

namespace {
// The bf16 planes of a prepared router (MOE_ROUTE_PREPARED), else NULL.
const uint16_t* prepared_planes(const float* router, int E, int H, unsigned flags) {
  if (!(flags & MOE_ROUTE_PREPARED) || !router) return nullptr;
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(router) +
                                           align256((size_t)E * H * 4));
}
}  // namespace

size_t moe_router_prepared_bytes(int E, int H) {
  if (E < 1 || E > 1024 || !valid_dim(H)) return 0;
  return align256((size_t)E * H * 4) + align256((size_t)3 * E * H * 2);
}

int moe_router_prepare(const float* router, int E, int H, void* prepared, moe_stream_t stream) {
  g_err[0] = 0;
  if (!moe_router_prepared_bytes(E, H)) return fail(MOE_E_ARG, "E=%d H=%d", E, H);
  if (!router || !prepared) return fail(MOE_E_ARG, "NULL router or prepared buffer");
  if (!aligned(router, 16) || !aligned(prepared, 256))
    return fail(MOE_E_ARG, "router must be 16-byte and prepared 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = (size_t)E * H;
  hipError_t e = hipSuccess;
  if (prepared != static_cast<const void*>(router))
    e = hipMemcpyAsync(prepared, router, n * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_router_split(router, E, H,
                            reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(prepared) + align256(n * 4)), s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_router_prepare");
}

size_t moe_route_workspace(int T, int H, int E, int k) {
  if (T < 0 || E < 1 || k < 1 || !valid_dim(H)) return 0;
  return route_ws_bytes(T, H, E, k);
}

int moe_route(const uint16_t* x, const float* router, int T, int H, int E, int k, unsigned flags,
              int32_t* topk_idx, float* topk_w, int32_t* pair_perm, int32_t* expert_off, void* ws,
              size_t ws_bytes, moe_stream_t stream) {
  g_err[0] = 0;
  int st = check_route_dims(T, H, E, k);
  if (st) return st;
  if (flags & ~(MOE_ROUTE_RENORM | MOE_ROUTE_PREPARED)) return fail(MOE_E_ARG, "unknown route flags 0x%x", flags);
  if (T > 0 && (pair_perm == nullptr) != (expert_off == nullptr))
    return fail(MOE_E_ARG, "pair_perm and expert_off must both be given or both be NULL");
  if (T > 0 && (!x || !router || !topk_idx || !topk_w))
    return fail(MOE_E_ARG, "NULL x/router/topk_idx/topk_w");
  if (!aligned(x, 16) || !aligned(router, 16)) return fail(MOE_E_ARG, "x and router must be 16-byte aligned");
  if (!ws || !aligned(ws, 256) || ws_bytes < route_ws_bytes(T, H, E, k))
    return fail(MOE_E_WORKSPACE, "route workspace needs %zu bytes, 256-aligned", route_ws_bytes(T, H, E, k));
  RouteArgs a{};
  a.x = x; a.router = router; a.T = T; a.H = H; a.E = E; a.k = k; a.flags = flags & MOE_ROUTE_RENORM;
  a.planes_ready = prepared_planes(router, E, H, flags);
  a.topk_idx = topk_idx; a.topk_w = topk_w; a.pair_perm = pair_perm; a.expert_off = expert_off;
  route_ws_carve(a, ws);
  hipError_t e = launch_route(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route");
}

// ------------------------------------------------------------------ cache

int moe_lru_reset(const moe_lru* lru, moe_stream_t stream) {
  g_err[0] = 0;
  if (!lru || !lru->slot_expert || !lru->expert_slot || !lru->slot_stamp || !lru->clock)
    return fail(MOE_E_ARG, "NULL lru state");
  if (lru->E < 1 || lru->E > 1024 || lru->S < 1 || lru->S > 1024)
    return fail(MOE_E_ARG, "E=%d S=%d outside [1, 1024]", lru->E, lru->S);
  hipError_t e = launch_lru_reset(*lru, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_lru_reset");
}

size_t moe_lru_resize_workspace(int S_new) {
  if (S_new < 1 || S_new > 1024) return 0;
  return align256((size_t)(1 + 2 * S_new) * 4);
}

int moe_lru_resize(const moe_lru* from, const void* from_pool, const moe_lru* to, void* to_pool,
                   size_t expert_bytes, size_t stride, void* ws, size_t ws_bytes, moe_stream_t stream) {
  g_err[0] = 0;
  for (const moe_lru* l : {from, to}) {
    if (!l || !l->slot_expert || !l->expert_slot || !l->slot_stamp || !l->clock)
      return fail(MOE_E_ARG, "NULL lru state");
    if (l->E < 1 || l->E > 1024 || l->S < 1 || l->S > 1024)
      return fail(MOE_E_ARG, "E=%d S=%d outside [1, 1024]", l->E, l->S);
  }
  if (from->E != to->E) return fail(MOE_E_ARG, "E %d -> %d: the expert count cannot change", from->E, to->E);
  if (!from_pool || !to_pool) return fail(MOE_E_ARG, "NULL pool");
  if (!expert_bytes || expert_bytes % 256 || stride < expert_bytes || stride % 256)
    return fail(MOE_E_ARG, "bad expert_bytes %zu / stride %zu", expert_bytes, stride);
  if (!aligned(from_pool, 16) || !aligned(to_pool, 16)) return fail(MOE_E_ARG, "pools must be 16-byte aligned");
  if (from_pool != to_pool) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(from_pool), a1 = a0 + (uintptr_t)from->S * stride;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(to_pool), b1 = b0 + (uintptr_t)to->S * stride;
    if (a0 < b1 && b0 < a1) return fail(MOE_E_ARG, "pools overlap without being the same pool");
  }
  const size_t need = moe_lru_resize_workspace(to->S);
  if (!ws || ws_bytes < need) return fail(MOE_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  if (!aligned(ws, 4)) return fail(MOE_E_ARG, "workspace must be 4-byte aligned");
  hipError_t e = launch_lru_resize(*from, static_cast<const uint8_t*>(from_pool), *to, static_cast<uint8_t*>(to_pool),
                                   expert_bytes, stride, static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_lru_resize");
}

size_t moe_miss_record_words(int T, int k, int S) {
  if (T < 0 || k < 1 || S < 1) return 0;
  const long long n = (long long)T * k;
  const long long nmax = n < S ? n : S;
  return (size_t)(5 + 2 * nmax);
}

int moe_cache_lookup(const moe_lru* lru, const int32_t* topk_idx, int T, int k, int32_t* pair_slot,
                     int32_t* pair_order, int32_t* miss_rec, moe_stream_t stream) {
  g_err[0] = 0;
  if (!lru || !lru->slot_expert || !lru->expert_slot || !lru->slot_stamp || !lru->clock)
    return fail(MOE_E_ARG, "NULL lru state");
  if (lru->E < 1 || lru->E > 1024 || lru->S < 1 || lru->S > 1024)
    return fail(MOE_E_ARG, "E=%d S=%d outside [1, 1024]", lru->E, lru->S);
  if (lru->key_base < 0 || lru->key_base >= lru->E)
    return fail(MOE_E_ARG, "key_base %d outside [0, E=%d)", lru->key_base, lru->E);
  if (T < 0 || k < 1 || k > lru->E - lru->key_base) return fail(MOE_E_ARG, "T=%d k=%d", T, k);
  if (!miss_rec) return fail(MOE_E_ARG, "NULL miss_rec");
  const int n = T * k;
  if (n > 0 && (!topk_idx || !pair_slot || !pair_order)) return fail(MOE_E_ARG, "NULL pair arrays");
  const int n_max = n < lru->S ? n : lru->S;
  hipError_t e = launch_lru_lookup(*lru, topk_idx, n, pair_slot, pair_order, miss_rec, n_max,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_cache_lookup");
}

int moe_cache_fill(const int32_t* rec, const void* host_pool, void* slot_pool, size_t expert_bytes,
                   size_t stride, moe_event_t slots_free, moe_stream_t copy_stream,
                   moe_event_t fill_done) {
  g_err[0] = 0;
  if (!rec || !host_pool || !slot_pool) return fail(MOE_E_ARG, "NULL record or pool");
  if (rec[0] != MOE_OK) return fail(MOE_E_CAPACITY, "miss record status %d", rec[0]);
  if (stride < expert_bytes || stride % 256) return fail(MOE_E_ARG, "bad stride %zu", stride);
  const int n_miss = rec[1], n_max = rec[4];
  if (n_miss < 0 || n_miss > n_max) return fail(MOE_E_ARG, "corrupt miss record");
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  hipError_t e;
  if (slots_free) {
    e = hipStreamWaitEvent(cs, static_cast<hipEvent_t>(slots_free), 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  const uint8_t* hp = static_cast<const uint8_t*>(host_pool);
  uint8_t* sp = static_cast<uint8_t*>(slot_pool);
  for (int r = 0; r < n_miss; ++r) {
    const int ex = rec[5 + r], sl = rec[5 + n_max + r];
    e = hipMemcpyAsync(sp + (size_t)sl * stride, hp + (size_t)ex * stride, expert_bytes,
                       hipMemcpyHostToDevice, cs);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  }
  if (fill_done) {
    e = hipEventRecord(static_cast<hipEvent_t>(fill_done), cs);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- expert FFN

size_t moe_ffn_workspace(int fmt, int T, int H, int F, int k, int E) {
  if (!valid_fmt(fmt) || T < 0 || k < 1 || E < 1 || !valid_dim(H) || !valid_dim(F)) return 0;
  return ffn_ws_bytes(fmt, T, H, F, k, E);
}

int moe_expert_ffn(int fmt, const void* slot_pool, size_t stride, int H, int F, int E,
                   const uint16_t* x, int T, int k, const int32_t* topk_idx,
                   const int32_t* pair_slot, const int32_t* pair_perm, const int32_t* expert_off,
                   const int32_t* pair_subset, int n_subset, const float* topk_w, float* y,
                   uint16_t* out, unsigned flags, void* ws, size_t ws_bytes, moe_stream_t stream) {
  g_err[0] = 0;
  int st = check_shape(fmt, H, F);
  if (st) return st;
  if (E < 1 || E > 1024) return fail(MOE_E_ARG, "E=%d outside [1, 1024]", E);
  if (T < 0 || k < 1 || k > E || k > 16) return fail(MOE_E_ARG, "T=%d k=%d", T, k);
  if ((flags & ~MOE_FFN_MX_NATIVE) > MOE_FFN_GROUPED) return fail(MOE_E_ARG, "unknown ffn flags 0x%x", flags);
  if (T == 0) return MOE_OK;
  if (!y && !out) return fail(MOE_E_ARG, "y and out are both NULL");
  if (out && !topk_w) return fail(MOE_E_ARG, "out needs topk_w");
  if (out && pair_subset) return fail(MOE_E_ARG, "the fused combine needs all pairs (pair_subset NULL)");
  if (pair_subset && (n_subset < 0 || n_subset > T * k)) return fail(MOE_E_ARG, "n_subset=%d", n_subset);
  const size_t eb = blob_layout(fmt, H, F).total;
  if (stride < eb || stride % 256) return fail(MOE_E_ARG, "stride %zu < blob %zu or not 256-multiple", stride, eb);
  if (!slot_pool || !aligned(slot_pool, 256)) return fail(MOE_E_ARG, "slot_pool NULL or not 256-aligned");
  if (T > 0 && (!x || !topk_idx)) return fail(MOE_E_ARG, "NULL x/topk_idx");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(out, 16))
    return fail(MOE_E_ARG, "x, y and out must be 16-byte aligned");
  const size_t need = moe_ffn_workspace(fmt, T, H, F, k, E);
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "ffn workspace needs %zu bytes, 256-aligned", need);

  bool grouped = false;
  const bool have_perm = pair_perm && expert_off;
  const unsigned path = flags & ~MOE_FFN_MX_NATIVE;
  if (path == MOE_FFN_GROUPED) {
    if (!have_perm) return fail(MOE_E_ARG, "grouped path needs pair_perm and expert_off");
    if (pair_subset) return fail(MOE_E_ARG, "grouped path computes all pairs (pair_subset NULL)");
    grouped = true;
  } else if (path == MOE_FFN_AUTO) {
    grouped = have_perm && !pair_subset && (long long)T * k >= 2LL * E;
  }
  if (!grouped && out && k > 16) return fail(MOE_E_ARG, "fused combine on the GEMV path needs k <= 16");

  FfnArgs a{};
  a.fmt = fmt; a.H = H; a.F = F; a.E = E; a.T = T; a.k = k;
  a.pool = static_cast<const uint8_t*>(slot_pool); a.stride = stride; a.L = blob_layout(fmt, H, F);
  a.x = x; a.topk_idx = topk_idx; a.pair_slot = pair_slot; a.pair_perm = pair_perm;
  a.expert_off = expert_off; a.pair_subset = pair_subset;
  a.n_pairs = pair_subset ? n_subset : T * k;
  a.topk_w = topk_w; a.y = y; a.out = out;
  a.mx_native = (flags & MOE_FFN_MX_NATIVE) ? 1 : 0;
  ffn_ws_carve(a, static_cast<uint8_t*>(ws));
  if (T == 0 || a.n_pairs == 0) return MOE_OK;
  hipError_t e = grouped ? launch_ffn_grouped(a, static_cast<hipStream_t>(stream))
                         : launch_ffn_gemv(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, grouped ? "moe_expert_ffn(grouped)" : "moe_expert_ffn(gemv)");
}

size_t moe_layer_workspace(int fmt, int T, int H, int F, int k, int E) {
  const size_t ffn = moe_ffn_workspace(fmt, T, H, F, k, E);
  if (!ffn || E > 1024) return 0;
  const size_t n = (size_t)T * k;
  return align256(route_ws_bytes(T, H, E, k)) + align256(n * 4) + align256((size_t)(E + 1) * 4) + ffn;
}

int moe_layer_forward(int fmt, const void* pool, size_t stride, int H, int F, int E, int k,
                      unsigned route_flags, const uint16_t* x, int T, const float* router,
                      int32_t* topk_idx, float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                      moe_stream_t stream) {
  return moe_layer_forward_prefetch(fmt, pool, stride, H, F, E, k, route_flags, x, T, router, topk_idx, topk_w,
                                    out, ws, ws_bytes, nullptr, 0, stream);
}

int moe_layer_forward_prefetch(int fmt, const void* pool, size_t stride, int H, int F, int E, int k,
                               unsigned route_flags, const uint16_t* x, int T, const float* router,
                               int32_t* topk_idx, float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                               const void* warm, size_t warm_bytes, moe_stream_t stream) {
  g_err[0] = 0;
  if ((warm == nullptr) != (warm_bytes == 0)) return fail(MOE_E_ARG, "warm and warm_bytes: both set or both 0");
  if (warm && !aligned(warm, 16)) return fail(MOE_E_ARG, "warm must be 16-byte aligned");
  int st = check_shape(fmt, H, F);
  if (st) return st;
  st = check_route_dims(T, H, E, k);
  if (st) return st;
  if (route_flags & ~(MOE_ROUTE_RENORM | MOE_ROUTE_PREPARED | MOE_LAYER_MX_NATIVE))
    return fail(MOE_E_ARG, "unknown route flags 0x%x", route_flags);
  if (k > 16) return fail(MOE_E_ARG, "moe_layer_forward needs k <= 16");
  const size_t eb = blob_layout(fmt, H, F).total;
  if (stride < eb || stride % 256) return fail(MOE_E_ARG, "stride %zu < blob %zu or not 256-multiple", stride, eb);
  if (!pool || !aligned(pool, 256)) return fail(MOE_E_ARG, "pool NULL or not 256-aligned");
  if (T == 0) return MOE_OK;
  if (!x || !router || !topk_idx || !topk_w || !out) return fail(MOE_E_ARG, "NULL argument");
  if (!aligned(x, 16) || !aligned(router, 16) || !aligned(out, 16))
    return fail(MOE_E_ARG, "x, router and out must be 16-byte aligned");
  const size_t need = moe_layer_workspace(fmt, T, H, F, k, E);
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "layer workspace needs %zu bytes, 256-aligned", need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* p = static_cast<uint8_t*>(ws);
  RouteArgs r{};
  r.x = x; r.router = router; r.T = T; r.H = H; r.E = E; r.k = k; r.flags = route_flags & MOE_ROUTE_RENORM;
  r.planes_ready = prepared_planes(router, E, H, route_flags);
  r.topk_idx = topk_idx; r.topk_w = topk_w;
  route_ws_carve(r, p);
  p += align256(route_ws_bytes(T, H, E, k));
  int32_t* perm = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)T * k * 4);
  int32_t* off = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)(E + 1) * 4);
  FfnArgs a{};
  a.fmt = fmt; a.H = H; a.F = F; a.E = E; a.T = T; a.k = k;
  a.pool = static_cast<const uint8_t*>(pool); a.stride = stride; a.L = blob_layout(fmt, H, F);
  a.x = x; a.topk_idx = topk_idx; a.topk_w = topk_w; a.out = out; a.n_pairs = T * k;
  a.mx_native = (route_flags & MOE_LAYER_MX_NATIVE) ? 1 : 0;
  ffn_ws_carve(a, p);
  a.warm = static_cast<const uint8_t*>(warm);
  a.warm_bytes = warm_bytes;
  hipError_t e;
  if (T <= 4) {
    e = launch_router_logits(x, router, T, H, E, r.logits, s);
    if (e == hipSuccess) e = launch_decode_layer(a, r.logits, route_flags & MOE_ROUTE_RENORM, topk_idx, topk_w, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_layer_forward(decode)");
  }
  r.pair_perm = perm;
  r.expert_off = off;
  const bool grouped = (long long)T * k >= 2LL * E;
  if (grouped) {  // the permutation kernel also writes the grouped path's tile list
    r.tiles = a.tiles;
    r.tile_rows = grouped_tile_rows(fmt, a.mx_native);
    r.max_tiles = grouped_max_tiles(fmt, a.mx_native, T * k, E);
    a.tiles_ready = 1;
  }
  e = launch_route(r, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward(route)");
  a.pair_perm = perm;
  a.expert_off = off;
  e = grouped ? launch_ffn_grouped(a, s) : launch_ffn_gemv(a, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_layer_forward(ffn)");
}

// ------------------------------------------------- allocation-free layer call

// The workspace of moe_layer_forward_static: one static device array, held by
// every GPU the library runs on until the process ends.  Host code must never
// pass `scratch` itself to a kernel or a copy (on the host the name stands for
// a host-side symbol, not the device address); the device address comes from
// hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on the first call
// on each device); MOE_OK or an error status.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_E_ARG, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

int moe_layer_forward_static(int fmt, const void* pool, size_t stride, int H, int F, int E, int k,
                             unsigned route_flags, const uint16_t* x, int T, const float* router,
                             int32_t* topk_idx, float* topk_w, uint16_t* out, moe_stream_t stream) {
  g_err[0] = 0;
  int st = check_shape(fmt, H, F);
  if (st) return st;
  st = check_route_dims(T, H, E, k);
  if (st) return st;
  const size_t need = moe_layer_workspace(fmt, T, H, F, k, E);
  if (!need) return fail(MOE_E_ARG, "bad shape or format");
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES)
    return fail(MOE_E_WORKSPACE, "this call needs %zu bytes of workspace, more than the %u of the static scratch array "
                "(use moe_layer_forward with a caller workspace)", need, (unsigned)MOE_STATIC_SCRATCH_BYTES);
  if (route_flags & ~(MOE_ROUTE_RENORM | MOE_ROUTE_PREPARED))
    return fail(MOE_E_ARG, "unknown route flags 0x%x", route_flags);
  const size_t eb = blob_layout(fmt, H, F).total;
  if (stride < eb || stride % 256) return fail(MOE_E_ARG, "stride %zu < blob %zu or not 256-multiple", stride, eb);
  if (!pool || !aligned(pool, 256)) return fail(MOE_E_ARG, "pool NULL or not 256-aligned");
  if (T == 0) return MOE_OK;
  if (!x || !router || !topk_idx || !topk_w || !out) return fail(MOE_E_ARG, "NULL argument");
  if (!aligned(x, 16) || !aligned(router, 16) || !aligned(out, 16))
    return fail(MOE_E_ARG, "x, router and out must be 16-byte aligned");
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  return moe_layer_forward(fmt, pool, stride, H, F, E, k, route_flags, x, T, router, topk_idx, topk_w, out, ws,
                           (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

size_t moe_prefill_streamed_workspace(int fmt, int T, int H, int F, int k, int E) {
  return moe_layer_workspace(fmt, T, H, F, k, E);
}

int moe_prefill_streamed(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                         int n_layers, const void* const* host_pools, const float* const* routers,
                         const uint16_t* x, int T, uint16_t* const* outs, int32_t* topk_idx,
                         float* topk_w, void* const* pools, void* ws, size_t ws_bytes,
                         moe_stream_t stream, moe_stream_t copy_stream, const moe_event_t* events) {
  g_err[0] = 0;
  int st = check_shape(fmt, H, F);
  if (st) return st;
  st = check_route_dims(T, H, E, k);
  if (st) return st;
  if (n_layers < 0) return fail(MOE_E_ARG, "n_layers %d", n_layers);
  if (n_layers == 0 || T == 0) return MOE_OK;
  if (!host_pools || !routers || !outs || !pools || !events || !topk_idx || !topk_w)
    return fail(MOE_E_ARG, "NULL array argument");
  if (!pools[0] || !pools[1] || pools[0] == pools[1]) return fail(MOE_E_ARG, "need two distinct pools");
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return fail(MOE_E_ARG, "event %d is NULL", i);
  if (!copy_stream || copy_stream == stream) return fail(MOE_E_ARG, "copy_stream must be a second stream");
  for (int l = 0; l < n_layers; ++l)
    if (!host_pools[l] || !routers[l] || !outs[l]) return fail(MOE_E_ARG, "layer %d: NULL pointer", l);
  const size_t need = moe_prefill_streamed_workspace(fmt, T, H, F, k, E);
  if (!need) return fail(MOE_E_ARG, "bad shape or format");
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "prefill workspace needs %zu bytes, 256-aligned", need);
  hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(copy_stream);
  hipEvent_t ev[4];
  for (int i = 0; i < 4; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  const size_t bytes = (size_t)E * stride;
  // copy of layer l into pool l % 2, after the pool's previous reader (layer l-2)
  auto copy_layer = [&](int l) -> hipError_t {
    const int p = l & 1;
    hipError_t e = hipSuccess;
    if (l >= 2) e = hipStreamWaitEvent(cs, ev[2 + p], 0);
    if (e == hipSuccess) e = hipMemcpyAsync(pools[p], host_pools[l], bytes, hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipEventRecord(ev[p], cs);
    return e;
  };
  hipError_t e = copy_layer(0);
  if (e == hipSuccess && n_layers > 1) e = copy_layer(1);
  if (e != hipSuccess) return hip_fail(e, "moe_prefill_streamed(copy)");
  const size_t tk = (size_t)T * k;
  for (int l = 0; l < n_layers; ++l) {
    const int p = l & 1;
    e = hipStreamWaitEvent(s, ev[p], 0);
    if (e != hipSuccess) return hip_fail(e, "moe_prefill_streamed(wait copy)");
    st = moe_layer_forward(fmt, pools[p], stride, H, F, E, k, route_flags, x, T, routers[l], topk_idx + l * tk,
                           topk_w + l * tk, outs[l], ws, ws_bytes, stream);
    if (st) return st;
    e = hipEventRecord(ev[2 + p], s);
    if (e == hipSuccess && l + 2 < n_layers) e = copy_layer(l + 2);
    if (e != hipSuccess) return hip_fail(e, "moe_prefill_streamed(layer)");
  }
  return MOE_OK;
}

int moe_combine(const float* y, const float* topk_w, int T, int H, int k, uint16_t* out,
                moe_stream_t stream) {
  g_err[0] = 0;
  if (T < 0 || k < 1 || !valid_dim(H)) return fail(MOE_E_ARG, "T=%d H=%d k=%d", T, H, k);
  if (T > 0 && (!y || !topk_w || !out)) return fail(MOE_E_ARG, "NULL y/topk_w/out");
  if (!aligned(y, 16) || !aligned(out, 16)) return fail(MOE_E_ARG, "y and out must be 16-byte aligned");
  hipError_t e = launch_combine(y, topk_w, T, H, k, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine");
}

}  // extern "C"

// ------------------------------------------------------- cached layer executor

size_t moe_cached_layer_workspace(int fmt, int T, int H, int F, int k, int E) {
  const size_t ffn = moe_ffn_workspace(fmt, T, H, F, k, E), route = moe_route_workspace(T, H, E, k);
  if (!ffn || !route) return 0;
  return align256((size_t)T * k * H * 4) + align256(route) + ffn;
}

int moe_cached_layer_forward(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                             const moe_cached_layer* L, const uint16_t* x, int T, int32_t* topk_idx,
                             float* topk_w, int32_t* pair_slot, int32_t* pair_order, uint16_t* out,
                             void* ws, size_t ws_bytes, moe_stream_t stream, moe_stream_t copy_stream,
                             int32_t* n_hits, int32_t* n_miss) {
  g_err[0] = 0;
  if (!L || !L->router || !L->host_pool || !L->slot_pool || !L->miss_rec || !L->lookup_done)
    return fail(MOE_E_ARG, "incomplete moe_cached_layer");
  {
    // the record is read on the host after the lookup: it must be host memory
    hipPointerAttribute_t at{};
    const hipError_t pe = hipPointerGetAttributes(&at, L->miss_rec);
    if (pe == hipSuccess && at.type == hipMemoryTypeDevice)
      return fail(MOE_E_ARG, "miss_rec is device memory; moe_cached_layer_forward needs a [pinned] record");
    (void)hipGetLastError();  // an unregistered host pointer reports an error here; it is host memory
  }
  const size_t need = moe_cached_layer_workspace(fmt, T, H, F, k, E);
  if (!need) return fail(MOE_E_ARG, "bad shape or format");
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "cached layer workspace needs %zu bytes, 256-aligned", need);
  if (T == 0) return MOE_OK;
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* y = reinterpret_cast<float*>(p);
  p += align256((size_t)T * k * H * 4);
  const size_t route_bytes = moe_route_workspace(T, H, E, k);
  void* route_ws = p;
  p += align256(route_bytes);
  void* ffn_ws = p;
  const size_t ffn_bytes = moe_ffn_workspace(fmt, T, H, F, k, E);
  int st = moe_route(x, L->router, T, H, E, k, route_flags, topk_idx, topk_w, nullptr, nullptr, route_ws,
                     route_bytes, stream);
  if (st) return st;
  st = moe_cache_lookup(&L->lru, topk_idx, T, k, pair_slot, pair_order, L->miss_rec, stream);
  if (st) return st;
  hipEvent_t lk = static_cast<hipEvent_t>(L->lookup_done);
  hipError_t e = hipEventRecord(lk, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipEventSynchronize(lk);
  if (e != hipSuccess) return hip_fail(e, "lookup event");
  const int32_t* rec = L->miss_rec;
  if (n_hits) *n_hits = rec[3];
  if (n_miss) *n_miss = rec[1];
  if (rec[0] != MOE_OK) return fail(MOE_E_CAPACITY, "layer cache: %d misses exceed the evictable slots", rec[1]);
  const size_t eb = moe_expert_bytes(fmt, H, F);
  st = moe_cache_fill(rec, L->host_pool, L->slot_pool, eb, stride, L->slots_free, copy_stream, L->fill_done);
  if (st) return st;
  const int n_pairs = T * k, n_hit = rec[2];
  if (n_hit > 0) {
    st = moe_expert_ffn(fmt, L->slot_pool, stride, H, F, E, x, T, k, topk_idx, pair_slot, nullptr, nullptr,
                        pair_order, n_hit, nullptr, y, nullptr, MOE_FFN_GEMV, ffn_ws, ffn_bytes, stream);
    if (st) return st;
  }
  if (L->fill_done) {
    e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(L->fill_done), 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(fill_done)");
  }
  if (n_hit < n_pairs) {
    st = moe_expert_ffn(fmt, L->slot_pool, stride, H, F, E, x, T, k, topk_idx, pair_slot, nullptr, nullptr,
                        pair_order + n_hit, n_pairs - n_hit, nullptr, y, nullptr, MOE_FFN_GEMV, ffn_ws,
                        ffn_bytes, stream);
    if (st) return st;
  }
  if (L->slots_free) {
    e = hipEventRecord(static_cast<hipEvent_t>(L->slots_free), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(slots_free)");
  }
  return moe_combine(y, topk_w, T, H, k, out, stream);
}

size_t moe_cached_layer_split_host_bytes(int T, int H, int F, int k) {
  if (T < 0 || k < 1 || H < 1 || F < 1) return 0;
  const size_t n = (size_t)T * k;
  return align256((size_t)T * H * 2) + align256(n * 4) * 2 + align256(n * H * 4) + align256(n * (H + F) * 4);
}

int moe_cached_layer_forward_split(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                                   const moe_cached_layer* L, const uint16_t* x, int T, int32_t* topk_idx,
                                   float* topk_w, int32_t* pair_slot, int32_t* pair_order, uint16_t* out,
                                   void* ws, size_t ws_bytes, moe_stream_t stream, moe_stream_t copy_stream,
                                   float q, void* host_ws, size_t host_ws_bytes, int n_threads,
                                   moe_event_t defer_done, int32_t* n_hits, int32_t* n_miss, int32_t* n_cpu) {
  g_err[0] = 0;
  if (!L || !L->router || !L->host_pool || !L->slot_pool || !L->miss_rec || !L->lookup_done || !L->fill_done)
    return fail(MOE_E_ARG, "incomplete moe_cached_layer (needs its lookup_done and fill_done events)");
  if (!(q >= 0.0f && q <= 1.0f)) return fail(MOE_E_ARG, "q=%g outside [0, 1]", q);
  if (!defer_done || !copy_stream || copy_stream == stream)
    return fail(MOE_E_ARG, "needs a defer_done event and a copy stream other than stream");
  {
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, L->miss_rec) == hipSuccess && at.type == hipMemoryTypeDevice)
      return fail(MOE_E_ARG, "miss_rec is device memory; the split executor reads it on the host");
    (void)hipGetLastError();
  }
  const size_t need = moe_cached_layer_workspace(fmt, T, H, F, k, E);
  if (!need) return fail(MOE_E_ARG, "bad shape or format");
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "cached layer workspace needs %zu bytes, 256-aligned", need);
  const size_t hneed = moe_cached_layer_split_host_bytes(T, H, F, k);
  if (!host_ws || !aligned(host_ws, 256) || host_ws_bytes < hneed)
    return fail(MOE_E_WORKSPACE, "host workspace needs %zu bytes of pinned memory, 256-aligned", hneed);
  if (T == 0) return MOE_OK;
  if (T * k > 64) return fail(MOE_E_ARG, "the split executor takes at most 64 pairs per step (T=%d k=%d)", T, k);
  hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(copy_stream);
  const int n_pairs = T * k;
  // host workspace: x, topk_idx, the GPU-served missed pairs, y of the CPU pairs, scratch
  uint8_t* hp = static_cast<uint8_t*>(host_ws);
  uint16_t* hx = reinterpret_cast<uint16_t*>(hp);
  hp += align256((size_t)T * H * 2);
  int32_t* hidx = reinterpret_cast<int32_t*>(hp);
  hp += align256((size_t)n_pairs * 4);
  int32_t* hsub = reinterpret_cast<int32_t*>(hp);
  hp += align256((size_t)n_pairs * 4);
  float* hy = reinterpret_cast<float*>(hp);
  hp += align256((size_t)n_pairs * H * 4);
  float* hscr = reinterpret_cast<float*>(hp);
  // device workspace: y, routing, then the expert FFN's
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* y = reinterpret_cast<float*>(p);
  p += align256((size_t)n_pairs * H * 4);
  const size_t route_bytes = moe_route_workspace(T, H, E, k);
  void* route_ws = p;
  p += align256(route_bytes);
  void* ffn_ws = p;
  const size_t ffn_bytes = moe_ffn_workspace(fmt, T, H, F, k, E);
  // the previous call's deferred fills land before anything reads the slots
  hipError_t e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(defer_done), 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(defer_done)");
  int st = moe_route(x, L->router, T, H, E, k, route_flags, topk_idx, topk_w, nullptr, nullptr, route_ws,
                     route_bytes, stream);
  if (st) return st;
  e = hipMemcpyAsync(hidx, topk_idx, (size_t)n_pairs * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(hx, x, (size_t)T * H * 2, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "split: copies to the host");
  st = moe_cache_lookup(&L->lru, topk_idx, T, k, pair_slot, pair_order, L->miss_rec, stream);
  if (st) return st;
  hipEvent_t lk = static_cast<hipEvent_t>(L->lookup_done);
  e = hipEventRecord(lk, s);
  if (e == hipSuccess) e = hipEventSynchronize(lk);
  if (e != hipSuccess) return hip_fail(e, "lookup event");
  const int32_t* rec = L->miss_rec;
  if (rec[0] != MOE_OK) return fail(MOE_E_CAPACITY, "layer cache: %d misses exceed the evictable slots", rec[1]);
  const int nm = rec[1], n_max = rec[4], n_hit = rec[2];
  const int nc = (int)(q * (float)nm);  // the last nc distinct misses go to the CPU
  if (n_hits) *n_hits = rec[3];
  if (n_miss) *n_miss = nm;
  if (n_cpu) *n_cpu = nc;
  const size_t eb = moe_expert_bytes(fmt, H, F);
  const uint8_t* hpool = static_cast<const uint8_t*>(L->host_pool);
  uint8_t* spool = static_cast<uint8_t*>(L->slot_pool);
  // the copy stream: the GPU-served fills, fill_done, then the CPU-served
  // experts' fills (they still enter the cache), defer_done
  if (L->slots_free) {
    e = hipStreamWaitEvent(cs, static_cast<hipEvent_t>(L->slots_free), 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(slots_free)");
  }
  for (int r = 0; r < nm; ++r) {
    if (r == nm - nc) {
      e = hipEventRecord(static_cast<hipEvent_t>(L->fill_done), cs);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord(fill_done)");
    }
    e = hipMemcpyAsync(spool + (size_t)rec[5 + n_max + r] * stride, hpool + (size_t)rec[5 + r] * stride, eb,
                       hipMemcpyHostToDevice, cs);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(fill)");
  }
  if (nc == 0) {
    e = hipEventRecord(static_cast<hipEvent_t>(L->fill_done), cs);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(fill_done)");
  }
  e = hipEventRecord(static_cast<hipEvent_t>(defer_done), cs);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(defer_done)");
  // the hit pairs on the GPU meanwhile
  if (n_hit > 0) {
    st = moe_expert_ffn(fmt, L->slot_pool, stride, H, F, E, x, T, k, topk_idx, pair_slot, nullptr, nullptr,
                        pair_order, n_hit, nullptr, y, nullptr, MOE_FFN_GEMV, ffn_ws, ffn_bytes, stream);
    if (st) return st;
  }
  // which missed pairs the GPU computes (expert among the first nm - nc misses)
  auto cpu_served = [&](int ex) {
    for (int r = nm - nc; r < nm; ++r)
      if (rec[5 + r] == ex) return true;
    return false;
  };
  auto resident = [&](int ex) {
    for (int r = 0; r < nm; ++r)
      if (rec[5 + r] == ex) return false;
    return true;
  };
  int n_gpu_miss = 0, n_cpu_pairs = 0;
  for (int qp = 0; qp < n_pairs; ++qp) {
    const int ex = hidx[qp];
    if (resident(ex)) continue;
    if (cpu_served(ex)) ++n_cpu_pairs;
    else hsub[n_gpu_miss++] = qp;
  }
  e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(L->fill_done), 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(fill_done)");
  if (n_gpu_miss > 0) {
    // the list sits in pinned host memory, which the kernel reads directly; the
    // next call rewrites it only after its own lookup, i.e. after this kernel
    st = moe_expert_ffn(fmt, L->slot_pool, stride, H, F, E, x, T, k, topk_idx, pair_slot, nullptr, nullptr,
                        hsub, n_gpu_miss, nullptr, y, nullptr, MOE_FFN_GEMV, ffn_ws, ffn_bytes, stream);
    if (st) return st;
  }
  if (L->slots_free) {
    e = hipEventRecord(static_cast<hipEvent_t>(L->slots_free), s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(slots_free)");
  }
  // the CPU-served pairs on this thread, from the pinned blobs, while the GPU works
  if (n_cpu_pairs > 0) {
    const void* blobs[64];
    const uint16_t* xs[64];
    float* ys[64];
    int qs[64], n = 0;
    for (int qp = 0; qp < n_pairs && n < 64; ++qp) {
      const int ex = hidx[qp];
      if (resident(ex) || !cpu_served(ex)) continue;
      blobs[n] = hpool + (size_t)ex * stride;
      xs[n] = hx + (size_t)(qp / k) * H;
      ys[n] = hy + (size_t)n * H;
      qs[n++] = qp;
    }
    st = moe_host_expert_ffn(fmt, H, F, n, blobs, xs, ys, hscr, n_threads);
    if (st) return fail(st, "host expert FFN");
    for (int i = 0; i < n; ++i) {
      e = hipMemcpyAsync(y + (size_t)qs[i] * H, ys[i], (size_t)H * 4, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(y)");
    }
  }
  return moe_combine(y, topk_w, T, H, k, out, stream);
}

int moe_cache_fill_device(const int32_t* miss_rec, const void* host_pool, void* slot_pool,
                          size_t expert_bytes, size_t stride, moe_event_t record_ready,
                          moe_event_t slots_free, moe_stream_t copy_stream, moe_event_t fill_done) {
  g_err[0] = 0;
  if (!miss_rec || !host_pool || !slot_pool) return fail(MOE_E_ARG, "NULL record or pool");
  if (!expert_bytes || expert_bytes % 256 || stride < expert_bytes || stride % 256)
    return fail(MOE_E_ARG, "bad expert_bytes %zu / stride %zu", expert_bytes, stride);
  if (!aligned(host_pool, 16) || !aligned(slot_pool, 16)) return fail(MOE_E_ARG, "pools must be 16-byte aligned");
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  hipError_t e;
  for (moe_event_t ev : {record_ready, slots_free}) {
    if (!ev) continue;
    e = hipStreamWaitEvent(cs, static_cast<hipEvent_t>(ev), 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  e = launch_cache_fill(miss_rec, static_cast<const uint8_t*>(host_pool), static_cast<uint8_t*>(slot_pool),
                        expert_bytes, stride, cs);
  if (e != hipSuccess) return hip_fail(e, "cache fill kernel");
  if (fill_done) {
    e = hipEventRecord(static_cast<hipEvent_t>(fill_done), cs);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return MOE_OK;
}

namespace {
// Optional predictive prefetch of one cached decode layer (T = 1).
struct PrefetchArgs {
  int m;
  uint8_t* buf;
  hipStream_t stream;
};

int cached_enqueue(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                   const moe_cached_layer* L, const uint16_t* x, int T, int32_t* topk_idx, float* topk_w,
                   int32_t* pair_slot, int32_t* pair_order, uint16_t* out, void* ws, size_t ws_bytes,
                   moe_stream_t stream, const PrefetchArgs* pf) {
  if (!L || !L->router || !L->host_pool || !L->slot_pool || !L->miss_rec)
    return fail(MOE_E_ARG, "incomplete moe_cached_layer");
  int st = check_shape(fmt, H, F);
  if (st) return st;
  const size_t need = moe_cached_layer_workspace(fmt, T, H, F, k, E);
  if (!need) return fail(MOE_E_ARG, "bad shape or format");
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "cached layer workspace needs %zu bytes, 256-aligned", need);
  if (!pair_slot || !pair_order || !out || !topk_idx || !topk_w) return fail(MOE_E_ARG, "NULL output");
  if (stride < moe_expert_bytes(fmt, H, F) || stride % 256) return fail(MOE_E_ARG, "bad stride %zu", stride);
  if (!aligned(L->host_pool, 256) || !aligned(L->slot_pool, 256)) return fail(MOE_E_ARG, "pools must be 256-byte aligned");
  if (route_flags & ~(MOE_ROUTE_RENORM | MOE_ROUTE_PREPARED))
    return fail(MOE_E_ARG, "unknown route flags 0x%x", route_flags);
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* y = reinterpret_cast<float*>(p);
  p += align256((size_t)T * k * H * 4);
  const size_t route_bytes = moe_route_workspace(T, H, E, k);
  void* route_ws = p;
  p += align256(route_bytes);
  if (L->lru.key_base < 0 || L->lru.key_base + E > L->lru.E || L->lru.E > 1024 || L->lru.S < 1 || L->lru.S > 1024)
    return fail(MOE_E_ARG, "LRU state of %d keys (this layer from key %d), %d slots, for E=%d", L->lru.E,
                L->lru.key_base, L->lru.S, E);
  if (T < 0 || k < 1 || k > E || k > 16) return fail(MOE_E_ARG, "T=%d k=%d E=%d", T, k, E);
  if (T <= 4 && k <= 16) {
    // router GEMV, then the lookup kernel selects the experts itself (one kernel fewer)
    RouteArgs r{};
    r.T = T; r.H = H; r.E = E; r.k = k;
    route_ws_carve(r, route_ws);
    if (!aligned(x, 16) || !aligned(L->router, 16)) return fail(MOE_E_ARG, "x and router must be 16-byte aligned");
    float* keep = pf ? reinterpret_cast<float*>(pf->buf) : nullptr;  // the logits, for the prefetch step
    hipError_t e = launch_router_logits(x, L->router, T, H, E, r.logits, s);
    if (e == hipSuccess)
      e = launch_lru_lookup_topk(L->lru, r.logits, E, T, k, route_flags & MOE_ROUTE_RENORM, topk_idx, topk_w,
                                 pair_slot, pair_order,
                                 L->miss_rec, T * k < L->lru.S ? T * k : L->lru.S, s, keep);
    if (e != hipSuccess) return hip_fail(e, "cached layer (route + lookup)");
    if (pf) {
      // on the prefetch stream, after this lookup: one more LRU step over the
      // token's top-(k+m) experts in rank order (the routed k are hits and keep
      // their slots; runner-ups that miss take victims), then the copy of those
      // blobs from the host pool, overlapping this stream's work
      const int kp = k + pf->m, n_max = kp < L->lru.S ? kp : L->lru.S;
      int32_t* rec = reinterpret_cast<int32_t*>(pf->buf + align256((size_t)E * 4));
      int32_t* dummy = reinterpret_cast<int32_t*>(pf->buf + align256((size_t)E * 4) +
                                                  align256((size_t)(5 + 2 * n_max) * 4));
      e = hipEventRecord(static_cast<hipEvent_t>(L->lookup_done), s);
      if (e == hipSuccess) e = hipStreamWaitEvent(pf->stream, static_cast<hipEvent_t>(L->lookup_done), 0);
      if (e == hipSuccess)
        e = launch_lru_lookup_topk(L->lru, keep, E, 1, kp, route_flags & MOE_ROUTE_RENORM, dummy,
                                   reinterpret_cast<float*>(dummy + 16),
                                   dummy + 32, dummy + 48, rec, n_max, pf->stream);
      if (e == hipSuccess)
        e = launch_cache_fill(rec, static_cast<const uint8_t*>(L->host_pool), static_cast<uint8_t*>(L->slot_pool),
                              moe_expert_bytes(fmt, H, F), stride, pf->stream, 32);
      if (e != hipSuccess) return hip_fail(e, "cached layer (prefetch)");
    }
  } else {
    st = moe_route(x, L->router, T, H, E, k, route_flags, topk_idx, topk_w, nullptr, nullptr, route_ws,
                   route_bytes, stream);
    if (st) return st;
    st = moe_cache_lookup(&L->lru, topk_idx, T, k, pair_slot, pair_order, L->miss_rec, stream);
    if (st) return st;
  }
  FfnArgs a{};
  a.fmt = fmt; a.H = H; a.F = F; a.E = E; a.T = T; a.k = k;
  a.pool = static_cast<const uint8_t*>(L->slot_pool); a.stride = stride; a.L = blob_layout(fmt, H, F);
  a.x = x; a.topk_idx = topk_idx; a.pair_slot = pair_slot; a.pair_subset = pair_order;
  a.n_pairs = T * k; a.subset_rec = L->miss_rec;
  a.miss_src = static_cast<const uint8_t*>(L->host_pool); a.y = nullptr;
  a.hbuf = reinterpret_cast<uint16_t*>(p);
  a.ybuf = y;  // only if the fused down + combine does not fit
  a.out = out; a.topk_w = topk_w;
  // gate/up: mode 3 (misses streamed from the host pool into their slots, down
  // matrix included); down: mode 4 (every pair from its slot) with the combine
  hipError_t e = launch_ffn_gemv_split(a, 3, 4, s);
  // (the combine is fused into the down kernel, or follows it guarded by the record)
  return e == hipSuccess ? MOE_OK : hip_fail(e, "cached layer (experts)");
}
}  // namespace

int moe_cached_layer_enqueue(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                             const moe_cached_layer* L, const uint16_t* x, int T, int32_t* topk_idx,
                             float* topk_w, int32_t* pair_slot, int32_t* pair_order, uint16_t* out, void* ws,
                             size_t ws_bytes, moe_stream_t stream) {
  g_err[0] = 0;
  return cached_enqueue(fmt, stride, H, F, E, k, route_flags, L, x, T, topk_idx, topk_w, pair_slot, pair_order, out,
                        ws, ws_bytes, stream, nullptr);
}

size_t moe_prefetch_buffer_bytes(int E, int k, int m, int S) {
  if (E < 1 || E > 1024 || k < 1 || m < 1 || k + m > 16 || S < 1) return 0;
  const int n_max = k + m < S ? k + m : S;
  return align256((size_t)E * 4) + align256((size_t)(5 + 2 * n_max) * 4) + 256;
}

size_t moe_prefetch_record_offset(int E) { return E < 1 ? 0 : align256((size_t)E * 4); }

int moe_cached_layer_enqueue_prefetch(int fmt, size_t stride, int H, int F, int E, int k, unsigned route_flags,
                                      const moe_cached_layer* L, const uint16_t* x, int T, int32_t* topk_idx,
                                      float* topk_w, int32_t* pair_slot, int32_t* pair_order, uint16_t* out,
                                      void* ws, size_t ws_bytes, int m, void* pf_buf, size_t pf_bytes,
                                      moe_stream_t stream, moe_stream_t pf_stream) {
  g_err[0] = 0;
  if (T != 1) return fail(MOE_E_ARG, "prefetch runs one token per step (T=%d)", T);
  if (m < 1 || k + m > 16) return fail(MOE_E_ARG, "m=%d: need 1 <= m and k + m <= 16", m);
  if (!L || !L->lookup_done) return fail(MOE_E_ARG, "the layer needs its lookup_done event");
  if (!pf_stream || pf_stream == stream) return fail(MOE_E_ARG, "pf_stream must be a second stream");
  const size_t need = moe_prefetch_buffer_bytes(E, k, m, L->lru.S);
  if (!need || !pf_buf || !aligned(pf_buf, 256) || pf_bytes < need)
    return fail(MOE_E_WORKSPACE, "prefetch buffer needs %zu bytes, 256-aligned", need);
  PrefetchArgs pf{m, static_cast<uint8_t*>(pf_buf), static_cast<hipStream_t>(pf_stream)};
  return cached_enqueue(fmt, stride, H, F, E, k, route_flags, L, x, T, topk_idx, topk_w, pair_slot, pair_order, out,
                        ws, ws_bytes, stream, &pf);
}
