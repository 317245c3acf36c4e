// Batch-1 (decode-shaped) expert FFN: weight-streaming GEMV on block-scaled
// weights, dequantized in registers.
//
// Expert FFN h = bf16(silu(G x) * (U x)), y = D h  (each expert an independent
// FFN: page "FreeToken：753B大模型塞进单卡的本地部署硬件账该怎么算", section
// "混合专家架构（MoE）的天然稀疏性"; dequantization at compute time: page
// "8GB显存跑35B MoE模型：FreeToken引擎本地部署实战", §2.1).
//
// Mapping onto 64-lane wavefronts: the blob stores every matrix as fragments of
// 16 rows x 128 k in which lane l owns row l%16 and 32 consecutive k (common.h).
// A workgroup owns one 16-row group (of gate and up together for gate/up); its
// waves take the K steps round-robin.  Every lane issues all loads of a batch
// of steps first (one contiguous 1 KiB load per fragment per wavefront), then
// dots its 32 elements with the matching slice of the input vector using the
// gfx950 FP4/FP8 -> bf16 conversions and v_dot2_f32_bf16 (fp32 accumulate).
// A row is finished by two lane shuffles (its four lanes) and a fixed-order sum
// over the waves in LDS, so results do not depend on timing.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace {

constexpr int kMaxDim = 8192;

template <int FMT>
struct Frag {
  static constexpr bool kFP8 = FMT == MOE_FMT_FP8_E4M3;
  uint4 c[kFP8 ? 2 : 1];
  uint32_t sc;

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales, size_t f, int lane) {
    if constexpr (kFP8) {
      c[0] = reinterpret_cast<const uint4*>(codes + f * 2048)[lane];
      c[1] = reinterpret_cast<const uint4*>(codes + f * 2048 + 1024)[lane];
      sc = reinterpret_cast<const uint32_t*>(scales + f * 64)[lane & 15];
    } else {
      c[0] = reinterpret_cast<const uint4*>(codes + f * 1024)[lane];
      if constexpr (FMT == MOE_FMT_NVFP4)
        sc = reinterpret_cast<const uint16_t*>(scales + f * 128)[lane];
      else
        sc = scales[f * 64 + lane];
    }
  }

  // Write the fragment back at the same place of another blob (cache fill of a
  // streamed miss): every lane stores its codes, and the lanes holding a
  // distinct scale store it.
  __device__ __forceinline__ void store(uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, size_t f,
                                        int lane) const {
    if constexpr (kFP8) {
      reinterpret_cast<uint4*>(codes + f * 2048)[lane] = c[0];
      reinterpret_cast<uint4*>(codes + f * 2048 + 1024)[lane] = c[1];
      if (lane < 16) reinterpret_cast<uint32_t*>(scales + f * 64)[lane] = sc;
    } else {
      reinterpret_cast<uint4*>(codes + f * 1024)[lane] = c[0];
      if constexpr (FMT == MOE_FMT_NVFP4)
        reinterpret_cast<uint16_t*>(scales + f * 128)[lane] = (uint16_t)sc;
      else
        scales[f * 64 + lane] = (uint8_t)sc;
    }
  }

  // The lane's 32 elements against xs (16 bf16 pairs of the same k).
  __device__ __forceinline__ float dot(const uint32_t* xs) const {
    if constexpr (FMT == MOE_FMT_NVFP4)
      return chunk_dot_nvfp4(c[0], e4m3_byte0_to_f32(sc), e4m3_byte0_to_f32(sc >> 8), xs);
    else if constexpr (FMT == MOE_FMT_MXFP4)
      return chunk_dot_mxfp4(c[0], e8m0_to_f32(sc), xs, 0.0f);
    else
      return __uint_as_float(sc) * chunk_dot_fp8(c[1], xs + 8, chunk_dot_fp8(c[0], xs, 0.0f));
  }
};

// 32 bf16 (16 pairs) starting at p (16-byte aligned).
__device__ __forceinline__ void load_xslice(const uint16_t* p, uint32_t (&xs)[16]) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 u = v[j];
    xs[4 * j + 0] = u.x;
    xs[4 * j + 1] = u.y;
    xs[4 * j + 2] = u.z;
    xs[4 * j + 3] = u.w;
  }
}

// Sum of the four lanes l, l^16, l^32, l^48 (the lanes of one fragment row).
__device__ __forceinline__ float row_lanes_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Waves per workgroup and steps per load batch for S steps of 128 k.
constexpr int gemv_waves(int S) { return S < 8 ? S : 8; }
inline int gemv_batch(int S) {
  const int per = (S + gemv_waves(S) - 1) / gemv_waves(S);
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 8;
}

// Pair handled by workgroup row blockIdx.y; -1 if this workgroup has nothing to
// do.  With a miss record (subset_rec) the entries of pair_subset are split on
// the device: mode 1 takes the first rec[2] (the hits), mode 2 the rest, mode 3
// all of them and flags the rest as misses to stream from host memory, mode 4
// all of them from their slots; nothing runs unless rec[0] == MOE_OK.
__device__ __forceinline__ int pair_of_block(const int32_t* __restrict__ pair_subset,
                                             const int32_t* __restrict__ subset_rec, int subset_mode,
                                             bool& miss) {
  const int i = blockIdx.y;
  miss = false;
  if (subset_rec) {
    if (subset_rec[0] != MOE_OK) return -1;
    const int nh = subset_rec[2];
    if (subset_mode == 1 && i >= nh) return -1;
    if (subset_mode == 2 && i < nh) return -1;
    miss = subset_mode == 3 && i >= nh;  // mode 4: every entry, all from their slots
    return pair_subset ? pair_subset[i] : i;
  }
  return pair_subset ? pair_subset[i] : i;
}

// Gate and up rows 16g.. of one pair: steps w, w+nw, ... of S, in batches of NB
// with every load of a batch issued before its arithmetic.
// With fill != NULL (a streamed miss) the fragments read from blob are also
// written to the same places of fill.
template <int FMT, int NB>
__device__ __forceinline__ void gateup_partial(const uint8_t* __restrict__ blob, const BlobLayout& L,
                                               int S, int g, const uint16_t* xl, int w, int nw,
                                               int lane, float& ag, float& au, uint8_t* fill = nullptr) {
  const int q = lane >> 4;
  for (int s0 = w; s0 < S; s0 += NB * nw) {
    Frag<FMT> fg[NB], fu[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = s0 + i * nw;
      if (s < S) {
        const size_t f = (size_t)g * S + s;
        fg[i].load(blob + L.cg, blob + L.sg, f, lane);
        fu[i].load(blob + L.cu, blob + L.su, f, lane);
      }
    }
    if (fill) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int s = s0 + i * nw;
        if (s < S) {
          const size_t f = (size_t)g * S + s;
          fg[i].store(fill + L.cg, fill + L.sg, f, lane);
          fu[i].store(fill + L.cu, fill + L.su, f, lane);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = s0 + i * nw;
      if (s < S) {
        uint32_t xs[16];
        load_xslice(xl + kFragK * s + 32 * q, xs);
        ag += fg[i].dot(xs);
        au += fu[i].dot(xs);
      }
    }
  }
}

// Rows 16g.. of one matrix (down) for one pair over steps w, w+nw, ... of S in
// batches of NB.  The caller issues the first batch (load) before staging the
// pair's h row in LDS, so the weight latency overlaps the staging.
template <int FMT, int NB>
struct DownRows {
  Frag<FMT> fd[NB];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                       int S, int g, int s0, int nw, int lane) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (s0 + i * nw < S) fd[i].load(codes, scales, (size_t)g * S + s0 + i * nw, lane);
  }

  // Steps s0 .. s0+NB-1 (one wave per row group), with steps past the end
  // re-loading the last one: the loads are unconditional, so a later wait for
  // an older batch never waits for this one.
  __device__ __forceinline__ void load_clamped(const uint8_t* __restrict__ codes,
                                               const uint8_t* __restrict__ scales, int S, int g, int s0,
                                               int lane) {
#pragma unroll
    for (int i = 0; i < NB; ++i) fd[i].load(codes, scales, (size_t)g * S + min(s0 + i, S - 1), lane);
  }

  __device__ __forceinline__ void store(uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int S, int g,
                                        int s0, int nw, int lane) const {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (s0 + i * nw < S) fd[i].store(codes, scales, (size_t)g * S + s0 + i * nw, lane);
  }

  __device__ __forceinline__ float dot(const uint16_t* xrow, int S, int s0, int nw, int lane) const {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = s0 + i * nw;
      if (s < S) {
        uint32_t xs[16];
        load_xslice(xrow + kFragK * s + 32 * (lane >> 4), xs);
        a += fd[i].dot(xs);
      }
    }
    return a;
  }
};

// Gate/up + SwiGLU for rows 16*blockIdx.x.. of pair blockIdx.y (or pair_subset
// entry).  TOPK: the pair's expert comes from the softmax/top-k of `logits`,
// which one extra wave of every workgroup computes (identical everywhere);
// column group 0 of the token's first pair writes topk_idx / topk_w.  When the
// selection alone fixes the top-k set (no candidate beyond k), workgroup row j
// takes the set's j-th expert in index order and the other waves start its
// weight loads at once; the extra wave ranks the set meanwhile, and the h row
// goes to the expert's rank position, so hbuf and topk_idx agree as when
// ranked first.
template <int FMT, int NB, bool TOPK, int NV>
__global__ __launch_bounds__(TOPK ? 576 : 512) void k_gateup_gemv(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F, int E, int k,
    unsigned flags, const uint16_t* __restrict__ x, const float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, const int32_t* __restrict__ pair_slot,
    const int32_t* __restrict__ pair_subset, const int32_t* __restrict__ subset_rec, int subset_mode,
    const uint8_t* __restrict__ miss_src, uint16_t* __restrict__ hbuf) {
  __shared__ __attribute__((aligned(16))) uint16_t xl[kMaxDim];
  __shared__ float red[8][2][16];
  __shared__ int s_slot, s_row;
  __shared__ TopkScratch s_topk;
  // nw waves take the K steps; with TOPK wave nw runs the top-k
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x >> 6) - (TOPK ? 1 : 0);
  bool miss = false;
  const int q = TOPK ? (int)blockIdx.y : pair_of_block(pair_subset, subset_rec, subset_mode, miss);
  if (q < 0) return;
  const int t = q / k, j = q % k, g = blockIdx.x;
  const uint4* xs4 = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  // the logits are requested before the x staging waits on its loads, so the
  // two loads are in flight together
  float v[NV];
  if constexpr (TOPK)
    if (w == nw) wave_load_logits<NV>(logits + (size_t)t * E, E, v);
  for (int i = threadIdx.x; i < H / 8; i += blockDim.x) reinterpret_cast<uint4*>(xl)[i] = xs4[i];
  TopkSel<NV> sel;
  bool set_first = false;  // top-k wave: the set is known, its order comes later
  // order the selection, publish the outputs and the h row of expert `mine`
  const auto order = [&](int mine) {
    int idx;
    float wt;
    wave_topk_order<NV>(v, E, k, flags, sel, idx, wt, s_topk);
    const uint64_t at = __ballot(lane < k && idx == mine);
    if (lane == 0) s_row = t * k + __builtin_ctzll(at);
    if (g == 0 && j == 0 && lane < k) {
      topk_idx[(size_t)t * k + lane] = idx;
      topk_w[(size_t)t * k + lane] = wt;
    }
  };
  if constexpr (TOPK) {
    if (w == nw) {
      set_first = wave_topk_select<NV>(v, E, k, sel);
      if (set_first) {
        if (lane == 0) s_slot = topk_candidate<NV>(sel, j);
      } else {
        int idx;
        float wt;
        wave_topk_order<NV>(v, E, k, flags, sel, idx, wt, s_topk);
        if (lane == j) s_slot = idx;
        if (lane == 0) s_row = q;
        if (g == 0 && j == 0 && lane < k) {
          topk_idx[(size_t)t * k + lane] = idx;
          topk_w[(size_t)t * k + lane] = wt;
        }
      }
    }
  } else {
    if (threadIdx.x == 0) {
      s_slot = pair_slot ? pair_slot[q] : topk_idx[q];
      s_row = q;
    }
  }
  __syncthreads();
  // a streamed miss reads the expert's blob from host memory and fills its slot
  const uint8_t* blob = miss ? miss_src + (size_t)topk_idx[q] * stride : pool + (size_t)s_slot * stride;
  uint8_t* fill = miss ? const_cast<uint8_t*>(pool) + (size_t)s_slot * stride : nullptr;
  if (fill && g == 0 && threadIdx.x < 3)
    reinterpret_cast<float*>(fill + L.tau)[threadIdx.x] = reinterpret_cast<const float*>(blob + L.tau)[threadIdx.x];
  // NVFP4 tensor scales, requested with the weights so the epilogue does not wait for them
  float tau_g = 1.0f, tau_u = 1.0f;
  if constexpr (FMT == MOE_FMT_NVFP4) {
    tau_g = reinterpret_cast<const float*>(blob + L.tau)[0];
    tau_u = reinterpret_cast<const float*>(blob + L.tau)[1];
  }
  // the workgroups of a streamed miss also bring its down matrix (codes and
  // scales) into the slot, so the down kernel reads every pair from VRAM; the
  // first chunks of each thread are requested before the gate/up fragments,
  // so that their round trips over the link overlap
  constexpr int kEarly = 4;
  const size_t cdb = (size_t)H * F / (FMT == MOE_FMT_FP8_E4M3 ? 1 : 2);
  const size_t sdb = FMT == MOE_FMT_NVFP4 ? (size_t)H * F / 16 : FMT == MOE_FMT_MXFP4 ? (size_t)H * F / 32
                                                                                    : (size_t)H * (F / 128) * 4;
  const size_t nc = cdb / 16, ns = sdb / 16, step = (size_t)gridDim.x * blockDim.x;
  const size_t c0 = (size_t)g * blockDim.x + threadIdx.x;
  uint4 early[kEarly], early_s = make_uint4(0u, 0u, 0u, 0u);
  if (fill) {
#pragma unroll
    for (int i = 0; i < kEarly; ++i)
      if (c0 + i * step < nc) early[i] = reinterpret_cast<const uint4*>(blob + L.cd)[c0 + i * step];
    if (c0 < ns) early_s = reinterpret_cast<const uint4*>(blob + L.sd)[c0];
  }
  float ag = 0.0f, au = 0.0f;
  if (w < nw) {
    gateup_partial<FMT, NB>(blob, L, H / kFragK, g, xl, w, nw, lane, ag, au, fill);
  } else {
    if constexpr (TOPK)
      if (set_first) order(topk_candidate<NV>(sel, j));
  }
  if (fill) {
    const uint4* sc4 = reinterpret_cast<const uint4*>(blob + L.cd);
    uint4* dc4 = reinterpret_cast<uint4*>(fill + L.cd);
#pragma unroll
    for (int i = 0; i < kEarly; ++i)
      if (c0 + i * step < nc) dc4[c0 + i * step] = early[i];
    for (size_t c = c0 + kEarly * step; c < nc; c += step) dc4[c] = sc4[c];
    const uint4* ss4 = reinterpret_cast<const uint4*>(blob + L.sd);
    uint4* ds4 = reinterpret_cast<uint4*>(fill + L.sd);
    if (c0 < ns) ds4[c0] = early_s;
    for (size_t c = c0 + step; c < ns; c += step) ds4[c] = ss4[c];
  }
  ag = row_lanes_sum(ag);
  au = row_lanes_sum(au);
  if (w < nw && lane < 16) {
    red[w][0][lane] = ag;
    red[w][1][lane] = au;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float G = 0.0f, U = 0.0f;
    for (int i = 0; i < nw; ++i) {
      G += red[i][0][threadIdx.x];
      U += red[i][1][threadIdx.x];
    }
    if constexpr (FMT == MOE_FMT_NVFP4) {
      G *= tau_g;
      U *= tau_u;
    }
    hbuf[(size_t)s_row * F + kFragRows * g + threadIdx.x] = f32_to_bf16_rne(silu_f32(G) * U);
  }
}

// Decode gate/up for layers with more (pair, 16-row group) units than the
// chip holds workgroups at once.  A persistent workgroup owns `upw`
// consecutive units of one token (units ordered by pair, then row group);
// wave 0 computes the token's softmax/top-k once, then every wave streams its
// k-steps of all those units through a ring of NB prefetched items (one item
// = the gate and up fragments of one k-step): the next unit's weights are in
// flight while the current unit is dotted, and no barrier runs inside the
// stream.  Each unit's per-wave sums meet in LDS after the stream, in wave
// order, so the results equal those of k_gateup_gemv bit for bit.
constexpr int kStreamMaxUnits = 8;

template <int FMT, int NB, int NV>
__global__ __launch_bounds__(512) void k_gateup_topk_stream(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F, int E, int k, int T,
    unsigned flags, const uint16_t* __restrict__ x, const float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int upw, uint16_t* __restrict__ hbuf) {
  __shared__ __attribute__((aligned(16))) uint16_t xl[kMaxDim];
  __shared__ float red[kStreamMaxUnits][8][2][16];
  __shared__ int s_slot[16];
  __shared__ TopkScratch s_topk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int G = F / kFragRows, S = H / kFragK, per = (S + nw - 1) / nw;
  const int u0 = blockIdx.x * upw, nu = min(upw, T * k * G - u0);
  const int t = u0 / (k * G);  // upw divides k*G: all units of this workgroup belong to token t
  const uint4* xs4 = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  float v[NV];
  if (w == 0) wave_load_logits<NV>(logits + (size_t)t * E, E, v);
  for (int i = threadIdx.x; i < H / 8; i += blockDim.x) reinterpret_cast<uint4*>(xl)[i] = xs4[i];
  if (w == 0) {
    int idx;
    float wt;
    wave_topk_regs<NV>(v, E, k, flags, idx, wt, s_topk);
    if (lane < k) {
      s_slot[lane] = idx;
      if (u0 % (k * G) == 0) {
        topk_idx[(size_t)t * k + lane] = idx;
        topk_w[(size_t)t * k + lane] = wt;
      }
    }
  }
  __syncthreads();
  // NVFP4 tensor scales of the unit this thread finishes, requested before the stream
  float tau_g = 1.0f, tau_u = 1.0f;
  if constexpr (FMT == MOE_FMT_NVFP4) {
    if (threadIdx.x < 16 * nu) {
      const float* tp = reinterpret_cast<const float*>(pool + (size_t)s_slot[((u0 + (threadIdx.x >> 4)) / G) % k] * stride + L.tau);
      tau_g = tp[0];
      tau_u = tp[1];
    }
  }
  const int n_items = nu * per;
  // load cursor (unit, item within unit); items past the end re-load the last
  // one, so every load is unconditional
  int lu = 0, lj = 0;
  const auto load_item = [&](Frag<FMT>& fg, Frag<FMT>& fu) {
    const int cu = lu < nu ? lu : nu - 1, cj = lu < nu ? lj : per - 1;
    const int u = u0 + cu, g = u % G, pj = (u / G) % k;
    const uint8_t* blob = pool + (size_t)s_slot[pj] * stride;
    const size_t f = (size_t)g * S + min(w + nw * cj, S - 1);
    fg.load(blob + L.cg, blob + L.sg, f, lane);
    fu.load(blob + L.cu, blob + L.su, f, lane);
    if (++lj == per) {
      lj = 0;
      ++lu;
    }
  };
  Frag<FMT> fg[NB], fu[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) load_item(fg[r], fu[r]);
  float ag = 0.0f, au = 0.0f;
  int cu = 0, cj = 0;  // compute cursor
  for (int i0 = 0; i0 < n_items; i0 += NB) {
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      if (i0 + r < n_items) {
        const int st = w + nw * cj;
        if (st < S) {
          uint32_t xs[16];
          load_xslice(xl + kFragK * st + 32 * (lane >> 4), xs);
          ag += fg[r].dot(xs);
          au += fu[r].dot(xs);
        }
        if (cj == per - 1) {  // this wave's last step of unit cu
          ag = row_lanes_sum(ag);
          au = row_lanes_sum(au);
          if (lane < 16) {
            red[cu][w][0][lane] = ag;
            red[cu][w][1][lane] = au;
          }
          ag = 0.0f;
          au = 0.0f;
          cj = 0;
          ++cu;
        } else {
          ++cj;
        }
      }
      load_item(fg[r], fu[r]);
    }
  }
  __syncthreads();
  if (threadIdx.x < 16 * nu) {
    const int ul = threadIdx.x >> 4, row = threadIdx.x & 15;
    const int u = u0 + ul, g = u % G, q = u / G;
    float Gs = 0.0f, Us = 0.0f;
    for (int i = 0; i < nw; ++i) {
      Gs += red[ul][i][0][row];
      Us += red[ul][i][1][row];
    }
    if constexpr (FMT == MOE_FMT_NVFP4) {
      Gs *= tau_g;
      Us *= tau_u;
    }
    hbuf[(size_t)q * F + kFragRows * g + row] = f32_to_bf16_rne(silu_f32(Gs) * Us);
  }
}

// y rows 16*blockIdx.x.. of pair blockIdx.y (or pair_subset entry).
template <int FMT, int NB>
__global__ __launch_bounds__(512) void k_down_gemv(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F, int k,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ pair_slot,
    const int32_t* __restrict__ pair_subset, const int32_t* __restrict__ subset_rec, int subset_mode,
    const uint8_t* __restrict__ miss_src, const uint16_t* __restrict__ hbuf, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t hl[kMaxDim];
  __shared__ float red[8][16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  bool miss = false;
  const int q = pair_of_block(pair_subset, subset_rec, subset_mode, miss);
  if (q < 0) return;
  const int slot = pair_slot ? pair_slot[q] : topk_idx[q];
  const uint8_t* blob = miss ? miss_src + (size_t)topk_idx[q] * stride : pool + (size_t)slot * stride;
  uint8_t* fill = miss ? const_cast<uint8_t*>(pool) + (size_t)slot * stride : nullptr;
  const int g = blockIdx.x;
  const int S = F / kFragK;
  DownRows<FMT, NB> d;
  d.load(blob + L.cd, blob + L.sd, S, g, w, nw, lane);
  const float tau_d = FMT == MOE_FMT_NVFP4 ? reinterpret_cast<const float*>(blob + L.tau)[2] : 1.0f;
  const uint4* h4 = reinterpret_cast<const uint4*>(hbuf + (size_t)q * F);
  for (int i = threadIdx.x; i < F / 8; i += blockDim.x) reinterpret_cast<uint4*>(hl)[i] = h4[i];
  __syncthreads();
  if (fill) d.store(fill + L.cd, fill + L.sd, S, g, w, nw, lane);
  float a = d.dot(hl, S, w, nw, lane);
  for (int s0 = w + NB * nw; s0 < S; s0 += NB * nw) {
    d.load(blob + L.cd, blob + L.sd, S, g, s0, nw, lane);
    if (fill) d.store(fill + L.cd, fill + L.sd, S, g, s0, nw, lane);
    a += d.dot(hl, S, s0, nw, lane);
  }
  a = row_lanes_sum(a);
  if (lane < 16) red[w][lane] = a;
  __syncthreads();
  if (threadIdx.x < 16) {
    float v = 0.0f;
    for (int i = 0; i < nw; ++i) v += red[i][threadIdx.x];
    if constexpr (FMT == MOE_FMT_NVFP4) v *= tau_d;
    y[(size_t)q * H + kFragRows * g + threadIdx.x] = v;
  }
}

// Down for all k pairs of token blockIdx.y (wave j = pair j) on rows
// 16*blockIdx.x.., with the gate-weighted combine fused:
// out[t] = bf16(sum_j w_j * y_j) accumulated in fp32 in j order.
// Dynamic LDS: k rows of h (F bf16 each).  Workgroups past the H/16 row groups
// (token 0 only) read an equal share of `warm` and discard it, so that a later
// kernel finds those bytes in the memory-side cache.
template <int FMT, int NB>
__global__ __launch_bounds__(1024) void k_down_combine_gemv(
    const uint8_t* __restrict__ pool, size_t stride, BlobLayout L, int H, int F, int k,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ pair_slot,
    const uint16_t* __restrict__ hbuf, const float* __restrict__ topk_w, float* __restrict__ y,
    uint16_t* __restrict__ out, const int32_t* __restrict__ rec, const uint8_t* __restrict__ warm,
    size_t warm_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hl_dyn[];
  if ((int)blockIdx.x >= H / kFragRows) {
    if (blockIdx.y != 0) return;
    const int nb = gridDim.x - H / kFragRows, b = blockIdx.x - H / kFragRows;
    const size_t n16 = warm_bytes / 16, per = (n16 + nb - 1) / nb, i0 = (size_t)b * per;
    const size_t i1 = min(n16, i0 + per);
    const uint4* p4 = reinterpret_cast<const uint4*>(warm);
    uint32_t acc = 0;
    for (size_t i = i0 + threadIdx.x; i < i1; i += 4 * blockDim.x) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t iu = i + (size_t)u * blockDim.x;
        v[u] = iu < i1 ? p4[iu] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].w;
    }
    if (H == 0 && acc == 1u) out[0] = 0;  // never (H > 0): keeps the loads
    return;
  }
  if (rec && rec[0] != MOE_OK) return;  // cache capacity error: the pairs did not run
  __shared__ float ys[16][16], ws[16];
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int t = blockIdx.y, q = t * k + j, g = blockIdx.x;
  const int slot = pair_slot ? pair_slot[q] : topk_idx[q];
  const uint8_t* blob = pool + (size_t)slot * stride;
  // the pair's mixing weight and NVFP4 down scale, requested with the weights
  // so that the combine does not wait for them
  const float wq = topk_w[q];
  const float tau_d = FMT == MOE_FMT_NVFP4 ? reinterpret_cast<const float*>(blob + L.tau)[2] : 1.0f;
  uint16_t* hl = hl_dyn + (size_t)j * F;
  const int S = F / kFragK;
  // batches of NB steps through two register sets: batch b+2 is requested as
  // soon as batch b is consumed, so one batch is always in flight
  const int nb = (S + NB - 1) / NB;
  DownRows<FMT, NB> d0, d1;
  d0.load_clamped(blob + L.cd, blob + L.sd, S, g, 0, lane);
  if (nb > 1) d1.load_clamped(blob + L.cd, blob + L.sd, S, g, NB, lane);
  const uint4* h4 = reinterpret_cast<const uint4*>(hbuf + (size_t)q * F);
  for (int i = lane; i < F / 8; i += 64) reinterpret_cast<uint4*>(hl)[i] = h4[i];
  if (lane == 0) ws[j] = wq;
  __syncthreads();
  float a = 0.0f;
  int b = 0;
  for (; b + 2 < nb; b += 2) {
    a += d0.dot(hl, S, b * NB, 1, lane);
    d0.load_clamped(blob + L.cd, blob + L.sd, S, g, (b + 2) * NB, lane);
    a += d1.dot(hl, S, (b + 1) * NB, 1, lane);
    d1.load_clamped(blob + L.cd, blob + L.sd, S, g, (b + 3) * NB, lane);
  }
  a += d0.dot(hl, S, b * NB, 1, lane);
  if (b + 1 < nb) a += d1.dot(hl, S, (b + 1) * NB, 1, lane);
  a = row_lanes_sum(a);
  if (lane < 16) {
    if constexpr (FMT == MOE_FMT_NVFP4) a *= tau_d;
    ys[j][lane] = a;
    if (y) y[(size_t)q * H + kFragRows * g + lane] = a;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float acc = 0.0f;
    for (int jj = 0; jj < k; ++jj) acc = fmaf(ws[jj], ys[jj][threadIdx.x], acc);
    out[(size_t)t * H + kFragRows * g + threadIdx.x] = f32_to_bf16_rne(acc);
  }
}

// Compute units of the current device (one device model per process).
int compute_units() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      n = cu;
  }
  return n;
}

template <int FMT, bool TOPK, int NV>
hipError_t launch_gateup_t(const FfnArgs& a, const float* logits, unsigned flags, int32_t* idx, float* w,
                           hipStream_t s) {
  const int S = a.H / kFragK, nw = gemv_waves(S);
  dim3 grid(a.F / kFragRows, TOPK ? a.T * a.k : a.n_pairs), block(64 * (nw + (TOPK ? 1 : 0)));
  // the top-k wave lowers the register budget: FP8 batches of 8 would spill
  constexpr int kNB8 = TOPK && FMT == MOE_FMT_FP8_E4M3 ? 4 : 8;
#define L(CASE, NB)                                                                                    \
  case CASE:                                                                                           \
    hipLaunchKernelGGL((k_gateup_gemv<FMT, NB, TOPK, NV>), grid, block, 0, s, a.pool, a.stride, a.L, \
                       a.H, a.F, a.E, a.k, flags, a.x, logits, TOPK ? idx : const_cast<int32_t*>(a.topk_idx), \
                       w, a.pair_slot, a.pair_subset, a.subset_rec, a.subset_mode, a.miss_src, a.hbuf); \
    break;
  switch (gemv_batch(S)) {
    L(1, 1) L(2, 2) L(4, 4) L(8, kNB8)
    default: return hipErrorInvalidValue;
  }
#undef L
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gateup(const FfnArgs& a, hipStream_t s) {
  return launch_gateup_t<FMT, false, 1>(a, nullptr, 0, nullptr, nullptr, s);
}

// Workgroups of k_gateup_topk_stream<FMT, NB, NV> the current device holds at once.
template <int FMT, int NB, int NV>
int stream_capacity(int block) {
  static int cap = 0;  // per process: one device model
  if (cap == 0) {
    int dev = 0, n_cu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&k_gateup_topk_stream<FMT, NB, NV>), block, 0) != hipSuccess)
      return 0;
    cap = n_cu * per_cu;
  }
  return cap;
}

// Decode gate/up with in-block top-k: one unit (pair, 16-row group) per
// workgroup when the chip holds them all at once, else the streaming kernel
// with `upw` units per workgroup (a power of two <= 8, so it divides k*G).
template <int FMT, int NV>
hipError_t launch_gateup_topk_nv(const FfnArgs& a, const float* logits, unsigned flags, int32_t* idx, float* w,
                                 hipStream_t s) {
  constexpr int NB = 2;  // ring depth: the fastest of 1, 2, 3, 4 and 8 measured at hidden 6144
  const int S = a.H / kFragK, nw = gemv_waves(S), G = a.F / kFragRows;
  const int n_units = a.T * a.k * G;
  const int cap = stream_capacity<FMT, NB, NV>(64 * nw);
  const int old_cap = 256;  // k_gateup_gemv with one 8-wave workgroup per compute unit
  if (n_units <= old_cap || cap <= 0) return launch_gateup_t<FMT, true, NV>(a, logits, flags, idx, w, s);
  int upw = 1;
  while (upw < kStreamMaxUnits && (n_units + upw - 1) / upw > cap) upw *= 2;
  hipLaunchKernelGGL((k_gateup_topk_stream<FMT, NB, NV>), dim3((n_units + upw - 1) / upw), dim3(64 * nw), 0, s,
                     a.pool, a.stride, a.L, a.H, a.F, a.E, a.k, a.T, flags, a.x, logits, idx, w, upw, a.hbuf);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gateup_topk(const FfnArgs& a, const float* logits, unsigned flags, int32_t* idx, float* w,
                              hipStream_t s) {
  if (a.E <= 64) return launch_gateup_topk_nv<FMT, 1>(a, logits, flags, idx, w, s);
  if (a.E <= 256) return launch_gateup_topk_nv<FMT, 4>(a, logits, flags, idx, w, s);
  return launch_gateup_topk_nv<FMT, 16>(a, logits, flags, idx, w, s);
}

template <int FMT>
hipError_t launch_down(const FfnArgs& a, hipStream_t s) {
  const int S = a.F / kFragK;
#define LC(NB)                                                                                         \
  case NB:                                                                                             \
    hipLaunchKernelGGL((k_down_combine_gemv<FMT, NB>), grid, dim3(64 * a.k), lds, s, a.pool, a.stride, a.L, \
                       a.H, a.F, a.k, a.topk_idx, a.pair_slot, a.hbuf, a.topk_w, a.y, a.out, a.subset_rec, \
                       a.warm, a.warm_bytes);                                                         \
    break;
#define LD(NB)                                                                                         \
  case NB:                                                                                             \
    hipLaunchKernelGGL((k_down_gemv<FMT, NB>), grid, dim3(64 * nw), 0, s, a.pool, a.stride, a.L, a.H, \
                       a.F, a.k, a.topk_idx, a.pair_slot, a.pair_subset, a.subset_rec, a.subset_mode, \
                       a.miss_src, a.hbuf, y);                                                         \
    break;
  const size_t lds = (size_t)a.k * a.F * 2;
  // fused down + combine: all pairs of each token (a miss record only guards it, mode 4)
  if (a.out && a.k <= 16 && lds <= 64 * 1024 && !a.pair_subset && (!a.subset_rec || a.subset_mode == 4)) {
    // warming workgroups: the compute units the row groups leave idle, at least 64
    const int n_warm = a.warm && a.warm_bytes >= 16 ? max(64, compute_units() - a.H / kFragRows) : 0;
    dim3 grid(a.H / kFragRows + n_warm, a.T);
    switch (S <= 1 ? 1 : S <= 2 ? 2 : 4) {  // one wave per pair: batches of <= 4 steps
      LC(1) LC(2) LC(4)
      default: return hipErrorInvalidValue;
    }
  } else {
    // plain down into y; with `out`, the combine follows as its own kernel
    float* y = a.y ? a.y : (a.out ? a.ybuf : nullptr);
    if (!y) return hipErrorInvalidValue;
    const int nw = gemv_waves(S);
    dim3 grid(a.H / kFragRows, a.n_pairs);
    switch (gemv_batch(S)) {
      LD(1) LD(2) LD(4) LD(8)
      default: return hipErrorInvalidValue;
    }
    if (a.out) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return a.subset_rec ? launch_combine_rec(y, a.topk_w, a.T, a.H, a.k, a.out, a.subset_rec, s)
                          : launch_combine(y, a.topk_w, a.T, a.H, a.k, a.out, s);
    }
  }
#undef LC
#undef LD
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t s) {
  if (a.n_pairs == 0) return hipSuccess;
  if (a.H > kMaxDim || a.H % kFragK || a.F % kFragK) return hipErrorInvalidValue;
  hipError_t e;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: e = launch_gateup<MOE_FMT_NVFP4>(a, s); break;
    case MOE_FMT_MXFP4: e = launch_gateup<MOE_FMT_MXFP4>(a, s); break;
    default: e = launch_gateup<MOE_FMT_FP8_E4M3>(a, s); break;
  }
  if (e != hipSuccess) return e;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: return launch_down<MOE_FMT_NVFP4>(a, s);
    case MOE_FMT_MXFP4: return launch_down<MOE_FMT_MXFP4>(a, s);
    default: return launch_down<MOE_FMT_FP8_E4M3>(a, s);
  }
}

hipError_t launch_ffn_gemv_split(const FfnArgs& a0, int gateup_mode, int down_mode, hipStream_t s) {
  FfnArgs a = a0;
  a.subset_mode = gateup_mode;
  if (a.n_pairs == 0) return hipSuccess;
  if (a.H > kMaxDim || a.H % kFragK || a.F % kFragK) return hipErrorInvalidValue;
  hipError_t e;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: e = launch_gateup<MOE_FMT_NVFP4>(a, s); break;
    case MOE_FMT_MXFP4: e = launch_gateup<MOE_FMT_MXFP4>(a, s); break;
    default: e = launch_gateup<MOE_FMT_FP8_E4M3>(a, s); break;
  }
  if (e != hipSuccess) return e;
  a.subset_mode = down_mode;
  if (down_mode == 4 && a.out) a.pair_subset = nullptr;  // every pair from its slot, combine fused
  switch (a.fmt) {
    case MOE_FMT_NVFP4: return launch_down<MOE_FMT_NVFP4>(a, s);
    case MOE_FMT_MXFP4: return launch_down<MOE_FMT_MXFP4>(a, s);
    default: return launch_down<MOE_FMT_FP8_E4M3>(a, s);
  }
}

hipError_t launch_decode_layer(const FfnArgs& a0, const float* logits, unsigned route_flags,
                               int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (a0.T == 0) return hipSuccess;
  if (a0.H > kMaxDim || a0.H % kFragK || a0.F % kFragK) return hipErrorInvalidValue;
  hipError_t e;
  switch (a0.fmt) {
    case MOE_FMT_NVFP4: e = launch_gateup_topk<MOE_FMT_NVFP4>(a0, logits, route_flags, topk_idx, topk_w, s); break;
    case MOE_FMT_MXFP4: e = launch_gateup_topk<MOE_FMT_MXFP4>(a0, logits, route_flags, topk_idx, topk_w, s); break;
    default: e = launch_gateup_topk<MOE_FMT_FP8_E4M3>(a0, logits, route_flags, topk_idx, topk_w, s); break;
  }
  if (e != hipSuccess) return e;
  FfnArgs a = a0;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.pair_slot = nullptr;
  a.pair_subset = nullptr;
  a.n_pairs = a.T * a.k;
  switch (a.fmt) {
    case MOE_FMT_NVFP4: return launch_down<MOE_FMT_NVFP4>(a, s);
    case MOE_FMT_MXFP4: return launch_down<MOE_FMT_MXFP4>(a, s);
    default: return launch_down<MOE_FMT_FP8_E4M3>(a, s);
  }
}
