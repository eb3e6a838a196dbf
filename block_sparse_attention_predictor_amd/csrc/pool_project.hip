// Tile mean-pooling of Q and K fused with the per-head predictor projection.
//
// Affine launch article, "Training the Selector, Not the Generator": the
// selector consists of query and key projections trained per layer ("How the
// SN120 Competition Works" gives one tensor per layer and projection).  Each
// projection is applied here to the mean of the token rows of one tile:
//     x_hat[b, h, t, :] = W[h] (1/|tile t|) sum_{n in tile t} X[b, n, h, :]
//
// HBM-bound: every Q row of the query segment and every K row of the key
// segments is read exactly once (2 * H * d bytes per token).  One workgroup
// owns four tiles of one kind and a group of 8 heads; for each tile its 256
// threads stream the rows with 16-byte loads (d/8 lanes per head row, 8 heads side
// by side, so a wave reads whole contiguous head rows; eight rows in flight per
// thread), sum in fp32 registers, combine the row-parallel partial sums through
// LDS and divide by the number of real tokens.  Then W[h] (bf16 or f16, read
// through L2 once for the four tiles, converted exactly) is applied with fp32 dot
// products.
#include "common.h"

namespace veda {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadsPerGroup = 8;
constexpr int kThreads = 256;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// predictor weights: the low / high 16-bit element of a word as fp32 (both exact)
template <bool F16>
__device__ __forceinline__ float wlo(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  else return bf16lo(w);
}
template <bool F16>
__device__ __forceinline__ float whi(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else return bf16hi(w);
}

// Tiles of one kind (query or key) per workgroup: each W row is read once for all of them.
constexpr int kTilesPerGroup = 4;

template <int D, bool F16>
__global__ __launch_bounds__(kThreads) void pool_project_kernel(
    LayerDev L, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk, float* __restrict__ q_hat,
    float* __restrict__ k_hat) {
  constexpr int TPR = D / 8;                               // lanes per head row
  constexpr int RP = kThreads / (kHeadsPerGroup * TPR);    // token rows in flight per step
  __shared__ float red[RP][kHeadsPerGroup * D];
  __shared__ float means[kTilesPerGroup][kHeadsPerGroup * D];

  const int qgroups = (L.Tq + kTilesPerGroup - 1) / kTilesPerGroup;
  const bool is_q = (int)blockIdx.x < qgroups;
  const int first = (is_q ? (int)blockIdx.x : (int)blockIdx.x - qgroups) * kTilesPerGroup;
  const int total = is_q ? L.Tq : L.Tk;
  const int ntiles = min(kTilesPerGroup, total - first);
  const uint16_t* const x = is_q ? q : k;
  const uint16_t* const W = is_q ? wq : wk;
  float* const out = is_q ? q_hat : k_hat;
  const int h0 = blockIdx.y * kHeadsPerGroup;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int hl = (tid / TPR) % kHeadsPerGroup;
  const int r0 = tid / (TPR * kHeadsPerGroup);
  const int c = (tid % TPR) * 8;
  const int h = h0 + hl;
  const bool hv = h < L.H;

  for (int tt = 0; tt < ntiles; ++tt) {
    const int j = first + tt;                   // tile index within q_hat or k_hat
    int64_t start, len;
    if (is_q) {
      start = L.q0 + (int64_t)j * L.tile;
      len = min((int64_t)L.tile, L.qlen - (int64_t)j * L.tile);
    } else {
      int s = 0;
#pragma unroll
      for (int t = 1; t < kMaxSeg; ++t)
        if (t < L.n_seg && j >= L.seg[t].toff) s = t;
      const int tl = j - L.seg[s].toff;
      start = L.seg[s].start + (int64_t)tl * L.tile;
      len = min((int64_t)L.tile, L.seg[s].len - (int64_t)tl * L.tile);
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (hv) {
      const uint16_t* base = x + (int64_t)b * L.sb + start * L.sn + (int64_t)h * L.sh + c;
      int64_t r = r0;
      // eight rows in flight per thread
      for (; r + 7 * RP < len; r += 8 * RP) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (r + u * RP) * L.sn));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc[0] += bf16lo(v[u].x); acc[1] += bf16hi(v[u].x);
          acc[2] += bf16lo(v[u].y); acc[3] += bf16hi(v[u].y);
          acc[4] += bf16lo(v[u].z); acc[5] += bf16hi(v[u].z);
          acc[6] += bf16lo(v[u].w); acc[7] += bf16hi(v[u].w);
        }
      }
      for (; r < len; r += RP) {
        u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + r * L.sn));
        acc[0] += bf16lo(v.x); acc[1] += bf16hi(v.x);
        acc[2] += bf16lo(v.y); acc[3] += bf16hi(v.y);
        acc[4] += bf16lo(v.z); acc[5] += bf16hi(v.z);
        acc[6] += bf16lo(v.w); acc[7] += bf16hi(v.w);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[r0][hl * D + c + e] = acc[e];
    __syncthreads();
    // combine the row-parallel partial sums; mean over the real tokens
    const float inv_len = 1.0f / (float)len;
    for (int i = tid; i < kHeadsPerGroup * D; i += kThreads) {
      float s = 0.f;
#pragma unroll
      for (int rr = 0; rr < RP; ++rr) s += red[rr][i];
      means[tt][i] = s * inv_len;
    }
    __syncthreads();
  }
  // the last workgroup of a kind may have fewer tiles: their slots hold zeros
  if (ntiles < kTilesPerGroup) {
    float* const spare = &means[0][0] + ntiles * kHeadsPerGroup * D;
    for (int i = tid; i < (kTilesPerGroup - ntiles) * kHeadsPerGroup * D; i += kThreads) spare[i] = 0.f;
    __syncthreads();
  }

  // projection: x_hat[h, o] = sum_c W[h, o, c] * mean[h, c], each W row read once for the tiles
  const int P = L.p;
  for (int o = tid; o < kHeadsPerGroup * P; o += kThreads) {
    const int ohl = o / P;
    const int oc = o - ohl * P;
    const int oh = h0 + ohl;
    if (oh >= L.H) continue;
    const uint4* wrow = reinterpret_cast<const uint4*>(W + ((int64_t)oh * P + oc) * D);
    float s0[kTilesPerGroup], s1[kTilesPerGroup];
#pragma unroll
    for (int tt = 0; tt < kTilesPerGroup; ++tt) s0[tt] = s1[tt] = 0.f;
#pragma unroll 2
    for (int cc = 0; cc < D / 8; ++cc) {
      const uint4 w = wrow[cc];
#pragma unroll
      for (int tt = 0; tt < kTilesPerGroup; ++tt) {
        const float* mm = &means[tt][ohl * D + cc * 8];
        s0[tt] = fmaf(wlo<F16>(w.x), mm[0], s0[tt]); s1[tt] = fmaf(whi<F16>(w.x), mm[1], s1[tt]);
        s0[tt] = fmaf(wlo<F16>(w.y), mm[2], s0[tt]); s1[tt] = fmaf(whi<F16>(w.y), mm[3], s1[tt]);
        s0[tt] = fmaf(wlo<F16>(w.z), mm[4], s0[tt]); s1[tt] = fmaf(whi<F16>(w.z), mm[5], s1[tt]);
        s0[tt] = fmaf(wlo<F16>(w.w), mm[6], s0[tt]); s1[tt] = fmaf(whi<F16>(w.w), mm[7], s1[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < kTilesPerGroup; ++tt)
      if (tt < ntiles) out[(((int64_t)b * L.H + oh) * total + first + tt) * P + oc] = s0[tt] + s1[tt];
  }
}

}  // namespace

hipError_t launch_pool_project(const LayerDev& L, const void* q, const void* k, const void* wq,
                               const void* wk, float* q_hat, float* k_hat, hipStream_t s) {
  dim3 grid((unsigned)((L.Tq + kTilesPerGroup - 1) / kTilesPerGroup + (L.Tk + kTilesPerGroup - 1) / kTilesPerGroup),
            (unsigned)((L.H + kHeadsPerGroup - 1) / kHeadsPerGroup), (unsigned)L.B);
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto wqq = static_cast<const uint16_t*>(wq);
  auto wkk = static_cast<const uint16_t*>(wk);
  const bool f16 = L.wdtype == 1;
  if (L.d == 128 && f16)
    hipLaunchKernelGGL((pool_project_kernel<128, true>), grid, dim3(kThreads), 0, s, L, qq, kk, wqq,
                       wkk, q_hat, k_hat);
  else if (L.d == 128)
    hipLaunchKernelGGL((pool_project_kernel<128, false>), grid, dim3(kThreads), 0, s, L, qq, kk, wqq,
                       wkk, q_hat, k_hat);
  else if (f16)
    hipLaunchKernelGGL((pool_project_kernel<64, true>), grid, dim3(kThreads), 0, s, L, qq, kk, wqq,
                       wkk, q_hat, k_hat);
  else
    hipLaunchKernelGGL((pool_project_kernel<64, false>), grid, dim3(kThreads), 0, s, L, qq, kk, wqq,
                       wkk, q_hat, k_hat);
  return hipGetLastError();
}

}  // namespace veda
