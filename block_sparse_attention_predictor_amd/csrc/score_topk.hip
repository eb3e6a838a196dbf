// Pooled-score GEMM fused with the per-row, per-segment top-k selection.
//
// Veda R2VA record, first paragraph: a fixed budget of key tiles is kept per
// query tile and head, and the reference and current-video segments are chosen
// independently.  The score of a (query tile i, key tile j) pair is the plain
// dot product <q_hat_i, k_hat_j> of the projected pooled vectors; ties go to
// the lower tile index and the chosen ids are written ascending.
//
// One workgroup (4 waves) owns R consecutive query-tile rows of one (b, h):
//  1. S[R x Tk] on bf16 matrix cores: each fp32 operand x is split into
//     hi = bf16(x) and lo = bf16(x - hi); S = hi*hi + hi*lo + lo*hi (the lo*lo
//     term is below 2^-16 relative).  v_mfma_f32_16x16x32_bf16 blocks of 16 key
//     tiles are spread over the waves; the scores land in LDS as order-preserving
//     uint32 keys (and optionally in HBM as fp32).
//  2. Each (row, segment) pair is reduced by one wave: a most-significant-digit
//     radix select (four 8-bit passes, histograms in LDS, one wave-wide scan per
//     pass) finds the k-th largest key exactly and how many keys equal to it are
//     kept; one ordered pass with wave ballots then writes every key above the
//     threshold and the first of the equal ones, which yields the lowest-index
//     tie-break and an ascending list without sorting.
#include "common.h"

namespace veda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsScoreBudget = 128 * 1024;   // bytes of LDS for the score block

// float -> uint32 whose unsigned order is the float order; -0 maps like +0
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const __bf16 h = (__bf16)x[t];
    hi[t] = h;
    lo[t] = (__bf16)(x[t] - (float)h);
  }
}

__device__ __forceinline__ int prefix_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ __launch_bounds__(kThreads) void score_topk_kernel(LayerDev L, int R,
                                                              const float* __restrict__ q_hat,
                                                              const float* __restrict__ k_hat,
                                                              int32_t* __restrict__ idx,
                                                              float* __restrict__ scores) {
  extern __shared__ uint32_t smem[];
  const int Tk = L.Tk;
  uint32_t* keys = smem;                       // [R][Tk]
  uint32_t* hist_all = smem + (size_t)R * Tk;  // [kWaves][256]

  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int nrows = min(R, L.Tq - row0);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int P = L.p;
  const int64_t bh = (int64_t)b * L.H + h;

  // ---- 1. scores ------------------------------------------------------------------
  {
    // A operand (query rows): lane holds row (lane % 16), k = 8*(lane/16) .. +7 per 32-step
    const int arow = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int ksteps = (P + 31) / 32;
    const float* qrow = q_hat + (bh * L.Tq + row0 + arow) * P;
    const bool arow_ok = arow < nrows;
    for (int cb = wave; cb * 16 < Tk; cb += kWaves) {
      const int kcol = cb * 16 + (lane & 15);
      const bool kcol_ok = kcol < Tk;
      const float* krow = k_hat + (bh * Tk + kcol) * P;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < ksteps; ++ks) {
        const int c0 = ks * 32 + kq;
        float xa[8], xb[8];
        const bool in_p = c0 < P;   // P is a multiple of 16 and kq a multiple of 8
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          xa[t] = (arow_ok && in_p) ? qrow[c0 + t] : 0.f;
          xb[t] = (kcol_ok && in_p) ? krow[c0 + t] : 0.f;
        }
        bf16x8 ah, al, bh8, bl8;
        split8(xa, ah, al);
        split8(xb, bh8, bl8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh8, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl8, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh8, acc, 0, 0, 0);
      }
      // C layout: lane holds column (lane % 16), rows 4*(lane/16) + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = (lane >> 4) * 4 + j;
        if (r < nrows && kcol_ok) {
          keys[r * Tk + kcol] = order_key(acc[j]);
          if (scores) scores[(bh * L.Tq + row0 + r) * Tk + kcol] = acc[j];
        }
      }
    }
  }
  __syncthreads();

  // ---- 2. top-k per (row, segment), one wave each ------------------------------------
  uint32_t* hist = hist_all + wave * 256;
  for (int item = wave; item < nrows * L.n_seg; item += kWaves) {
    const int r = item / L.n_seg;
    const int s = item - r * L.n_seg;
    const SegDev sg = L.seg[s];
    const int T = sg.T;
    const int K = sg.K;
    const uint32_t* row = keys + r * Tk + sg.toff;
    int32_t* out = idx + (bh * L.Tq + row0 + r) * L.Ktot + sg.koff;
    if (K == 0) continue;
    if (K == T) {
      for (int j = lane; j < T; j += 64) out[j] = j;
      continue;
    }
    // radix select of the K-th largest key
    uint32_t prefix = 0, pmask = 0;
    int remaining = K;   // how many still to take from the elements matching `prefix`
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int t = 0; t < 4; ++t) hist[lane * 4 + t] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < T; j += 64) {
        const uint32_t key = row[j];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFFu], 1u);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane i owns digits 255-4i .. 252-4i (descending); inclusive scan of counts
      uint32_t c[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) c[t] = hist[255 - (lane * 4 + t)];
      const uint32_t local = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      const uint32_t excl = incl - local;
      // the lane whose range crosses `remaining`
      const bool mine = excl < (uint32_t)remaining && (uint32_t)remaining <= incl;
      const uint64_t bal = __ballot(mine);
      const int owner = bal ? __builtin_ctzll(bal) : 0;
      uint32_t digit = 0, above = 0;
      if (lane == owner) {
        uint32_t acc_above = excl;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (acc_above + c[t] >= (uint32_t)remaining) {
            digit = 255 - (lane * 4 + t);
            break;
          }
          acc_above += c[t];
        }
        above = acc_above;
      }
      digit = __shfl(digit, owner, 64);
      above = __shfl(above, owner, 64);
      remaining -= (int)above;
      prefix |= digit << shift;
      pmask |= 0xFFu << shift;
      __builtin_amdgcn_wave_barrier();
    }
    // prefix is now the K-th largest key; keep all keys above it and the first
    // `remaining` keys equal to it, in ascending tile order
    const uint32_t thr = prefix;
    int taken = 0, eq_seen = 0;
    for (int base = 0; base < T && taken < K; base += 64) {
      const int j = base + lane;
      const uint32_t key = j < T ? row[j] : 0u;
      const bool gt = j < T && key > thr;
      const bool eq = j < T && key == thr;
      const uint64_t beq = __ballot(eq);
      const int eq_rank = eq_seen + prefix_below(beq);
      const bool take = gt || (eq && eq_rank < remaining);
      const uint64_t bt = __ballot(take);
      const int pos = taken + prefix_below(bt);
      if (take && pos < K) out[pos] = j;
      taken += __popcll(bt);
      eq_seen += __popcll(beq);
    }
  }
}

}  // namespace

int score_rows_per_block(int Tk) {
  int r = kLdsScoreBudget / (Tk * 4);
  if (r > 16) r = 16;
  if (r < 1) r = 1;
  return r;
}

hipError_t launch_score_topk(const LayerDev& L, const float* q_hat, const float* k_hat,
                             int32_t* idx, float* scores, hipStream_t s) {
  const int R = score_rows_per_block(L.Tk);
  const size_t lds = (size_t)R * L.Tk * 4 + kWaves * 256 * 4;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)score_topk_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)((L.Tq + R - 1) / R), (unsigned)L.H, (unsigned)L.B);
  hipLaunchKernelGGL(score_topk_kernel, grid, dim3(kThreads), lds, s, L, R, q_hat, k_hat, idx,
                     scores);
  return hipGetLastError();
}

}  // namespace veda
