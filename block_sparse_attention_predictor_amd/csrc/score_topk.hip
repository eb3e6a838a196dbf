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
constexpr int kHistCopies = 4;                 // radix histograms per wave

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

template <int kMaxKSteps>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(LayerDev L, int R,
                                                              const float* __restrict__ q_hat,
                                                              const float* __restrict__ k_hat,
                                                              int32_t* __restrict__ idx,
                                                              float* __restrict__ scores) {
  extern __shared__ uint32_t smem[];
  const int Tk = L.Tk;
  uint32_t* keys = smem;                       // [R][Tk]
  uint32_t* hist_all = smem + (size_t)R * Tk;  // [kWaves][kHistCopies][256]

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
    // A operand (query rows): lane holds row (lane % 16), k = 8*(lane/16) .. +7 of each
    // 32-wide step; split into hi/lo once.  B operand (key tiles): 16-byte loads of
    // k_hat, prefetched one column block ahead, split per block.
    const int arow = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int ksteps = (P + 31) / 32;
    const float* __restrict__ qrow = q_hat + (bh * L.Tq + row0 + arow) * P;
    const bool arow_ok = arow < nrows;
    bf16x8 ah[kMaxKSteps], al[kMaxKSteps];
#pragma unroll
    for (int ks = 0; ks < kMaxKSteps; ++ks) {
      float xa[8];
      const int c0 = ks * 32 + kq;
      const bool ok = ks < ksteps && arow_ok && c0 < P;
      const float4 lo4 = ok ? *reinterpret_cast<const float4*>(qrow + c0) : make_float4(0, 0, 0, 0);
      const float4 hi4 = ok ? *reinterpret_cast<const float4*>(qrow + c0 + 4) : make_float4(0, 0, 0, 0);
      xa[0] = lo4.x; xa[1] = lo4.y; xa[2] = lo4.z; xa[3] = lo4.w;
      xa[4] = hi4.x; xa[5] = hi4.y; xa[6] = hi4.z; xa[7] = hi4.w;
      split8(xa, ah[ks], al[ks]);
    }
    auto load_b = [&](int cb, float4 (&buf)[kMaxKSteps][2]) {
      const int kcol = cb * 16 + (lane & 15);
      const bool kcol_ok = kcol < Tk;
      const float* __restrict__ krow = k_hat + (bh * Tk + (kcol_ok ? kcol : 0)) * P;
#pragma unroll
      for (int ks = 0; ks < kMaxKSteps; ++ks) {
        const int c0 = ks * 32 + kq;
        const bool ok = ks < ksteps && kcol_ok && c0 < P;
        buf[ks][0] = ok ? *reinterpret_cast<const float4*>(krow + c0) : make_float4(0, 0, 0, 0);
        buf[ks][1] = ok ? *reinterpret_cast<const float4*>(krow + c0 + 4) : make_float4(0, 0, 0, 0);
      }
    };
    // up to 256 predictor columns the next column block is prefetched; beyond that the
    // two buffers would not fit the register file, so each block is loaded in place
    constexpr bool kPrefetch = kMaxKSteps <= 8;
    float4 cur[kMaxKSteps][2], nxt[kPrefetch ? kMaxKSteps : 1][2];
    int cb = wave;
    if (kPrefetch && cb * 16 < Tk) load_b(cb, cur);
    for (; cb * 16 < Tk; cb += kWaves) {
      const int cb_next = cb + kWaves;
      if constexpr (kPrefetch) {
        if (cb_next * 16 < Tk) load_b(cb_next, nxt);
      } else {
        load_b(cb, cur);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kMaxKSteps; ++ks) {
        if (ks < ksteps) {
          float xb[8] = {cur[ks][0].x, cur[ks][0].y, cur[ks][0].z, cur[ks][0].w,
                         cur[ks][1].x, cur[ks][1].y, cur[ks][1].z, cur[ks][1].w};
          bf16x8 bh8, bl8;
          split8(xb, bh8, bl8);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], bh8, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bl8, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bh8, acc, 0, 0, 0);
        }
      }
      // C layout: lane holds column (lane % 16), rows 4*(lane/16) + j
      const int kcol = cb * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = (lane >> 4) * 4 + j;
        if (r < nrows && kcol < Tk) {
          keys[r * Tk + kcol] = order_key(acc[j]);
          if (scores) scores[(bh * L.Tq + row0 + r) * Tk + kcol] = acc[j];
        }
      }
      if constexpr (kPrefetch) {
#pragma unroll
        for (int ks = 0; ks < kMaxKSteps; ++ks) {
          cur[ks][0] = nxt[ks][0];
          cur[ks][1] = nxt[ks][1];
        }
      }
    }
  }
  __syncthreads();

  // ---- 2. top-k per (row, segment), one wave each ------------------------------------
  // each wave keeps kHistCopies histograms (lane % kHistCopies picks one) so lanes
  // whose keys share a digit rarely hit the same LDS word in one atomic
  uint32_t* hist = hist_all + wave * (kHistCopies * 256);
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
      for (int t = 0; t < kHistCopies * 4; ++t) hist[t * 64 + lane] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < T; j += 64) {
        const uint32_t key = row[j];
        if ((key & pmask) == prefix)
          atomicAdd(&hist[(lane % kHistCopies) * 256 + ((key >> shift) & 0xFFu)], 1u);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane i owns digits 255-4i .. 252-4i (descending); inclusive scan of counts
      uint32_t c[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        c[t] = 0u;
#pragma unroll
        for (int cp = 0; cp < kHistCopies; ++cp) c[t] += hist[cp * 256 + 255 - (lane * 4 + t)];
      }
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
  // Prefer a block that lets two workgroups share a CU (<= 78 KB of LDS each); fall
  // back to one workgroup per CU with up to 144 KB when fewer than 8 rows would fit.
  const int hist = kWaves * kHistCopies * 256 * 4;
  int r = (78 * 1024 - hist) / (Tk * 4);
  if (r < 8) r = (144 * 1024 - hist) / (Tk * 4);
  if (r > 16) r = 16;
  if (r < 1) r = 1;
  return r;
}

hipError_t launch_score_topk(const LayerDev& L, const float* q_hat, const float* k_hat,
                             int32_t* idx, float* scores, hipStream_t s) {
  const int R = score_rows_per_block(L.Tk);
  const size_t lds = (size_t)R * L.Tk * 4 + kWaves * kHistCopies * 256 * 4;
  dim3 grid((unsigned)((L.Tq + R - 1) / R), (unsigned)L.H, (unsigned)L.B);
  // the kernel is instantiated for 32-wide predictor steps: p <= 64, 128, 256, 384
  auto run = [&](auto kern) -> hipError_t {
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, L, R, q_hat, k_hat, idx, scores);
    return hipSuccess;
  };
  hipError_t e;
  if (L.p <= 64)
    e = run(score_topk_kernel<2>);
  else if (L.p <= 128)
    e = run(score_topk_kernel<4>);
  else if (L.p <= 256)
    e = run(score_topk_kernel<8>);
  else
    e = run(score_topk_kernel<12>);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace veda
