// Pooled-score GEMM fused with the per-row, per-segment top-k selection.
//
// Veda R2VA record, first paragraph: a fixed budget of key tiles is kept per
// query tile and head, and the reference and current-video segments are chosen
// independently.  The score of a (query tile i, key tile j) pair is the plain
// dot product <q_hat_i, k_hat_j> of the projected pooled vectors; ties go to
// the lower tile index and the chosen ids are written ascending.
//
// One workgroup (8 or 16 waves for predictor widths up to 64, as topk_plan picks; 8 up to
// 128, else 4) owns R consecutive query-tile rows of one (b, h):
//  1. S[R x Tk] on bf16 matrix cores: each fp32 operand x is split into
//     hi = bf16(x) and lo = bf16(x - hi); S = hi*hi + hi*lo + lo*hi (the lo*lo
//     term is below 2^-16 relative).  v_mfma_f32_16x16x32_bf16 blocks of 16 key
//     tiles are spread over the waves; the scores land in LDS as order-preserving
//     uint32 keys (and optionally in HBM as fp32).
//  2. Each (row, segment) pair is reduced by one wave: a most-significant-digit
//     radix select (up to four 8-bit steps, histograms in LDS, one wave-wide scan per
//     step, stopping once the fixed bits decide the set) finds the k-th largest key
//     exactly and how many keys equal to it are kept; one ordered pass with wave
//     ballots then writes every key above the threshold and the first of the equal
//     ones, which yields the lowest-index tie-break and an ascending list without
//     sorting.  Each step is a chain of dependent LDS round trips, so the many waves
//     of a workgroup (one row each) are what keeps the CU busy.
#include "common.h"

namespace veda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 16;                     // keys per lane read ahead in a radix pass

// histogram words of one wave: kCopies histograms of 256 digits, plus one word per lane
// that takes the updates of keys outside the current prefix (no branch per key)
constexpr int hist_words(int copies) { return copies * 256 + 64; }

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

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS round trip):
// Hillis-Steele steps inside each row of 16 lanes, then the last lane of row 0 (2) is
// added to row 1 (3), and lane 31 to rows 2 and 3.  Moves from outside a row or masked
// rows contribute 0.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Largest and smallest value of x over the wave (inclusive DPP scans as above, then lane 63)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x111, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x112, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x114, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x118, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x142, 0xA, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x143, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(x, 63);
}

constexpr int kBoundGroups = 4;   // key groups per lane for the radix's starting bound
// Rows shorter than this start the radix at the top bit: the bound's extra pass over the
// row costs more than the steps it saves there (measured: 1.03-1.04x slower at 1008 and
// 252 key tiles, 0.81x at 2741)
constexpr int kBoundMinTiles = 2048;

template <int kMaxKSteps, int kWaves, int kHistCopies>
__global__ __launch_bounds__(64 * kWaves) void score_topk_kernel(LayerDev L, int R,
                                                              const float* __restrict__ q_hat,
                                                              const float* __restrict__ k_hat,
                                                              int32_t* __restrict__ idx,
                                                              float* __restrict__ scores) {
  extern __shared__ uint32_t smem[];
  const int Tk = L.Tk;
  uint32_t* keys = smem;                       // [R][Tk]
  uint32_t* hist_all = smem + (size_t)R * Tk;  // [kWaves][hist_words(kHistCopies)]

  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int nrows = min(R, L.Tq - row0);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // each wave keeps kHistCopies histograms (lane % kHistCopies picks one) so lanes whose
  // keys share a digit rarely hit the same LDS word in one atomic
  constexpr int kHW = hist_words(kHistCopies);
  uint32_t* hist = hist_all + wave * kHW;
  uint32_t* const trash = hist + kHistCopies * 256 + lane;
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
    // radix select of the K-th largest key, up to 8 bits per step from the top.  After a
    // step, the keys whose fixed bits (pmask) exceed `prefix` are all taken, and
    // `remaining` more are taken from those equal to it; when that is every one of them,
    // the fixed bits already decide the selection and the remaining steps are skipped.
    uint32_t prefix = 0, pmask = 0;
    int remaining = K;   // how many still to take from the keys matching `prefix`
    int hi = 31;         // highest bit not yet fixed
    // Starting point.  The 64 * kBoundGroups groups of keys (lane, position mod
    // kBoundGroups) are disjoint, so the smallest of their maxima is at most the
    // (64 * kBoundGroups)-th largest key, hence at most the K-th largest when K is no more
    // than that.  Every key from that bound up to the largest key shares the bits above
    // the highest bit in which the two differ: those bits are fixed before the first
    // step, and the K selected keys all have them.
    if (K <= 64 * kBoundGroups && T >= kBoundMinTiles) {
      uint32_t gmax[kBoundGroups] = {};
      uint32_t kmx = 0;
      for (int base = 0; base < T; base += 64 * kChunk) {
        uint32_t kc[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
          const int j = base + 64 * u + lane;
          kc[u] = j < T ? row[j] : 0u;     // 0 is the smallest key: an empty group bounds nothing
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
          gmax[u % kBoundGroups] = max(gmax[u % kBoundGroups], kc[u]);
          kmx = max(kmx, kc[u]);
        }
      }
      uint32_t gmin = gmax[0];
#pragma unroll
      for (int g = 1; g < kBoundGroups; ++g) gmin = min(gmin, gmax[g]);
      const uint32_t lb = wave_min_u32(gmin);
      const uint32_t top = wave_max_u32(kmx);
      if (lb == top) {                   // at least K keys equal the largest: all bits decided
        pmask = 0xFFFFFFFFu;
        prefix = top;
        hi = -1;
      } else {
        hi = 31 - __builtin_clz(lb ^ top);
        pmask = ~((2u << hi) - 1u);      // hi = 31 gives 0
        prefix = top & pmask;
      }
    }
    while (hi >= 0) {
      const int shift = hi >= 7 ? hi - 7 : 0;
      const uint32_t dmask = (2u << (hi - shift)) - 1u;   // the step's digit: bits shift..hi
#pragma unroll
      for (int t = 0; t < kHW / 64; ++t) hist[t * 64 + lane] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // keys in chunks of kChunk per lane: every read of a chunk is issued before the
      // first one is used, so a step pays the LDS latency once per chunk, not per key
      for (int base = 0; base < T; base += 64 * kChunk) {
        uint32_t kc[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
          const int j = base + 64 * u + lane;
          kc[u] = j < T ? row[j] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
          const bool match = base + 64 * u + lane < T && (kc[u] & pmask) == prefix;
          atomicAdd(match ? hist + (lane % kHistCopies) * 256 + ((kc[u] >> shift) & dmask) : trash, 1u);
        }
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
      const uint32_t incl = wave_inclusive_sum(local);
      const uint32_t excl = incl - local;
      // the lane whose range crosses `remaining`
      const bool mine = excl < (uint32_t)remaining && (uint32_t)remaining <= incl;
      const uint64_t bal = __ballot(mine);
      const int owner = bal ? __builtin_ctzll(bal) : 0;
      uint32_t digit = 0, above = 0, cnt = 0;
      if (lane == owner) {
        uint32_t acc_above = excl;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (acc_above + c[t] >= (uint32_t)remaining) {
            digit = 255 - (lane * 4 + t);
            cnt = c[t];
            break;
          }
          acc_above += c[t];
        }
        above = acc_above;
      }
      digit = __builtin_amdgcn_readlane(digit, owner);
      above = __builtin_amdgcn_readlane(above, owner);
      cnt = __builtin_amdgcn_readlane(cnt, owner);
      remaining -= (int)above;
      prefix |= digit << shift;
      pmask |= dmask << shift;
      __builtin_amdgcn_wave_barrier();
      if ((uint32_t)remaining == cnt) break;
      hi = shift - 1;
    }
    // keep every key whose fixed bits exceed `prefix` and the first `remaining` keys whose
    // fixed bits equal it, in ascending tile order
    int taken = 0, eq_seen = 0;
    for (int base = 0; base < T && taken < K; base += 64 * kChunk) {
      uint32_t kc[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int j = base + 64 * u + lane;
        kc[u] = j < T ? row[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int j = base + 64 * u + lane;
        const uint32_t fixed = kc[u] & pmask;
        const bool gt = j < T && fixed > prefix;
        const bool eq = j < T && fixed == prefix;
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
}

// Waves per workgroup and histogram copies per wave for a predictor width: more waves
// (one row each in the top-k phase) hide the latency of each row's serial radix steps, as
// far as the kernel's registers allow.
template <int kMaxKSteps>
struct TopkShape {
  static constexpr int waves = kMaxKSteps <= 2 ? 16 : kMaxKSteps <= 4 ? 8 : 4;
  static constexpr int copies = kMaxKSteps <= 2 ? 1 : 4;
};
// Predictor widths up to 64 also have an 8-wave form: two of its workgroups share a CU
// (its registers allow 16 waves per CU, not the 32 two 16-wave workgroups would need), so
// one workgroup's top-k phase runs beside the other's score phase.
struct TopkHalf {
  static constexpr int waves = 8;
  static constexpr int copies = 1;
};

}  // namespace

// Launch plan of the selection kernel for Tk key tiles and predictor width p: the form
// (waves, histogram copies) and the rows R of the score block per workgroup.  Two
// workgroups share a CU when each needs at most 78 KB of LDS and holds at least 8 rows;
// otherwise one workgroup takes up to 150 KB.  At most 16 rows (one MFMA row block).
struct TopkPlan {
  int waves, copies, rows;
  size_t lds;
};

static TopkPlan topk_plan(int Tk, int p) {
  auto rows = [&](int waves, int copies, int budget) {
    return (budget - waves * hist_words(copies) * 4) / (Tk * 4);
  };
  auto make = [&](int waves, int copies, int r) {
    r = r > 16 ? 16 : (r < 1 ? 1 : r);
    return TopkPlan{waves, copies, r, (size_t)r * Tk * 4 + (size_t)waves * hist_words(copies) * 4};
  };
  if (p <= 64) {
    const int r2 = rows(TopkHalf::waves, TopkHalf::copies, 78 * 1024);
    if (r2 >= 8) return make(TopkHalf::waves, TopkHalf::copies, r2);
    return make(TopkShape<2>::waves, TopkShape<2>::copies,
                rows(TopkShape<2>::waves, TopkShape<2>::copies, 150 * 1024));
  }
  auto generic = [&](auto shape) {
    using S = decltype(shape);
    const int r2 = rows(S::waves, S::copies, 78 * 1024);
    return make(S::waves, S::copies, r2 >= 8 ? r2 : rows(S::waves, S::copies, 150 * 1024));
  };
  if (p <= 128) return generic(TopkShape<4>{});
  if (p <= 256) return generic(TopkShape<8>{});
  return generic(TopkShape<12>{});
}

int score_rows_per_block(int Tk, int p) { return topk_plan(Tk, p).rows; }

hipError_t launch_score_topk(const LayerDev& L, const float* q_hat, const float* k_hat,
                             int32_t* idx, float* scores, hipStream_t s) {
  const TopkPlan plan = topk_plan(L.Tk, L.p);
  const int R = plan.rows;
  dim3 grid((unsigned)((L.Tq + R - 1) / R), (unsigned)L.H, (unsigned)L.B);
  // the kernel is instantiated for 32-wide predictor steps: p <= 64, 128, 256, 384
  auto run = [&](auto kern) -> hipError_t {
    if (plan.lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan.lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * plan.waves), plan.lds, s, L, R, q_hat, k_hat, idx, scores);
    return hipSuccess;
  };
  hipError_t e;
  if (L.p <= 64 && plan.waves == TopkHalf::waves)
    e = run(score_topk_kernel<2, TopkHalf::waves, TopkHalf::copies>);
  else if (L.p <= 64)
    e = run(score_topk_kernel<2, TopkShape<2>::waves, TopkShape<2>::copies>);
  else if (L.p <= 128)
    e = run(score_topk_kernel<4, TopkShape<4>::waves, TopkShape<4>::copies>);
  else if (L.p <= 256)
    e = run(score_topk_kernel<8, TopkShape<8>::waves, TopkShape<8>::copies>);
  else
    e = run(score_topk_kernel<12, TopkShape<12>::waves, TopkShape<12>::copies>);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace veda
