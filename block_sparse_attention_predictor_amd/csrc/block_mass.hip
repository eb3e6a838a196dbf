// Teacher block attention mass and the recall of an index set under it.
//
// Affine launch article, "Training the Selector, Not the Generator": the Veda
// predictor is distilled from the attention patterns of a full-attention teacher.
// At block granularity that pattern is, per (b, h, query tile i, key tile j), the
// dense softmax probability that the rows of tile i put on the keys of tile j,
// averaged over the rows:
//     M[i, j] = (1 / rows_i) * sum_{n in tile i} sum_{m in tile j} P_n(m),
//     P_n(m)  = exp(scale * <q_n, k_m> - lse_n),  lse_n over every key (all tiles of
//               every segment and every dense range).
// Rows of M plus the dense ranges' share sum to one.  The recall of an index set is
// the part of the segment tiles' mass that the selected tiles hold.
//
// Two passes over all keys, each one workgroup per (b, h, query tile) with 32
// query rows per wave and keys streamed HBM -> LDS (global_load_lds, 16 bytes per
// lane, two-stage ring, XOR-swizzled rows) as in the block-sparse attention kernel:
//   pass 1: S^T = K Q^T on v_mfma_f32_32x32x16_bf16, running max and sum in the exp2
//           domain -> lse_n (fp32);
//   pass 2: the same product, p = exp2(s - lse_n), summed per lane, across the wave
//           (DPP row rotations and lane swaps, no LDS) and across the waves (one LDS
//           slot per wave and block, read after the pipeline's barrier) -> one value
//           per key tile, stored by wave 0.
#include "common.h"

#include <type_traits>

namespace veda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_t;

constexpr int KB = 64;            // keys per block
constexpr float kLazyRescale = 8.0f;

struct KeyBlock {
  int64_t start;
  int n;                          // 0 marks the end
  int col;                        // key-tile column over all segments; -1 for a dense range
};

// Every key in order: each segment cut into 64-token blocks (a block never crosses
// a tile boundary: tiles are 64 or 128 tokens from the segment start), then every
// dense range.
struct KeyWalk {
  int r = 0;
  int64_t off = 0;

  __device__ __forceinline__ KeyBlock next(const LayerDev& L, const DenseDev& DN) {
    for (;;) {
      if (r >= L.n_seg + DN.n) return KeyBlock{0, 0, -1};
      const bool seg = r < L.n_seg;
      const int64_t st = seg ? L.seg[r].start : DN.r[r - L.n_seg].start;
      const int64_t len = seg ? L.seg[r].len : DN.r[r - L.n_seg].len;
      if (off >= len) {
        ++r;
        off = 0;
        continue;
      }
      const int64_t rem = len - off;
      const KeyBlock b{st + off, (int)(rem < KB ? rem : KB),
                       seg ? L.seg[r].toff + (int)(off / L.tile) : -1};
      off += KB;
      return b;
    }
  }
};

template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }

// Sum over the 64 lanes without LDS: rotations within each 16-lane row (DPP), then
// the row pairs (lane ^ 16) and the halves (lane ^ 32) through lane swaps.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x120 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int NW, bool MASS>
__global__ __launch_bounds__(64 * NW, 2) void block_mass_kernel(
    LayerDev L, DenseDev DN, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    float scale_log2, float* __restrict__ lse, float* __restrict__ mass,
    float* __restrict__ dense_mass) {
  constexpr int NT = 64 * NW;
  constexpr int CPR = D / 8;
  constexpr int SLOTS = KB * CPR;
  constexpr int LPT = SLOTS / NT;
  static_assert(SLOTS % NT == 0, "block split");

  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * KB * D];
  __shared__ float red[2][NW];
  uint16_t* const Ks0 = smem;
  uint16_t* const Ks1 = smem + KB * D;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // work item: the attention kernel's XCD-aware order (one head at a time per XCD)
  const int per_xcd = (L.Tq + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int bh = slot / per_xcd;
  const int qt = xcd * per_xcd + (slot - bh * per_xcd);
  if (qt >= L.Tq) return;
  const int h = bh % L.H;
  const int b = bh / L.H;

  const int64_t q_first = L.q0 + (int64_t)qt * L.tile;
  const int64_t q_end = L.q0 + L.qlen;
  const int64_t head_off = (int64_t)b * L.sb + (int64_t)h * L.sh;

  const int64_t my_q = q_first + wave * 32 + l32;
  const bool q_ok = my_q < q_end;
  bf16x8 qv[D / 16];
  {
    const uint16_t* qp = q + head_off + (q_ok ? my_q : q_first) * L.sn + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 w = q_ok ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qv[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // pass 2: this row's lse in the exp2 domain; rows past the end weigh nothing
  float row_l2 = INFINITY;
  if constexpr (MASS) {
    if (q_ok) row_l2 = lse[(int64_t)bh * L.qlen + (my_q - L.q0)] * 1.44269504088896340736f;
  }

  auto dma_row = [&](int i) { return ((wave * LPT + i) * 64 + lane) / CPR; };
  auto dma_col = [&](int i) {
    const int r = dma_row(i);
    const int pc = ((wave * LPT + i) * 64 + lane) % CPR;
    return (pc ^ swz_k<CPR>(r)) * 8;
  };
  uint32_t koff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) koff[i] = (uint32_t)(((int64_t)dma_row(i) * L.sn + dma_col(i)) * 2);
  const char* kbase = reinterpret_cast<const char*>(k + head_off);
  auto dma = [&](const KeyBlock& blk, uint16_t* dst) {
    const char* g = kbase + blk.start * L.sn * 2;
    if (blk.n == KB) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        uint32_t o = koff[i];
        asm volatile("" : "+v"(o));
        __builtin_amdgcn_global_load_lds((const void*)(g + o),
                                         (lds_void_t)(reinterpret_cast<char*>(dst) + (wave * LPT + i) * 1024),
                                         16, 0, 0);
      }
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln) : : "memory");
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int r = ((wave * LPT + i) * 64 + ln) / CPR;
        const int rc = r < blk.n ? r : blk.n - 1;
        const uint32_t o = koff[i] - (uint32_t)((r - rc) * (int)L.sn * 2);
        __builtin_amdgcn_global_load_lds((const void*)(g + o),
                                         (lds_void_t)(reinterpret_cast<char*>(dst) + (wave * LPT + i) * 1024),
                                         16, 0, 0);
      }
    }
  };

  // K operand (row l32 [+32], chunk 2kk+hi) of a block: kR ^ (kk << 5) [+ 32 rows]
  const uint32_t kR = (uint32_t)l32 * (D * 2) + ((uint32_t)(hi ^ swz_k<CPR>(l32)) << 4);
  float m_run = -INFINITY, l_run = 0.f;   // pass 1
  float acc = 0.f, dacc = 0.f;            // pass 2 (wave 0): current tile, dense ranges
  const int rows = (int)((q_end - q_first) < L.tile ? (q_end - q_first) : L.tile);
  const float inv_rows = 1.0f / (float)rows;
  float* mrow = MASS ? mass + ((int64_t)bh * L.Tq + qt) * L.Tk : nullptr;

  KeyWalk it;
  KeyBlock b0 = it.next(L, DN);
  KeyBlock b1 = it.next(L, DN);
  if (b0.n > 0) dma(b0, Ks0);
  if (b1.n > 0) dma(b1, Ks1);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();

  // Iteration i: S^T of block i from Ks[i%2]; barrier; DMA block i+2 into Ks[i%2].
  auto step = [&](auto stage) {
    constexpr int ST = decltype(stage)::value;
    uint16_t* Kc = ST ? Ks1 : Ks0;
    const int n = b0.n;
    f32x16 s[2];
    bf16x8 ka[2][D / 16];
    const char* Kb = reinterpret_cast<const char*>(Kc);
    uint32_t kRi = kR;   // one register; the per-kk addresses are formed here
    asm volatile("" : "+v"(kRi));
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        ka[mb][kk] = *reinterpret_cast<const bf16x8*>(Kb + (kRi ^ (kk << 5)) + mb * 32 * D * 2);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[mb][kk], qv[kk], s[mb], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, D / 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, D / 8, 0);
    if (n < KB) {
      int kb = hi * 4;                      // key = kb + c for accumulator entry (mb, e)
      float ninf = -INFINITY;
      asm volatile("" : "+v"(kb), "+v"(ninf) : : "memory");
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = mb * 32 + (e >> 2) * 8 + (e & 3);
          if (kb >= n - c) s[mb][e] = ninf;
        }
    }
    if constexpr (!MASS) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale) != 0) {
        const float m_new = fmaxf(m_run, mx);
        l_run *= __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
      }
      float part = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) part += __builtin_amdgcn_exp2f(fmaf(s[mb][e], scale_log2, -m_run));
      l_run += part;
    } else {
      float part = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) part += __builtin_amdgcn_exp2f(fmaf(s[mb][e], scale_log2, -row_l2));
      part = wave_sum(part);
      if (lane == 0) red[ST][wave] = part;
    }

    const KeyBlock b2 = it.next(L, DN);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA of block i+1 landed
    __syncthreads();
    if (b2.n > 0) dma(b2, Kc);
    if constexpr (MASS) {
      if (wave == 0) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += red[ST][w];
        if (b0.col >= 0) {
          acc += tot;
          if (b1.n == 0 || b1.col != b0.col) {   // last block of this key tile
            if (lane == 0) mrow[b0.col] = acc * inv_rows;
            acc = 0.f;
          }
        } else {
          dacc += tot;
        }
      }
    }
    b0 = b1;
    b1 = b2;
  };
  while (b0.n > 0) {
    step(std::integral_constant<int, 0>{});
    if (b0.n <= 0) break;
    step(std::integral_constant<int, 1>{});
  }

  if constexpr (!MASS) {
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    if (q_ok && hi == 0)
      lse[(int64_t)bh * L.qlen + (my_q - L.q0)] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  } else {
    if (dense_mass && wave == 0 && lane == 0) dense_mass[(int64_t)bh * L.Tq + qt] = dacc * inv_rows;
  }
}

// Recall of one index row per wave: selected tiles' mass over all segment tiles'
// mass.  Within a segment's block of entries, a -1 ends the block.
__global__ __launch_bounds__(256) void block_recall_kernel(LayerDev L, const float* __restrict__ mass,
                                                           const int32_t* __restrict__ idx,
                                                           float* __restrict__ recall) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)L.B * L.H * L.Tq) return;
  const float* m = mass + row * L.Tk;
  const int32_t* ir = idx + row * L.Ktot;
  float all = 0.f, sel = 0.f;
  for (int j = lane; j < L.Tk; j += 64) all += m[j];
  for (int s = 0; s < L.n_seg; ++s) {
    const int end = L.seg[s].koff + L.seg[s].K;
    for (int base = L.seg[s].koff; base < end; base += 64) {
      const int c = base + lane;
      const int t = c < end ? ir[c] : 0;
      const uint64_t neg = __builtin_amdgcn_ballot_w64(c < end && t < 0);
      const int first = neg ? base + (int)__builtin_ctzll(neg) : end;
      if (c < first) sel += m[L.seg[s].toff + t];
      if (neg) break;
    }
  }
  all = wave_sum(all);
  sel = wave_sum(sel);
  if (lane == 0) recall[row] = all > 0.f ? sel / all : 1.0f;
}

template <int D, int NW>
hipError_t launch_pair(const LayerDev& L, const DenseDev& DN, const uint16_t* q, const uint16_t* k,
                       float scale_log2, float* lse, float* mass, float* dense_mass, hipStream_t s,
                       dim3 grid) {
  hipLaunchKernelGGL((block_mass_kernel<D, NW, false>), grid, dim3(64 * NW), 0, s, L, DN, q, k,
                     scale_log2, lse, mass, dense_mass);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((block_mass_kernel<D, NW, true>), grid, dim3(64 * NW), 0, s, L, DN, q, k,
                     scale_log2, lse, mass, dense_mass);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_mass(const LayerDev& L, const DenseDev& DN, const void* q, const void* k,
                             float scale, float* lse, float* mass, float* dense_mass, hipStream_t s) {
  const int64_t per_xcd = (L.Tq + 7) / 8;
  const int64_t nwork = (int64_t)L.B * L.H * per_xcd * 8;
  if (nwork > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.44269504088896340736f;
  const dim3 grid((unsigned)nwork);
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  if (L.d == 128 && L.tile == 128) return launch_pair<128, 4>(L, DN, qq, kk, scale_log2, lse, mass, dense_mass, s, grid);
  if (L.d == 128) return launch_pair<128, 2>(L, DN, qq, kk, scale_log2, lse, mass, dense_mass, s, grid);
  if (L.tile == 128) return launch_pair<64, 4>(L, DN, qq, kk, scale_log2, lse, mass, dense_mass, s, grid);
  return launch_pair<64, 2>(L, DN, qq, kk, scale_log2, lse, mass, dense_mass, s, grid);
}

hipError_t launch_block_recall(const LayerDev& L, const float* mass, const int32_t* idx, float* recall,
                               hipStream_t s) {
  const int64_t rows = (int64_t)L.B * L.H * L.Tq;
  if ((rows + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_recall_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, L, mass,
                     idx, recall);
  return hipGetLastError();
}

}  // namespace veda
