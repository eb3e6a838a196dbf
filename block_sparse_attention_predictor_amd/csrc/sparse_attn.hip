// Block-sparse flash attention over the selected key tiles plus dense key ranges.
//
// Affine launch article, "Training the Selector, Not the Generator": the
// predictor selects blocks for a sparse execution kernel; Veda R2VA record,
// first paragraph: the selected reference and video tiles are attended per
// query tile and head, while text, VLM conditioning and audio stay dense.
//
// One workgroup computes one (b, h, query tile); each of its tile/32 waves owns
// 32 query rows.  Keys stream through LDS in blocks of 64 tokens: first the
// tiles named by the index row (gathered by id), then every dense range, cut
// into 64-token blocks.  The next block's K/V rows are loaded into registers
// while the current block is multiplied, then written to LDS (K row-major, V
// transposed), so HBM latency hides behind the matrix work.
//
// Both products are computed transposed on v_mfma_f32_32x32x16_bf16:
//     S^T (keys x queries)  = K . Q^T     A = K rows from LDS, B = Q^T held in VGPRs
//     O^T (d x queries)    += V^T . P^T   A = V^T rows from LDS, B = P^T from S^T's accumulator
// With this orientation every accumulator value a lane holds belongs to one
// query row (lane % 32), so the online softmax needs a single cross-lane
// exchange (lane ^ 32) per block for the running maximum, and P^T is formed
// from S^T's accumulator registers without any shuffle: the key order inside
// each 16-key slice of the O^T contraction is permuted to match the
// accumulator layout, and V^T is stored in LDS in that same permuted order.
// Softmax runs in fp32 in the exp2 domain; P is rounded to bf16 for the second
// product; O is accumulated in fp32 and rounded to bf16 once at the end.
#include "common.h"

namespace veda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KB = 64;          // keys per block
constexpr int VP = KB + 8;      // V^T row pitch in LDS (bf16): 144 B, conflict-free 16 B reads

// position of key k (0..63) inside V^T's permuted row
__device__ __forceinline__ int vt_pos(int k) {
  const int kl = k & 15;
  const int g = kl >> 2;
  return (k & ~15) + (g & 1) * 8 + (g >> 1) * 4 + (kl & 3);
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) {
  return (uint32_t)a | ((uint32_t)b << 16);
}

struct Block {
  int64_t start;
  int n;
};

// Key block `bi` of the current (b, h, query tile): selected tiles first (ids from
// the index row, segment blocks in order), then the dense ranges.
__device__ __forceinline__ Block key_block(const LayerDev& L, const DenseDev& DN,
                                           const int32_t* __restrict__ idx_row, int nsel_blocks,
                                           int bpt, int bi) {
  Block blk;
  if (bi < nsel_blocks) {
    const int sel = bi / bpt;
    const int sub = bi - sel * bpt;
    int s = 0;
#pragma unroll
    for (int t = 1; t < kMaxSeg; ++t)
      if (t < L.n_seg && sel >= L.seg[t].koff) s = t;
    const int tile_id = __builtin_amdgcn_readfirstlane(idx_row[sel]);
    const int64_t rel = (int64_t)tile_id * L.tile + (int64_t)sub * KB;
    blk.start = L.seg[s].start + rel;
    const int64_t rem = L.seg[s].len - rel;
    blk.n = (int)(rem < KB ? (rem > 0 ? rem : 0) : KB);
  } else {
    int bd = bi - nsel_blocks;
    blk.start = 0;
    blk.n = 0;
    for (int r = 0; r < DN.n; ++r) {
      const int nb = (int)((DN.r[r].len + KB - 1) / KB);
      if (bd < nb) {
        blk.start = DN.r[r].start + (int64_t)bd * KB;
        const int64_t rem = DN.r[r].len - (int64_t)bd * KB;
        blk.n = (int)(rem < KB ? rem : KB);
        break;
      }
      bd -= nb;
    }
  }
  return blk;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attn_kernel(
    LayerDev L, DenseDev DN, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = 64 * NW;                 // threads
  constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  constexpr int KPT = KB * CPR / NT;          // keys per thread in a block (2, 4 or 8)
  constexpr int KP = D + 8;                   // K row pitch in LDS (bf16)
  static_assert(KPT == 2 || KPT == 4 || KPT == 8, "unsupported block split");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[KB * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work item, XCD-aware: XCD x (= blockIdx % 8) gets a contiguous run of items
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int per = nwg >> 3;
  const int rem = nwg & 7;
  const int work = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
  const int qt = work % L.Tq;
  const int bh = work / L.Tq;
  const int h = bh % L.H;
  const int b = bh / L.H;

  const int64_t q_first = L.q0 + (int64_t)qt * L.tile;              // first row of the tile
  const int64_t q_end = L.q0 + L.qlen;                              // end of the query segment
  const int64_t head_off = (int64_t)b * L.sb + (int64_t)h * L.sh;
  const int32_t* idx_row = idx ? idx + ((int64_t)bh * L.Tq + qt) * L.Ktot : nullptr;

  // ---- Q^T operand: lane holds query (32*wave + l32), d = 16*kk + 8*hi .. +7
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

  const int bpt = L.tile / KB;
  const int nsel_blocks = L.Ktot * bpt;
  int ndense_blocks = 0;
  for (int r = 0; r < DN.n; ++r) ndense_blocks += (int)((DN.r[r].len + KB - 1) / KB);
  const int nblk = nsel_blocks + ndense_blocks;

  // ---- loader mapping: thread holds keys kg*KPT .. +KPT-1, d-chunk c
  const int lc = (tid % CPR) * 8;
  const int lkg = tid / CPR;
  uint4 kr[KPT], vr[KPT];

  auto load_block = [&](int bi) -> int {
    const Block blk = key_block(L, DN, idx_row, nsel_blocks, bpt, bi);
    const uint16_t* kb = k + head_off + blk.start * L.sn + lc;
    const uint16_t* vb = v + head_off + blk.start * L.sn + lc;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int key = lkg * KPT + u;
      if (key < blk.n) {
        kr[u] = *reinterpret_cast<const uint4*>(kb + (int64_t)key * L.sn);
        vr[u] = *reinterpret_cast<const uint4*>(vb + (int64_t)key * L.sn);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    return blk.n;
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  int cur_n = nblk > 0 ? load_block(0) : 0;
  for (int bi = 0; bi < nblk; ++bi) {
    const int n = cur_n;
    __syncthreads();
    if (n > 0) {
      // K rows as they are
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        *reinterpret_cast<uint4*>(&Ks[(lkg * KPT + u) * KP + lc]) = kr[u];
      // V transposed, keys in the permuted order of the P^T operand
      const uint16_t* vs = reinterpret_cast<const uint16_t*>(vr);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (KPT == 2) {
          const int k0 = lkg * 2;
          *reinterpret_cast<uint32_t*>(&Vt[(lc + e) * VP + vt_pos(k0)]) =
              pack2(vs[0 * 8 + e], vs[1 * 8 + e]);
        } else {
#pragma unroll
          for (int g4 = 0; g4 < KPT / 4; ++g4) {
            const int k0 = lkg * KPT + g4 * 4;
            uint2 w;
            w.x = pack2(vs[(g4 * 4 + 0) * 8 + e], vs[(g4 * 4 + 1) * 8 + e]);
            w.y = pack2(vs[(g4 * 4 + 2) * 8 + e], vs[(g4 * 4 + 3) * 8 + e]);
            *reinterpret_cast<uint2*>(&Vt[(lc + e) * VP + vt_pos(k0)]) = w;
          }
        }
      }
    }
    __syncthreads();
    if (bi + 1 < nblk) cur_n = load_block(bi + 1);
    if (n <= 0) continue;

    // ---- S^T = K Q^T for 64 keys: two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&Ks[(mb * 32 + l32) * KP + kk * 16 + hi * 8]);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qv[kk], s[mb], 0, 0, 0);
      }
    }
    // ---- mask keys past the end of a partial block (tile-uniform branch)
    if (n < KB) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = mb * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
          if (key >= n) s[mb][e] = -INFINITY;
        }
    }
    // ---- online softmax, exp2 domain
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[mb][e], scale_log2, -m_new));
        psum += pe;
        pb[mb * 2 + (e >> 3)][e & 7] = (__bf16)pe;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vt[(db * 32 + l32) * VP + c * 16 + hi * 8]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], o[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q_ok) {
    uint16_t* op = out + head_off + my_q * L.sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + i * 8 + hi * 4;
        uint2 w;
        const __bf16 o0 = (__bf16)(o[db][i * 4 + 0] * inv);
        const __bf16 o1 = (__bf16)(o[db][i * 4 + 1] * inv);
        const __bf16 o2 = (__bf16)(o[db][i * 4 + 2] * inv);
        const __bf16 o3 = (__bf16)(o[db][i * 4 + 3] * inv);
        w.x = pack2(__builtin_bit_cast(uint16_t, o0), __builtin_bit_cast(uint16_t, o1));
        w.y = pack2(__builtin_bit_cast(uint16_t, o2), __builtin_bit_cast(uint16_t, o3));
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (lse && hi == 0) {
      lse[(int64_t)bh * L.qlen + (my_q - L.q0)] =
          (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
    }
  }
}

}  // namespace

hipError_t launch_sparse_attn(const LayerDev& L, const DenseDev& DN, const void* q, const void* k,
                              const void* v, const int32_t* idx, float scale, void* out, float* lse,
                              hipStream_t s) {
  const int64_t nwork = (int64_t)L.B * L.H * L.Tq;
  if (nwork > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.44269504088896340736f;
  dim3 grid((unsigned)nwork);
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(out);
  if (L.d == 128 && L.tile == 128)
    hipLaunchKernelGGL((sparse_attn_kernel<128, 4>), grid, dim3(256), 0, s, L, DN, qq, kk, vv, idx,
                       scale_log2, oo, lse);
  else if (L.d == 128 && L.tile == 64)
    hipLaunchKernelGGL((sparse_attn_kernel<128, 2>), grid, dim3(128), 0, s, L, DN, qq, kk, vv, idx,
                       scale_log2, oo, lse);
  else if (L.d == 64 && L.tile == 128)
    hipLaunchKernelGGL((sparse_attn_kernel<64, 4>), grid, dim3(256), 0, s, L, DN, qq, kk, vv, idx,
                       scale_log2, oo, lse);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<64, 2>), grid, dim3(128), 0, s, L, DN, qq, kk, vv, idx,
                       scale_log2, oo, lse);
  return hipGetLastError();
}

}  // namespace veda
