// Block-sparse flash attention over the selected key tiles plus dense key ranges.
//
// Affine launch article, "Training the Selector, Not the Generator": the
// predictor selects blocks for a sparse execution kernel; Veda R2VA record,
// first paragraph: the selected reference and video tiles are attended per
// query tile and head, while text, VLM conditioning and audio stay dense.
//
// One workgroup computes one (b, h, query tile), or two 64-row tiles, taken in the
// caller's processing order of the query tiles when one is given (work_order.hip), else
// in tile order; the results do not depend on it.  Keys stream
// through LDS in blocks of 64 tokens (32 for 64-row tiles): first the tiles named by the
// index row (gathered by id), then every dense range, cut into blocks.  The kernels
// share the math below:
//  * sparse_attn_pingpong_kernel (128-row tiles): two groups of four waves split the
//    key blocks and alternate products and softmax slot by slot (see its comment);
//  * sparse_attn_pingpong_pair_kernel (64-row tiles): the same, with two query tiles per
//    workgroup, each half of a group streaming its own tile's 32-key blocks;
//  * sparse_attn_kernel (rows whose block list exceeds the two-group tables):
//    tile/32 waves, one pipeline (64-row tiles with 32-key blocks and four workgroups
//    per CU);
//  * sparse_attn_fp8qk_pingpong_kernel: the two-group kernel with Q and K as FP8
//    (E4M3FN) codes and the first product on the FP8 matrix cores;
//  * sparse_attn_fp8_pingpong_kernel: the same with V as FP8 too (d-major 64-token
//    blocks) and P rounded to E4M3FN, both products on the FP8 matrix cores.
//
// Memory path (gfx950):
//  * K and V rows go HBM -> LDS directly (global_load_lds_dwordx4, 16 bytes per
//    lane, no VGPR staging) into two-stage rings; the next blocks are in flight while
//    the current one is multiplied.
//  * Rows are stored unpadded with their 16-byte chunks XOR-swizzled by row, so
//    the matrix-core operand reads below are free of LDS bank conflicts.
//  * V stays row-major; the transposing LDS read (ds_read_b64_tr_b16) hands each
//    lane four consecutive keys of one head-dimension column, which is exactly
//    the V^T operand layout.
//
// Both products are computed transposed on v_mfma_f32_32x32x16_bf16:
//     S^T (keys x queries)  = K . Q^T     A = K rows from LDS, B = Q^T held in VGPRs
//     O^T (d x queries)    += V^T . P^T   A = V^T via transposing reads, B = P^T
// Every accumulator value a lane holds then belongs to one query row
// (lane % 32): the online softmax needs one cross-lane exchange (lane ^ 32, a
// v_permlane32_swap) per block, and P^T is built from S^T's accumulator registers
// without a shuffle
// (the key order inside each 16-key slice of the O^T contraction is permuted to
// match the accumulator layout; the V^T reads use the same permutation).
// Softmax is fp32 in the exp2 domain against a lazily updated running maximum.
// A block's weights are first taken against the running maximum as it stands and
// kept when no lane's sum of them exceeds 2^8 (then no single weight does); the
// stale maximum leaves the result unchanged, since numerator and denominator share
// it.  Otherwise (always on a row's first block, rarely after) the maximum moves
// to the block's maximum, the output is rescaled and the weights are redone, so
// the block maximum itself is only computed on that path.
// P is rounded to bf16 for the second product; O accumulates in fp32 and is
// rounded to bf16 once at the end.
#include "common.h"

#include <type_traits>

namespace veda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;
typedef const __attribute__((address_space(4))) int32_t* const_i32_t;

constexpr int KB = 64;            // keys per block (the single-pipeline kernel also runs 32)
constexpr float kLazySum = 256.0f;   // largest per-lane weight sum kept against a stale maximum
// FP8 weights: 2^(x + kW8Shift) for exponents x (against the running maximum) up to kW8Lazy,
// so every weight stays below 2^8.5 < 448 and weights down to 2^-13 of the row maximum
// still round to a nonzero code (the smallest subnormal E4M3 value is 2^-9)
constexpr float kW8Shift = 4.0f;
constexpr float kW8Lazy = 4.5f;

struct Block {
  int64_t start;
  int n;                          // 0 marks the end of the key list
};

// Walks the key blocks of one (b, h, query tile): the selected tiles of every
// segment in index order (tiles longer than a block give several blocks; the
// empty tail of a short last tile gives none; an index entry of -1 ends its
// segment's block: it and the later entries of that block give none), then every
// dense range.  Without an index row every tile of every
// segment is taken, in order.
struct BlockIter {
  int sel = 0, sub = 0, seg = 0, dr = 0;
  int64_t doff = 0;

  template <int KBK = KB>
  __device__ __forceinline__ Block next(const LayerDev& L, const DenseDev& DN, const_i32_t idx_row) {
    const int bpt = L.tile / KBK;
    for (;;) {
      if (sel < L.Ktot) {
        while (sel >= L.seg[seg].koff + L.seg[seg].K) ++seg;
        const int t = idx_row ? idx_row[sel] : sel - L.seg[seg].koff;
        if (t < 0) {   // padding: the rest of this segment's block is unused
          sel = L.seg[seg].koff + L.seg[seg].K;
          sub = 0;
          continue;
        }
        const int64_t rel = (int64_t)t * L.tile + (int64_t)sub * KBK;
        const int64_t rem = L.seg[seg].len - rel;
        const int64_t st = L.seg[seg].start + rel;
        if (++sub == bpt) {
          sub = 0;
          ++sel;
        }
        if (rem > 0) return Block{st, (int)(rem < KBK ? rem : KBK)};
        continue;
      }
      if (dr < DN.n) {
        const int64_t rem = DN.r[dr].len - doff;
        const int64_t st = DN.r[dr].start + doff;
        doff += KBK;
        if (doff >= DN.r[dr].len) {
          ++dr;
          doff = 0;
        }
        return Block{st, (int)(rem < KBK ? rem : KBK)};
      }
      return Block{0, 0};
    }
  }
};

// 16-byte chunk swizzles (CPR = chunks per row).
template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int swz_v(int row) { return (row & 3) * (CPR / 4); }

// Work item of a workgroup, XCD-aware: workgroups are dispatched round-robin over the
// 8 XCDs (blockIdx % 8).
//  * by tiles (index rows given): every XCD works on the same (b, h) at a time and takes
//    a contiguous slice of its query tiles.  The head's K/V (tens of MB) then stays in the
//    shared Infinity Cache while it is in use, and neighbouring query tiles, whose
//    selections overlap, share each XCD's L2.
//  * by heads: every XCD takes whole heads, so the query tiles of one head run side by
//    side and share that XCD's L2, and no other XCD fetches that head's keys.  Mode 1
//    (no index: every tile of every segment, e.g. the dense query rows of a layer) runs
//    a head's tiles in tile order; mode 2 (index rows given, and the K/V of the eight
//    heads in flight small enough to stay in the Infinity Cache together) runs them in
//    the caller's processing order.
// n is the number of work items per (b, h): query tiles, or pairs of them.
// Returns false for a padding workgroup (a uniform exit before any barrier).
__device__ __forceinline__ bool work_item(const LayerDev& L, int n, int by_heads, int& bh, int& it) {
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  if (by_heads) {
    bh = (slot / n) * 8 + xcd;
    it = slot % n;
    return bh < L.B * L.H;
  }
  const int per_xcd = (n + 7) >> 3;               // items per XCD and head
  bh = slot / per_xcd;
  it = xcd * per_xcd + (slot - bh * per_xcd);
  return it < n;
}
__device__ __forceinline__ bool work_item(const LayerDev& L, int by_heads, int& bh, int& qt) {
  return work_item(L, L.Tq, by_heads, bh, qt);
}
// Query tile at processing position pos of (b, h): pos itself, or the caller's order
// entry for it; -1 for none (pos past the last tile, or an entry outside [0, Tq)).
__device__ __forceinline__ int tile_at(const LayerDev& L, const int32_t* order, int bh, int pos) {
  if (pos >= L.Tq) return -1;
  if (order == nullptr) return pos;
  const int t = order[(int64_t)bh * L.Tq + pos];
  return t >= 0 && t < L.Tq ? t : -1;
}

template <int D, int NW, int KBK>
__global__ __launch_bounds__(64 * NW, KBK == 32 ? 4 : 2) void sparse_attn_kernel(
    LayerDev L, DenseDev DN, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, int by_heads) {
  constexpr int NT = 64 * NW;                 // threads
  constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  constexpr int SLOTS = KBK * CPR;            // 16-byte slots per K (or V) block
  constexpr int LPT = SLOTS / NT;             // DMA loads per thread per tensor and block
  constexpr int MBN = KBK / 32;               // 32-key halves of S^T per block
  constexpr int PCN = KBK / 16;               // 16-key slices of the PV contraction
  static_assert(SLOTS % NT == 0 && (KBK == 32 || KBK == 64), "block split");

  // two stages each for K and V
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * KBK * D];
  uint16_t* const Ks0 = smem;
  uint16_t* const Ks1 = smem + KBK * D;
  uint16_t* const Vs0 = smem + 2 * KBK * D;
  uint16_t* const Vs1 = smem + 3 * KBK * D;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt;
  if (!work_item(L, by_heads, bh, qt)) return;     // padding workgroup (uniform exit)
  if (by_heads != 1 && (qt = tile_at(L, order, bh, qt)) < 0) return;   // no tile at this position
  const int h = bh % L.H;
  const int b = bh / L.H;

  const int64_t q_first = L.q0 + (int64_t)qt * L.tile;
  const int64_t q_end = L.q0 + L.qlen;
  const int64_t head_off = (int64_t)b * L.sb + (int64_t)h * L.sh;
  const const_i32_t idx_row =
      (const_i32_t)(idx ? idx + ((int64_t)bh * L.Tq + qt) * L.Ktot : idx);

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

  // ---- DMA mapping: load i of this thread fills 16-byte slot (wave*LPT + i)*64 + lane.
  // Byte offsets from the block's first row are 32-bit and block-independent for
  // full blocks; the base pointer of a block is wave-uniform.
  auto dma_row = [&](int i) { return ((wave * LPT + i) * 64 + lane) / CPR; };
  auto dma_col = [&](int i, bool is_v) {
    const int r = dma_row(i);
    const int pc = ((wave * LPT + i) * 64 + lane) % CPR;   // physical chunk
    return (pc ^ (is_v ? swz_v<CPR>(r) : swz_k<CPR>(r))) * 8;
  };
  uint32_t koff[LPT], voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    koff[i] = (uint32_t)(((int64_t)dma_row(i) * L.sn + dma_col(i, false)) * 2);
    voff[i] = (uint32_t)(((int64_t)dma_row(i) * L.sn + dma_col(i, true)) * 2);
  }
  const char* kbase = reinterpret_cast<const char*>(k + head_off);
  const char* vbase = reinterpret_cast<const char*>(v + head_off);
  auto dma = [&](const char* base, const uint32_t* off, bool is_v, const Block& blk,
                 uint16_t* dst) {
    const char* g = base + blk.start * L.sn * 2;
    if (blk.n == KBK) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        uint32_t o = off[i];
        asm volatile("" : "+v"(o));
        __builtin_amdgcn_global_load_lds((const void*)(g + o),
                                         (lds_void_t)(reinterpret_cast<char*>(dst) + (wave * LPT + i) * 1024),
                                         16, 0, 0);
      }
    } else {
      // partial block: rows past the end repeat the last row (masked later).  The lane
      // id is re-read here so that nothing of this rare path stays live in registers.
      int ln = lane;
      asm volatile("" : "+v"(ln) : : "memory");   // also keeps this path a real branch
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int r = ((wave * LPT + i) * 64 + ln) / CPR;
        const int rc = r < blk.n ? r : blk.n - 1;
        const uint32_t o = off[i] - (uint32_t)((r - rc) * (int)L.sn * 2);
        __builtin_amdgcn_global_load_lds((const void*)(g + o),
                                         (lds_void_t)(reinterpret_cast<char*>(dst) + (wave * LPT + i) * 1024),
                                         16, 0, 0);
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int vg2 = (lane >> 4) & 1;
  const int vj = lane & 15;
  // LDS byte addresses.  K operand (row l32 [+32], chunk 2kk+hi) of a block: kR ^ (kk << 5)
  // [+ 32 rows]; the XOR swizzle only touches chunk bits, so kk enters as an XOR and the
  // row half and the stage as plain offsets.  V^T operand (rows 16c + 8r + vrow0, columns
  // 32db + vdcol0 ..): (vR ^ (db << 6)) + (16c + 8r) rows, likewise.
  const uint32_t kR = (uint32_t)l32 * (D * 2) + ((uint32_t)(hi ^ swz_k<CPR>(l32)) << 4);
  const int vrow0 = 4 * hi + (vj >> 2);
  const int vdcol0 = 16 * vg2 + 4 * (vj & 3);
  const uint32_t vR = (uint32_t)vrow0 * (D * 2) +
                      ((uint32_t)((vdcol0 >> 3) ^ swz_v<CPR>(vrow0)) << 4) + (uint32_t)(vdcol0 & 7) * 2;

  // ---- pipeline.  Block i's K sits in Ks[i%2], its V in Vs[i%2].  In iteration i:
  //   S^T = K_i Q^T and the softmax (reads Ks[i%2])
  //   wait for this wave's DMA, barrier          -> V_i and K_{i+1} visible to all waves
  //   V_i^T reads (Vs[i%2])
  //   DMA K_{i+2} -> Ks[i%2], V_{i+1} -> Vs[(i+1)%2]   (both stages were last read
  //                                                       before this barrier)
  //   O^T += V_i^T P_i^T
  // so every DMA has a whole iteration to land and there is one barrier per block.
  BlockIter it;
  Block b0 = it.next<KBK>(L, DN, idx_row);
  Block b1 = it.next<KBK>(L, DN, idx_row);
  if (b0.n > 0) {
    dma(kbase, koff, false, b0, Ks0);
    dma(vbase, voff, true, b0, Vs0);
  }
  if (b1.n > 0) dma(kbase, koff, false, b1, Ks1);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();

  auto step = [&](auto stage) {
    constexpr int ST = decltype(stage)::value;
    uint16_t* Kc = ST ? Ks1 : Ks0;
    uint16_t* Vc = ST ? Vs1 : Vs0;
    const int n = b0.n;

    // ---- S^T = K Q^T for the block's keys, in 32-key halves
    f32x16 s[MBN];
    bf16x8 ka[MBN][D / 16];
    const char* Kb = reinterpret_cast<const char*>(Kc);
    uint32_t kRi = kR;   // kept in one register: the per-kk addresses are formed in the loop
    asm volatile("" : "+v"(kRi));
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mb = 0; mb < MBN; ++mb)
        ka[mb][kk] = *reinterpret_cast<const bf16x8*>(Kb + (kRi ^ (kk << 5)) + mb * 32 * D * 2);
#pragma unroll
    for (int mb = 0; mb < MBN; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mb = 0; mb < MBN; ++mb)
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[mb][kk], qv[kk], s[mb], 0, 0, 0);
    // all operand reads first, then the products (the reads' latency is paid once)
    __builtin_amdgcn_sched_group_barrier(0x100, MBN * D / 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MBN * D / 16, 0);
    // ---- mask keys past the end of a partial block (tile-uniform branch)
    if (n < KBK) {
      int kb = hi * 4;                      // key = kb + c for accumulator entry (mb, e)
      float ninf = -INFINITY;
      asm volatile("" : "+v"(kb), "+v"(ninf) : : "memory");   // a real branch, not selects
#pragma unroll
      for (int mb = 0; mb < MBN; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = mb * 32 + (e >> 2) * 8 + (e & 3);
          if (kb >= n - c) s[mb][e] = ninf;
        }
    }
    // ---- online softmax, exp2 domain.  Weights against the running maximum as it
    // stands, and this lane's sum of them (of the bf16 values the second product uses)
    bf16x8 pb[PCN];
    auto weights = [&]() {
#pragma unroll
      for (int mb = 0; mb < MBN; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          pb[mb * 2 + (e >> 3)][e & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[mb][e], scale_log2, -m_run));
      float bs = 0.f;
#pragma unroll
      for (int c = 0; c < PCN; ++c) {
        const bf16x2 p01 = {pb[c][0], pb[c][1]}, p23 = {pb[c][2], pb[c][3]};
        const bf16x2 p45 = {pb[c][4], pb[c][5]}, p67 = {pb[c][6], pb[c][7]};
        bs = __builtin_amdgcn_fdot2_f32_bf16(p01, ones, bs, false);
        bs = __builtin_amdgcn_fdot2_f32_bf16(p23, ones, bs, false);
        bs = __builtin_amdgcn_fdot2_f32_bf16(p45, ones, bs, false);
        bs = __builtin_amdgcn_fdot2_f32_bf16(p67, ones, bs, false);
      }
      return bs;
    };
    float bs = weights();
    // Kept while no lane's weights sum above kLazySum (so none exceeds it);
    // otherwise (always on the first block, where m_run = -inf gives inf or NaN) the
    // running maximum moves to this block's maximum and the weights are redone.
    if (__builtin_amdgcn_ballot_w64(!(bs <= kLazySum)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < MBN; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      bs = weights();
    }
    l_run += bs;

    // next block two ahead (its scalar index load overlaps the barrier wait)
    const Block b2 = it.next<KBK>(L, DN, idx_row);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA (V_i, K_{i+1}) landed
    __syncthreads();

    // ---- V^T operands of this block, then the next DMA, then O^T += V^T P^T
    uint32_t vRi = vR;
    asm volatile("" : "+v"(vRi));
    bf16x8 va[D / 32][PCN];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int c = 0; c < PCN; ++c) {
        s16x4 part[2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t)(reinterpret_cast<char*>(Vc) + (vRi ^ (db << 6)) + (16 * c + 8 * r) * D * 2));
        // the two halves as one 16-byte operand (whole-vector cast: building it
        // element by element through bf16 scalars is lowered wrongly by the compiler)
        const s16x8 both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
        va[db][c] = __builtin_bit_cast(bf16x8, both);
      }
    if (b2.n > 0) dma(kbase, koff, false, b2, Kc);
    if (b1.n > 0) dma(vbase, voff, true, b1, ST ? Vs0 : Vs1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int c = 0; c < PCN; ++c)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][c], pb[c], o[db], 0, 0, 0);
    b0 = b1;
    b1 = b2;
  };
  while (b0.n > 0) {
    step(std::integral_constant<int, 0>{});
    if (b0.n <= 0) break;
    step(std::integral_constant<int, 1>{});
  }

  // ---- normalise and store (a row with no key at all, possible only when every index
  // entry is padding and there is no dense range, is written as zeros)
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* op = out + head_off + my_q * L.sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + i * 8 + hi * 4;
        const __bf16 o0 = (__bf16)(o[db][i * 4 + 0] * inv);
        const __bf16 o1 = (__bf16)(o[db][i * 4 + 1] * inv);
        const __bf16 o2 = (__bf16)(o[db][i * 4 + 2] * inv);
        const __bf16 o3 = (__bf16)(o[db][i * 4 + 3] * inv);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, o0) | ((uint32_t)__builtin_bit_cast(uint16_t, o1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, o2) | ((uint32_t)__builtin_bit_cast(uint16_t, o3) << 16);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (lse && hi == 0) {
      lse[(int64_t)bh * L.qlen + (my_q - L.q0)] =
          (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
    }
  }
}

// Block table of one (b, h, query tile) for the ping-pong kernel: the key blocks in the
// order BlockIter yields them, as (first token, rows), built once per workgroup by one
// wave with vector loads and lane ballots (tiles hold at most two 64-key blocks), so
// that the main loop reads one LDS entry per block instead of walking the index row.
constexpr int kTabCap = 3072;

template <int KBK, int CAP>
__device__ __forceinline__ int build_block_table(const LayerDev& L, const DenseDev& DN,
                                                 const int32_t* idx_row, int lane, int2* tab) {
  int count = 0;
  const int bpt = L.tile / KBK;   // 1 or 2
  for (int s = 0; s < L.n_seg; ++s) {
    const int koff = L.seg[s].koff, K = L.seg[s].K;
    const int64_t len = L.seg[s].len, start = L.seg[s].start;
    for (int c0 = 0; c0 < K; c0 += 64) {
      const int e = c0 + lane;
      const bool in = e < K;
      const int t = in ? (idx_row ? idx_row[koff + e] : e) : 0;
      // the first -1 ends this segment's block
      const uint64_t negm = __builtin_amdgcn_ballot_w64(in && t < 0);
      const int limit = negm ? (int)__builtin_ctzll(negm) : 64;
      int nb = 0;
      int64_t rem = 0;
      if (in && lane < limit) {
        rem = len - (int64_t)t * L.tile;
        nb = rem <= 0 ? 0 : (rem >= (int64_t)bpt * KBK ? bpt : (int)((rem + KBK - 1) / KBK));
      }
      const uint64_t b1 = __builtin_amdgcn_ballot_w64(nb == 1);
      const uint64_t b2 = __builtin_amdgcn_ballot_w64(nb == 2);
      const int pre = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b1, 0)) +
                      2 * (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b2 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b2, 0));
      for (int sb = 0; sb < nb; ++sb) {
        const int64_t r2 = rem - (int64_t)sb * KBK;
        const int pos = count + pre + sb;
        if (pos < CAP)
          tab[pos] = make_int2((int)(start + (int64_t)t * L.tile + (int64_t)sb * KBK), (int)(r2 < KBK ? r2 : KBK));
      }
      count += __builtin_popcountll(b1) + 2 * __builtin_popcountll(b2);
      if (negm) break;
    }
  }
  for (int r = 0; r < DN.n; ++r) {
    const int64_t len = DN.r[r].len, st = DN.r[r].start;
    const int nbr = (int)((len + KBK - 1) / KBK);
    for (int b0 = 0; b0 < nbr; b0 += 64) {
      const int bi = b0 + lane;
      const int pos = count + bi;
      if (bi < nbr && pos < CAP) {
        const int64_t r2 = len - (int64_t)bi * KBK;
        tab[pos] = make_int2((int)(st + (int64_t)bi * KBK), (int)(r2 < KBK ? r2 : KBK));
      }
    }
    count += nbr;
  }
  return count;
}

// Two-group ("ping-pong") form for 128-row tiles.  Eight waves in two groups of four
// work on the same 128 query rows: group 0 takes the even key blocks of the row's block
// list, group 1 the odd ones, each with its own two-stage K and V rings.  Workgroup
// barriers cut time into slots; in every slot one group runs its products (PV of its
// previous block, then S^T of its current block: MFMAs and LDS reads only) while the
// other runs the softmax of its current block, so the two waves sharing a SIMD keep the
// matrix core and the vector ALU busy at once.  Group 1 runs one slot behind group 0.
// DMA: a group's K tile is loaded by its own softmax slot, its V tile by the other
// group's products slot after the last product (where that wave would otherwise wait at
// the barrier); every wave ends each slot by waiting for the loads it issued two slots
// earlier.  The two partial results (each with its own running maximum) are merged
// through LDS at the end.
//
// T2: two 64-row query tiles per workgroup.  Waves 0-1 of each group take the first
// tile and waves 2-3 the second; each half has its own block table (half of the LDS
// table) and its own K and V stages (half of the group's array), and blocks are 32
// keys.  Every wave runs the slot count of the longer of the two block lists.
//
// K8: Q and K are FP8 (E4M3FN) codes and the first product runs on
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales); V, P and the second product stay
// bf16.  A K row is then d bytes: the K stages use the first half of their space, a
// block's K DMA is half as many loads, and S^T takes 2 * d / 64 products instead of d / 8.
//
// V8 (with K8): V is FP8 too, in d-major blocks of 64 tokens (one contiguous DMA of d x 64
// bytes per block, see the V quantiser), and P is rounded to E4M3FN for the second product, also on the
// f8f6f4 matrix cores: O^T += V^T . P^T, A = V^T rows straight from LDS, B = P^T packed
// from S^T's accumulators.  For that, S^T's K operand rows are read in a permuted order:
// accumulator row 8 g + 4 h + t of the 32-row tile mb holds key 32 h + 16 mb + 4 g + t, so
// the 32 weights a lane holds are keys 32 h .. 32 h + 31 in order, which is the B
// operand's layout.  The row sums come from one more product with an all-ones A operand,
// so the normaliser is the sum of exactly the rounded weights the numerator used.  The
// weights are 2^(x + kW8Shift) for exponents x against the running maximum, kept while no
// x exceeds kW8Lazy (every weight < 2^8.5, inside E4M3's range of 448).
template <int D, bool K8, bool T2, bool V8 = false>
__device__ __forceinline__ void pingpong_attn(
    const LayerDev& L, const DenseDev& DN, const std::conditional_t<K8, uint8_t, uint16_t>* __restrict__ q,
    const std::conditional_t<K8, uint8_t, uint16_t>* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ order, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, int by_heads, int64_t vt_head_bytes = 0,
    float out_scale = 1.0f) {
  using KT = std::conditional_t<K8, uint8_t, uint16_t>;
  static_assert(!(K8 && T2), "the FP8 form runs 128-row tiles only");
  static_assert(!V8 || K8, "FP8 V needs FP8 Q and K");
  constexpr int NW = 4;                       // waves per group
  constexpr int KBK = T2 ? 32 : KB;           // keys per block
  constexpr int MB = KBK / 32;                // 32-key S^T tiles per block
  constexpr int PC = KBK / 16;                // 16-key slices of the PV contraction
  constexpr int WS = T2 ? 2 : NW;             // waves that share one block stream (one query tile)
  constexpr int TS = 64 * WS;                 // threads per stream
  constexpr int CAP = T2 ? kTabCap / 2 : kTabCap;   // block-table entries per stream
  constexpr int CPR = D / 8;                  // 16-byte chunks per bf16 row
  constexpr int SLOTS = V8 ? KBK * D / 16 : KBK * CPR;   // 16-byte slots of a V block
  constexpr int LPT = SLOTS / TS;             // V DMA loads per thread per block
  constexpr int KCPR = K8 ? D / 16 : CPR;     // 16-byte chunks per K row
  constexpr int LPK = KBK * KCPR / TS;        // K DMA loads per thread per block
  constexpr int NPV = (D / 32) * PC;          // PV products per block
  constexpr int NS = K8 ? 2 * (D / 64) : MB * (D / 16);   // S^T products per block
  static_assert(SLOTS % TS == 0 && (KBK * KCPR) % TS == 0 && LPK + LPT < 16, "block split");

  // one array per group: K stage 0, K stage 1, V stage 0, V stage 1 (the DMA is issued
  // from inline assembly, so no compiler-inserted wait depends on their aliasing)
  __shared__ __attribute__((aligned(1024))) uint16_t sg0[4 * KB * D], sg1[4 * KB * D];
  __shared__ float2 sml[NW * 64];
  __shared__ int2 stab[kTabCap];
  __shared__ int snblk[2];

  const int tid = threadIdx.x;
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
  const int half = T2 ? (wave >> 1) : 0;          // the stream (query tile) of this wave
  const int wsi = T2 ? (wave & 1) : wave;         // this wave's index inside its stream
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // A work item is processing position it (T2: the pair of positions 2 it and 2 it + 1, the
  // second one absent for the last item of an odd tile count); its query tile is the
  // position itself or the caller's order entry for it (no tile: nothing to do)
  int bh, it;
  if (!work_item(L, T2 ? (L.Tq + 1) >> 1 : L.Tq, by_heads, bh, it)) return;   // padding workgroup
  const int h = bh % L.H;
  const int b = bh / L.H;
  auto tile_of = [&](int pos) { return by_heads == 1 ? (pos < L.Tq ? pos : -1) : tile_at(L, order, bh, pos); };
  const int qt_at = tile_of(T2 ? 2 * it + half : it);
  if (!T2 && qt_at < 0) return;                   // uniform over the workgroup
  const bool tile_ok = qt_at >= 0;
  const int qt = tile_ok ? qt_at : 0;

  const int64_t q_first = L.q0 + (int64_t)qt * L.tile;
  const int64_t q_end = L.q0 + L.qlen;
  const int64_t head_off = (int64_t)b * L.sb + (int64_t)h * L.sh;

  const int64_t my_q = q_first + wsi * 32 + l32;
  const bool q_ok = tile_ok && my_q < q_end;
  // Q^T operand: bf16, 8 head-dim values per product; FP8, 32 bytes per product
  // (bytes 64 ks + 32 hi .. +31 of the row, the same bytes the K operand reads)
  bf16x8 qv[K8 ? 1 : D / 16];
  i32x8 qv8[K8 ? D / 64 : 1];
  if constexpr (K8) {
    const uint8_t* qp = q + head_off + (q_ok ? my_q : q_first) * L.sn + 32 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const uint4 w0 = q_ok ? *reinterpret_cast<const uint4*>(qp + 64 * ks) : make_uint4(0, 0, 0, 0);
      const uint4 w1 = q_ok ? *reinterpret_cast<const uint4*>(qp + 64 * ks + 16) : make_uint4(0, 0, 0, 0);
      qv8[ks] = i32x8{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
    }
  } else {
    const uint16_t* qp = q + head_off + (q_ok ? my_q : q_first) * L.sn + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 w = q_ok ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qv[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // A products slot with no previous block multiplies P = 0 by a V stage: both V stages of
  // each stream start zeroed, so that a stage no DMA has filled yet holds finite values.
  // The stores are 1 KB stripes that cross the slices the stream's waves later fill by
  // LDS DMA, so they go before the workgroup barrier below: no wave issues a DMA into a
  // stage while another wave's zero stores to it may still be pending.
  {
    uint4* const z = reinterpret_cast<uint4*>((grp ? sg1 : sg0) + half * 4 * KBK * D + 2 * KBK * D);
#pragma unroll
    for (int i = 0; i < 2 * KBK * D * 2 / 16 / TS; ++i) z[i * TS + (tid & (TS - 1))] = make_uint4(0, 0, 0, 0);
  }
  // wave s (s < number of streams) builds stream s's table; a stream without a tile has none
  // (its index-row loads go out while Q's are still in flight)
  if (tid < (T2 ? 128 : 64)) {
    const int st = tid >> 6;
    const int qts = tile_of(T2 ? 2 * it + st : it);
    int n = 0;
    if (qts >= 0) {
      const int32_t* const row = idx ? idx + ((int64_t)bh * L.Tq + qts) * L.Ktot : nullptr;
      n = build_block_table<KBK, CAP>(L, DN, row, lane, stab + st * CAP);
    }
    if (lane == 0) snblk[st] = n;
  }
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): Q is in registers before any DMA is issued
  const int nblk = __builtin_amdgcn_readfirstlane(snblk[half]);
  // slots: every wave runs as many as the longer stream needs (the barriers are shared)
  const int nmax = T2 ? __builtin_amdgcn_readfirstlane(max(snblk[0], snblk[1])) : nblk;
  const int2* const tab = stab + half * CAP;

  // K row swizzle: bf16 rows (256 or 128 bytes) as in the single-pipeline kernel; FP8
  // rows (128 or 64 bytes) by row pair (quad for 64 bytes), so that the 16 rows one
  // 16-lane operand read touches cover every 16-byte bank group once
  auto kswz = [](int r) {
    if constexpr (K8) return (r >> (KCPR == 8 ? 1 : 2)) & (KCPR - 1);
    else return swz_k<CPR>(r);
  };
  // load i of this thread fills 16-byte LDS slot (wsi * loads + i) * 64 + lane of its stream
  uint32_t koff[LPK], voff[LPT];
#pragma unroll
  for (int i = 0; i < LPK; ++i) {
    const int slot = (wsi * LPK + i) * 64 + lane;
    const int r = slot / KCPR;
    koff[i] = (uint32_t)((int64_t)r * L.sn * (int64_t)sizeof(KT) + (((slot % KCPR) ^ kswz(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int slot = (wsi * LPT + i) * 64 + lane;
    if constexpr (V8) {
      voff[i] = (uint32_t)slot * 16u;           // a V block is one contiguous run of d x 64 bytes
    } else {
      const int r = slot / CPR;
      voff[i] = (uint32_t)((int64_t)r * L.sn * 2 + (((slot % CPR) ^ swz_v<CPR>(r)) << 4));
    }
  }
  const char* kbase = reinterpret_cast<const char*>(k + head_off);
  const char* vbase = V8 ? static_cast<const char*>(v) + (int64_t)bh * vt_head_bytes
                         : reinterpret_cast<const char*>(static_cast<const uint16_t*>(v) + head_off);
  // One 16-byte-per-lane HBM -> LDS load.  Issued from inline assembly so that the
  // compiler's wait-count pass does not see it: it would otherwise wait for every LDS
  // DMA in flight before each LDS operand read.  All waits for these loads are explicit
  // (s_waitcnt vmcnt) and ordered by the workgroup barriers.
  // NL such loads fill consecutive 1 KB LDS slots from lds_addr; one asm block steps M0
  // by 1 KB between them, so that no per-load address has to stay in a scalar register.
  auto dma_n = [](auto nl, const char* g, const uint32_t (&o)[4], uint32_t lds_addr) {
    constexpr int NL = decltype(nl)::value;
    static_assert(NL == 1 || NL == 2 || NL == 4, "loads per block and thread");
    if constexpr (NL == 1) {
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(lds_addr), "v"(o[0]), "s"(g)
                   : "memory", "m0");
    } else if constexpr (NL == 2) {
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3\n\t"
                   "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3"
                   :
                   : "s"(lds_addr), "v"(o[0]), "v"(o[1]), "s"(g)
                   : "memory", "m0", "scc");
    } else {
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %5\n\t"
                   "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %5\n\t"
                   "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %5\n\t"
                   "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %5"
                   :
                   : "s"(lds_addr), "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "s"(g)
                   : "memory", "m0", "scc");
    }
  };
  // a block's K (IS_V = 0) or V (IS_V = 1) rows; rows past a partial block's end load
  // its last row again
  auto dma = [&](auto is_v, const char* base, const uint32_t* off, const Block& blk, uint16_t* dst) {
    constexpr bool IS_V = decltype(is_v)::value;
    constexpr int NL = IS_V ? LPT : LPK;
    constexpr int CP = IS_V ? CPR : KCPR;
    constexpr int EB = IS_V ? 2 : (int)sizeof(KT);
    constexpr bool BLOCKED = IS_V && V8;        // FP8 V: the 64-token block of the first key
    const char* g = BLOCKED ? base + (blk.start >> 6) * (int64_t)(D * 64) : base + blk.start * L.sn * EB;
    const uint32_t l0 = (uint32_t)(uintptr_t)(lds_void_t)(reinterpret_cast<char*>(dst) + wsi * NL * 1024);
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (BLOCKED || blk.n == KBK) {
#pragma unroll
      for (int i = 0; i < NL; ++i) o[i] = off[i];
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln) : : "memory");
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int r = ((wsi * NL + i) * 64 + ln) / CP;
        const int rc = r < blk.n ? r : blk.n - 1;
        o[i] = off[i] - (uint32_t)((r - rc) * (int)L.sn * EB);
      }
    }
    dma_n(std::integral_constant<int, NL>{}, g, o, l0);
  };
  const std::integral_constant<bool, false> kK{};
  const std::integral_constant<bool, true> kV{};
  // workgroup barrier without a memory fence (outstanding DMA is waited for explicitly)
  auto barrier = []() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // wait until at most n of this wave's DMA loads are outstanding (n in {0, LPK, LPT, LPK + LPT})
  auto wait_vm = [](int n) {
    if (n == LPK + LPT) __builtin_amdgcn_s_waitcnt(0x0F70 | (LPK + LPT));
    else if (n == LPT) __builtin_amdgcn_s_waitcnt(0x0F70 | LPT);
    else if (n == LPK) __builtin_amdgcn_s_waitcnt(0x0F70 | LPK);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  f32x16 osum;                                // V8: every entry of a lane is its row's sum of weights
#pragma unroll
  for (int e = 0; e < 16; ++e) osum[e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int vg2 = (lane >> 4) & 1;
  const int vj = lane & 15;
  const uint32_t kR = (uint32_t)l32 * (D * 2) + ((uint32_t)(hi ^ swz_k<CPR>(l32)) << 4);
  const int vrow0 = 4 * hi + (vj >> 2);
  const int vdcol0 = 16 * vg2 + 4 * (vj & 3);
  const uint32_t vR = (uint32_t)vrow0 * (D * 2) +
                      ((uint32_t)((vdcol0 >> 3) ^ swz_v<CPR>(vrow0)) << 4) + (uint32_t)(vdcol0 & 7) * 2;

  auto body = [&](auto G) {
    constexpr int GRP = decltype(G)::value;
    int j = 0;
    // this group's stages for this wave's stream (T2: each half of the group array)
    uint16_t* const Gb = (GRP ? sg1 : sg0) + half * 4 * KBK * D;
    uint16_t* const Ks0 = Gb;
    uint16_t* const Ks1 = Gb + KBK * D;
    uint16_t* const Vs0 = Gb + 2 * KBK * D;
    uint16_t* const Vs1 = Gb + 3 * KBK * D;
    // operand addresses: group base plus the lane's swizzled offset for every K column
    // step and every V column block; stage and row offsets are instruction immediates
    const uint32_t gbase = (uint32_t)(uintptr_t)(lds_void_t)Gb;
    uint32_t kA[K8 ? 2 * (D / 64) : D / 16], vA[D / 32], vB[2];
    if constexpr (K8) {
      // FP8: product ks reads the 16-byte chunks 4 ks + 2 hi and 4 ks + 2 hi + 1 of row l32
      // (V8: of the permuted row, 16 rows further for the second 32-row tile)
      const int kr = V8 ? 32 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3) : l32;
#pragma unroll
      for (int c = 0; c < 2 * (D / 64); ++c) {
        kA[c] = gbase + (uint32_t)kr * D + ((uint32_t)((4 * (c >> 1) + 2 * hi + (c & 1)) ^ kswz(kr)) << 4);
        asm volatile("" : "+v"(kA[c]));
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        kA[kk] = gbase + (kR ^ (kk << 5));
        asm volatile("" : "+v"(kA[kk]));
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      vA[db] = gbase + (vR ^ (db << 6));
      asm volatile("" : "+v"(vA[db]));
    }
    if constexpr (V8) {
      // V^T operand: row 32 db + l32 of the block (64 bytes), keys 32 hi .. 32 hi + 31, i.e.
      // logical chunks 2 hi and 2 hi + 1, swizzled by (row >> 1) & 3 like the quantiser
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        vB[part] = gbase + (uint32_t)l32 * 64 + ((uint32_t)((2 * hi + part) ^ ((l32 >> 1) & 3)) << 4);
        asm volatile("" : "+v"(vB[part]));
      }
    }
    // this group's j-th block c_j is block 2j + GRP of the table; K(c_j) and V(c_j)
    // live in stage j % 2
    auto entry = [&](int i) {
      if (i >= nblk) return Block{0, 0};
      const int2 e = tab[i];
      return Block{(int64_t)__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y)};
    };
    Block cur = entry(GRP);                   // c_j
    Block nx1 = entry(2 + GRP);               // c_{j+1}
    Block nx2 = entry(4 + GRP);               // c_{j+2}
    Block prev{0, 0};                         // c_{j-1}
    if (cur.n > 0) dma(kK, kbase, koff, cur, Ks0);
    if (nx1.n > 0) dma(kK, kbase, koff, nx1, Ks1);
    int np = 0;                               // this wave's loads issued in the previous phase
    if (cur.n > 0) {
      dma(kV, vbase, voff, cur, Vs0);
      np = LPT;
    }
    wait_vm(np);                              // K(c_0) and K(c_1) landed
    barrier();
    if (GRP) {                                // group 1 runs one slot behind
      barrier();
      np = 0;
    }
    // V tile the products slot issues for the other group: group 1's slot j loads group 0's
    // block j + 1, group 0's slot j (j >= 1) loads group 1's block j
    Block xo = GRP ? entry(2) : Block{0, 0};
    uint16_t* const Go = (GRP ? sg0 : sg1) + half * 4 * KBK * D;

    f32x16 s[MB];
    bf16x8 pb[PC];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
    for (int c = 0; c < PC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[c][e] = (__bf16)0.f;
    // V8: P^T as the second product's B operand, byte 16 mb + e of a lane = weight of
    // accumulator entry (mb, e) = key 32 hi + 16 mb + e
    i32x8 pb8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const i32x8 ones8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                         0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3FN 1.0

    typedef __attribute__((address_space(3))) const bf16x8* lds_bf16x8_t;
    auto read_v = [&](int ST, bf16x8 (&va)[D / 32][PC]) {   // V stage ST
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int c = 0; c < PC; ++c) {
          s16x4 part[2];
#pragma unroll
          for (int r = 0; r < 2; ++r)
            part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t)(uintptr_t)(vA[db] + (2 + ST) * KBK * D * 2 + (16 * c + 8 * r) * D * 2));
          const s16x8 both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
          va[db][c] = __builtin_bit_cast(bf16x8, both);
        }
    };
    auto read_k = [&](int ST, auto& ka) {   // K stage ST, bf16: ka[MB][D / 16]
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          ka[mb][kk] = *(lds_bf16x8_t)(uintptr_t)(kA[kk] + ST * KBK * D * 2 + mb * 32 * D * 2);
    };
    typedef __attribute__((address_space(3))) const i32x4* lds_i32x4_t;
    auto read_k8 = [&](int ST, auto& ka) {  // K stage ST, FP8: ka[2][D / 64], two chunks each
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const i32x4 a = *(lds_i32x4_t)(uintptr_t)(kA[2 * ks] + ST * KBK * D * 2 + mb * (V8 ? 16 : 32) * D);
          const i32x4 b = *(lds_i32x4_t)(uintptr_t)(kA[2 * ks + 1] + ST * KBK * D * 2 + mb * (V8 ? 16 : 32) * D);
          ka[mb][ks] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    auto mul_pv = [&](const bf16x8 (&va)[D / 32][PC]) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int c = 0; c < PC; ++c)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][c], pb[c], o[db], 0, 0, 0);
    };
    auto mul_s = [&](const auto& ka) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[mb][kk], qv[kk], s[mb], 0, 0, 0);
    };
    // FP8 E4M3 operands (format code 0 for A and B), unit block scales (E8M0 code 127)
    auto mul_s8 = [&](const auto& ka) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          s[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[mb][ks], qv8[ks], s[mb], 0, 0, 0, 127, 0, 127);
    };

    // products slot of c_j: PV of c_{j-1} (V stage (j-1)%2), S^T of c_j (K stage j%2).
    // Always both, with no branch: a missing c_{j-1} has P = 0 against finite V stage
    // contents (adds exactly zero), a missing c_j gives S^T values that nothing reads.
    // Operand reads run four products ahead; no VALU instruction is left in this slot.
    auto mphase = [&](auto stage) {
      constexpr int ST = decltype(stage)::value;
      bf16x8 va[D / 32][PC];
      if constexpr (!V8) read_v(1 - ST, va);
      // V reads (2 per PV product), then K reads; 8 reads go first, then each PV
      // product is followed by two reads, the last four by one
      if constexpr (V8) {
        // V^T operands (two 16-byte reads per 32-row block), K operands, then the products:
        // PV of c_{j-1} per 32 rows of d, the row sums, S^T of c_j
        i32x8 va8[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const i32x4 a = *(lds_i32x4_t)(uintptr_t)(vB[0] + (2 + (1 - ST)) * KBK * D * 2 + db * 32 * 64);
          const i32x4 b = *(lds_i32x4_t)(uintptr_t)(vB[1] + (2 + (1 - ST)) * KBK * D * 2 + db * 32 * 64);
          va8[db] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        i32x8 ka[2][D / 64];
        read_k8(ST, ka);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va8[db], pb8, o[db], 0, 0, 0, 127, 0, 127);
        osum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, pb8, osum, 0, 0, 0, 127, 0, 127);
        mul_s8(ka);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 32), 0);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * NS / (D / 32), 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1 + NS, 0);
      } else if constexpr (K8) {
        i32x8 ka[2][D / 64];
        read_k8(ST, ka);
        mul_pv(va);
        mul_s8(ka);
        constexpr int NKR = 2 * NS;             // two 16-byte reads per S^T product
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < NPV - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (NKR > 4) __builtin_amdgcn_sched_group_barrier(0x100, NKR - 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
      } else {
        bf16x8 ka[MB][D / 16];
        read_k(ST, ka);
        mul_pv(va);
        mul_s(ka);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < NPV - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < NS - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      if constexpr (K8) {
        // The FP8 products have no side effects and nothing in this block reads their
        // results, so the compiler would move them past the DMA's branch below, behind
        // a DMA issue that can stall for hundreds of cycles.  An empty use keeps them here.
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(s[mb]));
        if constexpr (V8) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(o[db]));
          asm volatile("" : "+v"(osum));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      int nc = 0;
      if (xo.n > 0) {
        // group 1 fills group 0's V stage (j+1)%2, group 0 fills group 1's V stage j%2
        dma(kV, vbase, voff, xo, Go + (2 + (GRP ? 1 - ST : ST)) * KBK * D);
        nc = LPT;
      }
      wait_vm(nc + np);                       // loads of two phases ago have landed
      np = nc;
      barrier();
    };
    // softmax slot of c_j.  First the DMA of K(c_{j+2}) into the K stage the products slot
    // has just released (j%2), then the softmax; the table entries of c_{j+3} and of the
    // other group's next V tile are read here for the following slots.
    auto vphase = [&](auto stage) {
      constexpr int ST = decltype(stage)::value;
      uint16_t* Kf = ST ? Ks1 : Ks0;
      const int i3 = 2 * (j + 3) + GRP;
      const int2 e3 = i3 < nblk ? tab[i3] : make_int2(0, 0);
      const int io = GRP ? 2 * (j + 2) : 2 * (j + 1) + 1;
      const int2 eo = io < nblk ? tab[io] : make_int2(0, 0);
      int nc = 0;
      if (nx2.n > 0) {
        dma(kK, kbase, koff, nx2, Kf);
        nc = LPK;
      }
      if (cur.n > 0) {
        const int n = cur.n;
        if (n < KBK) {
          int kb = V8 ? hi * 32 : hi * 4;
          float ninf = -INFINITY;
          asm volatile("" : "+v"(kb), "+v"(ninf) : : "memory");
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              // key of accumulator entry (mb, e) is kb + c (V8: the permuted K rows)
              const int c = V8 ? mb * 16 + e : mb * 32 + (e >> 2) * 8 + (e & 3);
              if (kb >= n - c) s[mb][e] = ninf;
            }
        }
        // weights against the running maximum as it stands, and this lane's sum of them
        auto weights = [&]() {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              pb[mb * 2 + (e >> 3)][e & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[mb][e], scale_log2, -m_run));
          // four independent sums (one chain of PC * 4 dependent dot products is slower)
          float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
#pragma unroll
          for (int c = 0; c < PC; ++c) {
            const bf16x2 p01 = {pb[c][0], pb[c][1]}, p23 = {pb[c][2], pb[c][3]};
            const bf16x2 p45 = {pb[c][4], pb[c][5]}, p67 = {pb[c][6], pb[c][7]};
            b0 = __builtin_amdgcn_fdot2_f32_bf16(p01, ones, b0, false);
            b1 = __builtin_amdgcn_fdot2_f32_bf16(p23, ones, b1, false);
            b2 = __builtin_amdgcn_fdot2_f32_bf16(p45, ones, b2, false);
            b3 = __builtin_amdgcn_fdot2_f32_bf16(p67, ones, b3, false);
          }
          return (b0 + b1) + (b2 + b3);
        };
        if constexpr (V8) {
          // Weights are kept against the running maximum while no exponent exceeds kW8Lazy;
          // otherwise (the first block too) the maximum moves to this block's.  The row sum
          // comes from the products slot (an all-ones MFMA over the FP8 weights).
          // four independent max chains (a single chain of 16 dependent max3 waits on each)
          float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mq[e & 3] = fmaxf(mq[e & 3], s[mb][e]);
          float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
          if (__builtin_amdgcn_ballot_w64(!(fmaf(mx, scale_log2, -m_run) <= kW8Lazy)) != 0) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
              for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
#pragma unroll
            for (int e = 0; e < 16; ++e) osum[e] *= alpha;
          }
          // dword w of the B operand: keys 4w..4w+3 of this lane's 32, E4M3FN nearest even
          const float off = kW8Shift - m_run;
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int mb = w >> 2, e = 4 * (w & 3);
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[mb][e + 0], scale_log2, off));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[mb][e + 1], scale_log2, off));
            const float p2 = __builtin_amdgcn_exp2f(fmaf(s[mb][e + 2], scale_log2, off));
            const float p3 = __builtin_amdgcn_exp2f(fmaf(s[mb][e + 3], scale_log2, off));
            // the first conversion writes bytes 0-1 and the second bytes 2-3, so the old
            // value passed to the first (the previous block's dword) is fully replaced
            const int dw = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pb8[w], false);
            pb8[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, dw, true);
          }
        } else {
        float bs = weights();
        // Weights are kept while no lane's weights (16 per 32 keys) sum above kLazySum
        // (none exceeds it then).  Otherwise (the first block: m_run = -inf gives inf or NaN)
        // the running maximum moves to this block's maximum and the weights are redone.
        if (__builtin_amdgcn_ballot_w64(!(bs <= kLazySum)) != 0) {
          float mx = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
          const float m_new = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
          bs = weights();
        }
        l_run += bs;
        }
      } else {
        // no block: the next PV adds zero
#pragma unroll
        for (int c = 0; c < PC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[c][e] = (__bf16)0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) pb8[w] = 0;
      }
      const Block nx3{(int64_t)__builtin_amdgcn_readfirstlane(e3.x), __builtin_amdgcn_readfirstlane(e3.y)};
      xo = Block{(int64_t)__builtin_amdgcn_readfirstlane(eo.x), __builtin_amdgcn_readfirstlane(eo.y)};
      wait_vm(nc + np);                       // loads of two phases ago have landed
      np = nc;
      __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): no scalar load stays in flight
      barrier();
      prev = cur;
      cur = nx1;
      nx1 = nx2;
      nx2 = nx3;
      ++j;
    };
    // slots: ceil(nmax / 2) + 1 products/softmax pairs, the same count in every wave
    const int iters = nmax > 0 ? (nmax + 1) / 2 + 1 : 0;
    while (j < iters) {
      mphase(std::integral_constant<int, 0>{});
      vphase(std::integral_constant<int, 0>{});
      if (j >= iters) break;
      mphase(std::integral_constant<int, 1>{});
      vphase(std::integral_constant<int, 1>{});
    }
    if (!GRP) barrier();                      // group 0 matches group 1's first slot
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): no DMA left in flight
  };
  if (grp == 0)
    body(std::integral_constant<int, 0>{});
  else
    body(std::integral_constant<int, 1>{});

  if constexpr (V8) l_run = osum[0];            // the whole row's sum, in both halves
  // ---- merge group 1's partial result into group 0's (K/V stages are free now).  Each
  // wave of group 1 parks its D/32 accumulator tiles (16 floats per lane each) in sg0:
  // (D/32) * 4 float4 per lane, so NW waves fill exactly sg0 at either head dimension.
  constexpr int kMergeF4 = (D / 32) * 4 * 64;     // float4 slots per wave
  static_assert(NW * kMergeF4 * sizeof(float4) <= sizeof(sg0), "merge area exceeds sg0");
  __syncthreads();
  float4* const mo = reinterpret_cast<float4*>(sg0) + wave * kMergeF4 + lane;
  if (grp) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        mo[(db * 4 + e4) * 64] = make_float4(o[db][4 * e4], o[db][4 * e4 + 1], o[db][4 * e4 + 2], o[db][4 * e4 + 3]);
    sml[wave * 64 + lane] = make_float2(m_run, l_run);
  }
  __syncthreads();
  if (grp) return;
  {
    const float2 ml = sml[wave * 64 + lane];
    const float m = fmaxf(m_run, ml.x);
    const float fa = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    const float fb = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - m);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const float4 w = mo[(db * 4 + e4) * 64];
        o[db][4 * e4 + 0] = o[db][4 * e4 + 0] * fa + w.x * fb;
        o[db][4 * e4 + 1] = o[db][4 * e4 + 1] * fa + w.y * fb;
        o[db][4 * e4 + 2] = o[db][4 * e4 + 2] * fa + w.z * fb;
        o[db][4 * e4 + 3] = o[db][4 * e4 + 3] * fa + w.w * fb;
      }
    l_run = l_run * fa + ml.y * fb;
    m_run = m;
  }

  float l_tot = l_run;
  if constexpr (!V8) {
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  }
  const float inv = l_tot > 0.f ? out_scale / l_tot : 0.f;
  if (q_ok) {
    uint16_t* op = out + head_off + my_q * L.sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + i * 8 + hi * 4;
        const __bf16 o0 = (__bf16)(o[db][i * 4 + 0] * inv);
        const __bf16 o1 = (__bf16)(o[db][i * 4 + 1] * inv);
        const __bf16 o2 = (__bf16)(o[db][i * 4 + 2] * inv);
        const __bf16 o3 = (__bf16)(o[db][i * 4 + 3] * inv);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, o0) | ((uint32_t)__builtin_bit_cast(uint16_t, o1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, o2) | ((uint32_t)__builtin_bit_cast(uint16_t, o3) << 16);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (lse && hi == 0) {
      const float m_lse = V8 ? m_run - kW8Shift : m_run;   // V8: the weights carry 2^kW8Shift
      lse[(int64_t)bh * L.qlen + (my_q - L.q0)] =
          (m_lse + __log2f(l_tot)) * 0.69314718055994530942f;
    }
  }
}

template <int D>
__global__ __launch_bounds__(512, 1) void sparse_attn_pingpong_kernel(
    LayerDev L, DenseDev DN, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, int by_heads) {
  pingpong_attn<D, false, false>(L, DN, q, k, v, idx, order, scale_log2, out, lse, by_heads);
}

// 64-row tiles: one workgroup takes two neighbouring query tiles, waves 0-1 and 2-3 of each
// group one tile each, with 32-key blocks (each tile's own block stream and table).
template <int D>
__global__ __launch_bounds__(512, 1) void sparse_attn_pingpong_pair_kernel(
    LayerDev L, DenseDev DN, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, int by_heads) {
  pingpong_attn<D, false, true>(L, DN, q, k, v, idx, order, scale_log2, out, lse, by_heads);
}

// Q and K as FP8 codes with per-tensor scales (device floats): logits are
// scale * q_scale * k_scale * <q8, k8>.
template <int D>
__global__ __launch_bounds__(512, 1) void sparse_attn_fp8qk_pingpong_kernel(
    LayerDev L, DenseDev DN, const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    float scale_log2, const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    uint16_t* __restrict__ out, float* __restrict__ lse, int by_heads) {
  pingpong_attn<D, true, false>(L, DN, q, k, v, idx, order, scale_log2 * q_scale[0] * k_scale[0], out, lse,
                                by_heads);
}

// Q and K as above, V as FP8 codes in d-major 64-token blocks, P rounded to E4M3FN: both
// products on the f8f6f4 matrix cores; the output is v_scale * sum(p v) / sum(p).
template <int D>
__global__ __launch_bounds__(512, 1) void sparse_attn_fp8_pingpong_kernel(
    LayerDev L, DenseDev DN, const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ vt, int64_t vt_head_bytes, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ order, float scale_log2, const float* __restrict__ q_scale,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse, int by_heads) {
  pingpong_attn<D, true, false, true>(L, DN, q, k, vt, idx, order, scale_log2 * q_scale[0] * k_scale[0], out,
                                      lse, by_heads, vt_head_bytes, v_scale[0]);
}

}  // namespace

// 128-row tiles take the two-group kernel when the row's block list fits its LDS table
// and every token index fits the table's 32-bit entries
namespace {
// the block list of one query tile fits a two-group table of cap entries of kbk keys, and
// every token index fits the table's 32-bit entries
bool table_fits(const LayerDev& L, const DenseDev& DN, int kbk, int64_t cap) {
  int64_t bound = (int64_t)L.Ktot * (L.tile / kbk);
  int64_t last = 0;
  for (int i = 0; i < DN.n; ++i) {
    bound += (DN.r[i].len + kbk - 1) / kbk;
    last = DN.r[i].start + DN.r[i].len > last ? DN.r[i].start + DN.r[i].len : last;
  }
  for (int i = 0; i < L.n_seg; ++i)
    last = L.seg[i].start + L.seg[i].len > last ? L.seg[i].start + L.seg[i].len : last;
  return bound <= cap && last < ((int64_t)1 << 31);
}

// grid of n work items per (b, h), in work_item's XCD-aware order
// by_heads: 0 by tiles, 1 by heads in tile order, 2 by heads in the caller's order (eight
// heads' K and V, 2 * 2 bytes * d per key token each, within 160 MB of the 256 MB
// Infinity Cache; larger layers keep every XCD on one head so that its keys stay there)
bool grid_of(const LayerDev& L, const DenseDev& DN, int64_t n, const int32_t* idx, dim3& grid, int& by_heads) {
  int64_t keys = 0;
  for (int i = 0; i < L.n_seg; ++i) keys += L.seg[i].len;
  for (int i = 0; i < DN.n; ++i) keys += DN.r[i].len;
  const bool fits = (int64_t)8 * 2 * keys * L.d * 2 <= ((int64_t)160 << 20);
  by_heads = L.B * L.H < 8 ? 0 : idx == nullptr ? 1 : fits ? 2 : 0;
  const int64_t per_xcd = (n + 7) / 8;
  const int64_t nwork = by_heads ? ((int64_t)L.B * L.H + 7) / 8 * 8 * n : (int64_t)L.B * L.H * per_xcd * 8;
  if (nwork > 0x7FFFFFFF) return false;
  grid = dim3((unsigned)nwork);
  return true;
}
}  // namespace

// 128-row tiles take the two-group kernel when the row's block list fits its LDS table
bool two_group_fits(const LayerDev& L, const DenseDev& DN) {
  return L.tile == 128 && table_fits(L, DN, KB, kTabCap);
}

// 64-row tiles take the paired two-group kernel when each tile's list of 32-key blocks
// fits half the table
bool pair_fits(const LayerDev& L, const DenseDev& DN) {
  return L.tile == 64 && table_fits(L, DN, 32, kTabCap / 2);
}

hipError_t launch_sparse_attn(const LayerDev& L, const DenseDev& DN, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* order, float scale, void* out,
                              float* lse, hipStream_t s) {
  const bool two_group = two_group_fits(L, DN);
  const bool pair = pair_fits(L, DN);
  dim3 grid;
  int by_heads;
  if (!grid_of(L, DN, pair ? ((int64_t)L.Tq + 1) / 2 : L.Tq, idx, grid, by_heads)) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.44269504088896340736f;
  const int32_t* const ord = idx ? order : nullptr;
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(out);
  if (pair && L.d == 128)
    hipLaunchKernelGGL((sparse_attn_pingpong_pair_kernel<128>), grid, dim3(512), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  else if (pair)
    hipLaunchKernelGGL((sparse_attn_pingpong_pair_kernel<64>), grid, dim3(512), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  else if (two_group && L.d == 128)
    hipLaunchKernelGGL((sparse_attn_pingpong_kernel<128>), grid, dim3(512), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  else if (two_group)
    hipLaunchKernelGGL((sparse_attn_pingpong_kernel<64>), grid, dim3(512), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  else if (L.d == 128 && L.tile == 128)
    hipLaunchKernelGGL((sparse_attn_kernel<128, 4, 64>), grid, dim3(256), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  else if (L.d == 128 && L.tile == 64)
    hipLaunchKernelGGL((sparse_attn_kernel<128, 2, 32>), grid, dim3(128), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  else if (L.d == 64 && L.tile == 128)
    hipLaunchKernelGGL((sparse_attn_kernel<64, 4, 64>), grid, dim3(256), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<64, 2, 32>), grid, dim3(128), 0, s, L, DN, qq, kk, vv, idx,
                       ord, scale_log2, oo, lse, by_heads);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_fp8(const LayerDev& L, const DenseDev& DN, const void* q8, const void* k8,
                                  const void* vt, int64_t n_tokens, const int32_t* idx, const int32_t* order,
                                  float scale, const float* q_scale, const float* k_scale, const float* v_scale,
                                  void* out, float* lse, hipStream_t s) {
  dim3 grid;
  int by_heads;
  if (!grid_of(L, DN, L.Tq, idx, grid, by_heads) || !two_group_fits(L, DN)) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.44269504088896340736f;
  const int64_t vt_head_bytes = (n_tokens + 63) / 64 * (int64_t)L.d * 64;
  auto qq = static_cast<const uint8_t*>(q8);
  auto kk = static_cast<const uint8_t*>(k8);
  auto vv = static_cast<const uint8_t*>(vt);
  auto oo = static_cast<uint16_t*>(out);
  if (L.d == 128)
    hipLaunchKernelGGL((sparse_attn_fp8_pingpong_kernel<128>), grid, dim3(512), 0, s, L, DN, qq, kk, vv,
                       vt_head_bytes, idx, idx ? order : nullptr, scale_log2, q_scale, k_scale, v_scale, oo, lse,
                       by_heads);
  else
    hipLaunchKernelGGL((sparse_attn_fp8_pingpong_kernel<64>), grid, dim3(512), 0, s, L, DN, qq, kk, vv,
                       vt_head_bytes, idx, idx ? order : nullptr, scale_log2, q_scale, k_scale, v_scale, oo, lse,
                       by_heads);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_fp8qk(const LayerDev& L, const DenseDev& DN, const void* q8, const void* k8,
                                    const void* v, const int32_t* idx, const int32_t* order, float scale,
                                    const float* q_scale, const float* k_scale, void* out, float* lse,
                                    hipStream_t s) {
  dim3 grid;
  int by_heads;
  if (!grid_of(L, DN, L.Tq, idx, grid, by_heads) || !two_group_fits(L, DN)) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.44269504088896340736f;
  auto qq = static_cast<const uint8_t*>(q8);
  auto kk = static_cast<const uint8_t*>(k8);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(out);
  if (L.d == 128)
    hipLaunchKernelGGL((sparse_attn_fp8qk_pingpong_kernel<128>), grid, dim3(512), 0, s, L, DN, qq, kk, vv, idx,
                       idx ? order : nullptr, scale_log2, q_scale, k_scale, oo, lse, by_heads);
  else
    hipLaunchKernelGGL((sparse_attn_fp8qk_pingpong_kernel<64>), grid, dim3(512), 0, s, L, DN, qq, kk, vv, idx,
                       idx ? order : nullptr, scale_log2, q_scale, k_scale, oo, lse, by_heads);
  return hipGetLastError();
}

}  // namespace veda
