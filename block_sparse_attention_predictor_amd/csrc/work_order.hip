// Processing order of the query tiles for the block-sparse attention kernels.
//
// The pages fix what the sparse execution kernel computes for each (b, h, query tile)
// (Affine launch article, "Training the Selector, Not the Generator"; Veda R2VA record,
// first paragraph), not the order in which the tiles are worked on; the results do not
// depend on it.  The order does decide how often a gathered K/V block is found in an
// XCD's L2: the attention kernels hand each XCD a contiguous run of processing
// positions of one (b, h), 32 workgroups at a time, and each workgroup walks its
// tile's selected blocks in ascending order.  Tiles whose selections start alike then
// read the same blocks at about the same time.  So the order sorts the query tiles of
// every (b, h) by their index rows, lexicographically, on the first segment that
// actually selects (budget below its tile count): the row's first E entries packed
// into the top 50 bits of a 64-bit key (E = 50 / bits, bits = the width of the
// segment's largest tile id, at least 4; an entry at or after the first -1 packs as all
// ones), the tile id in the low 14 bits, so that ties go to the lower tile id.
//
// Each workgroup takes 256 query tiles of one (b, h): it packs the keys of all of that
// (b, h)'s tiles into LDS, then ranks each of its tiles by comparison with every key
// (Tq compares per tile, eight keys per step from 16-byte broadcast reads).  Layers with more query tiles than the LDS array holds, or
// with no selecting segment, get the identity order.
#include "common.h"

namespace veda {
namespace {

constexpr int kOrderThreads = 256;      // query tiles ranked per work unit
constexpr int kOrderGrid = 4096;        // workgroups at most (a grid-stride loop over the units)
constexpr int kIdBits = 14;             // tile id in the low bits of a key (kOrderCap = 2^14)
constexpr int kMaxKeyEntries = 12;      // index entries per key at most ((64 - 14) / 4-bit ids)
static_assert(kOrderCap == 1 << kIdBits, "tile ids fill the low key bits");

// Work unit u: (b, h) = u / chunks, ranks of tiles (u % chunks) * 256 .. + 255.  Every unit
// packs all Tq keys of its (b, h) into LDS (padded to a multiple of 8 with all-ones keys),
// then each thread counts the keys below its own: keys are distinct (the tile id is part
// of each), so that count is the tile's position.
__global__ __launch_bounds__(kOrderThreads) void tile_order_kernel(int32_t Tq, int32_t Ktot, int32_t koff,
                                                                   int32_t nent, int32_t bits, int64_t units,
                                                                   int32_t chunks,
                                                                   const int32_t* __restrict__ idx,
                                                                   int32_t* __restrict__ order) {
  __shared__ __attribute__((aligned(16))) uint64_t keys[kOrderCap];
  const uint64_t ones = (1ull << bits) - 1;
  const int Tp = (Tq + 7) & ~7;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t bh = u / chunks;
    const int32_t* rows = idx + bh * Tq * Ktot + koff;
    __syncthreads();                            // the previous unit's ranking has read keys
    // (every entry loaded unconditionally, so that a row's loads and those of the next
    // rows are in flight together)
#pragma unroll 4
    for (int i = threadIdx.x; i < Tp; i += kOrderThreads) {
      uint64_t key = ~0ull;
      if (i < Tq) {
        const int32_t* r = rows + (int64_t)i * Ktot;
        int32_t t[kMaxKeyEntries];
#pragma unroll
        for (int e = 0; e < kMaxKeyEntries; ++e) t[e] = e < nent ? r[e] : 0;
        uint64_t packed = 0;
        bool ended = false;
#pragma unroll
        for (int e = 0; e < kMaxKeyEntries; ++e) {
          if (e >= nent) break;
          ended = ended || t[e] < 0;
          packed = (packed << bits) | (ended ? ones : (uint64_t)t[e]);
        }
        key = (packed << kIdBits) | (uint64_t)i;
      }
      keys[i] = key;
    }
    __syncthreads();
    const int i = (int)(u % chunks) * kOrderThreads + threadIdx.x;
    if (i < Tq) {
      const uint64_t ki = keys[i];
      int rank = 0;
      const ulonglong2* const kp = reinterpret_cast<const ulonglong2*>(keys);
#pragma unroll 2
      for (int j = 0; j < Tp; j += 8) {
        ulonglong2 k4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) k4[c] = kp[(j >> 1) + c];
#pragma unroll
        for (int c = 0; c < 4; ++c) rank += (int)(k4[c].x < ki) + (int)(k4[c].y < ki);
      }
      order[bh * Tq + rank] = i;
    }
  }
}

__global__ void identity_order_kernel(int32_t Tq, int64_t n, int32_t* __restrict__ order) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    order[i] = (int32_t)(i % Tq);
}

}  // namespace

hipError_t launch_tile_order(const LayerDev& L, const int32_t* idx, int32_t* order, hipStream_t s) {
  const int64_t nbh = (int64_t)L.B * L.H;
  int seg = -1;
  for (int i = 0; i < L.n_seg && seg < 0; ++i)
    if (L.seg[i].K < L.seg[i].T) seg = i;
  if (nbh == 0 || L.Tq == 0) return hipSuccess;
  if (seg < 0 || L.Tq > kOrderCap) {
    const int64_t n = nbh * L.Tq;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(identity_order_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                       L.Tq, n, order);
    return hipGetLastError();
  }
  int bits = 4;                                 // so that a key holds at most 12 entries
  while ((1ll << bits) < L.seg[seg].T) ++bits;
  const int room = (64 - kIdBits) / bits;
  const int nent = room < L.seg[seg].K ? room : L.seg[seg].K;
  const int32_t chunks = (L.Tq + kOrderThreads - 1) / kOrderThreads;
  const int64_t units = nbh * chunks;
  const unsigned grid = (unsigned)(units < kOrderGrid ? units : kOrderGrid);
  hipLaunchKernelGGL(tile_order_kernel, dim3(grid), dim3(kOrderThreads), 0, s, L.Tq, L.Ktot, L.seg[seg].koff,
                     nent, bits, units, chunks, idx, order);
  return hipGetLastError();
}

}  // namespace veda
