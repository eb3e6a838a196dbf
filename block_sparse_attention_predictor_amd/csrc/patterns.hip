// Fixed-pattern index producer: sliding frame-chunk windows with boundary anchors.
//
// The VDN analysis ("The mechanism: solving instead of stepping") describes a
// softmax branch over chunks of consecutive latent frames, each chunk attending to
// itself and its neighbouring chunks, plus anchors: every frame also attends to the
// first and last frames, and those two frames attend to everything.  Here the
// pattern is produced at tile granularity for the block-sparse attention call: a
// query tile takes every key tile that overlaps the key frames of any of its query
// frames.  Rows have different lengths; they are written ascending and padded with
// -1 to a common width (a -1 ends the row's block for the attention kernel).
#include "common.h"

namespace veda {

// Up to three disjoint, ascending tile intervals [lo, hi] (inclusive) of the key
// segment that query tile `qt` attends to.  Returns how many intervals are used.
__host__ __device__ inline int window_intervals(int64_t q0, int64_t qlen, int64_t tile, int64_t seg_len,
                                                int qt, const WindowPattern& P, int64_t lo[3],
                                                int64_t hi[3]) {
  const int64_t T = (seg_len + tile - 1) / tile;
  const int64_t n_frames = (seg_len + P.frame_tokens - 1) / P.frame_tokens;
  // query and key segment are the same token range, so frames count from its start
  (void)q0;
  const int64_t a = (int64_t)qt * tile;                          // first and last query token
  const int64_t b = (a + tile < qlen ? a + tile : qlen) - 1;
  const int64_t qfa = a / P.frame_tokens, qfb = b / P.frame_tokens;
  if (P.anchors && (qfa == 0 || qfb >= n_frames - 1)) {   // an anchor frame among the queries
    lo[0] = 0;
    hi[0] = T - 1;
    return 1;
  }
  const int64_t ca = qfa / P.chunk_frames, cb = qfb / P.chunk_frames;
  const int64_t n_chunks = (n_frames + P.chunk_frames - 1) / P.chunk_frames;
  int64_t c_lo = ca - P.halo_chunks, c_hi = cb + P.halo_chunks;
  if (c_lo < 0) c_lo = 0;
  if (c_hi > n_chunks - 1) c_hi = n_chunks - 1;
  const int64_t f_lo = c_lo * P.chunk_frames;
  int64_t f_hi = (c_hi + 1) * P.chunk_frames - 1;
  if (f_hi > n_frames - 1) f_hi = n_frames - 1;
  auto frames_to_tiles = [&](int64_t f0, int64_t f1, int64_t& t0, int64_t& t1) {
    const int64_t tok0 = f0 * P.frame_tokens;
    int64_t tok1 = (f1 + 1) * P.frame_tokens - 1;
    if (tok1 > seg_len - 1) tok1 = seg_len - 1;
    t0 = tok0 / tile;
    t1 = tok1 / tile;
  };
  int64_t wl, wh;
  frames_to_tiles(f_lo, f_hi, wl, wh);
  if (!P.anchors) {
    lo[0] = wl;
    hi[0] = wh;
    return 1;
  }
  int64_t al, ah, zl, zh;
  frames_to_tiles(0, 0, al, ah);                         // first frame
  frames_to_tiles(n_frames - 1, n_frames - 1, zl, zh);   // last frame
  // merge [al,ah], [wl,wh], [zl,zh] (each ascending by start)
  int n = 0;
  const int64_t il[3] = {al, wl, zl}, ih[3] = {ah, wh, zh};
  for (int i = 0; i < 3; ++i) {
    if (n > 0 && il[i] <= hi[n - 1] + 1) {
      if (ih[i] > hi[n - 1]) hi[n - 1] = ih[i];
    } else {
      lo[n] = il[i];
      hi[n] = ih[i];
      ++n;
    }
  }
  return n;
}

namespace {

// One wave per (b*h, query tile) row: the row's intervals are computed once per lane,
// then the 64 lanes write consecutive entries (coalesced), -1 past the row's length.
__global__ __launch_bounds__(256) void window_indices_kernel(int64_t q0, int64_t qlen, int64_t tile,
                                                             int64_t seg_len, int32_t Tq, int32_t BH,
                                                             WindowPattern P, int32_t* __restrict__ idx,
                                                             int32_t kmax) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= (int64_t)BH * Tq) return;
  const int qt = (int)(g % Tq);
  int64_t lo[3], hi[3];
  const int n = window_intervals(q0, qlen, tile, seg_len, qt, P, lo, hi);
  int64_t len[3] = {0, 0, 0};
  for (int i = 0; i < n; ++i) len[i] = hi[i] - lo[i] + 1;
  int32_t* row = idx + g * kmax;
  for (int64_t w = lane; w < kmax; w += 64) {
    int64_t r = w, v = -1;
    for (int i = 0; i < n; ++i) {
      if (r < len[i]) {
        v = lo[i] + r;
        break;
      }
      r -= len[i];
    }
    row[w] = (int32_t)v;
  }
}

}  // namespace

int64_t window_max_tiles(int64_t q0, int64_t qlen, int64_t tile, int64_t seg_len, const WindowPattern& P) {
  const int64_t Tq = (qlen + tile - 1) / tile;
  int64_t best = 0;
  for (int64_t qt = 0; qt < Tq; ++qt) {
    int64_t lo[3], hi[3];
    const int n = window_intervals(q0, qlen, tile, seg_len, (int)qt, P, lo, hi);
    int64_t c = 0;
    for (int i = 0; i < n; ++i) c += hi[i] - lo[i] + 1;
    if (c > best) best = c;
  }
  return best;
}

hipError_t launch_window_indices(int64_t q0, int64_t qlen, int64_t tile, int64_t seg_len, int32_t Tq,
                                 int32_t BH, const WindowPattern& P, int32_t* idx, int32_t kmax,
                                 hipStream_t s) {
  const int64_t n = (int64_t)BH * Tq;
  if ((n + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(window_indices_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, q0, qlen,
                     tile, seg_len, Tq, BH, P, idx, kmax);
  return hipGetLastError();
}

}  // namespace veda
