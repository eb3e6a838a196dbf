// Recording stand-ins for the kernel launchers (see launch_stubs.h).  The checks restate
// the kernels' preconditions: tile geometry consistent with the layer, 32-bit counts and
// grids, strides the row addressing can form, dense ranges inside the sequence, scales
// finite and positive.
#include "launch_stubs.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "../../block_sparse_attention_predictor_amd/csrc/common.h"
#include "../../include/veda.h"

namespace stub {
int64_t n_tokens = 0;
long launches = 0;
bool fail_launch = false;
bool fits = true;
int64_t window_tiles = 1;
}  // namespace stub

namespace {

[[noreturn]] void violation(const char* what, const char* where) {
  std::fprintf(stderr, "launcher precondition violated in %s: %s\n", where, what);
  std::abort();
}

#define REQUIRE(cond) \
  do {                \
    if (!(cond)) violation(#cond, __func__); \
  } while (0)

int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipError_t done() {
  ++stub::launches;
  return stub::fail_launch ? hipErrorInvalidValue : hipSuccess;
}

// Geometry every launcher that takes a layer relies on.
void check_layer(const veda::LayerDev& L, const char* where, bool need_query = true) {
  auto req = [&](bool c, const char* what) {
    if (!c) violation(what, where);
  };
  req(L.B >= 1 && L.H >= 1, "B, H >= 1");
  req((int64_t)L.B * L.H <= INT32_MAX, "B * H fits int32");
  req(L.d == 64 || L.d == 128, "d in {64, 128}");
  req(L.tile == 64 || L.tile == 128, "tile in {64, 128}");
  req(L.n_seg >= 0 && L.n_seg <= veda::kMaxSeg, "segment count");
  req(L.sn > 0 && L.sn < ((int64_t)1 << 24) && L.sh >= L.d && L.sb >= 0, "strides");
  req(L.sb % 8 == 0 && L.sn % 8 == 0 && L.sh % 8 == 0, "strides multiples of 8");
  req(L.q0 >= 0 && L.qlen >= (need_query ? 1 : 0) && L.q0 + L.qlen <= stub::n_tokens, "query range");
  req(L.Tq == cdiv(L.qlen, L.tile), "Tq = ceil(qlen / tile)");
  int64_t koff = 0, toff = 0;
  for (int s = 0; s < L.n_seg; ++s) {
    const veda::SegDev& g = L.seg[s];
    req(g.start >= 0 && g.len >= 1 && g.start + g.len <= stub::n_tokens, "segment range");
    req(g.T == cdiv(g.len, L.tile), "T = ceil(len / tile)");
    req(g.K >= 0 && g.K <= g.T, "0 <= K <= T");
    req(g.koff == koff && g.toff == toff, "segment offsets");
    for (int t = 0; t < s; ++t)
      req(g.start + g.len <= L.seg[t].start || L.seg[t].start + L.seg[t].len <= g.start,
          "segments disjoint");
    koff += g.K;
    toff += g.T;
  }
  req(L.Tk == toff && L.Ktot == koff, "Tk, Ktot");
  req((__int128)L.B * L.H * L.Tq * (L.Tk > 0 ? L.Tk : 1) <= ((__int128)1 << 40), "index volume");
}

void check_dense(const veda::LayerDev& L, const veda::DenseDev& D, const char* where) {
  auto req = [&](bool c, const char* what) {
    if (!c) violation(what, where);
  };
  req(D.n >= 0 && D.n <= veda::kMaxDense, "dense count");
  int64_t tokens = 0;
  for (int i = 0; i < D.n; ++i) {
    const veda::RangeDev& r = D.r[i];
    req(r.start >= 0 && r.len >= 1 && r.start + r.len <= stub::n_tokens, "dense range");
    for (int s = 0; s < L.n_seg; ++s)
      req(r.start + r.len <= L.seg[s].start || L.seg[s].start + L.seg[s].len <= r.start,
          "dense range disjoint from the segments");
    for (int j = 0; j < i; ++j)
      req(r.start + r.len <= D.r[j].start || D.r[j].start + D.r[j].len <= r.start,
          "dense ranges disjoint");
    tokens += r.len;
  }
  req(L.Ktot > 0 || tokens > 0, "some key for every query tile");
}

void check_attn(const veda::LayerDev& L, const veda::DenseDev& D, const void* q, const void* k,
                const void* v, const int32_t* idx, float scale, const void* out, const float* lse,
                const char* where) {
  check_layer(L, where);
  check_dense(L, D, where);
  auto req = [&](bool c, const char* what) {
    if (!c) violation(what, where);
  };
  req(q && k && v && out, "tensors");
  req(aligned(v, 16) && aligned(out, 16), "16-byte alignment");
  req(!lse || aligned(lse, 16), "lse alignment");
  req(idx ? aligned(idx, 16) : L.Ktot == L.Tk, "index, or every tile");
  req(std::isfinite(scale) && scale > 0.f, "scale");
}

}  // namespace

namespace veda {

hipError_t launch_pool_project(const LayerDev& L, const void* q, const void* k, const void* wq,
                               const void* wk, float* q_hat, float* k_hat, hipStream_t) {
  check_layer(L, __func__, false);   // with an empty query segment it pools the keys only
  REQUIRE(L.p >= 16 && L.p <= 384 && L.p % 16 == 0);
  REQUIRE(L.n_seg >= 1 && L.Tk <= VEDA_MAX_KEY_TILES);
  REQUIRE(L.wdtype == 0 || L.wdtype == 1);
  REQUIRE(q && k && wq && wk && q_hat && k_hat);
  REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(wq, 16) && aligned(wk, 16));
  REQUIRE(aligned(q_hat, 16) && aligned(k_hat, 16));
  return done();
}

hipError_t launch_score_topk(const LayerDev& L, const float* q_hat, const float* k_hat, int32_t* idx,
                             float* scores, hipStream_t) {
  check_layer(L, __func__);
  REQUIRE(L.p >= 16 && L.p <= 384 && L.p % 16 == 0);
  REQUIRE(L.n_seg >= 1 && L.Tk <= VEDA_MAX_KEY_TILES && L.Tq >= 1);
  REQUIRE(q_hat && k_hat && idx && aligned(idx, 16));
  REQUIRE(!scores || aligned(scores, 16));
  return done();
}

hipError_t launch_sparse_attn(const LayerDev& L, const DenseDev& D, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* order, float scale, void* out,
                              float* lse, hipStream_t) {
  check_attn(L, D, q, k, v, idx, scale, out, lse, __func__);
  REQUIRE(!order || (idx && aligned(order, 4)));
  REQUIRE(aligned(q, 16) && aligned(k, 16));
  return done();
}

hipError_t launch_sparse_attn_fp8qk(const LayerDev& L, const DenseDev& D, const void* q8, const void* k8,
                                    const void* v, const int32_t* idx, const int32_t* order, float scale,
                                    const float* q_scale, const float* k_scale, void* out, float* lse,
                                    hipStream_t) {
  check_attn(L, D, q8, k8, v, idx, scale, out, lse, __func__);
  REQUIRE(!order || (idx && aligned(order, 4)));
  REQUIRE(L.tile == 128 && stub::fits);
  REQUIRE(L.sb % 16 == 0 && L.sn % 16 == 0 && L.sh % 16 == 0);
  REQUIRE(q_scale && k_scale && aligned(q_scale, 4) && aligned(k_scale, 4));
  return done();
}

hipError_t launch_sparse_attn_fp8(const LayerDev& L, const DenseDev& D, const void* q8, const void* k8,
                                  const void* vt, int64_t n_tokens, const int32_t* idx, const int32_t* order,
                                  float scale, const float* q_scale, const float* k_scale, const float* v_scale,
                                  void* out, float* lse, hipStream_t) {
  check_attn(L, D, q8, k8, vt, idx, scale, out, lse, __func__);
  REQUIRE(!order || (idx && aligned(order, 4)));
  REQUIRE(L.tile == 128 && stub::fits);
  REQUIRE(n_tokens == stub::n_tokens);
  REQUIRE(L.sb % 16 == 0 && L.sn % 16 == 0 && L.sh % 16 == 0);
  REQUIRE(q_scale && k_scale && v_scale && aligned(q_scale, 4) && aligned(k_scale, 4) && aligned(v_scale, 4));
  for (int s = 0; s < L.n_seg; ++s) REQUIRE(L.seg[s].start % 64 == 0);
  for (int i = 0; i < D.n; ++i) REQUIRE(D.r[i].start % 64 == 0);
  return done();
}

hipError_t launch_quantize_fp8_vt(const LayerDev& L, int64_t n_tokens, const void* v, uint8_t* vt,
                                  float* scale, hipStream_t) {
  check_layer(L, __func__, false);
  REQUIRE(n_tokens == stub::n_tokens);
  REQUIRE(v && vt && scale && aligned(v, 16) && aligned(vt, 16) && aligned(scale, 4));
  return done();
}

hipError_t launch_tile_order(const LayerDev& L, const int32_t* idx, int32_t* order, hipStream_t) {
  check_layer(L, __func__);
  REQUIRE(L.Tq >= 1 && idx && order && aligned(idx, 16) && aligned(order, 4));
  return done();
}

bool two_group_fits(const LayerDev& L, const DenseDev&) {
  check_layer(L, __func__);
  return stub::fits;
}

hipError_t launch_quantize_fp8(const LayerDev& L, int64_t n_tokens, const void* x, uint8_t* x8,
                               float* scale, hipStream_t) {
  check_layer(L, __func__, false);   // every token is quantised, query segment or not
  REQUIRE(n_tokens == stub::n_tokens);
  REQUIRE(x && x8 && scale && aligned(x, 16) && aligned(x8, 16) && aligned(scale, 4));
  return done();
}

hipError_t launch_dequant_e4m3(const uint8_t* src, void* dst, int64_t n, int32_t pow2_exp, hipStream_t) {
  REQUIRE(src && dst && n >= 1 && aligned(dst, 2));
  REQUIRE(pow2_exp >= -24 && pow2_exp <= 24);
  return done();
}

hipError_t launch_block_mass(const LayerDev& L, const DenseDev& D, const void* q, const void* k,
                             float scale, float* lse, float* mass, float* dense_mass, hipStream_t) {
  check_attn(L, D, q, k, k, nullptr, scale, mass, lse, __func__);
  for (int s = 0; s < L.n_seg; ++s) REQUIRE(L.seg[s].K == L.seg[s].T);
  REQUIRE(lse && aligned(lse, 16) && (!dense_mass || aligned(dense_mass, 16)));
  return done();
}

hipError_t launch_block_recall(const LayerDev& L, const float* mass, const int32_t* idx, float* recall,
                               hipStream_t) {
  check_layer(L, __func__);
  REQUIRE(L.Tq >= 1);
  REQUIRE(mass && idx && recall && aligned(mass, 16) && aligned(idx, 16) && aligned(recall, 16));
  return done();
}

int64_t window_max_tiles(int64_t q0, int64_t qlen, int64_t tile, int64_t seg_len, const WindowPattern& P) {
  REQUIRE(q0 >= 0 && qlen >= 1 && (tile == 64 || tile == 128) && seg_len == qlen);
  REQUIRE(P.frame_tokens >= 1 && P.chunk_frames >= 1 && P.halo_chunks >= 0);
  REQUIRE(P.anchors == 0 || P.anchors == 1);
  return stub::window_tiles;
}

hipError_t launch_window_indices(int64_t q0, int64_t qlen, int64_t tile, int64_t seg_len, int32_t Tq,
                                 int32_t BH, const WindowPattern& P, int32_t* idx, int32_t kmax,
                                 hipStream_t) {
  REQUIRE(q0 >= 0 && qlen >= 1 && (tile == 64 || tile == 128) && seg_len == qlen);
  REQUIRE(Tq == cdiv(qlen, tile) && BH >= 1);
  REQUIRE(P.frame_tokens >= 1 && P.chunk_frames >= 1 && P.halo_chunks >= 0);
  REQUIRE(kmax >= stub::window_tiles && kmax <= cdiv(seg_len, tile));
  REQUIRE(idx && aligned(idx, 16));
  return done();
}

int score_rows_per_block(int, int) { return 1; }

}  // namespace veda
