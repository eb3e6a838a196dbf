// Host side of the C ABI: validation (complete before any device call), derived
// layer geometry, workspace carving and kernel launches.
#include "../../include/veda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>

#include "common.h"

namespace {

using veda::LayerDev;

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (a may be close to INT64_MAX)
int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool inside(const veda_range& r, int64_t n) {
  return r.start >= 0 && r.len >= 0 && r.start <= n && r.len <= n - r.start;
}

bool overlap(const veda_range& a, const veda_range& b) {
  if (a.len == 0 || b.len == 0) return false;
  return a.start < b.start + b.len && b.start < a.start + a.len;
}

// Checks shared by every entry point that takes a layer.
int check_layer(const veda_layer* L, bool for_select) {
  if (!L) return VEDA_EINVAL;
  if (L->B < 1 || L->H < 1 || L->n_tokens < 1) return VEDA_EINVAL;
  // B * H is an int32 on the device
  if ((int64_t)L->B * L->H > INT32_MAX) return VEDA_EUNSUPPORTED;
  if (L->d != 64 && L->d != 128) return VEDA_EUNSUPPORTED;
  if (L->tile != 64 && L->tile != 128) return VEDA_EUNSUPPORTED;
  if (for_select && (L->p < 16 || L->p > 384 || (L->p % 16) != 0)) return VEDA_EUNSUPPORTED;
  if (L->wdtype != VEDA_W_BF16 && L->wdtype != VEDA_W_F16) return VEDA_EUNSUPPORTED;
  if (L->reserved != 0) return VEDA_EINVAL;
  if (L->n_seg < 0 || L->n_seg > VEDA_MAX_SEGMENTS) return VEDA_EUNSUPPORTED;
  if (for_select && L->n_seg < 1) return VEDA_EINVAL;
  if (L->stride_n <= 0 || L->stride_h <= 0 || L->stride_b < 0) return VEDA_EINVAL;
  if ((L->stride_b % 8) || (L->stride_n % 8) || (L->stride_h % 8)) return VEDA_EINVAL;
  if (L->stride_h < L->d) return VEDA_EINVAL;
  // the kernels form 64-row byte offsets in 32 bits
  if (L->stride_n >= ((int64_t)1 << 24)) return VEDA_EUNSUPPORTED;
  if (!inside(L->query, L->n_tokens)) return VEDA_ERANGE;
  int64_t tk = 0;
  for (int s = 0; s < L->n_seg; ++s) {
    if (L->seg[s].len < 1) return VEDA_EINVAL;
    if (!inside(L->seg[s], L->n_tokens)) return VEDA_ERANGE;
    if (L->budget[s] < 0) return VEDA_EINVAL;
    for (int t = 0; t < s; ++t)
      if (overlap(L->seg[s], L->seg[t])) return VEDA_ERANGE;
    tk += ceil_div(L->seg[s].len, L->tile);
  }
  if (for_select && tk > VEDA_MAX_KEY_TILES) return VEDA_EUNSUPPORTED;
  // tile counts are int32 on the device
  const int64_t tq = ceil_div(L->query.len, L->tile);
  if (tq > INT32_MAX || tk > INT32_MAX) return VEDA_EUNSUPPORTED;
  // index and mass rows: B * H * Tq * sum T_s entries at most 2^40, so that every offset
  // formed from them on the device stays far inside int64
  if ((__int128)L->B * L->H * tq * std::max<int64_t>(tk, 1) > (__int128)1 << 40) return VEDA_EUNSUPPORTED;
  return VEDA_OK;
}

int64_t k_total(const veda_layer* L) {
  int64_t k = 0;
  for (int s = 0; s < L->n_seg; ++s)
    k += std::min<int64_t>(L->budget[s], ceil_div(L->seg[s].len, L->tile));
  return k;
}

LayerDev to_dev(const veda_layer* L) {
  LayerDev D{};
  D.B = L->B;
  D.H = L->H;
  D.d = L->d;
  D.p = L->p;
  D.tile = L->tile;
  D.n_seg = L->n_seg;
  D.Tq = (int32_t)ceil_div(L->query.len, L->tile);
  D.sb = L->stride_b;
  D.sn = L->stride_n;
  D.sh = L->stride_h;
  D.wdtype = L->wdtype;
  D.q0 = L->query.start;
  D.qlen = L->query.len;
  int32_t koff = 0, toff = 0;
  for (int s = 0; s < L->n_seg; ++s) {
    veda::SegDev& g = D.seg[s];
    g.start = L->seg[s].start;
    g.len = L->seg[s].len;
    g.T = (int32_t)ceil_div(g.len, L->tile);
    g.K = std::min<int32_t>(L->budget[s], g.T);
    g.koff = koff;
    g.toff = toff;
    koff += g.K;
    toff += g.T;
  }
  D.Tk = toff;
  D.Ktot = koff;
  return D;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t qhat_bytes(const LayerDev& D) { return round256((size_t)D.B * D.H * D.Tq * D.p * 4); }
size_t khat_bytes(const LayerDev& D) { return round256((size_t)D.B * D.H * D.Tk * D.p * 4); }

int hip_status(hipError_t e) { return e == hipSuccess ? VEDA_OK : VEDA_EHIP; }

}  // namespace

extern "C" {

int veda_abi_version(void) { return VEDA_ABI_VERSION; }

const char* veda_status_string(int status) {
  switch (status) {
    case VEDA_OK: return "ok";
    case VEDA_EINVAL: return "invalid argument (null pointer, bad size, alignment or stride)";
    case VEDA_EUNSUPPORTED: return "unsupported configuration (d, tile, p or count limits)";
    case VEDA_EWORKSPACE: return "workspace too small";
    case VEDA_ERANGE: return "token range outside the sequence or overlapping ranges";
    case VEDA_ENOKEYS: return "a query tile would attend to no key";
    case VEDA_EHIP: return "HIP launch error";
    case VEDA_EIO: return "file could not be opened or read";
    case VEDA_EFORMAT: return "malformed safetensors file";
    default: return "unknown status";
  }
}

int64_t veda_k_total(const veda_layer* layer) {
  if (!layer || layer->tile <= 0 || layer->n_seg < 0 || layer->n_seg > VEDA_MAX_SEGMENTS) return -1;
  for (int s = 0; s < layer->n_seg; ++s)
    if (layer->seg[s].len < 0 || layer->budget[s] < 0) return -1;
  return k_total(layer);
}

int veda_layer_check(const veda_layer* layer, int for_select) {
  return check_layer(layer, for_select != 0);
}

size_t veda_select_workspace_bytes(const veda_layer* layer) {
  if (check_layer(layer, true) != VEDA_OK) return 0;
  LayerDev D = to_dev(layer);
  return qhat_bytes(D) + khat_bytes(D);
}

int veda_pool_project(const veda_layer* layer, const void* q, const void* k, const void* wq,
                      const void* wk, float* q_hat, float* k_hat, void* stream) {
  int st = check_layer(layer, true);
  if (st != VEDA_OK) return st;
  if (!q || !k || !wq || !wk || !q_hat || !k_hat) return VEDA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(wq) || !aligned16(wk) || !aligned16(q_hat) ||
      !aligned16(k_hat))
    return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  if (D.Tq == 0 && D.Tk == 0) return VEDA_OK;
  return hip_status(veda::launch_pool_project(D, q, k, wq, wk, q_hat, k_hat, (hipStream_t)stream));
}

int veda_score_topk(const veda_layer* layer, const float* q_hat, const float* k_hat, int32_t* idx,
                    float* scores_opt, void* stream) {
  int st = check_layer(layer, true);
  if (st != VEDA_OK) return st;
  if (!q_hat || !k_hat || !idx) return VEDA_EINVAL;
  if (!aligned16(q_hat) || !aligned16(k_hat) || !aligned16(idx)) return VEDA_EINVAL;
  if (scores_opt && !aligned16(scores_opt)) return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  if (D.Tq == 0) return VEDA_OK;
  return hip_status(veda::launch_score_topk(D, q_hat, k_hat, idx, scores_opt, (hipStream_t)stream));
}

int veda_select(const veda_layer* layer, const void* q, const void* k, const void* wq,
                const void* wk, int32_t* idx, float* scores_opt, void* ws, size_t ws_bytes,
                void* stream) {
  int st = check_layer(layer, true);
  if (st != VEDA_OK) return st;
  if (!q || !k || !wq || !wk || !idx || !ws) return VEDA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return VEDA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(wq) || !aligned16(wk) || !aligned16(idx))
    return VEDA_EINVAL;
  if (scores_opt && !aligned16(scores_opt)) return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  if (ws_bytes < qhat_bytes(D) + khat_bytes(D)) return VEDA_EWORKSPACE;
  if (D.Tq == 0) return VEDA_OK;
  float* qh = static_cast<float*>(ws);
  float* kh = reinterpret_cast<float*>(static_cast<char*>(ws) + qhat_bytes(D));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = veda::launch_pool_project(D, q, k, wq, wk, qh, kh, s);
  if (e != hipSuccess) return VEDA_EHIP;
  return hip_status(veda::launch_score_topk(D, qh, kh, idx, scores_opt, s));
}

}  // extern "C"

namespace {

// Every check veda_sparse_attn makes before launching; dd receives the dense ranges.
int sparse_attn_check(const veda_layer* layer, const void* q, const void* k, const void* v,
                      const int32_t* idx, const int32_t* order, const veda_range* dense, int32_t n_dense,
                      float scale, const void* out, veda::DenseDev* dd) {
  int st = check_layer(layer, false);
  if (st != VEDA_OK) return st;
  if (!q || !k || !v || !out) return VEDA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VEDA_EINVAL;
  if (order && (!idx || (reinterpret_cast<uintptr_t>(order) & 3u))) return VEDA_EINVAL;
  if (n_dense < 0) return VEDA_EINVAL;
  if (n_dense > VEDA_MAX_DENSE) return VEDA_EUNSUPPORTED;
  if (n_dense > 0 && !dense) return VEDA_EINVAL;
  if (!(std::isfinite(scale)) || scale < 0.f) return VEDA_EINVAL;
  int64_t dense_tokens = 0;
  veda::DenseDev DD{};
  for (int i = 0; i < n_dense; ++i) {
    if (dense[i].len < 0) return VEDA_EINVAL;
    if (!inside(dense[i], layer->n_tokens)) return VEDA_ERANGE;
    for (int s = 0; s < layer->n_seg; ++s)
      if (overlap(dense[i], layer->seg[s])) return VEDA_ERANGE;
    for (int j = 0; j < i; ++j)
      if (overlap(dense[i], dense[j])) return VEDA_ERANGE;
    dense_tokens += dense[i].len;
    if (dense[i].len == 0) continue;
    DD.r[DD.n].start = dense[i].start;
    DD.r[DD.n].len = dense[i].len;
    DD.n++;
  }
  LayerDev D = to_dev(layer);
  if (D.Tq == 0) {
    if (dd) *dd = DD;
    return VEDA_OK;
  }
  if (D.Ktot == 0 && dense_tokens == 0) return VEDA_ENOKEYS;
  if (!idx && D.Ktot != D.Tk) return VEDA_EINVAL;   // no index: every tile of every segment
  if (idx && !aligned16(idx)) return VEDA_EINVAL;
  if (dd) *dd = DD;
  return VEDA_OK;
}

}  // namespace

extern "C" {

int veda_sparse_attn_check(const veda_layer* layer, const void* q, const void* k, const void* v,
                           const int32_t* idx, const int32_t* order, const veda_range* dense,
                           int32_t n_dense, float scale, const void* out) {
  return sparse_attn_check(layer, q, k, v, idx, order, dense, n_dense, scale, out, nullptr);
}

int veda_tile_order(const veda_layer* layer, const int32_t* idx, int32_t* order, void* stream) {
  int st = check_layer(layer, false);
  if (st != VEDA_OK) return st;
  if (!idx || !order) return VEDA_EINVAL;
  if (!aligned16(idx) || (reinterpret_cast<uintptr_t>(order) & 3u)) return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  if (D.Tq == 0) return VEDA_OK;
  return hip_status(veda::launch_tile_order(D, idx, order, (hipStream_t)stream));
}

int veda_sparse_attn(const veda_layer* layer, const void* q, const void* k, const void* v,
                     const int32_t* idx, const int32_t* order, const veda_range* dense, int32_t n_dense,
                     float scale, void* out, float* lse_opt, void* stream) {
  veda::DenseDev DD{};
  int st = sparse_attn_check(layer, q, k, v, idx, order, dense, n_dense, scale, out, &DD);
  if (st != VEDA_OK) return st;
  if (lse_opt && !aligned16(lse_opt)) return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  if (D.Tq == 0) return VEDA_OK;
  if (scale == 0.f) scale = 1.0f / std::sqrt((float)layer->d);
  return hip_status(veda::launch_sparse_attn(D, DD, q, k, v, idx, order, scale, out, lse_opt,
                                             (hipStream_t)stream));
}

int veda_sparse_attn_fp8qk(const veda_layer* layer, const uint8_t* q8, const uint8_t* k8, const void* v,
                           const float* q_scale, const float* k_scale, const int32_t* idx,
                           const int32_t* order, const veda_range* dense, int32_t n_dense, float scale,
                           void* out, float* lse_opt, void* stream) {
  veda::DenseDev DD{};
  int st = sparse_attn_check(layer, q8, k8, v, idx, order, dense, n_dense, scale, out, &DD);
  if (st != VEDA_OK) return st;
  if (!q_scale || !k_scale) return VEDA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u))
    return VEDA_EINVAL;
  // one-byte rows: 16-byte loads need 16-element strides
  if ((layer->stride_b % 16) || (layer->stride_n % 16) || (layer->stride_h % 16)) return VEDA_EINVAL;
  if (lse_opt && !aligned16(lse_opt)) return VEDA_EINVAL;
  if (layer->tile != 128) return VEDA_EUNSUPPORTED;
  LayerDev D = to_dev(layer);
  if (D.Tq == 0) return VEDA_OK;
  if (!veda::two_group_fits(D, DD)) return VEDA_EUNSUPPORTED;
  if (scale == 0.f) scale = 1.0f / std::sqrt((float)layer->d);
  return hip_status(veda::launch_sparse_attn_fp8qk(D, DD, q8, k8, v, idx, order, scale, q_scale, k_scale, out,
                                                   lse_opt, (hipStream_t)stream));
}

int veda_quantize_fp8_e4m3(const veda_layer* layer, const void* x, uint8_t* x8, float* scale,
                           void* stream) {
  int st = check_layer(layer, false);
  if (st != VEDA_OK) return st;
  if (!x || !x8 || !scale) return VEDA_EINVAL;
  if (!aligned16(x) || !aligned16(x8) || (reinterpret_cast<uintptr_t>(scale) & 3u)) return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  return hip_status(veda::launch_quantize_fp8(D, layer->n_tokens, x, x8, scale, (hipStream_t)stream));
}

size_t veda_fp8_vt_bytes(const veda_layer* layer) {
  if (check_layer(layer, false) != VEDA_OK) return 0;
  const int64_t blocks = ceil_div(layer->n_tokens, 64);
  const int64_t bh = (int64_t)layer->B * layer->H;
  if (blocks > INT32_MAX / bh) return 0;   // the quantiser runs one workgroup per block
  return (size_t)(bh * blocks) * (size_t)layer->d * 64u;
}

int veda_quantize_fp8_e4m3_vt(const veda_layer* layer, const void* v, uint8_t* vt, float* v_scale,
                              void* stream) {
  int st = check_layer(layer, false);
  if (st != VEDA_OK) return st;
  if (!v || !vt || !v_scale) return VEDA_EINVAL;
  if (!aligned16(v) || !aligned16(vt) || (reinterpret_cast<uintptr_t>(v_scale) & 3u)) return VEDA_EINVAL;
  if (veda_fp8_vt_bytes(layer) == 0) return VEDA_EUNSUPPORTED;
  LayerDev D = to_dev(layer);
  return hip_status(veda::launch_quantize_fp8_vt(D, layer->n_tokens, v, vt, v_scale, (hipStream_t)stream));
}

int veda_sparse_attn_fp8(const veda_layer* layer, const uint8_t* q8, const uint8_t* k8, const uint8_t* vt,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         const int32_t* idx, const int32_t* order, const veda_range* dense, int32_t n_dense,
                         float scale, void* out, float* lse_opt, void* stream) {
  veda::DenseDev DD{};
  int st = sparse_attn_check(layer, q8, k8, vt, idx, order, dense, n_dense, scale, out, &DD);
  if (st != VEDA_OK) return st;
  if (!q_scale || !k_scale || !v_scale) return VEDA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(v_scale) & 3u))
    return VEDA_EINVAL;
  if ((layer->stride_b % 16) || (layer->stride_n % 16) || (layer->stride_h % 16)) return VEDA_EINVAL;
  if (lse_opt && !aligned16(lse_opt)) return VEDA_EINVAL;
  if (layer->tile != 128) return VEDA_EUNSUPPORTED;
  // every key block starts a 64-token block of vt
  for (int s = 0; s < layer->n_seg; ++s)
    if (layer->seg[s].start % 64) return VEDA_EUNSUPPORTED;
  for (int i = 0; i < DD.n; ++i)
    if (DD.r[i].start % 64) return VEDA_EUNSUPPORTED;
  if (veda_fp8_vt_bytes(layer) == 0) return VEDA_EUNSUPPORTED;
  LayerDev D = to_dev(layer);
  if (D.Tq == 0) return VEDA_OK;
  if (!veda::two_group_fits(D, DD)) return VEDA_EUNSUPPORTED;
  if (scale == 0.f) scale = 1.0f / std::sqrt((float)layer->d);
  return hip_status(veda::launch_sparse_attn_fp8(D, DD, q8, k8, vt, layer->n_tokens, idx, order, scale, q_scale,
                                                 k_scale, v_scale, out, lse_opt, (hipStream_t)stream));
}

int veda_layer_attn(const veda_layer* layer, const void* q, const void* k, const void* v,
                    const void* wq, const void* wk, const veda_range* dense, int32_t n_dense,
                    const veda_range* dense_queries, int32_t n_dense_queries, float scale,
                    void* out, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  int st = check_layer(layer, true);
  if (st != VEDA_OK) return st;
  if (!v || !out) return VEDA_EINVAL;
  if (n_dense_queries < 0) return VEDA_EINVAL;
  if (n_dense_queries > VEDA_MAX_DENSE) return VEDA_EUNSUPPORTED;
  if (n_dense_queries > 0 && !dense_queries) return VEDA_EINVAL;
  // every dense query range attends to every key: the same segments with full budgets
  veda_layer full = *layer;
  for (int s = 0; s < full.n_seg; ++s) full.budget[s] = (int32_t)((full.seg[s].len + full.tile - 1) / full.tile);
  for (int i = 0; i < n_dense_queries; ++i) {
    if (dense_queries[i].len < 0) return VEDA_EINVAL;
    if (!inside(dense_queries[i], layer->n_tokens)) return VEDA_ERANGE;
    if (overlap(dense_queries[i], layer->query)) return VEDA_ERANGE;
    for (int j = 0; j < i; ++j)
      if (overlap(dense_queries[i], dense_queries[j])) return VEDA_ERANGE;
  }
  // argument checks of the three stages, all before the first launch
  if (!q || !k || !wq || !wk || !idx || !ws) return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  if (ws_bytes < qhat_bytes(D) + khat_bytes(D)) return VEDA_EWORKSPACE;
  st = veda_sparse_attn_check(layer, q, k, v, idx, nullptr, dense, n_dense, scale, out);
  if (st != VEDA_OK) return st;
  for (int i = 0; i < n_dense_queries; ++i) {
    full.query = dense_queries[i];
    st = veda_sparse_attn_check(&full, q, k, v, nullptr, nullptr, dense, n_dense, scale, out);
    if (st != VEDA_OK) return st;
  }
  st = veda_select(layer, q, k, wq, wk, idx, nullptr, ws, ws_bytes, stream);
  if (st != VEDA_OK) return st;
  // the processing order goes into the workspace, free once the selection has run (its
  // q_hat part alone, B*H*Tq*p floats, is larger)
  int32_t* const order = static_cast<int32_t*>(ws);
  st = veda_tile_order(layer, idx, order, stream);
  if (st != VEDA_OK) return st;
  st = veda_sparse_attn(layer, q, k, v, idx, order, dense, n_dense, scale, out, nullptr, stream);
  if (st != VEDA_OK) return st;
  // dense query ranges that touch each other run as one launch (every row attends to the
  // same keys, so grouping rows into tiles across a boundary changes nothing)
  veda_range merged[VEDA_MAX_DENSE];
  int n_merged = 0;
  for (int i = 0; i < n_dense_queries; ++i)
    if (dense_queries[i].len > 0) merged[n_merged++] = dense_queries[i];
  std::sort(merged, merged + n_merged,
            [](const veda_range& a, const veda_range& b) { return a.start < b.start; });
  int n_runs = 0;
  for (int i = 0; i < n_merged; ++i) {
    if (n_runs > 0 && merged[n_runs - 1].start + merged[n_runs - 1].len == merged[i].start)
      merged[n_runs - 1].len += merged[i].len;
    else
      merged[n_runs++] = merged[i];
  }
  for (int i = 0; i < n_runs; ++i) {
    full.query = merged[i];
    st = veda_sparse_attn(&full, q, k, v, nullptr, nullptr, dense, n_dense, scale, out, nullptr, stream);
    if (st != VEDA_OK) return st;
  }
  return VEDA_OK;
}

}  // extern "C"

namespace {

int window_check(const veda_layer* layer, int64_t frame_tokens, int32_t chunk_frames,
                 int32_t halo_chunks, int32_t anchors, veda::WindowPattern* P) {
  int st = check_layer(layer, false);
  if (st != VEDA_OK) return st;
  if (layer->n_seg != 1) return VEDA_EUNSUPPORTED;
  if (layer->seg[0].start != layer->query.start || layer->seg[0].len != layer->query.len)
    return VEDA_ERANGE;
  if (frame_tokens < 1 || chunk_frames < 1 || halo_chunks < 0 || (anchors != 0 && anchors != 1))
    return VEDA_EINVAL;
  P->frame_tokens = frame_tokens;
  P->chunk_frames = chunk_frames;
  P->halo_chunks = halo_chunks;
  P->anchors = anchors;
  return VEDA_OK;
}

}  // namespace

extern "C" {

int64_t veda_window_width(const veda_layer* layer, int64_t frame_tokens, int32_t chunk_frames,
                          int32_t halo_chunks, int32_t anchors) {
  veda::WindowPattern P{};
  const int st = window_check(layer, frame_tokens, chunk_frames, halo_chunks, anchors, &P);
  if (st != VEDA_OK) return st;
  return veda::window_max_tiles(layer->query.start, layer->query.len, layer->tile, layer->seg[0].len, P);
}

int veda_window_indices(const veda_layer* layer, int64_t frame_tokens, int32_t chunk_frames,
                        int32_t halo_chunks, int32_t anchors, int32_t* idx, int32_t width,
                        void* stream) {
  veda::WindowPattern P{};
  int st = window_check(layer, frame_tokens, chunk_frames, halo_chunks, anchors, &P);
  if (st != VEDA_OK) return st;
  if (!idx || !aligned16(idx)) return VEDA_EINVAL;
  const int64_t need = veda::window_max_tiles(layer->query.start, layer->query.len, layer->tile,
                                              layer->seg[0].len, P);
  if (width < need || width > ceil_div(layer->seg[0].len, layer->tile)) return VEDA_EINVAL;
  const int64_t Tq = ceil_div(layer->query.len, layer->tile);
  if (Tq == 0) return VEDA_OK;
  return hip_status(veda::launch_window_indices(layer->query.start, layer->query.len, layer->tile,
                                                layer->seg[0].len, (int32_t)Tq, layer->B * layer->H, P,
                                                idx, width, (hipStream_t)stream));
}

int veda_block_mass(const veda_layer* layer, const void* q, const void* k, const veda_range* dense,
                    int32_t n_dense, float scale, float* lse, float* mass, float* dense_mass_opt,
                    void* stream) {
  if (!layer) return VEDA_EINVAL;
  veda_layer full = *layer;   // the teacher attends to every tile of every segment
  for (int s = 0; s < full.n_seg && s < VEDA_MAX_SEGMENTS; ++s)
    full.budget[s] = (int32_t)std::min<int64_t>(ceil_div(std::max<int64_t>(full.seg[s].len, 0),
                                                         std::max(full.tile, 1)), INT32_MAX);
  veda::DenseDev DD{};
  int st = sparse_attn_check(&full, q, k, k, nullptr, nullptr, dense, n_dense, scale, mass, &DD);
  if (st != VEDA_OK) return st;
  if (!lse || !aligned16(lse)) return VEDA_EINVAL;
  if (dense_mass_opt && !aligned16(dense_mass_opt)) return VEDA_EINVAL;
  LayerDev D = to_dev(&full);
  if (D.Tq == 0) return VEDA_OK;
  if (scale == 0.f) scale = 1.0f / std::sqrt((float)layer->d);
  return hip_status(veda::launch_block_mass(D, DD, q, k, scale, lse, mass, dense_mass_opt,
                                            (hipStream_t)stream));
}

int veda_block_recall(const veda_layer* layer, const float* mass, const int32_t* idx, float* recall,
                      void* stream) {
  int st = check_layer(layer, false);
  if (st != VEDA_OK) return st;
  if (!mass || !idx || !recall) return VEDA_EINVAL;
  if (!aligned16(mass) || !aligned16(idx) || !aligned16(recall)) return VEDA_EINVAL;
  LayerDev D = to_dev(layer);
  if (D.Tq == 0) return VEDA_OK;
  return hip_status(veda::launch_block_recall(D, mass, idx, recall, (hipStream_t)stream));
}

int veda_dequant_fp8_e4m3(const uint8_t* src, void* dst_bf16, int64_t n, int32_t pow2_exp,
                          void* stream) {
  if (n < 0) return VEDA_EINVAL;
  if (n == 0) return VEDA_OK;
  if (!src || !dst_bf16) return VEDA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(dst_bf16) & 1u) != 0) return VEDA_EINVAL;
  if (pow2_exp < -24 || pow2_exp > 24) return VEDA_EUNSUPPORTED;
  return hip_status(veda::launch_dequant_e4m3(src, dst_bf16, n, pow2_exp, (hipStream_t)stream));
}

}  // extern "C"
