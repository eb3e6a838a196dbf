// Shared definitions of the gfx950 kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace veda {

// Segment of key tiles as the kernels see it (derived on the host from veda_layer).
struct SegDev {
  int64_t start;   // first token
  int64_t len;     // tokens
  int32_t T;       // tiles = ceil(len / tile)
  int32_t K;       // selected tiles per query tile = min(budget, T)
  int32_t koff;    // first index column of this segment's block in idx rows
  int32_t toff;    // first column of this segment in the concatenated key-tile space
};

struct RangeDev {
  int64_t start;
  int64_t len;
};

struct LayerDev {
  int32_t B, H, d, p, tile, n_seg;
  int32_t Tq;      // query tiles
  int32_t Tk;      // key tiles over all segments
  int32_t Ktot;    // selected tiles per query tile over all segments
  int32_t wdtype;  // predictor weight type: 0 bf16, 1 f16
  int64_t sb, sn, sh;       // element strides of q, k, v, out
  int64_t q0, qlen;         // query segment
  SegDev seg[4];
};

constexpr int kMaxSeg = 4;
constexpr int kMaxDense = 8;

struct DenseDev {
  int32_t n;
  int32_t pad_;
  RangeDev r[kMaxDense];
};

// Launchers (return hipError_t of the launch).
hipError_t launch_pool_project(const LayerDev& L, const void* q, const void* k, const void* wq,
                               const void* wk, float* q_hat, float* k_hat, hipStream_t s);
hipError_t launch_score_topk(const LayerDev& L, const float* q_hat, const float* k_hat,
                             int32_t* idx, float* scores, hipStream_t s);
// order: NULL, or int32 [B, H, Tq], the query tile each (b, h)'s processing position
// takes (see work_order.hip); only read when idx is given.
hipError_t launch_sparse_attn(const LayerDev& L, const DenseDev& D, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* order, float scale, void* out,
                              float* lse, hipStream_t s);
// Q and K as E4M3FN codes (same element strides as the bf16 tensors, one byte each) with
// per-tensor scales in device memory; V, O as in launch_sparse_attn.  Needs 128-row tiles
// and a block list within the two-group kernel's table (two_group_fits).
hipError_t launch_sparse_attn_fp8qk(const LayerDev& L, const DenseDev& D, const void* q8, const void* k8,
                                    const void* v, const int32_t* idx, const int32_t* order, float scale,
                                    const float* q_scale,
                                    const float* k_scale, void* out, float* lse, hipStream_t s);
bool two_group_fits(const LayerDev& L, const DenseDev& D);
// bf16 tensor [B, n_tokens, H, d] (layer strides) -> E4M3FN codes at the same element
// offsets, with the per-tensor power-of-two scale written to *scale (device float).
hipError_t launch_quantize_fp8(const LayerDev& L, int64_t n_tokens, const void* x, uint8_t* x8,
                                float* scale, hipStream_t s);
hipError_t launch_dequant_e4m3(const uint8_t* src, void* dst, int64_t n, int32_t pow2_exp,
                               hipStream_t s);
// bf16 V [B, n_tokens, H, d] (layer strides) -> E4M3FN codes in d-major blocks of 64 tokens
// ([B, H, ceil(n_tokens / 64), d, 64], chunk-swizzled; see dequant.hip), per-tensor scale
// as launch_quantize_fp8.
hipError_t launch_quantize_fp8_vt(const LayerDev& L, int64_t n_tokens, const void* v, uint8_t* vt,
                                  float* scale, hipStream_t s);
// FP8 Q, K (as launch_sparse_attn_fp8qk) and V in the blocked layout above; P rounded to
// E4M3FN for the second product.  Needs 128-row tiles, block starts on multiples of 64 and
// a block list within the two-group kernel's table.
hipError_t launch_sparse_attn_fp8(const LayerDev& L, const DenseDev& D, const void* q8, const void* k8,
                                  const void* vt, int64_t n_tokens, const int32_t* idx, const int32_t* order,
                                  float scale,
                                  const float* q_scale, const float* k_scale, const float* v_scale, void* out,
                                  float* lse, hipStream_t s);

// Processing order of the query tiles (see work_order.hip): order int32 [B, H, Tq].
// Layers with more than kOrderCap query tiles get the identity order.
constexpr int kOrderCap = 16384;
hipError_t launch_tile_order(const LayerDev& L, const int32_t* idx, int32_t* order, hipStream_t s);

// Teacher block attention mass (two launches: dense lse, then per-tile mass) and the
// recall of an index set under it (see block_mass.hip).  L must carry full budgets.
hipError_t launch_block_mass(const LayerDev& L, const DenseDev& D, const void* q, const void* k,
                             float scale, float* lse, float* mass, float* dense_mass, hipStream_t s);
hipError_t launch_block_recall(const LayerDev& L, const float* mass, const int32_t* idx, float* recall,
                               hipStream_t s);

// Sliding frame-chunk window pattern (see patterns.hip).
struct WindowPattern {
  int64_t frame_tokens;   // tokens per latent frame
  int32_t chunk_frames;   // frames per chunk
  int32_t halo_chunks;    // neighbouring chunks on each side
  int32_t anchors;        // 1: first and last frame are global
};
int64_t window_max_tiles(int64_t q0, int64_t qlen, int64_t tile, int64_t seg_len, const WindowPattern& P);
hipError_t launch_window_indices(int64_t q0, int64_t qlen, int64_t tile, int64_t seg_len, int32_t Tq,
                                 int32_t BH, const WindowPattern& P, int32_t* idx, int32_t kmax,
                                 hipStream_t s);

// Rows of the score block one selection workgroup handles for Tk key tiles and
// predictor width p.
int score_rows_per_block(int Tk, int p);

}  // namespace veda
