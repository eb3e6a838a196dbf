// Drives the host code of the C ABI -- the argument validation of every entry point and the
// safetensors reader -- with random and malformed inputs.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer and linked against launch_stubs.cpp in place of the kernels, so
// it needs no device.
//
//   host_fuzz <dir for files> <seed> <layer iterations> <file iterations>
//
// Properties checked beside the sanitizers' own:
//   - a call that returns an error launches nothing;
//   - a launched kernel receives geometry its stand-in accepts (the kernels' preconditions);
//   - with valid pointers, each entry point returns veda_layer_check's status for the layer,
//     and veda_select_workspace_bytes is 0 exactly for layers selection rejects;
//   - a launch error comes back as VEDA_EHIP;
//   - a well-formed safetensors file reads back exactly (names with every kind of escape,
//     zero-size tensors, metadata); a damaged one is either rejected or, when the damage
//     left it well formed, reads back a consistent tiling of its data buffer.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/veda.h"
#include "launch_stubs.h"

namespace {

struct Rng {
  uint64_t s;
  uint64_t next() {   // splitmix64
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int64_t below(int64_t n) { return n <= 0 ? 0 : (int64_t)(next() % (uint64_t)n); }
  bool chance(int pct) { return below(100) < pct; }
  template <class T, size_t N>
  T pick(const T (&a)[N]) { return a[below(N)]; }
};

long g_checks = 0;

void fail(const char* what, const char* call, int st) {
  std::fprintf(stderr, "property failed after %s (status %d): %s\n", call, st, what);
  std::abort();
}

#define EXPECT(cond, call, st)        \
  do {                                \
    ++g_checks;                       \
    if (!(cond)) fail(#cond, call, st); \
  } while (0)

// ------------------------------------------------------------------------------------------
// layers

const int32_t kI32[] = {0, 1, -1, 2, 7, 8, 15, 16, 17, 32, 63, 64, 65, 127, 128, 129, 383, 384,
                        385, 8192, 8193, 46341, 65536, INT32_MAX, INT32_MIN, INT32_MAX / 2 + 1};
const int64_t kI64[] = {0, 1, -1, 8, 64, 127, 128, ((int64_t)1 << 24) - 8, (int64_t)1 << 24,
                        INT32_MAX, (int64_t)1 << 31, (int64_t)1 << 32, (int64_t)1 << 37,
                        (int64_t)1 << 40, ((int64_t)1 << 40) + 1, (int64_t)1 << 62, INT64_MAX,
                        INT64_MAX - 7, INT64_MIN};

// A plausible layer: query segment first, then up to three more key segments, then room for
// dense ranges; contiguous [B, n, H, d] strides, sometimes a padded head stride.
veda_layer plausible_layer(Rng& r, int64_t* dense_room) {
  veda_layer L{};
  L.B = 1 + (int32_t)r.below(3);
  L.H = 1 + (int32_t)r.below(5);
  L.d = r.chance(50) ? 64 : 128;
  L.p = 16 * (1 + (int32_t)r.below(r.chance(10) ? 24 : 6));
  L.tile = r.chance(50) ? 64 : 128;
  L.wdtype = (int32_t)r.below(2);
  const int64_t nq = r.chance(5) ? 0 : 1 + r.below(4000);
  int64_t at = 0;
  L.query = {0, nq};
  L.n_seg = 1 + (int32_t)r.below(4);
  for (int s = 0; s < L.n_seg; ++s) {
    const int64_t len = s == 0 ? nq : 1 + r.below(900);
    L.seg[s] = {at, len};
    L.budget[s] = r.chance(20) ? INT32_MAX : (int32_t)r.below(70);
    at += len;
  }
  *dense_room = at;
  L.n_tokens = at + r.below(3000);
  L.stride_h = L.d + (r.chance(20) ? 8 * r.below(4) : 0);
  L.stride_n = L.H * L.stride_h;
  L.stride_b = L.n_tokens * L.stride_n;
  return L;
}

void mutate(Rng& r, veda_layer& L) {
  const int n = 1 + (int)r.below(3);
  for (int i = 0; i < n; ++i) {
    const int s = (int)r.below(VEDA_MAX_SEGMENTS);
    const bool near = r.chance(30);   // near n_tokens instead of an extreme
    const int64_t v64 = near ? (int64_t)((uint64_t)L.n_tokens + (uint64_t)(r.below(5) - 2)) : r.pick(kI64);
    switch (r.below(18)) {
      case 0: L.B = r.pick(kI32); break;
      case 1: L.H = r.pick(kI32); break;
      case 2: L.d = r.pick(kI32); break;
      case 3: L.p = r.pick(kI32); break;
      case 4: L.tile = r.pick(kI32); break;
      case 5: L.n_seg = (int32_t)r.below(7) - 1; break;
      case 6: L.n_tokens = r.pick(kI64); break;
      case 7: L.stride_b = r.pick(kI64); break;
      case 8: L.stride_n = r.pick(kI64); break;
      case 9: L.stride_h = r.pick(kI64); break;
      case 10: L.query.start = v64; break;
      case 11: L.query.len = v64; break;
      case 12: L.seg[s].start = v64; break;
      case 13: L.seg[s].len = v64; break;
      case 14: L.budget[s] = r.pick(kI32); break;
      case 15: L.wdtype = (int32_t)r.below(4) - 1; break;
      case 16: L.reserved = r.chance(50) ? 1 : -1; break;
      default:   // a huge but consistent layer
        L.n_tokens = r.pick(kI64);
        L.query = {0, L.n_tokens};
        L.seg[0] = {0, L.n_tokens};
        L.stride_b = 0;
        break;
    }
  }
}

// Fake device addresses: never dereferenced by the host code or the stand-ins.
void* dev(uintptr_t slot, uintptr_t misalign = 0) {
  return reinterpret_cast<void*>((uintptr_t)0x100000000ull + slot * 0x10000 + misalign);
}

// A device pointer argument: valid and 256-byte aligned, or (rarely) null or misaligned.
void* arg(Rng& r, uintptr_t slot, bool* bad) {
  const int64_t c = r.below(100);
  if (c < 2) {
    *bad = true;
    return nullptr;
  }
  if (c < 4) {
    *bad = true;
    return dev(slot, 4);
  }
  return dev(slot);
}

std::vector<veda_range> dense_ranges(Rng& r, int64_t room) {
  std::vector<veda_range> d;
  const int n = (int)r.below(4) + (r.chance(5) ? 8 : 0);
  int64_t at = room;
  for (int i = 0; i < n; ++i) {
    if (r.chance(8)) {
      d.push_back({r.pick(kI64), r.pick(kI64)});
    } else {
      const int64_t len = r.chance(10) ? 0 : 1 + r.below(700);
      if (r.chance(10)) at -= r.below(50);   // may overlap the previous range or a segment
      d.push_back({at, len});
      at += len;
    }
  }
  return d;
}

struct Call {
  long before;
  explicit Call(const veda_layer& L) : before(stub::launches) { stub::n_tokens = L.n_tokens; }
  long launched() const { return stub::launches - before; }
};

// status of a call that launches when it succeeds: nothing launched on error, EHIP when the
// stand-ins report a launch error
void check_status(const char* name, int st, const Call& c) {
  EXPECT(st <= 0, name, st);
  if (st != VEDA_OK && st != VEDA_EHIP) EXPECT(c.launched() == 0, name, st);
  if (st == VEDA_EHIP) EXPECT(stub::fail_launch && c.launched() >= 1, name, st);
  if (stub::fail_launch && c.launched() >= 1) EXPECT(st == VEDA_EHIP, name, st);
}

void fuzz_layer(Rng& r, const veda_layer& L, int64_t room) {
  stub::fail_launch = r.chance(5);
  stub::fits = !r.chance(10);
  const int c0 = veda_layer_check(&L, 0);
  const int c1 = veda_layer_check(&L, 1);
  EXPECT(c0 <= 0 && c1 <= 0, "veda_layer_check", c1);
  if (c1 == VEDA_OK) EXPECT(c0 == VEDA_OK, "veda_layer_check", c0);
  (void)veda_k_total(&L);
  const size_t ws_need = veda_select_workspace_bytes(&L);
  EXPECT((ws_need > 0) == (c1 == VEDA_OK), "veda_select_workspace_bytes", c1);
  const bool empty_q = c0 == VEDA_OK && L.query.len == 0;
  const float scale = r.chance(3) ? (r.chance(50) ? -1.f : NAN) : (r.chance(50) ? 0.f : 0.125f);

  {   // selection
    bool bad = false;
    void* q = arg(r, 1, &bad);
    void* k = arg(r, 2, &bad);
    void* wq = arg(r, 3, &bad);
    void* wk = arg(r, 4, &bad);
    int32_t* idx = static_cast<int32_t*>(arg(r, 5, &bad));
    float* scores = r.chance(50) ? nullptr : static_cast<float*>(arg(r, 6, &bad));
    const size_t ws_bytes = r.chance(5) && ws_need > 0 ? ws_need - 1 : ws_need + (size_t)r.below(4096);
    Call c(L);
    int st = veda_select(&L, q, k, wq, wk, idx, scores, dev(7), ws_bytes, nullptr);
    check_status("veda_select", st, c);
    if (!bad && ws_bytes >= ws_need && !stub::fail_launch) EXPECT(st == c1, "veda_select", st);
    if (st == VEDA_OK) EXPECT(c.launched() == (empty_q ? 0 : 2), "veda_select", st);

    Call c2(L);
    float* qh = static_cast<float*>(dev(8));
    st = veda_pool_project(&L, q, k, wq, wk, qh, static_cast<float*>(dev(9)), nullptr);
    check_status("veda_pool_project", st, c2);
    if (!bad && !stub::fail_launch) EXPECT(st == c1, "veda_pool_project", st);

    Call c3(L);
    st = veda_score_topk(&L, qh, static_cast<float*>(dev(9)), idx, scores, nullptr);
    check_status("veda_score_topk", st, c3);
    if (!bad && !stub::fail_launch) EXPECT(st == c1, "veda_score_topk", st);
  }

  std::vector<veda_range> dense = dense_ranges(r, room);
  const int32_t nd = r.chance(3) ? -1 : (int32_t)dense.size();
  const veda_range* dp = dense.empty() && r.chance(50) ? nullptr : dense.data();
  {   // attention
    bool bad = false;
    void* q = arg(r, 11, &bad);
    void* k = arg(r, 12, &bad);
    void* v = arg(r, 13, &bad);
    void* out = arg(r, 14, &bad);
    const int32_t* idx = r.chance(20) ? nullptr : static_cast<const int32_t*>(arg(r, 15, &bad));
    float* lse = r.chance(50) ? nullptr : static_cast<float*>(dev(16, r.chance(3) ? 4 : 0));
    // a processing order: absent, aligned, or 2-byte aligned (rejected); with or without idx
    const int32_t* ord = r.chance(2) ? nullptr : static_cast<const int32_t*>(dev(22, r.chance(4) ? 2 : 0));
    const int chk = veda_sparse_attn_check(&L, q, k, v, idx, ord, dp, nd, scale, out);
    if (ord && !idx && !bad && c0 == VEDA_OK) EXPECT(chk == VEDA_EINVAL, "veda_sparse_attn_check order", chk);
    EXPECT(chk <= 0, "veda_sparse_attn_check", chk);
    if (c0 != VEDA_OK) EXPECT(chk == c0, "veda_sparse_attn_check", chk);
    Call c(L);
    int st = veda_sparse_attn(&L, q, k, v, idx, ord, dp, nd, scale, out, lse, nullptr);
    check_status("veda_sparse_attn", st, c);
    if (chk != VEDA_OK) EXPECT(st == chk, "veda_sparse_attn", st);
    if (st == VEDA_OK) EXPECT(c.launched() == (empty_q ? 0 : 1), "veda_sparse_attn", st);

    const float* qs = static_cast<const float*>(dev(17, r.chance(3) ? 2 : 0));
    Call c2(L);
    st = veda_sparse_attn_fp8qk(&L, static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k), v,
                                r.chance(2) ? nullptr : qs, qs, idx, ord, dp, nd, scale, out, lse, nullptr);
    check_status("veda_sparse_attn_fp8qk", st, c2);
    if (chk != VEDA_OK) EXPECT(st == chk, "veda_sparse_attn_fp8qk", st);

    Call c3(L);
    st = veda_quantize_fp8_e4m3(&L, q, static_cast<uint8_t*>(dev(18)), static_cast<float*>(dev(19)), nullptr);
    check_status("veda_quantize_fp8_e4m3", st, c3);
    if (!bad && !stub::fail_launch) EXPECT(st == c0, "veda_quantize_fp8_e4m3", st);

    // the FP8-V form: the fp8qk checks plus 64-aligned segment and dense starts
    Call c8(L);
    st = veda_sparse_attn_fp8(&L, static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k),
                              static_cast<const uint8_t*>(v), qs, qs, r.chance(2) ? nullptr : qs, idx, ord, dp,
                              nd, scale, out, lse, nullptr);
    check_status("veda_sparse_attn_fp8", st, c8);
    if (chk != VEDA_OK) EXPECT(st == chk, "veda_sparse_attn_fp8", st);

    Call c9(L);
    st = veda_quantize_fp8_e4m3_vt(&L, v, static_cast<uint8_t*>(dev(18)), static_cast<float*>(dev(19)), nullptr);
    check_status("veda_quantize_fp8_e4m3_vt", st, c9);
    const size_t vt_bytes = veda_fp8_vt_bytes(&L);
    if (c0 != VEDA_OK) EXPECT(vt_bytes == 0, "veda_fp8_vt_bytes", c0);
    const int c9w = c0 == VEDA_OK && vt_bytes == 0 ? VEDA_EUNSUPPORTED : c0;
    if (!bad && !stub::fail_launch) EXPECT(st == c9w, "veda_quantize_fp8_e4m3_vt", st);

    Call c4(L);
    float* mass = static_cast<float*>(dev(20));
    st = veda_block_mass(&L, q, k, dp, nd, scale, static_cast<float*>(dev(21)), mass,
                         r.chance(50) ? nullptr : static_cast<float*>(dev(22)), nullptr);
    check_status("veda_block_mass", st, c4);
    // the teacher replaces the budgets, so a layer rejected for its budgets alone may pass
    bool budgets_ok = true;
    for (int s = 0; s < L.n_seg && s < VEDA_MAX_SEGMENTS; ++s) budgets_ok = budgets_ok && L.budget[s] >= 0;
    if (c0 != VEDA_OK && budgets_ok) EXPECT(st == c0, "veda_block_mass", st);

    Call c5(L);
    st = veda_block_recall(&L, mass, static_cast<const int32_t*>(dev(23)), static_cast<float*>(dev(24)), nullptr);
    check_status("veda_block_recall", st, c5);
    if (!stub::fail_launch) EXPECT(st == c0, "veda_block_recall", st);
  }

  {   // the whole layer
    std::vector<veda_range> dq;
    const int n = (int)r.below(3);
    for (int i = 0; i < n; ++i) {
      if (r.chance(10)) dq.push_back({r.pick(kI64), r.pick(kI64)});
      else if (!dense.empty()) dq.push_back(dense[(size_t)r.below((int64_t)dense.size())]);
    }
    bool bad = false;
    Call c(L);
    const int st = veda_layer_attn(&L, arg(r, 31, &bad), arg(r, 32, &bad), arg(r, 33, &bad),
                                   arg(r, 34, &bad), arg(r, 35, &bad), dp, nd, dq.data(),
                                   r.chance(3) ? -1 : (int32_t)dq.size(), scale, arg(r, 36, &bad),
                                   static_cast<int32_t*>(arg(r, 37, &bad)), dev(38),
                                   ws_need + (size_t)r.below(2), nullptr);
    check_status("veda_layer_attn", st, c);
    if (c1 != VEDA_OK) EXPECT(st == c1, "veda_layer_attn", st);
  }

  {   // window pattern
    const int64_t ft = r.chance(5) ? r.pick(kI64) : 1 + r.below(1000);
    const int32_t cf = r.chance(5) ? r.pick(kI32) : 1 + (int32_t)r.below(8);
    const int32_t halo = r.chance(5) ? r.pick(kI32) : (int32_t)r.below(3);
    const int32_t anch = (int32_t)r.below(3) - (r.chance(5) ? 1 : 0);
    stub::window_tiles = 1 + r.below(6);
    const int64_t w = veda_window_width(&L, ft, cf, halo, anch);
    EXPECT(w < 0 || w == stub::window_tiles, "veda_window_width", (int)w);
    const int32_t width = r.chance(10) ? r.pick(kI32) : (int32_t)(stub::window_tiles + r.below(3) - 1);
    Call c(L);
    const int st = veda_window_indices(&L, ft, cf, halo, anch, static_cast<int32_t*>(dev(41)), width, nullptr);
    check_status("veda_window_indices", st, c);
    if (w < 0) EXPECT(st == w, "veda_window_indices", st);
  }
}

void fuzz_plain_calls(Rng& r) {
  for (int i = 0; i < 50; ++i) {
    const int64_t n = r.chance(20) ? r.pick(kI64) : r.below(5000);
    const int32_t e = (int32_t)r.below(60) - 30;
    veda_layer dummy{};
    stub::fail_launch = r.chance(10);
    Call c(dummy);
    const int st = veda_dequant_fp8_e4m3(static_cast<const uint8_t*>(dev(50)), dev(51, r.chance(5) ? 1 : 0),
                                         n, e, nullptr);
    check_status("veda_dequant_fp8_e4m3", st, c);
  }
  for (int s = -12; s <= 2; ++s) EXPECT(veda_status_string(s) != nullptr, "veda_status_string", s);
  EXPECT(veda_layer_check(nullptr, 0) == VEDA_EINVAL, "veda_layer_check", 0);
  EXPECT(veda_k_total(nullptr) == -1, "veda_k_total", 0);
  EXPECT(veda_select_workspace_bytes(nullptr) == 0, "veda_select_workspace_bytes", 0);
  EXPECT(veda_abi_version() == VEDA_ABI_VERSION, "veda_abi_version", 0);
}

// ------------------------------------------------------------------------------------------
// safetensors files

struct Tensor {
  std::string name;       // UTF-8
  std::string json_name;  // as written in the header
  int dtype;
  std::vector<int64_t> shape;
  std::string bytes;
};

const char* kDtName[] = {"", "F16", "BF16", "F32", "F64", "F8_E4M3", "F8_E5M2", "I8", "U8",
                         "I16", "U16", "I32", "U32", "I64", "U64", "BOOL"};
const int kDtSize[] = {0, 2, 2, 4, 8, 1, 1, 1, 1, 2, 2, 4, 4, 8, 8, 1};

void utf8(std::string& s, uint32_t cp) {
  if (cp < 0x80) {
    s += (char)cp;
  } else if (cp < 0x800) {
    s += (char)(0xC0 | (cp >> 6));
    s += (char)(0x80 | (cp & 0x3F));
  } else if (cp < 0x10000) {
    s += (char)(0xE0 | (cp >> 12));
    s += (char)(0x80 | ((cp >> 6) & 0x3F));
    s += (char)(0x80 | (cp & 0x3F));
  } else {
    s += (char)(0xF0 | (cp >> 18));
    s += (char)(0x80 | ((cp >> 12) & 0x3F));
    s += (char)(0x80 | ((cp >> 6) & 0x3F));
    s += (char)(0x80 | (cp & 0x3F));
  }
}

void escaped(std::string& s, uint32_t cp, bool upper) {
  char b[8];
  std::snprintf(b, sizeof b, upper ? "\\u%04X" : "\\u%04x", cp);
  s += b;
}

// a random string as (decoded UTF-8, JSON text with quotes)
void random_string(Rng& r, std::string& plain, std::string& json) {
  const uint32_t pool[] = {'a', 'q', '_', '.', '0', '7', ' ', '"', '\\', '/', '\n', '\t', '\b', '\f', '\r',
                           0x01, 0x1F, 0xE9, 0x3B1, 0x4E2D, 0xFFFD, 0x1F600, 0x10FFFF};
  plain.clear();
  json = "\"";
  const int n = (int)r.below(12);
  for (int i = 0; i < n; ++i) {
    const uint32_t cp = r.pick(pool);
    utf8(plain, cp);
    const bool must = cp < 0x20 || cp == '"' || cp == '\\';
    if (!must && r.chance(60)) {
      utf8(json, cp);
      continue;
    }
    switch (cp) {
      case '"': json += r.chance(50) ? "\\\"" : "\\u0022"; continue;
      case '\\': json += r.chance(50) ? "\\\\" : "\\u005c"; continue;
      case '/': json += "\\/"; continue;
      case '\n': json += "\\n"; continue;
      case '\t': json += "\\t"; continue;
      case '\b': json += "\\b"; continue;
      case '\f': json += "\\f"; continue;
      case '\r': json += "\\r"; continue;
      default: break;
    }
    if (cp >= 0x10000) {   // surrogate pair
      const uint32_t v = cp - 0x10000;
      escaped(json, 0xD800 + (v >> 10), r.chance(50));
      escaped(json, 0xDC00 + (v & 0x3FF), r.chance(50));
    } else {
      escaped(json, cp, r.chance(50));
    }
  }
  json += '"';
}

std::string ws(Rng& r) {
  static const char kWs[] = {' ', '\t', '\n', '\r'};
  std::string s;
  if (r.chance(30))
    for (int i = (int)r.below(3); i >= 0; --i) s += kWs[r.below(4)];
  return s;
}

struct Meta {
  std::string key, key_json, value, value_json;
};

std::string le64(uint64_t v) {
  std::string s(8, '\0');
  for (int i = 0; i < 8; ++i) s[(size_t)i] = (char)((v >> (8 * i)) & 0xFF);
  return s;
}

// A well-formed file: tensors tiling the data buffer in a random order, optional metadata,
// random whitespace and trailing spaces in the header.
std::string make_file(Rng& r, std::vector<Tensor>& ts, std::vector<Meta>& meta) {
  ts.clear();
  meta.clear();
  const int n = (int)r.below(7);
  for (int i = 0; i < n; ++i) {
    Tensor t;
    for (;;) {
      random_string(r, t.name, t.json_name);
      bool dup = t.name == "__metadata__";
      for (auto& o : ts) dup = dup || o.name == t.name;
      if (!dup) break;
    }
    t.dtype = 1 + (int)r.below(15);
    const int nd = (int)r.below(5);
    int64_t count = 1;
    for (int d = 0; d < nd; ++d) {
      t.shape.push_back(r.chance(10) ? 0 : 1 + r.below(5));
      count *= t.shape.back();
    }
    for (int64_t b = 0; b < count * kDtSize[t.dtype]; ++b) t.bytes += (char)r.below(256);
    ts.push_back(std::move(t));
  }
  const int nm = r.chance(50) ? 0 : (int)r.below(4);
  for (int i = 0; i < nm; ++i) {
    Meta m;
    for (;;) {
      random_string(r, m.key, m.key_json);
      bool dup = false;
      for (auto& o : meta) dup = dup || o.key == m.key;
      if (!dup) break;
    }
    random_string(r, m.value, m.value_json);
    meta.push_back(std::move(m));
  }
  // data order: a random permutation of the tensors
  std::vector<size_t> order(ts.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  for (size_t i = order.size(); i > 1; --i) std::swap(order[i - 1], order[(size_t)r.below((int64_t)i)]);
  std::vector<int64_t> begin(ts.size());
  std::string data;
  for (size_t i : order) {
    begin[i] = (int64_t)data.size();
    data += ts[i].bytes;
  }
  // header: metadata at a random place among the tensor entries
  std::vector<std::string> entries;
  for (size_t i = 0; i < ts.size(); ++i) {
    std::string e = ws(r) + ts[i].json_name + ws(r) + ":" + ws(r) + "{";
    std::string fields[3];
    fields[0] = ws(r) + "\"dtype\"" + ws(r) + ":" + ws(r) + "\"" + kDtName[ts[i].dtype] + "\"";
    std::string shape = "[";
    for (size_t d = 0; d < ts[i].shape.size(); ++d)
      shape += (d ? "," : "") + ws(r) + std::to_string(ts[i].shape[d]);
    shape += ws(r) + "]";
    fields[1] = ws(r) + "\"shape\"" + ws(r) + ":" + ws(r) + shape;
    fields[2] = ws(r) + "\"data_offsets\":[" + std::to_string(begin[i]) + "," + ws(r) +
                std::to_string(begin[i] + (int64_t)ts[i].bytes.size()) + "]";
    for (int k = 2; k > 0; --k) std::swap(fields[k], fields[r.below(k + 1)]);
    e += fields[0] + "," + fields[1] + "," + fields[2] + ws(r) + "}";
    entries.push_back(e);
  }
  if (!meta.empty() || r.chance(20)) {
    std::string e = ws(r) + "\"__metadata__\"" + ws(r) + ":{";
    for (size_t i = 0; i < meta.size(); ++i)
      e += (i ? "," : "") + ws(r) + meta[i].key_json + ":" + ws(r) + meta[i].value_json + ws(r);
    e += "}";
    entries.insert(entries.begin() + r.below((int64_t)entries.size() + 1), e);
  }
  std::string hdr = "{";
  for (size_t i = 0; i < entries.size(); ++i) hdr += (i ? "," : "") + entries[i];
  hdr += ws(r) + "}";
  hdr += std::string((size_t)r.below(8), ' ');
  return le64(hdr.size()) + hdr + data;
}

void write_file(const std::string& path, const std::string& bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(bytes.data(), 1, bytes.size(), f) != bytes.size() || std::fclose(f) != 0) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    std::exit(2);
  }
}

// Any file the reader accepts: the tensors tile the data buffer, each one reads back.
void check_opened(veda_st_file* f, int64_t file_size) {
  const int64_t n = veda_st_count(f);
  EXPECT(n >= 0, "veda_st_count", (int)n);
  int64_t total = 0;
  for (int64_t i = 0; i < n; ++i) {
    const char* name = nullptr;
    int32_t dtype = -1, ndim = -1;
    int64_t shape[VEDA_ST_MAX_DIMS], nbytes = -1;
    int st = veda_st_info(f, i, &name, &dtype, &ndim, shape, &nbytes);
    EXPECT(st == VEDA_OK && name && dtype >= 1 && dtype <= 15, "veda_st_info", st);
    EXPECT(ndim >= 0 && ndim <= VEDA_ST_MAX_DIMS && nbytes >= 0 && nbytes <= file_size, "veda_st_info", st);
    EXPECT(veda_st_find(f, name) <= i && veda_st_find(f, name) >= 0, "veda_st_find", 0);
    std::vector<char> buf((size_t)nbytes + 1);
    st = veda_st_read(f, i, buf.data(), nbytes);
    EXPECT(st == VEDA_OK, "veda_st_read", st);
    st = veda_st_read(f, i, buf.data(), nbytes + 1);
    EXPECT(st == VEDA_EINVAL, "veda_st_read", st);
    total += nbytes;
  }
  EXPECT(total <= file_size, "veda_st_open", 0);
  const int64_t nm = veda_st_metadata_count(f);
  for (int64_t i = 0; i < nm; ++i) {
    const char *k = nullptr, *v = nullptr;
    EXPECT(veda_st_metadata_at(f, i, &k, &v) == VEDA_OK && k && v, "veda_st_metadata_at", 0);
  }
  EXPECT(veda_st_info(f, n, nullptr, nullptr, nullptr, nullptr, nullptr) == VEDA_EINVAL, "veda_st_info", 0);
  EXPECT(veda_st_info(f, -1, nullptr, nullptr, nullptr, nullptr, nullptr) == VEDA_EINVAL, "veda_st_info", 0);
  EXPECT(veda_st_metadata_at(f, nm, nullptr, nullptr) == VEDA_EINVAL, "veda_st_metadata_at", 0);
}

// A well-formed file reads back exactly.
void check_round_trip(const std::string& path, const std::vector<Tensor>& ts, const std::vector<Meta>& meta,
                      int64_t size) {
  veda_st_file* f = nullptr;
  const int st = veda_st_open(path.c_str(), &f);
  EXPECT(st == VEDA_OK && f, "veda_st_open (well formed)", st);
  check_opened(f, size);
  EXPECT(veda_st_count(f) == (int64_t)ts.size(), "veda_st_count", 0);
  for (size_t i = 0; i < ts.size(); ++i) {
    const char* name = nullptr;
    int32_t dtype = 0, ndim = 0;
    int64_t shape[VEDA_ST_MAX_DIMS], nbytes = 0;
    EXPECT(veda_st_info(f, (int64_t)i, &name, &dtype, &ndim, shape, &nbytes) == VEDA_OK, "veda_st_info", 0);
    EXPECT(ts[i].name == name && dtype == ts[i].dtype, "veda_st_info (name, dtype)", 0);
    EXPECT(ndim == (int32_t)ts[i].shape.size(), "veda_st_info (ndim)", ndim);
    for (int d = 0; d < ndim; ++d) EXPECT(shape[d] == ts[i].shape[(size_t)d], "veda_st_info (shape)", d);
    EXPECT(nbytes == (int64_t)ts[i].bytes.size(), "veda_st_info (nbytes)", (int)nbytes);
    EXPECT(veda_st_find(f, ts[i].name.c_str()) == (int64_t)i, "veda_st_find", 0);
    std::string got((size_t)nbytes, '\0');
    EXPECT(veda_st_read(f, (int64_t)i, &got[0], nbytes) == VEDA_OK && got == ts[i].bytes, "veda_st_read", 0);
  }
  EXPECT(veda_st_find(f, "\x01no such tensor") == VEDA_ERANGE, "veda_st_find", 0);
  EXPECT(veda_st_metadata_count(f) == (int64_t)meta.size(), "veda_st_metadata_count", 0);
  for (size_t i = 0; i < meta.size(); ++i) {
    const char *k = nullptr, *v = nullptr;
    EXPECT(veda_st_metadata_at(f, (int64_t)i, &k, &v) == VEDA_OK, "veda_st_metadata_at", 0);
    EXPECT(meta[i].key == k && meta[i].value == v, "veda_st_metadata_at (text)", 0);
  }
  veda_st_close(f);
}

// Open a damaged file: a status, never a crash; whatever is accepted is consistent.
int open_damaged(const std::string& path, const std::string& bytes) {
  write_file(path, bytes);
  veda_st_file* f = reinterpret_cast<veda_st_file*>(1);
  const int st = veda_st_open(path.c_str(), &f);
  EXPECT(st == VEDA_OK || st == VEDA_EFORMAT || st == VEDA_EIO, "veda_st_open (damaged)", st);
  if (st != VEDA_OK) {
    EXPECT(f == nullptr, "veda_st_open (damaged)", st);
    return st;
  }
  check_opened(f, (int64_t)bytes.size());
  veda_st_close(f);
  return st;
}

// Hand-written headers, each with the status it must get.
void fixed_headers(const std::string& dir) {
  struct Case {
    const char* header;
    int data;       // bytes of data after the header
    int status;
  };
  const Case cases[] = {
      {"{}", 0, VEDA_OK},
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2],\"data_offsets\":[0,4]}}", 4, VEDA_OK},
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2],\"data_offsets\":[0,4]}}", 5, VEDA_EFORMAT},   // hole at the end
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2],\"data_offsets\":[0,4]}}", 3, VEDA_EFORMAT},   // past the end
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2],\"data_offsets\":[1,5]}}", 5, VEDA_EFORMAT},   // hole at the start
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[3],\"data_offsets\":[0,4]}}", 4, VEDA_EFORMAT},   // count
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2],\"data_offsets\":[4,0]}}", 4, VEDA_EFORMAT},   // reversed
      {"{\"a\":{\"dtype\":\"F17\",\"shape\":[2],\"data_offsets\":[0,4]}}", 4, VEDA_EFORMAT},   // dtype
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[-2],\"data_offsets\":[0,4]}}", 4, VEDA_EFORMAT},  // sign
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[02],\"data_offsets\":[0,4]}}", 4, VEDA_EFORMAT},  // leading zero
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2.0],\"data_offsets\":[0,4]}}", 4, VEDA_EFORMAT}, // float
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2],\"data_offsets\":[0,4],}}", 4, VEDA_EFORMAT},  // trailing comma
      {"{\"a\":{\"dtype\":\"F16\",\"shape\":[2]}}", 4, VEDA_EFORMAT},                          // missing field
      {"{\"a\":{\"dtype\":\"F16\",\"dtype\":\"F16\",\"shape\":[2],\"data_offsets\":[0,4]}}", 4, VEDA_EFORMAT},
      {"{\"a\":{\"dtype\":\"U8\",\"shape\":[1],\"data_offsets\":[0,1]},"
       "\"a\":{\"dtype\":\"U8\",\"shape\":[1],\"data_offsets\":[1,2]}}", 2, VEDA_EFORMAT},      // same name
      {"{\"a\":{\"dtype\":\"U8\",\"shape\":[2],\"data_offsets\":[0,2]},"
       "\"b\":{\"dtype\":\"U8\",\"shape\":[2],\"data_offsets\":[1,3]}}", 3, VEDA_EFORMAT},      // overlap
      {"{\"a\":{\"dtype\":\"U8\",\"shape\":[4611686018427387904,4],\"data_offsets\":[0,0]}}", 0, VEDA_EFORMAT},
      {"{\"a\":{\"dtype\":\"F64\",\"shape\":[2305843009213693952],\"data_offsets\":[0,0]}}", 0, VEDA_EFORMAT},
      {"{\"a\":{\"dtype\":\"U8\",\"shape\":[99999999999999999999],\"data_offsets\":[0,0]}}", 0, VEDA_EFORMAT},
      {"{\"a\":{\"dtype\":\"U8\",\"shape\":[1,1,1,1,1,1,1,1,1],\"data_offsets\":[0,1]}}", 1, VEDA_EFORMAT},
      {"{\"a\":{\"dtype\":\"U8\",\"shape\":[1,1,1,1,1,1,1,1],\"data_offsets\":[0,1]}}", 1, VEDA_OK},
      {"{\"a\":{\"dtype\":\"U8\",\"shape\":[0,5],\"data_offsets\":[0,0]}}", 0, VEDA_OK},
      {"{\"__metadata__\":{\"k\":\"v\"},\"__metadata__\":{}}", 0, VEDA_EFORMAT},
      {"{\"__metadata__\":{\"k\":\"v\",\"k\":\"w\"}}", 0, VEDA_EFORMAT},
      {"{\"__metadata__\":{\"k\":{\"x\":\"y\"}}}", 0, VEDA_EFORMAT},
      {"{\"__metadata__\":{\"k\":1}}", 0, VEDA_EFORMAT},
      {"{\"__metadata__\":{\"\\ud83d\\ude00\":\"\\u00e9\"}}", 0, VEDA_OK},
      {"{\"__metadata__\":{\"\\ud83d\":\"x\"}}", 0, VEDA_EFORMAT},      // lone high surrogate
      {"{\"__metadata__\":{\"\\ude00\":\"x\"}}", 0, VEDA_EFORMAT},      // lone low surrogate
      {"{\"__metadata__\":{\"\\u12\":\"x\"}}", 0, VEDA_EFORMAT},        // short escape
      {"{\"__metadata__\":{\"\\x41\":\"x\"}}", 0, VEDA_EFORMAT},        // unknown escape
      {"{\"__metadata__\":{\"a\\u0000b\":\"x\"}}", 0, VEDA_EFORMAT},   // U+0000
      {"{\"a\\u0000\":{\"dtype\":\"U8\",\"shape\":[1],\"data_offsets\":[0,1]}}", 1, VEDA_EFORMAT},
      {"{\"__metadata__\":{\"a\nb\":\"x\"}}", 0, VEDA_EFORMAT},         // raw control character
      {"{\"__metadata__\":{\"a\":\"x", 0, VEDA_EFORMAT},                // unterminated
      {"{} x", 0, VEDA_EFORMAT},                                          // trailing text
      {"[]", 0, VEDA_EFORMAT},
      {"{", 0, VEDA_EFORMAT},
      {"\"", 0, VEDA_EFORMAT},
  };
  int i = 0;
  for (const Case& c : cases) {
    const std::string h = c.header;
    std::string bytes = le64(h.size()) + h + std::string((size_t)c.data, 'z');
    const std::string path = dir + "/fixed_" + std::to_string(i++) + ".safetensors";
    write_file(path, bytes);
    veda_st_file* f = nullptr;
    const int st = veda_st_open(path.c_str(), &f);
    if (st != c.status) {
      std::fprintf(stderr, "header %s: status %d, expected %d\n", c.header, st, c.status);
      std::abort();
    }
    ++g_checks;
    if (st == VEDA_OK) {
      check_opened(f, (int64_t)bytes.size());
      veda_st_close(f);
    }
  }
  // the length field: too small, past the end, beyond the format's limit
  const std::string h = "{}";
  const uint64_t lens[] = {0, 1, 3, 1000, (uint64_t)100 << 20, ((uint64_t)100 << 20) + 1, UINT64_MAX,
                           (uint64_t)1 << 63};
  for (uint64_t n : lens) {
    const std::string path = dir + "/len.safetensors";
    write_file(path, le64(n) + h);
    veda_st_file* f = nullptr;
    const int st = veda_st_open(path.c_str(), &f);
    EXPECT(st == VEDA_EFORMAT && f == nullptr, "veda_st_open (length field)", st);
  }
  for (int n = 0; n < 8; ++n) {   // shorter than the length field
    const std::string path = dir + "/short.safetensors";
    write_file(path, std::string((size_t)n, '\0'));
    veda_st_file* f = nullptr;
    EXPECT(veda_st_open(path.c_str(), &f) == VEDA_EFORMAT, "veda_st_open (short)", n);
  }
  veda_st_file* f = nullptr;
  EXPECT(veda_st_open((dir + "/does/not/exist").c_str(), &f) == VEDA_EIO, "veda_st_open (missing)", 0);
  EXPECT(veda_st_open(dir.c_str(), &f) != VEDA_OK && f == nullptr, "veda_st_open (directory)", 0);
  EXPECT(veda_st_open(nullptr, &f) == VEDA_EINVAL, "veda_st_open (null path)", 0);
  EXPECT(veda_st_open(dir.c_str(), nullptr) == VEDA_EINVAL, "veda_st_open (null out)", 0);
  EXPECT(veda_st_count(nullptr) == VEDA_EINVAL && veda_st_metadata_count(nullptr) == VEDA_EINVAL,
         "null handle", 0);
  EXPECT(veda_st_find(nullptr, "a") == VEDA_EINVAL, "veda_st_find (null)", 0);
  char b[4];
  EXPECT(veda_st_read(nullptr, 0, b, 4) == VEDA_EINVAL, "veda_st_read (null)", 0);
  veda_st_close(nullptr);
}

void fuzz_files(Rng& r, const std::string& dir, long iters) {
  fixed_headers(dir);
  std::vector<Tensor> ts;
  std::vector<Meta> meta;
  long accepted = 0, rejected = 0;
  for (long it = 0; it < iters; ++it) {
    const std::string file = make_file(r, ts, meta);
    const std::string path = dir + "/f.safetensors";
    write_file(path, file);
    check_round_trip(path, ts, meta, (int64_t)file.size());
    std::string bad = file;
    uint64_t hlen = 0;
    for (int i = 7; i >= 0; --i) hlen = (hlen << 8) | (unsigned char)file[(size_t)i];
    switch (r.below(6)) {
      case 0:   // truncated
        bad.resize((size_t)r.below((int64_t)file.size()));
        break;
      case 1:   // bytes of the header changed
        for (int k = (int)r.below(4); k >= 0; --k)
          bad[8 + (size_t)r.below((int64_t)hlen)] = (char)r.below(256);
        break;
      case 2: {   // header length field changed
        const uint64_t v = r.chance(50) ? hlen + (uint64_t)r.below(9) - 4 : r.next() >> r.below(64);
        bad.replace(0, 8, le64(v));
        break;
      }
      case 3:   // bytes appended
        bad += std::string((size_t)(1 + r.below(9)), 'x');
        break;
      case 4: {   // a digit of the header changed
        std::vector<size_t> digits;
        for (size_t i = 8; i < 8 + hlen; ++i)
          if (bad[i] >= '0' && bad[i] <= '9') digits.push_back(i);
        if (!digits.empty()) bad[digits[(size_t)r.below((int64_t)digits.size())]] = (char)('0' + r.below(10));
        break;
      }
      default: {   // a header byte removed or inserted
        const size_t at = 8 + (size_t)r.below((int64_t)hlen);
        if (r.chance(50)) bad.erase(at, 1);
        else bad.insert(at, 1, "{}[],:\"\\ 0a"[r.below(11)]);
        break;
      }
    }
    (open_damaged(dir + "/bad.safetensors", bad) == VEDA_OK ? accepted : rejected)++;
  }
  std::printf("files: %ld well formed, damaged: %ld rejected, %ld still well formed\n", iters, rejected,
              accepted);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 5) {
    std::fprintf(stderr, "usage: %s <dir> <seed> <layer iterations> <file iterations>\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  Rng r{std::strtoull(argv[2], nullptr, 10)};
  const long layer_iters = std::strtol(argv[3], nullptr, 10);
  const long file_iters = std::strtol(argv[4], nullptr, 10);
  long ok[2] = {0, 0};
  for (long it = 0; it < layer_iters; ++it) {
    int64_t room = 0;
    veda_layer L = plausible_layer(r, &room);
    if (r.chance(60)) mutate(r, L);
    ok[veda_layer_check(&L, 0) == VEDA_OK]++;
    fuzz_layer(r, L, room);
  }
  fuzz_plain_calls(r);
  std::printf("layers: %ld valid for attention, %ld rejected; %ld launches recorded\n", ok[1], ok[0],
              stub::launches);
  fuzz_files(r, dir, file_iters);
  std::printf("checks: %ld\n", g_checks);
  return 0;
}
