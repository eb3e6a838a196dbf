// Host-side reader of safetensors files: predictor weights (the competition's
// selector file of float16 query/key projections, an FP8 predictor file) are
// loaded from this format.
//
// Layout: an 8-byte little-endian header length N, N bytes of JSON, then the data
// buffer.  The JSON object maps each tensor name to {"dtype", "shape",
// "data_offsets": [begin, end]} (offsets relative to the data buffer) and may hold a
// "__metadata__" object of string values.  The reader is strict: it checks every
// offset against the file, every byte count against dtype x shape, and that the
// tensors tile the data buffer without holes or overlaps.
#include "../../include/veda.h"

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

struct veda_st_file {
  struct Tensor {
    std::string name;
    int32_t dtype = VEDA_ST_UNKNOWN;
    std::vector<int64_t> shape;
    int64_t begin = 0, end = 0;
  };
  int fd = -1;
  int64_t data_start = 0;
  std::vector<Tensor> tensors;
  std::vector<std::pair<std::string, std::string>> meta;
  ~veda_st_file() {
    if (fd >= 0) close(fd);
  }
};

namespace {

constexpr int64_t kMaxHeader = (int64_t)100 << 20;   // the format's own limit

struct DType {
  const char* name;
  int32_t code;
  int32_t size;
};
const DType kDTypes[] = {
    {"F16", VEDA_ST_F16, 2},     {"BF16", VEDA_ST_BF16, 2},      {"F32", VEDA_ST_F32, 4},
    {"F64", VEDA_ST_F64, 8},     {"F8_E4M3", VEDA_ST_F8_E4M3, 1}, {"F8_E5M2", VEDA_ST_F8_E5M2, 1},
    {"I8", VEDA_ST_I8, 1},       {"U8", VEDA_ST_U8, 1},          {"I16", VEDA_ST_I16, 2},
    {"U16", VEDA_ST_U16, 2},     {"I32", VEDA_ST_I32, 4},        {"U32", VEDA_ST_U32, 4},
    {"I64", VEDA_ST_I64, 8},     {"U64", VEDA_ST_U64, 8},        {"BOOL", VEDA_ST_BOOL, 1},
};

// Minimal JSON reader for the header: objects, arrays, strings, non-negative integers.
struct Json {
  const char* p;
  const char* e;

  void ws() {
    while (p < e && (*p == ' ' || *p == '\t' || *p == '\n' || *p == '\r')) ++p;
  }
  bool eat(char c) {
    ws();
    if (p < e && *p == c) {
      ++p;
      return true;
    }
    return false;
  }
  static void put_utf8(std::string& s, uint32_t cp) {
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
  bool hex4(uint32_t& v) {
    if (e - p < 4) return false;
    v = 0;
    for (int i = 0; i < 4; ++i) {
      const char c = *p++;
      v <<= 4;
      if (c >= '0' && c <= '9') v |= (uint32_t)(c - '0');
      else if (c >= 'a' && c <= 'f') v |= (uint32_t)(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') v |= (uint32_t)(c - 'A' + 10);
      else return false;
    }
    return true;
  }
  bool str(std::string& out) {
    ws();
    if (p >= e || *p != '"') return false;
    ++p;
    out.clear();
    while (p < e) {
      const char c = *p++;
      if (c == '"') return true;
      if ((unsigned char)c < 0x20) return false;
      if (c != '\\') {
        out += c;
        continue;
      }
      if (p >= e) return false;
      const char x = *p++;
      switch (x) {
        case '"': out += '"'; break;
        case '\\': out += '\\'; break;
        case '/': out += '/'; break;
        case 'b': out += '\b'; break;
        case 'f': out += '\f'; break;
        case 'n': out += '\n'; break;
        case 'r': out += '\r'; break;
        case 't': out += '\t'; break;
        case 'u': {
          uint32_t cp;
          if (!hex4(cp)) return false;
          if (cp >= 0xD800 && cp < 0xDC00) {   // surrogate pair
            uint32_t lo;
            if (e - p < 2 || p[0] != '\\' || p[1] != 'u') return false;
            p += 2;
            if (!hex4(lo) || lo < 0xDC00 || lo >= 0xE000) return false;
            cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
          } else if (cp >= 0xDC00 && cp < 0xE000) {
            return false;
          } else if (cp == 0) {   // names and metadata are handed out as C strings
            return false;
          }
          put_utf8(out, cp);
          break;
        }
        default: return false;
      }
    }
    return false;
  }
  bool uint(int64_t& v) {
    ws();
    if (p >= e || *p < '0' || *p > '9') return false;
    if (*p == '0' && p + 1 < e && p[1] >= '0' && p[1] <= '9') return false;   // no leading zeros
    v = 0;
    while (p < e && *p >= '0' && *p <= '9') {
      if (v > (INT64_MAX - 9) / 10) return false;
      v = v * 10 + (*p++ - '0');
    }
    return true;
  }
  bool uint_array(std::vector<int64_t>& out) {
    out.clear();
    if (!eat('[')) return false;
    if (eat(']')) return true;
    for (;;) {
      int64_t v;
      if (!uint(v)) return false;
      out.push_back(v);
      if (eat(']')) return true;
      if (!eat(',')) return false;
    }
  }
};

int parse_header(const char* b, const char* e, veda_st_file* f) {
  Json j{b, e};
  if (!j.eat('{')) return VEDA_EFORMAT;
  if (j.eat('}')) {
    j.ws();
    return j.p == j.e ? VEDA_OK : VEDA_EFORMAT;
  }
  bool seen_meta = false;
  for (;;) {
    std::string key;
    if (!j.str(key) || !j.eat(':')) return VEDA_EFORMAT;
    if (key == "__metadata__") {
      if (seen_meta || !j.eat('{')) return VEDA_EFORMAT;
      seen_meta = true;
      if (!j.eat('}')) {
        for (;;) {
          std::string k2, v2;
          if (!j.str(k2) || !j.eat(':') || !j.str(v2)) return VEDA_EFORMAT;
          for (auto& kv : f->meta)
            if (kv.first == k2) return VEDA_EFORMAT;
          f->meta.emplace_back(std::move(k2), std::move(v2));
          if (j.eat('}')) break;
          if (!j.eat(',')) return VEDA_EFORMAT;
        }
      }
    } else {
      veda_st_file::Tensor t;
      t.name = key;
      if (!j.eat('{')) return VEDA_EFORMAT;
      bool has_dtype = false, has_shape = false, has_off = false;
      for (;;) {
        std::string field;
        if (!j.str(field) || !j.eat(':')) return VEDA_EFORMAT;
        if (field == "dtype" && !has_dtype) {
          std::string dt;
          if (!j.str(dt)) return VEDA_EFORMAT;
          for (const DType& d : kDTypes)
            if (dt == d.name) t.dtype = d.code;
          if (t.dtype == VEDA_ST_UNKNOWN) return VEDA_EFORMAT;
          has_dtype = true;
        } else if (field == "shape" && !has_shape) {
          if (!j.uint_array(t.shape) || t.shape.size() > VEDA_ST_MAX_DIMS) return VEDA_EFORMAT;
          has_shape = true;
        } else if (field == "data_offsets" && !has_off) {
          std::vector<int64_t> off;
          if (!j.uint_array(off) || off.size() != 2 || off[0] > off[1]) return VEDA_EFORMAT;
          t.begin = off[0];
          t.end = off[1];
          has_off = true;
        } else {
          return VEDA_EFORMAT;
        }
        if (j.eat('}')) break;
        if (!j.eat(',')) return VEDA_EFORMAT;
      }
      if (!has_dtype || !has_shape || !has_off) return VEDA_EFORMAT;
      for (auto& o : f->tensors)
        if (o.name == t.name) return VEDA_EFORMAT;
      f->tensors.push_back(std::move(t));
    }
    if (j.eat('}')) break;
    if (!j.eat(',')) return VEDA_EFORMAT;
  }
  j.ws();
  return j.p == j.e ? VEDA_OK : VEDA_EFORMAT;
}

int32_t item_size(int32_t code) {
  for (const DType& d : kDTypes)
    if (d.code == code) return d.size;
  return 0;
}

bool read_at(int fd, void* dst, int64_t n, int64_t off) {
  char* c = static_cast<char*>(dst);
  while (n > 0) {
    const ssize_t r = pread(fd, c, (size_t)std::min<int64_t>(n, (int64_t)1 << 30), (off_t)off);
    if (r <= 0) return false;
    c += r;
    n -= r;
    off += r;
  }
  return true;
}

}  // namespace

extern "C" {

int veda_st_open(const char* path, veda_st_file** out) {
  if (!path || !out) return VEDA_EINVAL;
  *out = nullptr;
  auto* f = new veda_st_file();
  f->fd = open(path, O_RDONLY);
  struct stat st;
  if (f->fd < 0 || fstat(f->fd, &st) != 0) {
    delete f;
    return VEDA_EIO;
  }
  const int64_t size = (int64_t)st.st_size;
  unsigned char lenb[8];
  if (size < 8 || !read_at(f->fd, lenb, 8, 0)) {
    delete f;
    return size < 8 ? VEDA_EFORMAT : VEDA_EIO;
  }
  uint64_t n = 0;
  for (int i = 7; i >= 0; --i) n = (n << 8) | lenb[i];
  if (n < 2 || n > (uint64_t)kMaxHeader || (int64_t)n > size - 8) {
    delete f;
    return VEDA_EFORMAT;
  }
  std::vector<char> hdr((size_t)n);
  if (!read_at(f->fd, hdr.data(), (int64_t)n, 8)) {
    delete f;
    return VEDA_EIO;
  }
  int rc = parse_header(hdr.data(), hdr.data() + n, f);
  if (rc != VEDA_OK) {
    delete f;
    return rc;
  }
  f->data_start = 8 + (int64_t)n;
  const int64_t data_size = size - f->data_start;
  // byte counts, bounds, and an exact tiling of the data buffer
  std::vector<std::pair<int64_t, int64_t>> spans;
  for (auto& t : f->tensors) {
    int64_t count = 1;
    for (int64_t d : t.shape) {
      if (d != 0 && count > INT64_MAX / d) {
        delete f;
        return VEDA_EFORMAT;
      }
      count *= d;
    }
    const int64_t isz = item_size(t.dtype);
    if (count > INT64_MAX / isz || t.end - t.begin != count * isz || t.end > data_size) {
      delete f;
      return VEDA_EFORMAT;
    }
    if (t.end > t.begin) spans.emplace_back(t.begin, t.end);
  }
  std::sort(spans.begin(), spans.end());
  int64_t at = 0;
  for (auto& s : spans) {
    if (s.first != at) {
      delete f;
      return VEDA_EFORMAT;
    }
    at = s.second;
  }
  if (at != data_size) {
    delete f;
    return VEDA_EFORMAT;
  }
  *out = f;
  return VEDA_OK;
}

void veda_st_close(veda_st_file* f) { delete f; }

int64_t veda_st_count(const veda_st_file* f) { return f ? (int64_t)f->tensors.size() : (int64_t)VEDA_EINVAL; }

int veda_st_info(const veda_st_file* f, int64_t i, const char** name, int32_t* dtype, int32_t* ndim,
                 int64_t* shape, int64_t* nbytes) {
  if (!f || i < 0 || i >= (int64_t)f->tensors.size()) return VEDA_EINVAL;
  const auto& t = f->tensors[(size_t)i];
  if (name) *name = t.name.c_str();
  if (dtype) *dtype = t.dtype;
  if (ndim) *ndim = (int32_t)t.shape.size();
  if (shape)
    for (size_t d = 0; d < t.shape.size(); ++d) shape[d] = t.shape[d];
  if (nbytes) *nbytes = t.end - t.begin;
  return VEDA_OK;
}

int64_t veda_st_find(const veda_st_file* f, const char* name) {
  if (!f || !name) return VEDA_EINVAL;
  for (size_t i = 0; i < f->tensors.size(); ++i)
    if (f->tensors[i].name == name) return (int64_t)i;
  return VEDA_ERANGE;
}

int veda_st_read(const veda_st_file* f, int64_t i, void* dst, int64_t nbytes) {
  if (!f || !dst || i < 0 || i >= (int64_t)f->tensors.size()) return VEDA_EINVAL;
  const auto& t = f->tensors[(size_t)i];
  if (nbytes != t.end - t.begin) return VEDA_EINVAL;
  if (nbytes == 0) return VEDA_OK;
  return read_at(f->fd, dst, nbytes, f->data_start + t.begin) ? VEDA_OK : VEDA_EIO;
}

int64_t veda_st_metadata_count(const veda_st_file* f) {
  return f ? (int64_t)f->meta.size() : (int64_t)VEDA_EINVAL;
}

int veda_st_metadata_at(const veda_st_file* f, int64_t i, const char** key, const char** value) {
  if (!f || i < 0 || i >= (int64_t)f->meta.size()) return VEDA_EINVAL;
  if (key) *key = f->meta[(size_t)i].first.c_str();
  if (value) *value = f->meta[(size_t)i].second.c_str();
  return VEDA_OK;
}

}  // extern "C"
