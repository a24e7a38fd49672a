// .ninfer v2 container: header and JSON directory validation.
// [ninfer-skill] §1: the 8-byte magic "NINFER\0\2", a little-endian uint64
// directory length, the compact UTF-8 JSON directory at offset 16, and the
// payload at align_up(16 + json_bytes, 4096) with payload-relative object
// offsets; the exact member sets of the root, identity, tensor and resource
// entries; kinds, the resource encoding, encoded sizes, ordered aligned
// non-overlapping in-payload ranges and unique names, with the error
// wording the page gives.  Readings where the page is silent (the layout
// names of the NInfer v3 layouts, the (format, layout) pairs whose size is
// known, compactness as "no whitespace outside strings") are stated in
// tq.h.  Host code only; no device work.

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <memory>
#include <string>
#include <vector>

#include "../../include/tq.h"

namespace tq {
tq_status fail(tq_status st, const char *fmt, ...);
}

namespace {

// ---- a minimal JSON reader (objects keep their member order)
struct JVal {
  enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
  bool b = false;
  bool integral = false;  // the number is a plain non-negative integer literal
  uint64_t u = 0;
  std::string s;
  std::vector<std::unique_ptr<JVal>> items;
  std::vector<std::pair<std::string, std::unique_ptr<JVal>>> members;

  const JVal *get(const char *key) const {
    for (const auto &m : members)
      if (m.first == key) return m.second.get();
    return nullptr;
  }
};

struct Parser {
  const char *p, *end;
  bool compact = true;
  std::string err;

  void ws() {
    while (p < end && (*p == ' ' || *p == '\t' || *p == '\n' || *p == '\r')) {
      compact = false;
      ++p;
    }
  }
  bool lit(const char *w) {
    const size_t n = strlen(w);
    if ((size_t)(end - p) < n || memcmp(p, w, n) != 0) return false;
    p += n;
    return true;
  }
  bool string(std::string &out) {
    if (p >= end || *p != '"') return false;
    ++p;
    while (p < end && *p != '"') {
      if ((unsigned char)*p < 0x20) return false;
      if (*p == '\\') {
        if (++p >= end) return false;
        switch (*p) {
          case '"': out += '"'; break;
          case '\\': out += '\\'; break;
          case '/': out += '/'; break;
          case 'b': out += '\b'; break;
          case 'f': out += '\f'; break;
          case 'n': out += '\n'; break;
          case 'r': out += '\r'; break;
          case 't': out += '\t'; break;
          case 'u': {
            if (end - p < 5) return false;
            unsigned cp = 0;
            for (int i = 1; i <= 4; ++i) {
              const char c = p[i];
              cp <<= 4;
              if (c >= '0' && c <= '9') cp |= c - '0';
              else if (c >= 'a' && c <= 'f') cp |= c - 'a' + 10;
              else if (c >= 'A' && c <= 'F') cp |= c - 'A' + 10;
              else return false;
            }
            p += 4;
            // UTF-8 of a BMP code point (surrogates kept as-is)
            if (cp < 0x80) out += (char)cp;
            else if (cp < 0x800) { out += (char)(0xC0 | (cp >> 6)); out += (char)(0x80 | (cp & 0x3F)); }
            else {
              out += (char)(0xE0 | (cp >> 12));
              out += (char)(0x80 | ((cp >> 6) & 0x3F));
              out += (char)(0x80 | (cp & 0x3F));
            }
            break;
          }
          default: return false;
        }
        ++p;
      } else {
        out += *p++;
      }
    }
    if (p >= end) return false;
    ++p;
    return true;
  }
  std::unique_ptr<JVal> value(int depth) {
    if (depth > 64) return nullptr;
    ws();
    if (p >= end) return nullptr;
    auto v = std::make_unique<JVal>();
    if (*p == '{') {
      ++p;
      v->kind = JVal::OBJ;
      ws();
      if (p < end && *p == '}') { ++p; return v; }
      for (;;) {
        ws();
        std::string key;
        if (!string(key)) return nullptr;
        for (const auto &m : v->members)
          if (m.first == key) { err = "directory object repeats a member"; return nullptr; }
        ws();
        if (p >= end || *p != ':') return nullptr;
        ++p;
        auto mv = value(depth + 1);
        if (!mv) return nullptr;
        v->members.emplace_back(key, std::move(mv));
        ws();
        if (p < end && *p == ',') { ++p; continue; }
        if (p < end && *p == '}') { ++p; return v; }
        return nullptr;
      }
    }
    if (*p == '[') {
      ++p;
      v->kind = JVal::ARR;
      ws();
      if (p < end && *p == ']') { ++p; return v; }
      for (;;) {
        auto iv = value(depth + 1);
        if (!iv) return nullptr;
        v->items.push_back(std::move(iv));
        ws();
        if (p < end && *p == ',') { ++p; continue; }
        if (p < end && *p == ']') { ++p; return v; }
        return nullptr;
      }
    }
    if (*p == '"') {
      v->kind = JVal::STR;
      if (!string(v->s)) return nullptr;
      return v;
    }
    if (lit("true")) { v->kind = JVal::BOOL; v->b = true; return v; }
    if (lit("false")) { v->kind = JVal::BOOL; return v; }
    if (lit("null")) return v;
    // number: a plain non-negative integer is kept exactly; anything else
    // (sign, fraction, exponent) is a number that is not one
    v->kind = JVal::NUM;
    const char *s = p;
    if (p < end && *p == '-') ++p;
    if (p >= end || *p < '0' || *p > '9') return nullptr;
    while (p < end && *p >= '0' && *p <= '9') ++p;
    bool plain = *s != '-';
    if (p < end && *p == '.') {
      plain = false;
      ++p;
      if (p >= end || *p < '0' || *p > '9') return nullptr;
      while (p < end && *p >= '0' && *p <= '9') ++p;
    }
    if (p < end && (*p == 'e' || *p == 'E')) {
      plain = false;
      ++p;
      if (p < end && (*p == '+' || *p == '-')) ++p;
      if (p >= end || *p < '0' || *p > '9') return nullptr;
      while (p < end && *p >= '0' && *p <= '9') ++p;
    }
    if (plain) {
      uint64_t u = 0;
      for (const char *q = s; q < p; ++q) {
        const uint64_t d = (uint64_t)(*q - '0');
        if (u > (UINT64_MAX - d) / 10) { plain = false; break; }
        u = u * 10 + d;
      }
      v->u = u;
    }
    v->integral = plain;
    return v;
  }
};

bool exact_members(const JVal *o, const char *const *keys, int n) {
  if (!o || o->kind != JVal::OBJ || (int)o->members.size() != n) return false;
  for (int i = 0; i < n; ++i)
    if (!o->get(keys[i])) return false;
  return true;
}

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Parsed and validated directory.
struct Directory {
  uint64_t payload_offset = 0;
  std::vector<tq_container_object> objects;
};

tq_status validate(const uint8_t *file, uint64_t file_bytes, Directory &dir) {
  static const uint8_t magic[8] = {'N', 'I', 'N', 'F', 'E', 'R', 0, 2};
  if (!file && file_bytes) return tq::fail(TQ_ERR_ARG, "file is null");
  if (file_bytes < 16 || memcmp(file, magic, 8) != 0) return tq::fail(TQ_ERR_FORMAT, "bad magic");
  uint64_t json_bytes = 0;
  for (int i = 7; i >= 0; --i) json_bytes = (json_bytes << 8) | file[8 + i];
  if (json_bytes > file_bytes - 16)
    return tq::fail(TQ_ERR_FORMAT, "directory runs past the end of the file");
  const uint64_t payload_offset = align_up(16 + json_bytes, 4096);
  if (payload_offset > file_bytes)
    return tq::fail(TQ_ERR_FORMAT, "payload starts past the end of the file");
  Parser ps{reinterpret_cast<const char *>(file + 16), reinterpret_cast<const char *>(file + 16 + json_bytes)};
  auto root = ps.value(0);
  ps.ws();
  if (!root || ps.p != ps.end) {
    if (!ps.err.empty()) return tq::fail(TQ_ERR_FORMAT, "%s", ps.err.c_str());
    return tq::fail(TQ_ERR_FORMAT, "directory is not valid JSON");
  }
  if (!ps.compact) return tq::fail(TQ_ERR_FORMAT, "directory is not compact JSON");
  static const char *const kRoot[] = {"identity", "objects"};
  static const char *const kIdent[] = {"model_id", "weights_id"};
  static const char *const kTensor[] = {"name", "kind", "shape", "format", "layout", "offset", "bytes"};
  static const char *const kRes[] = {"name", "kind", "encoding", "offset", "bytes"};
  if (!exact_members(root.get(), kRoot, 2))
    return tq::fail(TQ_ERR_FORMAT, "root members must be exactly identity, objects");
  const JVal *ident = root->get("identity");
  if (!exact_members(ident, kIdent, 2))
    return tq::fail(TQ_ERR_FORMAT, "identity members must be exactly model_id, weights_id");
  for (const char *key : kIdent) {
    const JVal *v = ident->get(key);
    if (v->kind != JVal::STR || v->s.empty())
      return tq::fail(TQ_ERR_FORMAT, "identity %s must be a non-empty string", key);
  }
  const JVal *objs = root->get("objects");
  if (objs->kind != JVal::ARR) return tq::fail(TQ_ERR_FORMAT, "objects must be an array");
  const uint64_t payload_bytes = file_bytes - payload_offset;
  uint64_t cursor = 0;
  dir.payload_offset = payload_offset;
  dir.objects.clear();
  for (const auto &op : objs->items) {
    const JVal *o = op.get();
    const JVal *kind = o->kind == JVal::OBJ ? o->get("kind") : nullptr;
    if (!kind) return tq::fail(TQ_ERR_FORMAT, "object entry without a kind");
    tq_container_object rec;
    memset(&rec, 0, sizeof(rec));
    const bool tensor = kind->kind == JVal::STR && kind->s == "tensor";
    const bool resource = kind->kind == JVal::STR && kind->s == "resource";
    if (tensor) {
      if (!exact_members(o, kTensor, 7))
        return tq::fail(TQ_ERR_FORMAT, "tensor members must be exactly bytes, format, kind, layout, name, offset, shape");
    } else if (resource) {
      if (!exact_members(o, kRes, 5))
        return tq::fail(TQ_ERR_FORMAT, "resource members must be exactly bytes, encoding, kind, name, offset");
    } else {
      return tq::fail(TQ_ERR_FORMAT, "kind must be tensor or resource");
    }
    const JVal *name = o->get("name");
    if (name->kind != JVal::STR || name->s.empty())
      return tq::fail(TQ_ERR_FORMAT, "object name must be a non-empty string");
    if (name->s.size() >= sizeof(rec.name))
      return tq::fail(TQ_ERR_UNSUPPORTED, "object name longer than %d bytes", (int)sizeof(rec.name) - 1);
    for (const auto &prev : dir.objects)
      if (name->s == prev.name) return tq::fail(TQ_ERR_FORMAT, "duplicate object name: %s", name->s.c_str());
    const char *nm = name->s.c_str();
    const JVal *off = o->get("offset"), *nb = o->get("bytes");
    if (off->kind != JVal::NUM || !off->integral || nb->kind != JVal::NUM || !nb->integral || nb->u == 0)
      return tq::fail(TQ_ERR_FORMAT, "object %s: offset and bytes must be integers (bytes > 0)", nm);
    uint64_t align = 1;
    if (tensor) {
      const JVal *shape = o->get("shape"), *fmt = o->get("format"), *lay = o->get("layout");
      if (shape->kind != JVal::ARR || shape->items.size() > 16)
        return tq::fail(TQ_ERR_FORMAT, "tensor %s: shape must be an array of positive integers", nm);
      rec.rank = (int32_t)shape->items.size();
      for (size_t i = 0; i < shape->items.size(); ++i) {
        const JVal *d = shape->items[i].get();
        if (d->kind != JVal::NUM || !d->integral || d->u == 0 || d->u > (uint64_t)INT64_MAX)
          return tq::fail(TQ_ERR_FORMAT, "tensor %s: shape must be an array of positive integers", nm);
        rec.shape[i] = (int64_t)d->u;
      }
      if (fmt->kind != JVal::STR || lay->kind != JVal::STR)
        return tq::fail(TQ_ERR_FORMAT, "tensor %s: format and layout must be strings", nm);
      if (fmt->s.size() >= sizeof(rec.format) || lay->s.size() >= sizeof(rec.layout))
        return tq::fail(TQ_ERR_FORMAT, "unknown numeric format: %s", fmt->s.c_str());
      const std::string &L = lay->s, &F = fmt->s;
      uint64_t need = 0;
      if (L == "row_split_k128_v1") {
        int32_t f = F == "PQ2_0_G128" ? TQ_PQ2_0_G128 : F == "PTQ1_0_G128" ? TQ_PTQ1_0_G128 : 0;
        if (!f) return tq::fail(TQ_ERR_FORMAT, "unknown numeric format: %s", F.c_str());
        if (rec.rank != 2) return tq::fail(TQ_ERR_FORMAT, "row_split_k128_v1 needs a rank-2 shape");
        tq_geometry g;
        const tq_status st = tq_geometry_get(f, rec.shape[0], rec.shape[1], &g);
        if (st != TQ_OK) return st;
        need = g.payload_bytes;
      } else if (L == "contiguous_le_v1") {
        const uint64_t es = F == "bf16" ? 2 : (F == "fp32" || F == "int32") ? 4 : 0;
        if (!es) return tq::fail(TQ_ERR_FORMAT, "unknown numeric format: %s", F.c_str());
        unsigned __int128 cnt = 1;
        for (int i = 0; i < rec.rank; ++i) cnt *= (uint64_t)rec.shape[i];
        cnt *= es;
        if (cnt > UINT64_MAX) return tq::fail(TQ_ERR_FORMAT, "tensor %s is too large", nm);
        need = (uint64_t)cnt;
      } else if (L == "block_scale_k16_m128x4_v1" || L == "row_scale_v1") {
        return tq::fail(TQ_ERR_UNSUPPORTED, "unsupported layout: %s", L.c_str());
      } else {
        return tq::fail(TQ_ERR_FORMAT, "unknown layout: %s", L.c_str());
      }
      if (nb->u != need)
        return tq::fail(TQ_ERR_FORMAT, "tensor %s stores %llu bytes; layout requires %llu", nm,
                        (unsigned long long)nb->u, (unsigned long long)need);
      align = 256;
      rec.kind = 0;
      snprintf(rec.format, sizeof(rec.format), "%s", F.c_str());
      snprintf(rec.layout, sizeof(rec.layout), "%s", L.c_str());
    } else {
      const JVal *enc = o->get("encoding");
      if (enc->kind != JVal::STR || enc->s != "raw-bytes-v1")
        return tq::fail(TQ_ERR_FORMAT, "resource %s: encoding must be raw-bytes-v1", nm);
      rec.kind = 1;
      snprintf(rec.format, sizeof(rec.format), "%s", "raw-bytes-v1");
    }
    if (off->u < cursor)
      return tq::fail(TQ_ERR_FORMAT, "object %s overlaps or precedes the previous object", nm);
    if (off->u % align)
      return tq::fail(TQ_ERR_FORMAT, "object %s offset is not a multiple of %llu", nm,
                      (unsigned long long)align);
    if (off->u > payload_bytes || nb->u > payload_bytes - off->u)
      return tq::fail(TQ_ERR_FORMAT, "object %s runs past the end of the payload", nm);
    cursor = off->u + nb->u;
    rec.offset = off->u;
    rec.bytes = nb->u;
    snprintf(rec.name, sizeof(rec.name), "%s", nm);
    dir.objects.push_back(rec);
  }
  return TQ_OK;
}

}  // namespace

extern "C" tq_status tq_container_parse(const uint8_t *file, uint64_t file_bytes,
                                        uint64_t *payload_offset, int64_t *count) {
  Directory dir;
  const tq_status st = validate(file, file_bytes, dir);
  if (st != TQ_OK) return st;
  if (payload_offset) *payload_offset = dir.payload_offset;
  if (count) *count = (int64_t)dir.objects.size();
  return TQ_OK;
}

extern "C" tq_status tq_container_object_at(const uint8_t *file, uint64_t file_bytes, int64_t index,
                                            tq_container_object *out) {
  if (!out) return tq::fail(TQ_ERR_ARG, "out is null");
  Directory dir;
  const tq_status st = validate(file, file_bytes, dir);
  if (st != TQ_OK) return st;
  if (index < 0 || index >= (int64_t)dir.objects.size())
    return tq::fail(TQ_ERR_ARG, "object index %lld outside [0, %lld)", (long long)index,
                    (long long)dir.objects.size());
  *out = dir.objects[(size_t)index];
  return TQ_OK;
}
