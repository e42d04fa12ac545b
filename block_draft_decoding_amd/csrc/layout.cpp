// Schema -> layout expansion (host only, no HIP).  See layout.h.
#include "layout.h"

#include <algorithm>
#include <map>

namespace fpd {

int32_t HostLayout::width() const {
  if (any_free()) return vocab;
  int32_t w = 0;
  for (int32_t s = 0; s < n_sets(); ++s) w = std::max(w, set_offsets[s + 1] - set_offsets[s]);
  return w;
}

bool HostLayout::any_free() const {
  for (int32_t p = 1; p < L; ++p)
    if (pos_set[p] == -1) return true;
  return false;
}

namespace {

using Set = std::vector<int32_t>;

Set canonical(Set s) {
  std::sort(s.begin(), s.end());
  s.erase(std::unique(s.begin(), s.end()), s.end());
  return s;
}

// Collects per-position roles and numbers distinct sets by first appearance.
struct Builder {
  std::vector<int32_t> pos_set{-2};
  std::vector<Set> sets;
  std::map<Set, int32_t> index;
  std::vector<int32_t> pairs, fields;

  int32_t next_pos() const { return (int32_t)pos_set.size(); }
  void free_pos() { pos_set.push_back(-1); }
  void add(const Set& s) {
    auto it = index.find(s);
    int32_t id;
    if (it == index.end()) {
      id = (int32_t)sets.size();
      index.emplace(s, id);
      sets.push_back(s);
    } else {
      id = it->second;
    }
    pos_set.push_back(id);
  }
};

bool fail(std::string* err, const std::string& msg) {
  if (err) *err = msg;
  return false;
}

bool check_id(int32_t id, int32_t vocab, const char* what, std::string* err) {
  if (id < 0 || id >= vocab)
    return fail(err, std::string(what) + " id " + std::to_string(id) + " outside [0, vocab)");
  return true;
}

}  // namespace

int32_t expand_schema(const fpd_schema& s, int32_t vocab, HostLayout* out, std::string* err) {
  if (vocab <= 0) {
    if (err) *err = "vocab must be positive";
    return FPD_E_ARG;
  }
  Builder b;
  const int32_t off = s.off_id;
  auto coords = [&]() {
    Set c;
    for (int32_t i = 0; i < s.coord_count; ++i) c.push_back(s.coord_base + i);
    return c;
  };
  auto need = [&](bool ok) { return ok ? FPD_OK : FPD_E_SCHEMA; };

  switch (s.kind) {
    case FPD_SCHEMA_TEXT: {
      if (s.block_len < 2) return need(fail(err, "text block_len must be >= 2"));
      for (int32_t p = 1; p < s.block_len; ++p) b.free_pos();
      break;
    }
    case FPD_SCHEMA_TRAJ2D:
    case FPD_SCHEMA_TRAJ2D3D:
    case FPD_SCHEMA_BOXES2D:
    case FPD_SCHEMA_POINTS3D_TEXT: {
      if (s.n_points < 1) return need(fail(err, "n_points must be >= 1"));
      if (!check_id(s.delim_id, vocab, "delimiter", err)) return FPD_E_SCHEMA;
      const Set delim{s.delim_id};
      if (s.kind != FPD_SCHEMA_POINTS3D_TEXT) {
        if (s.coord_count < 1) return need(fail(err, "coord_count must be >= 1"));
        if (!check_id(s.coord_base, vocab, "coordinate", err) ||
            !check_id(s.coord_base + s.coord_count - 1, vocab, "coordinate", err))
          return FPD_E_SCHEMA;
      }
      if (s.kind == FPD_SCHEMA_TRAJ2D) {
        const Set c = coords();
        for (int32_t i = 0; i < s.n_points; ++i) {
          b.add(c);
          b.add(c);
          b.add(delim);
        }
      } else if (s.kind == FPD_SCHEMA_BOXES2D) {
        const Set c = coords();
        for (int32_t i = 0; i < s.n_points; ++i) {
          for (int32_t j = 0; j < 4; ++j) b.add(c);
          b.add(delim);
        }
      } else if (s.kind == FPD_SCHEMA_TRAJ2D3D) {
        const Set c = coords();
        Set img = c;
        if (off >= 0) {
          if (!check_id(off, vocab, "off-frame", err)) return FPD_E_SCHEMA;
          img.push_back(off);
          img = canonical(img);
          if ((int32_t)img.size() != s.coord_count + 1)
            return need(fail(err, "off-frame id collides with a coordinate id"));
        }
        for (int32_t i = 0; i < s.n_points; ++i) {
          const int32_t p = b.next_pos();
          if (off >= 0) {
            b.pairs.push_back(p);
            b.pairs.push_back(p + 1);
          }
          b.add(img);
          b.add(img);
          b.add(c);
          b.add(c);
          b.add(c);
          b.add(delim);
        }
      } else {
        if (!check_id(s.plus_id, vocab, "plus", err) || !check_id(s.minus_id, vocab, "minus", err) ||
            !check_id(s.fill_id, vocab, "fill", err) || !check_id(s.digit0_id, vocab, "digit", err) ||
            !check_id(s.digit0_id + 9, vocab, "digit", err))
          return FPD_E_SCHEMA;
        const Set sign = canonical({s.plus_id, s.minus_id});
        Set dig;
        for (int32_t i = 0; i < 10; ++i) dig.push_back(s.digit0_id + i);
        dig.push_back(s.fill_id);
        dig = canonical(dig);
        if (sign.size() != 2 || dig.size() != 11)
          return need(fail(err, "sign, digit and fill ids must be distinct"));
        for (int32_t i = 0; i < s.n_points; ++i) {
          for (int32_t axis = 0; axis < 3; ++axis) {
            const int32_t p = b.next_pos();
            b.fields.push_back(p + 1);
            b.fields.push_back(5);
            b.add(sign);
            for (int32_t j = 0; j < 5; ++j) b.add(dig);
          }
          b.add(delim);
        }
      }
      break;
    }
    case FPD_SCHEMA_CUSTOM: {
      const int32_t L = s.block_len;
      if (L < 2) return need(fail(err, "custom block_len must be >= 2"));
      if (!s.pos_set) return need(fail(err, "custom schema needs pos_set"));
      if (s.n_sets < 0 || (s.n_sets > 0 && (!s.set_offsets || !s.set_ids)))
        return need(fail(err, "custom schema: bad set table"));
      if (s.n_sets > 0 && s.set_offsets[0] != 0) return need(fail(err, "set_offsets[0] must be 0"));
      std::vector<Set> sets;
      for (int32_t k = 0; k < s.n_sets; ++k) {
        const int32_t lo = s.set_offsets[k], hi = s.set_offsets[k + 1];
        if (hi <= lo) return need(fail(err, "custom schema: empty or inverted set " + std::to_string(k)));
        Set st(s.set_ids + lo, s.set_ids + hi);
        for (int32_t id : st)
          if (!check_id(id, vocab, "set", err)) return FPD_E_SCHEMA;
        sets.push_back(canonical(st));
      }
      if (s.pos_set[0] != -2) return need(fail(err, "pos_set[0] must be -2 (the anchor)"));
      for (int32_t p = 1; p < L; ++p) {
        const int32_t v = s.pos_set[p];
        if (v < -1 || v >= s.n_sets)
          return need(fail(err, "pos_set[" + std::to_string(p) + "] out of range"));
        b.pos_set.push_back(v);
      }
      b.sets = sets;
      if (s.n_pairs < 0 || (s.n_pairs > 0 && !s.pairs)) return need(fail(err, "bad pairs"));
      if (s.n_fields < 0 || (s.n_fields > 0 && !s.fields)) return need(fail(err, "bad fields"));
      for (int32_t i = 0; i < 2 * s.n_pairs; ++i) b.pairs.push_back(s.pairs[i]);
      for (int32_t i = 0; i < 2 * s.n_fields; ++i) b.fields.push_back(s.fields[i]);
      break;
    }
    default:
      if (err) *err = "unknown schema kind " + std::to_string(s.kind);
      return FPD_E_ARG;
  }

  HostLayout& o = *out;
  o = HostLayout();
  o.vocab = vocab;
  o.L = (int32_t)b.pos_set.size();
  o.pos_set = b.pos_set;
  o.set_offsets.push_back(0);
  for (const Set& st : b.sets) {
    o.set_ids.insert(o.set_ids.end(), st.begin(), st.end());
    o.set_offsets.push_back((int32_t)o.set_ids.size());
  }
  o.pairs = b.pairs;
  o.fields = b.fields;
  o.off_id = off;
  o.fill_id = s.fill_id;
  o.digit0_id = s.digit0_id;
  // coordinate positions: every id of the legal set is a coordinate or OFF,
  // and at least one is a coordinate
  o.coord.assign(o.L, 0);
  for (int32_t p = 1; p < o.L; ++p) {
    const int32_t st = o.pos_set[p];
    if (st < 0) continue;
    bool any = false, only = true;
    for (int32_t i = o.set_offsets[st]; i < o.set_offsets[st + 1]; ++i) {
      const int32_t id = o.set_ids[i];
      const bool c = s.coord_count > 0 && id >= s.coord_base && id - s.coord_base < s.coord_count;
      any = any || c;
      only = only && (c || (off >= 0 && id == off));
    }
    o.coord[p] = any && only;
  }

  // structural checks common to every kind
  std::vector<int32_t> used(o.L, 0);
  const int32_t npairs = (int32_t)o.pairs.size() / 2;
  if (npairs > 0 && off < 0) return need(fail(err, "pairs need an off-frame id"));
  for (int32_t i = 0; i < npairs; ++i) {
    for (int32_t j = 0; j < 2; ++j) {
      const int32_t p = o.pairs[2 * i + j];
      if (p < 1 || p >= o.L) return need(fail(err, "pair position out of range"));
      if (used[p]++) return need(fail(err, "position in more than one pair"));
      const int32_t st = o.pos_set[p];
      if (st < 0) return need(fail(err, "paired position must have a legal set"));
      const int32_t* lo = o.set_ids.data() + o.set_offsets[st];
      const int32_t* hi = o.set_ids.data() + o.set_offsets[st + 1];
      if (!std::binary_search(lo, hi, off)) return need(fail(err, "paired set lacks the off-frame id"));
      if (hi - lo < 2) return need(fail(err, "paired set needs an on-frame id"));
    }
  }
  const int32_t nfields = (int32_t)o.fields.size() / 2;
  if (nfields > 0 && (o.fill_id < 0 || o.digit0_id < 0))
    return need(fail(err, "fields need fill and digit ids"));
  std::fill(used.begin(), used.end(), 0);
  for (int32_t i = 0; i < nfields; ++i) {
    const int32_t p0 = o.fields[2 * i], w = o.fields[2 * i + 1];
    if (w < 1 || w > 16 || p0 < 1 || p0 + w > o.L) return need(fail(err, "field out of range"));
    for (int32_t j = 0; j < w; ++j)
      if (used[p0 + j]++) return need(fail(err, "overlapping fields"));
  }
  return FPD_OK;
}

}  // namespace fpd
