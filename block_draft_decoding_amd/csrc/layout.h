// Schema -> layout expansion (host only, no HIP).
//
// VFlash paper §2.2-§2.3: once a primitive's type, coordinate dimensions and
// length are declared, the block length and the role of every position are
// known before decoding; coordinates and delimiters are then limited to
// their legal vocabularies (§2.5).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/fpd.h"

namespace fpd {

struct HostLayout {
  int32_t L = 0;
  int32_t vocab = 0;
  std::vector<int32_t> pos_set;      // [L]: -2 anchor, -1 free, >= 0 set index
  std::vector<int32_t> set_offsets;  // [n_sets + 1] CSR offsets into set_ids
  std::vector<int32_t> set_ids;      // ascending within each set
  std::vector<int32_t> pairs;        // [n_pairs * 2] block positions (u, v)
  std::vector<int32_t> fields;       // [n_fields * 2] (first digit position, width)
  std::vector<int32_t> coord;        // [L]: 1 where the legal set is coordinate ids (and OFF) only
  int32_t off_id = -1, fill_id = -1, digit0_id = -1;

  int32_t n_sets() const { return (int32_t)set_offsets.size() - 1; }
  int32_t width() const;             // widest legal set, or vocab if any position is free
  bool any_free() const;
};

// Returns an FPD_* status; on error `err` describes the problem.
int32_t expand_schema(const fpd_schema& s, int32_t vocab, HostLayout* out, std::string* err);

}  // namespace fpd
