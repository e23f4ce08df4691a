// Shared-prefix groups read off block tables (host only): pkv_prefix_groups.
//
// Sequences that took a prefix by reference hold the same physical blocks at
// the start of their tables ([KVM §19.2.5]; [PFX §prefix]).  A group is a
// maximal run of consecutive sequences whose first valid table entry is the
// same block; its shared prefix is the longest run of leading entries that
// every member holds as valid entries (entry i of a sequence of length L is
// valid when i < ceil(L / B)) and that agree across members, in tokens; a
// group of one shares nothing.  Page keys are listed in include/pkv.h.
#include <algorithm>
#include <cstdint>

#include "pkv_internal.h"

extern "C" {

pkv_status pkv_prefix_groups(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks,
                             const int32_t* seq_lens, int32_t block_size,
                             int32_t* group_starts_out, int32_t* prefix_lens_out,
                             int32_t* num_groups_out, int32_t* max_group_size_out,
                             int32_t* max_prefix_len_out, int32_t* max_suffix_len_out) {
  const char* who = "pkv_prefix_groups";
  if (num_seqs < 0 || max_blocks < 0 || block_size <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: bad size", who);
  if (!group_starts_out || !prefix_lens_out || !num_groups_out || !max_group_size_out ||
      !max_prefix_len_out || !max_suffix_len_out || (num_seqs > 0 && (!seq_lens || (max_blocks > 0 && !block_tables))))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null pointer", who);
  auto valid = [&](int32_t s) -> int64_t {  // valid entries of sequence s
    const int64_t L = seq_lens[s] < 0 ? 0 : seq_lens[s];
    return std::min<int64_t>((L + block_size - 1) / block_size, max_blocks);
  };
  auto at = [&](int32_t s, int64_t i) { return block_tables[int64_t(s) * max_blocks + i]; };
  int32_t ng = 0, max_group = 0, max_prefix = 0, max_suffix = 0;
  int32_t s = 0;
  while (s < num_seqs) {
    int32_t e = s + 1;
    if (valid(s) > 0)
      while (e < num_seqs && valid(e) > 0 && at(e, 0) == at(s, 0)) ++e;
    int64_t k = 0;
    if (e - s >= 2) {
      int64_t limit = valid(s);
      for (int32_t i = s + 1; i < e; ++i) limit = std::min(limit, valid(i));
      while (k < limit) {
        bool same = true;
        for (int32_t i = s + 1; i < e && same; ++i) same = at(i, k) == at(s, k);
        if (!same) break;
        ++k;
      }
    }
    const int64_t tokens = k * block_size;
    if (tokens >= (int64_t(1) << 31)) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: prefix too long", who);
    group_starts_out[ng] = s;
    prefix_lens_out[ng] = static_cast<int32_t>(tokens);
    max_group = std::max(max_group, e - s);
    for (int32_t i = s; i < e; ++i) {  // positions after the shared prefix
      const int32_t L = seq_lens[i] < 0 ? 0 : seq_lens[i];
      max_suffix = std::max<int32_t>(max_suffix, static_cast<int32_t>(L - std::min<int64_t>(tokens, L)));
    }
    max_prefix = std::max(max_prefix, static_cast<int32_t>(tokens));
    ++ng;
    s = e;
  }
  group_starts_out[ng] = num_seqs;
  *num_groups_out = ng;
  *max_group_size_out = max_group;
  *max_prefix_len_out = max_prefix;
  *max_suffix_len_out = max_suffix;
  return PKV_OK;
}

}  // extern "C"
