// Host block manager of libpkv: free list, reference counts, per-sequence block
// tables, fork, prefix sharing and the copy-on-write decision.  Host memory
// only, no HIP; one handle is used by one thread at a time.
//
// Semantics follow [KVM §19.2.2]-[KVM §19.2.3] (pool, free list taken from the
// end, reference counts, block table with the number of filled tokens, release
// of every block including the partly filled last one), [KVM §19.2.2] Fig. 19-8
// (copy-on-write), [SLOT §locate] (logical block / offset / token slot),
// [ENG §3.2] (most recently freed first; out-of-blocks reported to the caller)
// and [KVM §19.2.6] (all-or-nothing).  Page keys are listed in include/pkv.h.
//
// Swap ([KVM §19.2.6] pausing a request and moving its KV cache to CPU memory;
// [ENG §8.2] CPU memory as a second-level block pool): an optional host pool
// with its own free list and reference counts, managed like the device pool.
// A swapped-out sequence's table names host blocks.
#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {

struct Seq {
  std::vector<int32_t> table;  // logical block -> physical block (host block if swapped)
  int32_t filled = 0;          // tokens written
  bool swapped = false;
};

// One reversible step of an append call.
struct Undo {
  enum Kind { kNewBlock, kCow, kFilled } kind;
  Seq* seq;
  int32_t lb;     // kCow: logical block remapped
  int32_t block;  // kCow: the old block
};

}  // namespace

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t shift = 0;                 // log2(block_size)
  std::vector<int32_t> free_list;    // taken from / returned to the back
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  int32_t num_host_blocks = 0;       // host tier; 0 = none
  std::vector<int32_t> host_free;
  std::vector<int32_t> host_ref;

  void drop_host(int32_t h) {
    if (--host_ref[h] == 0) host_free.push_back(h);
  }
  bool take(int32_t* out) {
    if (free_list.empty()) return false;
    *out = free_list.back();
    free_list.pop_back();
    ref[*out] = 1;
    return true;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
  }
  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
};

namespace {

pkv_status swapped_error(const char* what, int64_t seq) {
  return pkv::fail(PKV_ERR_INVALID_ARG, "%s: sequence %lld is swapped out", what, (long long)seq);
}

// Sequences of a swap call: known, distinct, all on the expected tier.
pkv_status swap_set(pkv_bm* bm, const int64_t* seqs, int32_t n, bool want_swapped,
                    const char* what, std::vector<Seq*>* out) {
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: negative count", what);
  if (n > 0 && !seqs) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: null sequence array", what);
  std::vector<int64_t> ids(seqs, seqs + n);
  std::sort(ids.begin(), ids.end());
  if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: repeated sequence", what);
  out->resize(n);
  for (int32_t i = 0; i < n; ++i) {
    Seq* s = bm->find(seqs[i]);
    if (!s) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: unknown sequence %lld", what, (long long)seqs[i]);
    if (s->swapped != want_swapped)
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s: sequence %lld is %s", what, (long long)seqs[i],
                       want_swapped ? "resident" : "swapped out");
    (*out)[i] = s;
  }
  return PKV_OK;
}

// Distinct ids named by the tables, in order of first appearance.
std::vector<int32_t> distinct_blocks(const std::vector<Seq*>& ss, int32_t pool_blocks) {
  std::vector<char> seen(pool_blocks, 0);
  std::vector<int32_t> order;
  for (const Seq* s : ss)
    for (int32_t b : s->table)
      if (!seen[b]) {
        seen[b] = 1;
        order.push_back(b);
      }
  return order;
}

// Move the sequences' tables from one tier to the other: every distinct block
// gets one block of the target pool (taken from the end of its free list),
// each entry is remapped and its old reference released, table by table.
pkv_status move_tier(pkv_bm* bm, const int64_t* seqs, int32_t n, bool to_host,
                     int32_t* pairs_out, int32_t cap, int32_t* n_pairs_out) {
  const char* what = to_host ? "swap_out" : "swap_in";
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  if (n_pairs_out) *n_pairs_out = 0;
  std::vector<Seq*> ss;
  if (pkv_status st = swap_set(bm, seqs, n, !to_host, what, &ss)) return st;
  const int32_t src_blocks = to_host ? bm->num_blocks : bm->num_host_blocks;
  const std::vector<int32_t> order = distinct_blocks(ss, src_blocks);
  const int32_t m = static_cast<int32_t>(order.size());
  if (m > 0 && (!pairs_out || cap < m))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s: pair capacity %d < %d blocks", what, cap, m);
  std::vector<int32_t>& dst_free = to_host ? bm->host_free : bm->free_list;
  std::vector<int32_t>& dst_ref = to_host ? bm->host_ref : bm->ref;
  if (m > static_cast<int32_t>(dst_free.size()))
    return pkv::fail(PKV_ERR_NO_FREE_BLOCKS, "%s: %d blocks needed, %zu free in the %s pool (state "
                     "unchanged)", what, m, dst_free.size(), to_host ? "host" : "device");
  std::vector<int32_t> map(src_blocks, -1);
  for (int32_t i = 0; i < m; ++i) {
    const int32_t d = dst_free.back();
    dst_free.pop_back();
    dst_ref[d] = 0;
    map[order[i]] = d;
    pairs_out[2 * i] = order[i];
    pairs_out[2 * i + 1] = d;
  }
  for (Seq* s : ss) {
    for (int32_t& b : s->table) {
      const int32_t d = map[b];
      ++dst_ref[d];
      if (to_host) bm->drop(b); else bm->drop_host(b);
      b = d;
    }
    s->swapped = to_host;
  }
  if (n_pairs_out) *n_pairs_out = m;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0 || (block_size & (block_size - 1)) != 0 ||
      static_cast<int64_t>(num_blocks) * block_size >= (int64_t(1) << 31)) {
    pkv::fail(PKV_ERR_INVALID_ARG, "pkv_bm_create: bad num_blocks/block_size (%d, %d)",
              num_blocks, block_size);
    return nullptr;
  }
  auto* bm = new pkv_bm();
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  while ((1 << bm->shift) < block_size) ++bm->shift;
  bm->ref.assign(num_blocks, 0);
  bm->free_list.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        pkv::fail(PKV_ERR_INVALID_ARG, "pkv_bm_create: free_order is not a permutation");
        return nullptr;
      }
      seen[b] = 1;
      bm->free_list[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = i;
  }
  return bm;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

pkv_status pkv_bm_add_seq(pkv_bm* bm, int64_t seq) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  if (bm->find(seq)) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld exists", (long long)seq);
  bm->seqs.emplace(seq, Seq{});
  return PKV_OK;
}

pkv_status pkv_bm_share_prefix(pkv_bm* bm, int64_t dst, int64_t src, int32_t num_tokens) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  Seq* d = bm->find(dst);
  const Seq* s = bm->find(src);
  if (!d || !s) return pkv::fail(PKV_ERR_INVALID_ARG, "share_prefix: unknown sequence");
  if (d->swapped) return swapped_error("share_prefix", dst);
  if (s->swapped) return swapped_error("share_prefix", src);
  if (d == s || !d->table.empty() || d->filled != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "share_prefix: destination must be a different, empty sequence");
  if (num_tokens < 0 || num_tokens > s->filled)
    return pkv::fail(PKV_ERR_INVALID_ARG, "share_prefix: %d tokens > source length %d", num_tokens,
                     s->filled);
  const int32_t nb = (num_tokens + bm->block_size - 1) >> bm->shift;
  d->table.assign(s->table.begin(), s->table.begin() + nb);
  d->filled = num_tokens;
  for (int32_t b : d->table) ++bm->ref[b];
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  const Seq* p = bm->find(parent);
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARG, "fork: unknown parent %lld", (long long)parent);
  if (p->swapped) return swapped_error("fork", parent);
  if (bm->find(child)) return pkv::fail(PKV_ERR_INVALID_ARG, "fork: child %lld exists", (long long)child);
  Seq c = *p;  // copy before emplace: emplace may rehash and move *p
  for (int32_t b : c.table) ++bm->ref[b];
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

pkv_status pkv_bm_append_slots(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t tokens_each,
                               int32_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  if (n < 0 || tokens_each < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "append: negative count");
  if (num_cow_out) *num_cow_out = 0;
  if (n == 0 || tokens_each == 0) return PKV_OK;
  if (!seqs || !slots_out) return pkv::fail(PKV_ERR_INVALID_ARG, "append: null array");
  std::vector<Seq*> ptr(n);
  for (int32_t i = 0; i < n; ++i) {
    ptr[i] = bm->find(seqs[i]);
    if (!ptr[i]) return pkv::fail(PKV_ERR_INVALID_ARG, "append: unknown sequence %lld", (long long)seqs[i]);
    if (ptr[i]->swapped) return swapped_error("append", seqs[i]);
    if (static_cast<int64_t>(ptr[i]->filled) + tokens_each >= (int64_t(1) << 31))
      return pkv::fail(PKV_ERR_INVALID_ARG, "append: sequence length overflow");
  }
  const int32_t B = bm->block_size, shift = bm->shift;
  std::vector<Undo> journal;
  std::vector<int32_t> taken;  // blocks popped from the free list, in order
  int32_t ncow = 0;
  pkv_status st = PKV_OK;
  int64_t k = 0;
  for (int32_t i = 0; i < n && st == PKV_OK; ++i) {
    Seq* s = ptr[i];
    journal.push_back({Undo::kFilled, s, 0, s->filled});
    for (int32_t t = 0; t < tokens_each; ++t) {
      const int32_t lb = s->filled >> shift;       // logical block
      const int32_t off = s->filled & (B - 1);     // offset in block
      if (lb == static_cast<int32_t>(s->table.size())) {
        int32_t b;
        if (!bm->take(&b)) { st = PKV_ERR_NO_FREE_BLOCKS; break; }
        taken.push_back(b);
        s->table.push_back(b);
        journal.push_back({Undo::kNewBlock, s, lb, b});
      } else if (bm->ref[s->table[lb]] > 1) {
        // Shared block about to be written: private copy (copy-on-write).
        int32_t b;
        if (!bm->take(&b)) { st = PKV_ERR_NO_FREE_BLOCKS; break; }
        if (!cow_pairs_out) {
          bm->free_list.push_back(b);
          bm->ref[b] = 0;
          st = PKV_ERR_INVALID_ARG;
          break;
        }
        taken.push_back(b);
        const int32_t old = s->table[lb];
        cow_pairs_out[2 * ncow] = old;
        cow_pairs_out[2 * ncow + 1] = b;
        ++ncow;
        s->table[lb] = b;
        --bm->ref[old];  // > 0 afterwards: it was shared
        journal.push_back({Undo::kCow, s, lb, old});
      }
      slots_out[k++] = s->table[lb] * B + off;  // token slot
      ++s->filled;
    }
  }
  if (st != PKV_OK) {
    // Roll back in reverse order; re-pushing the taken blocks in reverse
    // restores the free list exactly (they were popped from its end).
    for (auto it = journal.rbegin(); it != journal.rend(); ++it) {
      switch (it->kind) {
        case Undo::kNewBlock: it->seq->table.pop_back(); break;
        case Undo::kCow:
          it->seq->table[it->lb] = it->block;
          ++bm->ref[it->block];
          break;
        case Undo::kFilled: it->seq->filled = it->block; break;
      }
    }
    for (auto it = taken.rbegin(); it != taken.rend(); ++it) {
      bm->ref[*it] = 0;
      bm->free_list.push_back(*it);
    }
    if (num_cow_out) *num_cow_out = 0;
    if (st == PKV_ERR_NO_FREE_BLOCKS)
      return pkv::fail(st, "append: no free physical block (state unchanged)");
    return pkv::fail(st, "append: a copy-on-write pair is needed but cow_pairs_out is NULL");
  }
  if (num_cow_out) *num_cow_out = ncow;
  return PKV_OK;
}

pkv_status pkv_bm_free_seq(pkv_bm* bm, int64_t seq) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "free: unknown sequence %lld", (long long)seq);
  if (it->second.swapped) {
    for (int32_t h : it->second.table) bm->drop_host(h);
  } else {
    for (int32_t b : it->second.table) bm->drop(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_export(const pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t max_blocks,
                         int32_t* block_tables_out, int32_t* seq_lens_out) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  if (n < 0 || max_blocks < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "export: negative size");
  if (n > 0 && (!seqs || !seq_lens_out || (max_blocks > 0 && !block_tables_out)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "export: null array");
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seqs[i]);
    if (!s) return pkv::fail(PKV_ERR_INVALID_ARG, "export: unknown sequence %lld", (long long)seqs[i]);
    if (s->swapped) return swapped_error("export", seqs[i]);
    if (static_cast<int32_t>(s->table.size()) > max_blocks)
      return pkv::fail(PKV_ERR_INVALID_ARG, "export: sequence %lld has %zu blocks > %d",
                       (long long)seqs[i], s->table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seqs[i]);
    int32_t* row = block_tables_out + static_cast<int64_t>(i) * max_blocks;
    std::copy(s->table.begin(), s->table.end(), row);
    std::fill(row + s->table.size(), row + max_blocks, -1);
    seq_lens_out[i] = s->filled;
  }
  return PKV_OK;
}

int32_t pkv_bm_num_free(const pkv_bm* bm) {
  return bm ? static_cast<int32_t>(bm->free_list.size()) : -1;
}

int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int32_t pkv_bm_num_tokens(const pkv_bm* bm, int64_t seq) {
  if (!bm) return -1;
  const Seq* s = bm->find(seq);
  return s ? s->filled : -1;
}

pkv_status pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!bm || !n_out) return pkv::fail(PKV_ERR_INVALID_ARG, "free_list: null argument");
  const int32_t n = static_cast<int32_t>(bm->free_list.size());
  *n_out = n;
  if (cap < n) return pkv::fail(PKV_ERR_INVALID_ARG, "free_list: capacity %d < %d", cap, n);
  if (n) std::memcpy(out, bm->free_list.data(), sizeof(int32_t) * n);
  return PKV_OK;
}

pkv_status pkv_bm_check(const pkv_bm* bm) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  std::vector<int32_t> count(bm->num_blocks, 0);
  std::vector<int32_t> hcount(bm->num_host_blocks, 0);
  for (const auto& kv : bm->seqs) {
    const Seq& s = kv.second;
    const int64_t want = (static_cast<int64_t>(s.filled) + bm->block_size - 1) >> bm->shift;
    if (static_cast<int64_t>(s.table.size()) != want)
      return pkv::fail(PKV_ERR_INVALID_ARG, "check: sequence %lld has %zu blocks for %d tokens",
                       (long long)kv.first, s.table.size(), s.filled);
    const int32_t lim = s.swapped ? bm->num_host_blocks : bm->num_blocks;
    std::vector<int32_t>& cnt = s.swapped ? hcount : count;
    for (int32_t b : s.table) {
      if (b < 0 || b >= lim)
        return pkv::fail(PKV_ERR_INVALID_ARG, "check: block id %d out of range", b);
      ++cnt[b];
    }
  }
  const struct {
    const char* name;
    int32_t n;
    const std::vector<int32_t>& count;
    const std::vector<int32_t>& ref;
    const std::vector<int32_t>& free;
  } tiers[2] = {{"block", bm->num_blocks, count, bm->ref, bm->free_list},
                {"host block", bm->num_host_blocks, hcount, bm->host_ref, bm->host_free}};
  for (const auto& t : tiers) {
    std::vector<char> on_free(t.n, 0);
    for (int32_t b : t.free) {
      if (b < 0 || b >= t.n || on_free[b])
        return pkv::fail(PKV_ERR_INVALID_ARG, "check: bad or duplicate free %s id %d", t.name, b);
      on_free[b] = 1;
    }
    for (int32_t b = 0; b < t.n; ++b) {
      if (t.count[b] != t.ref[b])
        return pkv::fail(PKV_ERR_INVALID_ARG, "check: %s %d refcount %d != %d references", t.name,
                         b, t.ref[b], t.count[b]);
      if ((t.ref[b] > 0) == (on_free[b] != 0))
        return pkv::fail(PKV_ERR_INVALID_ARG, "check: %s %d is %s", t.name, b,
                         on_free[b] ? "referenced and free" : "neither referenced nor free (leak)");
    }
  }
  return PKV_OK;
}

pkv_status pkv_bm_add_host_pool(pkv_bm* bm, int32_t num_host_blocks, const int32_t* free_order) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null manager");
  if (bm->num_host_blocks != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "add_host_pool: the manager already has a host pool");
  if (num_host_blocks <= 0 ||
      static_cast<int64_t>(num_host_blocks) * bm->block_size >= (int64_t(1) << 31))
    return pkv::fail(PKV_ERR_INVALID_ARG, "add_host_pool: bad num_host_blocks %d", num_host_blocks);
  std::vector<int32_t> order(num_host_blocks);
  if (free_order) {
    std::vector<char> seen(num_host_blocks, 0);
    for (int32_t i = 0; i < num_host_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_host_blocks || seen[b])
        return pkv::fail(PKV_ERR_INVALID_ARG, "add_host_pool: free_order is not a permutation");
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_host_blocks; ++i) order[i] = i;
  }
  bm->num_host_blocks = num_host_blocks;
  bm->host_free = std::move(order);
  bm->host_ref.assign(num_host_blocks, 0);
  return PKV_OK;
}

pkv_status pkv_bm_swap_out(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                           int32_t cap, int32_t* num_pairs_out) {
  return move_tier(bm, seqs, n, true, pairs_out, cap, num_pairs_out);
}

pkv_status pkv_bm_swap_in(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* pairs_out,
                          int32_t cap, int32_t* num_pairs_out) {
  return move_tier(bm, seqs, n, false, pairs_out, cap, num_pairs_out);
}

int32_t pkv_bm_distinct_blocks(const pkv_bm* bm, const int64_t* seqs, int32_t n) {
  if (!bm || n < 0 || (n > 0 && !seqs)) return -1;
  std::vector<char> seen(bm->num_blocks, 0), hseen(bm->num_host_blocks, 0);
  int32_t m = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seqs[i]);
    if (!s) return -1;
    std::vector<char>& sn = s->swapped ? hseen : seen;
    for (int32_t b : s->table)
      if (!sn[b]) {
        sn[b] = 1;
        ++m;
      }
  }
  return m;
}

int32_t pkv_bm_is_swapped(const pkv_bm* bm, int64_t seq) {
  if (!bm) return -1;
  const Seq* s = bm->find(seq);
  return s ? (s->swapped ? 1 : 0) : -1;
}

int32_t pkv_bm_num_free_host(const pkv_bm* bm) {
  return bm ? static_cast<int32_t>(bm->host_free.size()) : -1;
}

int32_t pkv_bm_host_refcount(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_host_blocks) return -1;
  return bm->host_ref[block];
}

pkv_status pkv_bm_host_free_list(const pkv_bm* bm, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!bm || !n_out) return pkv::fail(PKV_ERR_INVALID_ARG, "host_free_list: null argument");
  const int32_t n = static_cast<int32_t>(bm->host_free.size());
  *n_out = n;
  if (cap < n) return pkv::fail(PKV_ERR_INVALID_ARG, "host_free_list: capacity %d < %d", cap, n);
  if (n) std::memcpy(out, bm->host_free.data(), sizeof(int32_t) * n);
  return PKV_OK;
}

}  // extern "C"
