// Host block manager; see pool.hpp for the model and its sources.
#include "pool.hpp"

#include <unordered_map>

#include <algorithm>
#include <cstring>
#include <new>

namespace pa {

namespace {
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

BlockPool::BlockPool(int32_t n, int32_t bs)
    : n_(n), bs_(bs), next_(n, -1), prev_(n, -1), in_queue_(n, 0), ref_(n, 0) {}

Status BlockPool::create(int32_t num_blocks, int32_t block_size, const int32_t* order,
                         BlockPool** out, std::string* err) {
  if (out == nullptr) {
    *err = "pa_pool_create: out is NULL";
    return kBadArg;
  }
  if (num_blocks < 1 || block_size < 1) {
    *err = "pa_pool_create: num_blocks and block_size must be >= 1";
    return kBadArg;
  }
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t(1) << 31)) {
    *err = "pa_pool_create: num_blocks * block_size must be < 2^31 (slots are int32)";
    return kBadArg;
  }
  BlockPool* p = nullptr;
  try {
    p = new BlockPool(num_blocks, block_size);
  } catch (const std::bad_alloc&) {
    *err = "pa_pool_create: out of host memory";
    return kBadArg;
  }
  if (order != nullptr) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        *err = "pa_pool_create: init_free_order is not a permutation of 0..num_blocks-1";
        return kBadArg;
      }
      seen[b] = 1;
    }
  }
  for (int32_t i = 0; i < num_blocks; ++i) p->push_back(order ? order[i] : i);
  *out = p;
  return kOk;
}

int32_t BlockPool::pop_front() {
  const int32_t b = head_;
  unlink(b);
  if (!cached_.empty()) {
    auto it = cached_.find(b);
    if (it != cached_.end()) {  // the block's cached K/V is about to be overwritten
      cache_.erase(it->second.key);
      cached_.erase(it);
      ++evictions_;
    }
  }
  return b;
}

void BlockPool::unlink(int32_t b) {
  const int32_t p = prev_[b], n = next_[b];
  if (p >= 0) next_[p] = n; else head_ = n;
  if (n >= 0) prev_[n] = p; else tail_ = p;
  next_[b] = prev_[b] = -1;
  in_queue_[b] = 0;
  --nfree_;
}

// SHA-256 over the parent's key (32 bytes) and the block's token ids (4 bytes
// each, little endian).  The first block's parent key is 32 zero bytes.
Digest BlockPool::block_key(const Digest& parent, const int32_t* ids) const {
  Sha256 h;
  h.update(parent.b, 32);
  for (int32_t i = 0; i < bs_; ++i) {
    const uint32_t t = static_cast<uint32_t>(ids[i]);
    const uint8_t le[4] = {static_cast<uint8_t>(t), static_cast<uint8_t>(t >> 8),
                           static_cast<uint8_t>(t >> 16), static_cast<uint8_t>(t >> 24)};
    h.update(le, 4);
  }
  return h.finish();
}

int32_t BlockPool::lookup(const Digest& key) const {
  const auto it = cache_.find(key);
  return it == cache_.end() ? -1 : it->second;
}

void BlockPool::push_back(int32_t b) {
  prev_[b] = tail_;
  next_[b] = -1;
  if (tail_ >= 0) next_[tail_] = b; else head_ = b;
  tail_ = b;
  in_queue_[b] = 1;
  ++nfree_;
}

Status BlockPool::seq_create(int32_t* id) {
  if (id == nullptr) return kBadArg;
  if (seqs_.size() >= static_cast<size_t>(INT32_MAX)) return kCapacity;
  try {
    seqs_.emplace_back();
  } catch (const std::bad_alloc&) {
    return kCapacity;
  }
  seqs_.back().live = true;
  *id = static_cast<int32_t>(seqs_.size() - 1);
  ++live_seqs_;
  return kOk;
}

Status BlockPool::alloc_append(int32_t seq, int32_t n, const int32_t* tokens, int32_t* slots,
                               int32_t* cow, std::string* err) {
  if (!live(seq)) {
    *err = "pa_alloc_append: unknown sequence";
    return kBadSeq;
  }
  if (n < 0) {
    *err = "pa_alloc_append: n_tokens < 0";
    return kBadArg;
  }
  if (n > 0 && slots == nullptr) {
    *err = "pa_alloc_append: slots_out is NULL";
    return kBadArg;
  }
  Seq& s = seqs_[seq];
  if (s.swapped) {
    *err = "pa_alloc_append: the sequence is swapped out";
    return kBadArg;
  }
  if (cow != nullptr) cow[0] = cow[1] = -1;
  if (n == 0) return kOk;
  const int64_t len = s.len;
  const int64_t nb = static_cast<int64_t>(s.table.size());
  const int64_t blocks_after = ceil_div(len + n, bs_);
  if (blocks_after * bs_ >= (int64_t(1) << 31)) {
    *err = "pa_alloc_append: sequence would exceed 2^31 tokens";
    return kBadArg;
  }
  const int64_t new_blocks = blocks_after - nb;
  // copy-on-write: tokens will land in a partly filled last block that others share
  const bool do_cow = (len % bs_) != 0 && ref_[s.table.back()] > 1;
  if (do_cow && cow == nullptr) {
    *err = "pa_alloc_append: copy-on-write needed but cow_out is NULL";
    return kBadArg;
  }
  const int64_t need = new_blocks + (do_cow ? 1 : 0);
  if (need > nfree_) {
    *err = "pa_alloc_append: not enough free blocks";
    return kNoBlocks;
  }
  const bool record = tokens != nullptr && static_cast<int64_t>(s.tokens.size()) == len;
  try {
    s.table.reserve(static_cast<size_t>(blocks_after));
    if (record) s.tokens.reserve(static_cast<size_t>(len + n));
  } catch (const std::bad_alloc&) {
    *err = "pa_alloc_append: out of host memory";
    return kCapacity;
  }
  // --- no failure past this point ---
  const int64_t waste_before = nb * bs_ - len;
  if (do_cow) {
    const int32_t src = s.table.back();
    const int32_t dst = pop_front();
    if (ref_[src] == 2) --shared_;
    --ref_[src];
    ref_[dst] = 1;
    s.table.back() = dst;
    cow[0] = src;
    cow[1] = dst;
    ++cow_copies_;
  }
  for (int64_t j = 0; j < new_blocks; ++j) {
    const int32_t b = pop_front();
    ref_[b] = 1;
    ++refs_;
    s.table.push_back(b);
  }
  const int32_t* tbl = s.table.data();
  for (int32_t i = 0; i < n; ++i) {
    const int64_t pos = len + i;
    slots[i] = tbl[pos / bs_] * bs_ + static_cast<int32_t>(pos % bs_);
  }
  s.len = len + n;
  tokens_ += n;
  waste_ += (blocks_after * bs_ - s.len) - waste_before;
  if (record) s.tokens.insert(s.tokens.end(), tokens, tokens + n);
  return kOk;
}

Status BlockPool::alloc_append_batch(const int32_t* seqs, int32_t n_seqs, const int32_t* counts,
                                     const int32_t* tokens, int32_t* slots, int32_t* cow,
                                     std::string* err) {
  if (n_seqs < 0 || (n_seqs > 0 && (seqs == nullptr || counts == nullptr || cow == nullptr))) {
    *err = "pa_alloc_append_batch: bad arguments";
    return kBadArg;
  }
  // Dry run in batch order: the checks of each single call, with the blocks
  // earlier calls take and the references their copies drop.
  int64_t total = 0, need = 0;
  std::unordered_map<int32_t, int32_t> dropped;  // shared last block -> references given up
  std::unordered_map<int32_t, char> seen;
  try {
    for (int32_t i = 0; i < n_seqs; ++i) {
      const int32_t sid = seqs[i], n = counts[i];
      if (!live(sid)) {
        *err = "pa_alloc_append_batch: unknown sequence";
        return kBadSeq;
      }
      const Seq& s = seqs_[sid];
      if (n < 0 || s.swapped || !seen.emplace(sid, 1).second) {
        *err = "pa_alloc_append_batch: negative count, swapped-out or repeated sequence";
        return kBadArg;
      }
      total += n;
      if (n == 0) continue;
      const int64_t blocks_after = ceil_div(s.len + n, bs_);
      if (blocks_after * bs_ >= (int64_t(1) << 31)) {
        *err = "pa_alloc_append_batch: sequence would exceed 2^31 tokens";
        return kBadArg;
      }
      need += blocks_after - static_cast<int64_t>(s.table.size());
      if (s.len % bs_ != 0) {
        const int32_t last = s.table.back();
        int32_t& d = dropped[last];
        if (ref_[last] - d > 1) {  // still shared when this call runs: it copies
          ++need;
          ++d;
        }
      }
      if (need > nfree_) {
        *err = "pa_alloc_append_batch: not enough free blocks";
        return kNoBlocks;
      }
    }
    if (total > 0 && slots == nullptr) {
      *err = "pa_alloc_append_batch: slots_out is NULL";
      return kBadArg;
    }
    // the only other failure of the single calls, a host allocation, happens here
    for (int32_t i = 0; i < n_seqs; ++i) {
      Seq& s = seqs_[seqs[i]];
      s.table.reserve(static_cast<size_t>(ceil_div(s.len + counts[i], bs_)));
      if (tokens != nullptr && static_cast<int64_t>(s.tokens.size()) == s.len)
        s.tokens.reserve(static_cast<size_t>(s.len + counts[i]));
    }
  } catch (const std::bad_alloc&) {
    *err = "pa_alloc_append_batch: out of host memory";
    return kCapacity;
  }
  // --- no failure past this point ---
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Status st = alloc_append(seqs[i], counts[i], tokens != nullptr ? tokens + off : nullptr,
                                   slots + off, cow + 2 * i, err);
    (void)st;  // kOk: every condition was checked above
    off += counts[i];
  }
  return kOk;
}

Status BlockPool::alloc_prompt(int32_t seq, const int32_t* tokens, int32_t n, int32_t* slots,
                               int32_t* hit_tokens, std::string* err) {
  if (!live(seq)) {
    *err = "pa_alloc_prompt: unknown sequence";
    return kBadSeq;
  }
  if (n < 0 || hit_tokens == nullptr || (n > 0 && (tokens == nullptr || slots == nullptr))) {
    *err = "pa_alloc_prompt: bad arguments";
    return kBadArg;
  }
  Seq& s = seqs_[seq];
  if (s.len != 0 || s.swapped) {
    *err = "pa_alloc_prompt: the sequence is not empty";
    return kBadArg;
  }
  const int64_t nblk = ceil_div(n, bs_);
  // the longest run of cached full blocks, leaving the last token to compute
  std::vector<int32_t> hits;
  try {
    hits.reserve(static_cast<size_t>(nblk));
    s.table.reserve(static_cast<size_t>(nblk));
    s.tokens.reserve(static_cast<size_t>(n));
  } catch (const std::bad_alloc&) {
    *err = "pa_alloc_prompt: out of host memory";
    return kCapacity;
  }
  int64_t free_hits = 0;
  if (!cache_.empty() && n > 0) {
    Digest parent{};
    for (int64_t i = 0; i < (n - 1) / bs_; ++i) {
      const int32_t* ids = tokens + i * bs_;
      const Digest key = block_key(parent, ids);
      const int32_t b = lookup(key);
      if (b < 0) break;
      hits.push_back(b);
      if (ref_[b] == 0) ++free_hits;
      parent = key;
    }
  }
  const int64_t new_blocks = nblk - static_cast<int64_t>(hits.size());
  if (new_blocks > nfree_ - free_hits) {
    *err = "pa_alloc_prompt: not enough free blocks";
    return kNoBlocks;
  }
  // --- no failure past this point ---
  for (int32_t b : hits) {
    if (ref_[b] == 0) unlink(b);
    if (ref_[b] == 1) ++shared_;
    ++ref_[b];
    ++refs_;
    s.table.push_back(b);
  }
  for (int64_t j = 0; j < new_blocks; ++j) {
    const int32_t b = pop_front();
    ref_[b] = 1;
    ++refs_;
    s.table.push_back(b);
  }
  const int64_t hit = static_cast<int64_t>(hits.size()) * bs_;
  for (int64_t pos = hit; pos < n; ++pos)
    slots[pos - hit] = s.table[pos / bs_] * bs_ + static_cast<int32_t>(pos % bs_);
  s.len = n;
  s.tokens.assign(tokens, tokens + n);
  tokens_ += n;
  waste_ += nblk * bs_ - n;
  prompt_tokens_ += n;
  hit_tokens_ += hit;
  *hit_tokens = static_cast<int32_t>(hit);
  return kOk;
}

Status BlockPool::cache_commit(int32_t seq, int32_t* added, std::string* err) {
  if (!live(seq)) {
    *err = "pa_cache_commit: unknown sequence";
    return kBadSeq;
  }
  const Seq& s = seqs_[seq];
  if (s.swapped) {
    *err = "pa_cache_commit: the sequence is swapped out";
    return kBadArg;
  }
  const int64_t full = static_cast<int64_t>(s.tokens.size()) / bs_;
  std::vector<int32_t> done;  // blocks inserted, for the roll-back
  int32_t count = 0;
  Digest parent{};
  try {
    for (int64_t i = 0; i < full; ++i) {
      const int32_t* ids = s.tokens.data() + i * bs_;
      const Digest key = block_key(parent, ids);
      const int32_t b = s.table[i];
      // one cached copy per prefix; a block is cached under one prefix only
      if (cache_.find(key) == cache_.end() && cached_.find(b) == cached_.end()) {
        done.push_back(b);
        cached_.emplace(b, Cached{key});
        cache_.emplace(key, b);
        ++count;
      }
      parent = key;
    }
  } catch (const std::bad_alloc&) {
    for (int32_t b : done) {
      auto it = cached_.find(b);
      if (it != cached_.end()) {
        cache_.erase(it->second.key);
        cached_.erase(it);
      }
    }
    *err = "pa_cache_commit: out of host memory";
    return kCapacity;
  }
  if (added) *added = count;
  return kOk;
}

Status BlockPool::fork(int32_t parent, int32_t* child) {
  if (!live(parent)) return kBadSeq;
  if (child == nullptr || seqs_[parent].swapped) return kBadArg;
  if (seqs_.size() >= static_cast<size_t>(INT32_MAX)) return kCapacity;
  Seq c;
  try {
    c.table = seqs_[parent].table;
    c.tokens = seqs_[parent].tokens;
    // room for the child before any state changes; grows geometrically, like
    // push_back would, so a run of forks does not move every record each time
    if (seqs_.size() == seqs_.capacity())
      seqs_.reserve(std::max<size_t>(2 * seqs_.capacity(), seqs_.size() + 1));
  } catch (const std::bad_alloc&) {
    return kCapacity;
  }
  c.len = seqs_[parent].len;
  c.live = true;
  for (int32_t b : c.table) {
    if (ref_[b] == 1) ++shared_;
    ++ref_[b];
    ++refs_;
  }
  tokens_ += c.len;
  waste_ += static_cast<int64_t>(c.table.size()) * bs_ - c.len;
  seqs_.push_back(std::move(c));
  *child = static_cast<int32_t>(seqs_.size() - 1);
  ++live_seqs_;
  return kOk;
}

Status BlockPool::seq_free(int32_t seq) {
  if (!live(seq)) return kBadSeq;
  Seq& s = seqs_[seq];
  if (s.swapped) {  // host blocks go back to the host queue; device counters were settled at swap-out
    for (int32_t h : s.table) host_push(h);
    std::vector<int32_t>().swap(s.table);
    std::vector<int32_t>().swap(s.tokens);
    s.len = 0;
    s.swapped = false;
    s.live = false;
    --swapped_seqs_;
    --live_seqs_;
    return kOk;
  }
  for (int32_t b : s.table) {
    if (ref_[b] == 2) --shared_;
    --ref_[b];
    --refs_;
    if (ref_[b] == 0) push_back(b);
  }
  tokens_ -= s.len;
  waste_ -= static_cast<int64_t>(s.table.size()) * bs_ - s.len;
  std::vector<int32_t>().swap(s.table);
  std::vector<int32_t>().swap(s.tokens);
  s.len = 0;
  s.live = false;
  --live_seqs_;
  return kOk;
}

Status BlockPool::block_tables(const int32_t* seqs, int32_t n, int32_t max_blocks,
                               int32_t* tables, int32_t* lens, std::string* err) const {
  if (n < 0 || max_blocks < 0 || (n > 0 && (seqs == nullptr || tables == nullptr))) {
    *err = "pa_block_tables: bad arguments";
    return kBadArg;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (!live(seqs[i])) {
      *err = "pa_block_tables: unknown sequence";
      return kBadSeq;
    }
    if (seqs_[seqs[i]].swapped) {
      *err = "pa_block_tables: a sequence is swapped out";
      return kBadArg;
    }
    if (seqs_[seqs[i]].table.size() > static_cast<size_t>(max_blocks)) {
      *err = "pa_block_tables: a table is longer than max_blocks";
      return kCapacity;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = seqs_[seqs[i]];
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    const int32_t nb = static_cast<int32_t>(s.table.size());
    for (int32_t j = 0; j < nb; ++j) row[j] = s.table[j];
    for (int32_t j = nb; j < max_blocks; ++j) row[j] = -1;
    if (lens) lens[i] = static_cast<int32_t>(s.len);
  }
  return kOk;
}

Status BlockPool::seq_table(int32_t seq, int32_t* table, int32_t cap, int32_t* n_out,
                            int32_t* len_out) const {
  if (!live(seq)) return kBadSeq;
  const Seq& s = seqs_[seq];
  const int32_t nb = static_cast<int32_t>(s.table.size());
  if (n_out) *n_out = nb;
  if (len_out) *len_out = static_cast<int32_t>(s.len);
  if (table == nullptr) return kOk;
  if (nb > cap) return kCapacity;
  for (int32_t j = 0; j < nb; ++j) table[j] = s.table[j];
  return kOk;
}

Status BlockPool::shared_prefix(const int32_t* seqs, int32_t n, int32_t* out,
                                std::string* err) const {
  if (n < 0 || (n > 0 && (seqs == nullptr || out == nullptr))) {
    *err = "pa_shared_prefix: bad arguments";
    return kBadArg;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (!live(seqs[i])) {
      *err = "pa_shared_prefix: unknown sequence";
      return kBadSeq;
    }
    if (seqs_[seqs[i]].swapped) {
      *err = "pa_shared_prefix: a sequence is swapped out";
      return kBadArg;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = seqs_[seqs[i]];
    int32_t k = 0;
    while (k < static_cast<int32_t>(s.table.size()) && ref_[s.table[k]] > 1) ++k;
    out[i] = k;
  }
  return kOk;
}

void BlockPool::state(PoolStats* st, int32_t* free_order, int32_t* ref_cnt) const {
  if (st) {
    st->num_blocks = n_;
    st->free_blocks = nfree_;
    st->used_blocks = n_ - nfree_;
    st->shared_blocks = shared_;
    st->total_refs = refs_;
    st->cow_copies = cow_copies_;
    st->live_seqs = live_seqs_;
    st->tokens = tokens_;
    st->waste_tokens = waste_;
    st->cached_blocks = static_cast<int64_t>(cached_.size());
    st->prompt_tokens = prompt_tokens_;
    st->hit_tokens = hit_tokens_;
    st->evictions = evictions_;
    st->host_blocks = host_n_;
    st->host_free_blocks = host_count_;
    st->swapped_seqs = swapped_seqs_;
  }
  if (free_order) {
    int32_t i = 0;
    for (int32_t b = head_; b >= 0; b = next_[b]) free_order[i++] = b;
  }
  if (ref_cnt) {
    for (int32_t b = 0; b < n_; ++b) ref_cnt[b] = ref_[b];
  }
}

int32_t BlockPool::host_pop() {
  const int32_t h = host_free_[host_head_];
  host_head_ = (host_head_ + 1) % host_n_;
  --host_count_;
  return h;
}

void BlockPool::host_push(int32_t h) {
  host_free_[(host_head_ + host_count_) % host_n_] = h;
  ++host_count_;
}

Status BlockPool::set_swap_space(int32_t n, std::string* err) {
  if (n < 0) {
    *err = "pa_swap_space: num_host_blocks < 0";
    return kBadArg;
  }
  if (swapped_seqs_ > 0) {
    *err = "pa_swap_space: sequences are swapped out";
    return kBadArg;
  }
  std::vector<int32_t> q;
  try {
    q.resize(static_cast<size_t>(n));
  } catch (const std::bad_alloc&) {
    *err = "pa_swap_space: out of host memory";
    return kCapacity;
  }
  for (int32_t i = 0; i < n; ++i) q[i] = i;
  host_free_.swap(q);
  host_n_ = n;
  host_head_ = 0;
  host_count_ = n;
  return kOk;
}

Status BlockPool::swap_out(int32_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs,
                           std::string* err) {
  if (!live(seq)) {
    *err = "pa_swap_out: unknown sequence";
    return kBadSeq;
  }
  Seq& s = seqs_[seq];
  const int32_t nb = static_cast<int32_t>(s.table.size());
  if (s.swapped || n_pairs == nullptr || (nb > 0 && pairs == nullptr)) {
    *err = s.swapped ? "pa_swap_out: the sequence is already swapped out" : "pa_swap_out: NULL argument";
    return kBadArg;
  }
  if (nb > cap) {
    *err = "pa_swap_out: pairs_out holds fewer than the sequence's blocks";
    return kCapacity;
  }
  if (nb > host_count_) {
    *err = "pa_swap_out: not enough free host blocks";
    return kNoBlocks;
  }
  // --- no failure past this point ---
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t b = s.table[i];
    const int32_t h = host_pop();
    pairs[2 * i] = b;
    pairs[2 * i + 1] = h;
    if (ref_[b] == 2) --shared_;
    --ref_[b];
    --refs_;
    if (ref_[b] == 0) push_back(b);
    s.table[i] = h;
  }
  tokens_ -= s.len;
  waste_ -= static_cast<int64_t>(nb) * bs_ - s.len;
  s.swapped = true;
  ++swapped_seqs_;
  *n_pairs = nb;
  return kOk;
}

Status BlockPool::swap_in(int32_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs,
                          std::string* err) {
  if (!live(seq)) {
    *err = "pa_swap_in: unknown sequence";
    return kBadSeq;
  }
  Seq& s = seqs_[seq];
  const int32_t nb = static_cast<int32_t>(s.table.size());
  if (!s.swapped || n_pairs == nullptr || (nb > 0 && pairs == nullptr)) {
    *err = !s.swapped ? "pa_swap_in: the sequence is not swapped out" : "pa_swap_in: NULL argument";
    return kBadArg;
  }
  if (nb > cap) {
    *err = "pa_swap_in: pairs_out holds fewer than the sequence's blocks";
    return kCapacity;
  }
  if (nb > nfree_) {
    *err = "pa_swap_in: not enough free blocks";
    return kNoBlocks;
  }
  // --- no failure past this point ---
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t h = s.table[i];
    const int32_t b = pop_front();
    ref_[b] = 1;
    ++refs_;
    pairs[2 * i] = h;
    pairs[2 * i + 1] = b;
    host_push(h);
    s.table[i] = b;
  }
  tokens_ += s.len;
  waste_ += static_cast<int64_t>(nb) * bs_ - s.len;
  s.swapped = false;
  --swapped_seqs_;
  *n_pairs = nb;
  return kOk;
}

}  // namespace pa
