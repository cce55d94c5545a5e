// Host block manager for the paged KV cache.
//
// Model ([p2] "PagedAttention: KV cache as virtual memory", sections "Direct
// answer" and "Deep dive"; [p3] "PagedAttention: Why Static Batching Wastes Your
// KV Cache", sections on on-demand blocks and copy-on-write):
//   * a pool of fixed-size physical blocks shared by every sequence;
//   * a free queue, doubly linked through two int32 arrays, giving O(1) take
//     from the front, return to the back and (for later prefix caching) removal
//     from the middle;
//   * a reference count per block; a block returns to the queue at zero;
//   * per sequence: a block table (logical -> physical) and a token count.
// Prefix caching ([p2] "Deep dive", prefix-caching bullet; [p1] "Automatic
// Prefix Caching (APC)"): a full block is keyed by a chained digest of its
// token ids and its parent block's key (SHA-256 over the parent's 32-byte key
// and the block's ids), so a key names the whole token prefix that ends with
// the block and a hit means that prefix matches (up to a SHA-256 collision).
// Freed blocks keep their entry while they wait in the free queue and lose it
// when the queue front hands them out again; a hit on a waiting block takes it
// out of the middle of the queue.  Blocks enter the cache on cache_commit(),
// once the caller has written their K/V.
// Preemption by swapping ([p3] "What happens when the GPU runs out of KV
// blocks?"): an optional pool of host (CPU RAM) blocks with its own FIFO free
// queue; swapping a sequence out moves its table to host blocks and drops its
// references to device blocks, swapping it in takes device blocks again.  The
// byte copies are the caller's (pa_swap_blocks), ordered on its stream.
// Every mutating call is all-or-nothing: it validates and reserves host memory
// first, and only then changes state.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "sha256.hpp"

namespace pa {

enum Status : int32_t {
  kOk = 0,
  kNoBlocks = 1,
  kBadSeq = 2,
  kBadArg = 3,
  kCapacity = 4,
};

struct PoolStats {
  int64_t num_blocks, free_blocks, used_blocks, shared_blocks, total_refs, cow_copies,
      live_seqs, tokens, waste_tokens, cached_blocks, prompt_tokens, hit_tokens, evictions,
      host_blocks, host_free_blocks, swapped_seqs;
};

class BlockPool {
 public:
  // order: nullptr for 0..n-1, else a permutation (validated by create()).
  static Status create(int32_t num_blocks, int32_t block_size, const int32_t* order,
                       BlockPool** out, std::string* err);

  Status seq_create(int32_t* id);
  // slots: n entries; cow: {src, dst} or {-1, -1}.  tokens: the new tokens'
  // ids (recorded for prefix caching) or nullptr (the sequence's later
  // blocks are then never cached).
  Status alloc_append(int32_t seq, int32_t n, const int32_t* tokens, int32_t* slots, int32_t* cow,
                      std::string* err);
  // alloc_append for seqs[0], seqs[1], ... in that order (counts[i] tokens
  // each; tokens: their ids back to back, or nullptr), all or nothing: the
  // first call that would fail decides the status and nothing is changed.
  // slots: sum(counts) entries in batch order; cow: 2 entries per sequence.
  // A sequence may appear once.
  Status alloc_append_batch(const int32_t* seqs, int32_t n_seqs, const int32_t* counts,
                            const int32_t* tokens, int32_t* slots, int32_t* cow, std::string* err);
  // Admit a prompt into an empty sequence, reusing cached full blocks; slots
  // gets the slots of tokens hit..n-1; at most (n - 1) / block_size blocks are
  // reused (the last token is always computed).
  Status alloc_prompt(int32_t seq, const int32_t* tokens, int32_t n, int32_t* slots,
                      int32_t* hit_tokens, std::string* err);
  // Enter the sequence's full, token-known blocks into the prefix cache.
  Status cache_commit(int32_t seq, int32_t* added, std::string* err);
  // Host swap space of n blocks (only while no sequence is swapped out).
  Status set_swap_space(int32_t n, std::string* err);
  // pairs: 2 * blocks entries {device, host} (out) / {host, device} (in).
  Status swap_out(int32_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs, std::string* err);
  Status swap_in(int32_t seq, int32_t* pairs, int32_t cap, int32_t* n_pairs, std::string* err);
  Status fork(int32_t parent, int32_t* child);
  Status seq_free(int32_t seq);
  Status block_tables(const int32_t* seqs, int32_t n, int32_t max_blocks, int32_t* tables,
                      int32_t* lens, std::string* err) const;
  Status seq_table(int32_t seq, int32_t* table, int32_t cap, int32_t* n_out,
                   int32_t* len_out) const;
  // Per sequence: how many leading table entries are shared (ref_cnt > 1).
  Status shared_prefix(const int32_t* seqs, int32_t n, int32_t* out, std::string* err) const;
  void state(PoolStats* st, int32_t* free_order, int32_t* ref_cnt) const;

  int32_t num_blocks() const { return n_; }
  int32_t block_size() const { return bs_; }

 private:
  BlockPool(int32_t n, int32_t bs);
  bool live(int32_t seq) const {
    return seq >= 0 && seq < static_cast<int32_t>(seqs_.size()) && seqs_[seq].live;
  }
  int32_t pop_front();  // evicts the block's cache entry, if any
  void push_back(int32_t b);
  void unlink(int32_t b);  // remove from the middle of the free queue
  int32_t host_pop();
  void host_push(int32_t h);
  Digest block_key(const Digest& parent, const int32_t* ids) const;
  // cached block for this prefix key, or -1
  int32_t lookup(const Digest& key) const;

  struct Seq {
    std::vector<int32_t> table;  // device blocks, or host blocks while swapped
    bool swapped = false;
    std::vector<int32_t> tokens;  // ids of the leading tokens, while every append gave them
    int64_t len = 0;
    bool live = false;
  };
  struct Cached {
    Digest key;
  };

  int32_t n_, bs_;
  // free queue: next_/prev_ links, -1 terminated; in_queue_ marks membership
  std::vector<int32_t> next_, prev_;
  std::vector<uint8_t> in_queue_;
  int32_t head_ = -1, tail_ = -1, nfree_ = 0;
  std::vector<int32_t> ref_;
  std::vector<Seq> seqs_;  // indexed by id; ids are never reused
  int64_t live_seqs_ = 0, tokens_ = 0, waste_ = 0, cow_copies_ = 0, shared_ = 0, refs_ = 0;
  std::unordered_map<Digest, int32_t, DigestHash> cache_;   // prefix key -> block
  std::unordered_map<int32_t, Cached> cached_;    // block -> its entry
  int64_t prompt_tokens_ = 0, hit_tokens_ = 0, evictions_ = 0;
  // host swap space: FIFO free queue of host block ids
  int32_t host_n_ = 0;
  std::vector<int32_t> host_free_;  // ring buffer of host_n_ entries
  int32_t host_head_ = 0, host_count_ = 0;
  int64_t swapped_seqs_ = 0;
};

}  // namespace pa
