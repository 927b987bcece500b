// Host block manager: the memory-management side of the paged KV cache.
//
// A fixed pool of physical blocks; each sequence owns a block table (logical
// block j -> physical block) that grows on demand as tokens are appended, and
// its blocks return to the pool when the sequence is freed.  Sequences that
// share a prefix share physical blocks (reference counts); a sequence that
// appends into a shared, partially filled last block first gets its own copy
// of it (copy-on-write), reported as a (src, dst) pair for pa_copy_blocks.
// Pages: "Paged Attention and Memory Efficiency in Production LLM Serving",
// section "How PagedAttention borrows OS paging to eliminate KV cache
// fragmentation"; "PagedAttention in Production", section "Core Principle";
// "PagedAttention - The KV Cache Problem", sections "How It Works" and "Why
// This Matters for Production".
//
// Policies the pages leave open: free blocks are handed out last-freed-first
// (a fresh pool hands out 0, 1, 2, ...); a full shared block is never
// written, so only a partial last block is copied; an append that cannot get
// every block it needs fails and changes nothing.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> table;
    int64_t length = 0;
  };
  int32_t block_size;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) free_stack.push_back(b);
  }
  // blocks an append of n tokens to s needs, copy included
  int64_t blocks_needed(const Seq& s, int64_t n) const {
    const int64_t bs = block_size;
    const bool cow = n > 0 && s.length % bs != 0 && refcount[s.table.back()] > 1;
    const int64_t grow = n > 0 ? (s.length + n + bs - 1) / bs - (int64_t)s.table.size() : 0;
    return grow + (cow ? 1 : 0);
  }
  // append n tokens (the caller checked the pool); returns whether a copy was made
  bool append(Seq& s, int64_t n, int64_t* slots, int64_t* pair) {
    const int64_t bs = block_size;
    bool copied = false;
    if (n > 0 && s.length % bs != 0 && refcount[s.table.back()] > 1) {
      const int32_t old = s.table.back();
      const int32_t fresh = take();
      release(old);
      s.table.back() = fresh;
      pair[0] = old;
      pair[1] = fresh;
      copied = true;
    }
    const int64_t grow = n > 0 ? (s.length + n + bs - 1) / bs - (int64_t)s.table.size() : 0;
    for (int64_t i = 0; i < grow; ++i) s.table.push_back(take());
    for (int64_t i = 0; i < n; ++i) {
      const int64_t t = s.length + i;
      slots[i] = (int64_t)s.table[t / bs] * bs + t % bs;
    }
    s.length += n;
    return copied;
  }
};

using pa::set_error;

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size) {
  if (num_blocks < 0 || num_blocks > INT32_MAX || block_size < 1) {
    set_error("pa_bm_create: need 0 <= num_blocks <= 2^31-1 and block_size >= 1");
    return nullptr;
  }
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) {
    set_error("pa_bm_create: out of host memory");
    return nullptr;
  }
  try {
    bm->block_size = block_size;
    bm->refcount.assign((size_t)num_blocks, 0);
    bm->free_stack.resize((size_t)num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) bm->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
  } catch (...) {
    delete bm;
    set_error("pa_bm_create: out of host memory");
    return nullptr;
  }
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add(pa_block_manager* bm, int64_t seq) {
  if (!bm) return set_error("pa_bm_add: null manager"), PA_ERR_INVALID_ARG;
  if (bm->seqs.count(seq)) return set_error("pa_bm_add: sequence %lld exists", (long long)seq), PA_ERR_INVALID_ARG;
  bm->seqs.emplace(seq, pa_block_manager::Seq());
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return set_error("pa_bm_fork: null manager"), PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return set_error("pa_bm_fork: no sequence %lld", (long long)parent), PA_ERR_INVALID_ARG;
  if (bm->seqs.count(child)) return set_error("pa_bm_fork: sequence %lld exists", (long long)child), PA_ERR_INVALID_ARG;
  pa_block_manager::Seq copy = it->second;
  for (int32_t b : copy.table) ++bm->refcount[b];
  bm->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t n, int64_t* slots, int64_t* copy_pair,
                       int32_t* copied) {
  if (!bm || n < 0 || (n > 0 && !slots) || !copy_pair || !copied)
    return set_error("pa_bm_append: null pointer or n < 0"), PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return set_error("pa_bm_append: no sequence %lld", (long long)seq), PA_ERR_INVALID_ARG;
  const int64_t need = bm->blocks_needed(it->second, n);
  if (need > (int64_t)bm->free_stack.size())
    return set_error("pa_bm_append: %lld blocks needed, %zu free", (long long)need, bm->free_stack.size()),
           PA_ERR_NO_BLOCKS;
  *copied = bm->append(it->second, n, slots, copy_pair) ? 1 : 0;
  return PA_OK;
}

pa_status pa_bm_append_batch(pa_block_manager* bm, const int64_t* seqs, int32_t count, const int32_t* n_tokens,
                             int64_t* slots, int64_t* copy_pairs, int32_t* n_pairs) {
  if (!bm || count < 0 || (count > 0 && (!seqs || !n_tokens || !slots || !copy_pairs)) || !n_pairs)
    return set_error("pa_bm_append_batch: null pointer or count < 0"), PA_ERR_INVALID_ARG;
  std::vector<pa_block_manager::Seq*> ss((size_t)count);
  int64_t need = 0;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return set_error("pa_bm_append_batch: no sequence %lld", (long long)seqs[i]), PA_ERR_INVALID_ARG;
    if (n_tokens[i] < 0) return set_error("pa_bm_append_batch: n_tokens[%d] < 0", i), PA_ERR_INVALID_ARG;
    ss[(size_t)i] = &it->second;
    need += bm->blocks_needed(it->second, n_tokens[i]);
  }
  for (int32_t i = 1; i < count; ++i)
    for (int32_t j = 0; j < i && count <= 64; ++j)
      if (seqs[i] == seqs[j]) return set_error("pa_bm_append_batch: sequence %lld twice", (long long)seqs[i]), PA_ERR_INVALID_ARG;
  if (count > 64) {  // duplicates: one pass over a sorted copy
    std::vector<int64_t> sorted(seqs, seqs + count);
    std::sort(sorted.begin(), sorted.end());
    for (int32_t i = 1; i < count; ++i)
      if (sorted[(size_t)i] == sorted[(size_t)i - 1])
        return set_error("pa_bm_append_batch: sequence %lld twice", (long long)sorted[(size_t)i]), PA_ERR_INVALID_ARG;
  }
  if (need > (int64_t)bm->free_stack.size())
    return set_error("pa_bm_append_batch: %lld blocks needed, %zu free", (long long)need, bm->free_stack.size()),
           PA_ERR_NO_BLOCKS;
  int64_t off = 0;
  int32_t pairs = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (bm->append(*ss[(size_t)i], n_tokens[i], slots + off, copy_pairs + 2 * (int64_t)pairs)) ++pairs;
    off += n_tokens[i];
  }
  *n_pairs = pairs;
  return PA_OK;
}

pa_status pa_bm_evict(pa_block_manager* bm, int64_t seq, int64_t sink_tokens, int64_t window_tokens,
                      int64_t* dropped) {
  if (!bm || sink_tokens < 0 || window_tokens < 0)
    return set_error("pa_bm_evict: null manager or negative sink/window"), PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return set_error("pa_bm_evict: no sequence %lld", (long long)seq), PA_ERR_INVALID_ARG;
  pa_block_manager::Seq& s = it->second;
  const int64_t bs = bm->block_size;
  const int64_t nblk = (int64_t)s.table.size();
  const int64_t head = (sink_tokens + bs - 1) / bs;  // blocks kept in front
  // first block kept behind: the window's first, never past the newest block
  const int64_t tail = std::min(s.length > window_tokens ? (s.length - window_tokens) / bs : 0, nblk - 1);
  int64_t n = 0;
  if (tail > head) {
    for (int64_t j = head; j < tail; ++j) bm->release(s.table[(size_t)j]);
    s.table.erase(s.table.begin() + head, s.table.begin() + tail);
    n = (tail - head) * bs;
    s.length -= n;
  }
  if (dropped) *dropped = n;
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return set_error("pa_bm_free: null manager"), PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return set_error("pa_bm_free: no sequence %lld", (long long)seq), PA_ERR_INVALID_ARG;
  for (int32_t b : it->second.table) bm->release(b);
  bm->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* table, int32_t capacity) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  const auto& t = it->second.table;
  const int32_t n = (int32_t)t.size();
  if (table)
    for (int32_t i = 0; i < n && i < capacity; ++i) table[i] = t[(size_t)i];
  return n;
}

pa_status pa_bm_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t count, int32_t* tables,
                       int32_t width, int32_t* context_lens, int32_t pad) {
  if (!bm || count < 0 || width < 1 || (count > 0 && (!seqs || !tables)))
    return set_error("pa_bm_tables: null pointer or bad size"), PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return set_error("pa_bm_tables: no sequence %lld", (long long)seqs[i]), PA_ERR_INVALID_ARG;
    if ((int64_t)it->second.table.size() > width)
      return set_error("pa_bm_tables: sequence %lld has %zu blocks, width %d", (long long)seqs[i],
                       it->second.table.size(), width), PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < count; ++i) {
    const auto& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + (int64_t)i * width;
    const size_t n = s.table.size();
    if (n) std::memcpy(row, s.table.data(), n * sizeof(int32_t));
    if (pad) std::fill_n(row + n, (size_t)width - n, -1);
    if (context_lens) context_lens[i] = (int32_t)s.length;
  }
  return PA_OK;
}

int64_t pa_bm_length(const pa_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.length;
}

pa_status pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* out) {
  if (!bm || !out) return set_error("pa_bm_get_stats: null pointer"), PA_ERR_INVALID_ARG;
  pa_bm_stats st{};
  st.blocks_free = (int64_t)bm->free_stack.size();
  st.blocks_in_use = (int64_t)bm->refcount.size() - st.blocks_free;
  for (int32_t c : bm->refcount) st.shared_blocks += c > 1;
  for (const auto& kv : bm->seqs) {
    st.slots_held += (int64_t)kv.second.table.size() * bm->block_size;
    st.tokens += kv.second.length;
  }
  st.sequences = (int64_t)bm->seqs.size();
  *out = st;
  return PA_OK;
}

}  // extern "C"
