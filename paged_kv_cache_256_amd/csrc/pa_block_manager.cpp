// pa_block_manager.cpp -- host-side block manager: the step before the kernels, which turns
// "sequence s gets a token" into cache slots, block tables and copy-on-write copies.
//
// What it does (codebumble.net, "The Block Table Mapping Subsystem"; bicarait.com,
// "Architectural Blueprint 2"; infoisland, section 2):
//  * The cache holds NB fixed-size frames.  Free frames wait in a FIFO free list: allocation
//    takes the head, release appends to the tail.
//  * A sequence's block table lists its frames in logical order.  Token position p lives in
//    logical block p / bs at offset p % bs, so a new frame is taken exactly when a token starts
//    a block (offset 0): allocation is on demand and waste is confined to the last block.
//  * fork(parent, child) gives the child the parent's table; every frame gains a reference.
//  * Copy-on-write: a token written into a frame that other tables also reference (offset != 0
//    in a shared last frame) first moves the writer to a fresh frame.  The (old, new) pair is
//    returned so the caller copies the frame's contents with pa_copy_blocks before writing.
//  * free(s) drops one reference from each of s's frames; frames no table references any more
//    return to the free list in table order.
//  * Prefix caching (codebumble.net, "CUDA Shared Memory Optimization": a prefix tree of token
//    blocks lets a new prompt reference the blocks an earlier prompt already computed):
//    append_prompt matches the prompt's full blocks in a tree whose nodes are keyed by
//    (parent node, the block's token ids) -- compared exactly, so no two different prefixes can
//    share a frame -- references every matched frame, and registers the full blocks it fills.
//    A released frame keeps its registration while it waits in the free list (a later prompt
//    can revive it) and loses it when allocation reuses the frame.
// Every mutating call either succeeds completely or changes nothing.

#include <algorithm>
#include <climits>
#include <cstdint>
#include <deque>
#include <functional>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

// A prefix-tree edge: the parent node (-1 for a prompt's first block) and the block's tokens.
struct BlockKey {
  int64_t parent = -1;
  std::vector<int32_t> tokens;
  bool operator==(const BlockKey& o) const { return parent == o.parent && tokens == o.tokens; }
};
struct BlockKeyHash {
  size_t operator()(const BlockKey& k) const {
    uint64_t h = 0x9e3779b97f4a7c15ull ^ (uint64_t)k.parent;
    for (int32_t t : k.tokens) h = (h ^ (uint32_t)t) * 0x100000001b3ull;
    return (size_t)h;
  }
};

}  // namespace

struct pa_block_manager {
  int64_t nb = 0;
  int bs = 0;
  // Free list: FIFO of (frame, generation).  An entry is live while its frame is free and the
  // generation matches; reviving a cached frame just marks it used (its entry goes stale).
  std::deque<std::pair<int32_t, uint32_t>> free_list;
  std::vector<uint32_t> free_gen;
  std::vector<char> is_free;
  int64_t n_free = 0;
  std::vector<int32_t> refs;  // tables referencing each frame
  struct Seq {
    std::vector<int32_t> frames;
    int64_t len = 0;  // tokens written
  };
  std::unordered_map<int64_t, Seq> seqs;
  // Prefix tree: key -> frame; per frame its node id (-1: not registered) and key.
  std::unordered_map<BlockKey, int32_t, BlockKeyHash> tree;
  std::vector<int64_t> node_of;
  std::vector<BlockKey> key_of;
  int64_t next_node = 0;

  void push_free(int32_t f) {
    is_free[f] = 1;
    free_list.emplace_back(f, ++free_gen[f]);
    ++n_free;
  }
  void unregister(int32_t f) {
    if (node_of[f] < 0) return;
    tree.erase(key_of[f]);
    key_of[f].tokens.clear();
    node_of[f] = -1;
  }
  // Take the frame at the head of the free list (there must be one); a frame still registered
  // in the prefix tree is evicted from it.
  int32_t pop_free() {
    for (;;) {
      const auto e = free_list.front();
      free_list.pop_front();
      if (is_free[e.first] && e.second == free_gen[e.first]) {
        is_free[e.first] = 0;
        --n_free;
        unregister(e.first);
        return e.first;
      }
    }
  }
  // A registered frame referenced again (it may be waiting in the free list).
  void revive(int32_t f) {
    if (is_free[f]) {
      is_free[f] = 0;
      --n_free;
    }
    ++refs[f];
  }
};

namespace {

// What appending one token to `s` needs: a new frame (block start, or copy-on-write of a shared
// last frame) and, for copy-on-write, the frame it replaces.
struct AppendPlan {
  bool new_frame = false;
  int32_t cow_from = -1;
};

AppendPlan plan_append(const pa_block_manager::Seq& s, int bs, const std::vector<int32_t>& refs) {
  AppendPlan p;
  const int64_t off = s.len % bs;
  if (off == 0) {
    p.new_frame = true;
  } else {
    const int32_t last = s.frames.back();
    if (refs[last] > 1) {
      p.new_frame = true;
      p.cow_from = last;
    }
  }
  return p;
}

}  // namespace

extern "C" {

int pa_bm_create(int64_t num_frames, int block_size, pa_block_manager** out) {
  if (!out) return pa::set_error(PA_EINVAL, "null output pointer");
  *out = nullptr;
  if (num_frames < 1 || num_frames > INT32_MAX)
    return pa::set_error(PA_EINVAL, "num_frames %lld outside [1, 2^31)", (long long)num_frames);
  if (block_size < 1) return pa::set_error(PA_EINVAL, "block_size %d must be positive", block_size);
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return pa::set_error(PA_ENOSPC, "out of host memory");
  bm->nb = num_frames;
  bm->bs = block_size;
  bm->refs.assign((size_t)num_frames, 0);
  bm->free_gen.assign((size_t)num_frames, 0);
  bm->is_free.assign((size_t)num_frames, 0);
  bm->node_of.assign((size_t)num_frames, -1);
  bm->key_of.resize((size_t)num_frames);
  for (int64_t f = 0; f < num_frames; ++f) bm->push_free((int32_t)f);
  *out = bm;
  return pa::clear_error();
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, int64_t n, int64_t* slots,
                 int64_t* copy_pairs, int64_t* num_copies) {
  if (!bm) return pa::set_error(PA_EINVAL, "null block manager");
  if (n < 0) return pa::set_error(PA_EINVAL, "n %lld must not be negative", (long long)n);
  if (n > 0 && (!seq_ids || !slots || !copy_pairs || !num_copies))
    return pa::set_error(PA_EINVAL, "null pointer argument");
  if (num_copies) *num_copies = 0;
  if (n == 0) return pa::clear_error();
  // Pass 1 (no state change): frames needed, with the reference counts and lengths each
  // entry would see after the earlier entries of the same call.
  // A sequence is summarised by its length and last frame (-1: a fresh frame of this call,
  // referenced once); only those change within one call.
  struct Tail {
    int64_t len;
    int32_t last;
  };
  std::unordered_map<int32_t, int32_t> ref_delta;
  std::unordered_map<int64_t, Tail> touched;
  touched.reserve((size_t)n);
  int64_t need = 0;
  auto ref_of = [&](int32_t f) {
    auto it = ref_delta.find(f);
    return bm->refs[f] + (it == ref_delta.end() ? 0 : it->second);
  };
  for (int64_t i = 0; i < n; ++i) {
    const int64_t id = seq_ids[i];
    auto t = touched.find(id);
    if (t == touched.end()) {
      auto it = bm->seqs.find(id);
      Tail tl{0, -1};
      if (it != bm->seqs.end()) {
        tl.len = it->second.len;
        tl.last = it->second.frames.empty() ? -1 : it->second.frames.back();
      }
      t = touched.emplace(id, tl).first;
    }
    Tail& s = t->second;
    if (s.len % bm->bs == 0) {
      ++need;
      s.last = -1;  // a fresh frame, referenced once
    } else if (s.last >= 0 && ref_of(s.last) > 1) {
      ++need;
      --ref_delta[s.last];
      s.last = -1;
    }
    ++s.len;
  }
  if (need > bm->n_free)
    return pa::set_error(PA_ENOSPC, "%lld free frames needed, %lld free", (long long)need,
                         (long long)bm->n_free);
  // Pass 2: apply.
  int64_t nc = 0;
  for (int64_t i = 0; i < n; ++i) {
    pa_block_manager::Seq& s = bm->seqs[seq_ids[i]];
    const AppendPlan p = plan_append(s, bm->bs, bm->refs);
    if (p.new_frame) {
      const int32_t f = bm->pop_free();
      bm->refs[f] = 1;
      if (p.cow_from >= 0) {
        --bm->refs[p.cow_from];
        s.frames.back() = f;
        copy_pairs[2 * nc] = p.cow_from;
        copy_pairs[2 * nc + 1] = f;
        ++nc;
      } else {
        s.frames.push_back(f);
      }
    }
    const int64_t pos = s.len++;
    slots[i] = (int64_t)s.frames[pos / bm->bs] * bm->bs + pos % bm->bs;
  }
  *num_copies = nc;
  return pa::clear_error();
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return pa::set_error(PA_EINVAL, "null block manager");
  auto p = bm->seqs.find(parent);
  if (p == bm->seqs.end()) return pa::set_error(PA_EINVAL, "unknown parent sequence %lld", (long long)parent);
  if (bm->seqs.count(child)) return pa::set_error(PA_EINVAL, "sequence %lld already exists", (long long)child);
  pa_block_manager::Seq copy = p->second;
  for (int32_t f : copy.frames) ++bm->refs[f];
  bm->seqs.emplace(child, std::move(copy));
  return pa::clear_error();
}

int pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return pa::set_error(PA_EINVAL, "null block manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::set_error(PA_EINVAL, "unknown sequence %lld", (long long)seq);
  for (int32_t f : it->second.frames)
    if (--bm->refs[f] == 0) bm->push_free(f);
  bm->seqs.erase(it);
  return pa::clear_error();
}

int pa_bm_num_free(const pa_block_manager* bm, int64_t* out) {
  if (!bm || !out) return pa::set_error(PA_EINVAL, "null pointer argument");
  *out = bm->n_free;
  return pa::clear_error();
}

int pa_bm_seq_len(const pa_block_manager* bm, int64_t seq, int64_t* out) {
  if (!bm || !out) return pa::set_error(PA_EINVAL, "null pointer argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::set_error(PA_EINVAL, "unknown sequence %lld", (long long)seq);
  *out = it->second.len;
  return pa::clear_error();
}

int pa_bm_ref_count(const pa_block_manager* bm, int64_t frame, int32_t* out) {
  if (!bm || !out) return pa::set_error(PA_EINVAL, "null pointer argument");
  if (frame < 0 || frame >= bm->nb)
    return pa::set_error(PA_ERANGE, "frame %lld outside [0, %lld)", (long long)frame, (long long)bm->nb);
  *out = bm->refs[(size_t)frame];
  return pa::clear_error();
}

int pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int64_t capacity, int64_t* count) {
  if (!bm || !count) return pa::set_error(PA_EINVAL, "null pointer argument");
  *count = bm->n_free;
  if (capacity < *count) return pa::set_error(PA_ERANGE, "capacity %lld < %lld free frames", (long long)capacity, (long long)*count);
  if (*count > 0 && !out) return pa::set_error(PA_EINVAL, "null output pointer");
  int64_t i = 0;
  for (const auto& e : bm->free_list)
    if (bm->is_free[e.first] && e.second == bm->free_gen[e.first]) out[i++] = e.first;
  return pa::clear_error();
}

int pa_bm_append_prompt(pa_block_manager* bm, int64_t seq, const int32_t* tokens, int64_t n,
                        int64_t* slots, int64_t* num_cached) {
  if (!bm) return pa::set_error(PA_EINVAL, "null block manager");
  if (n < 1) return pa::set_error(PA_EINVAL, "a prompt needs at least one token (n %lld)", (long long)n);
  if (!tokens || !slots || !num_cached) return pa::set_error(PA_EINVAL, "null pointer argument");
  if (bm->seqs.count(seq)) return pa::set_error(PA_EINVAL, "sequence %lld already exists", (long long)seq);
  const int bs = bm->bs;
  const int64_t full = n / bs, blocks = (n + bs - 1) / bs;
  // match the longest run of cached full blocks
  std::vector<int32_t> matched;
  BlockKey key;
  int64_t revived = 0;
  for (int64_t k = 0; k < full; ++k) {
    key.tokens.assign(tokens + k * bs, tokens + (k + 1) * bs);
    const auto it = bm->tree.find(key);
    if (it == bm->tree.end()) break;
    matched.push_back(it->second);
    if (bm->is_free[it->second]) ++revived;
    key.parent = bm->node_of[it->second];
  }
  const int64_t need = blocks - (int64_t)matched.size();
  if (need > bm->n_free - revived)
    return pa::set_error(PA_ENOSPC, "%lld free frames needed, %lld free", (long long)need,
                         (long long)(bm->n_free - revived));
  for (int32_t f : matched) bm->revive(f);
  pa_block_manager::Seq& s = bm->seqs[seq];
  s.frames = matched;
  for (int64_t k = (int64_t)matched.size(); k < blocks; ++k) {
    const int32_t f = bm->pop_free();
    bm->refs[f] = 1;
    s.frames.push_back(f);
    if (k < full) {  // a full block of this prompt: register it under its parent
      key.tokens.assign(tokens + k * bs, tokens + (k + 1) * bs);
      bm->tree.emplace(key, f);
      bm->key_of[f] = key;
      bm->node_of[f] = bm->next_node++;
      key.parent = bm->node_of[f];
    }
  }
  s.len = n;
  for (int64_t i = 0; i < n; ++i) slots[i] = (int64_t)s.frames[i / bs] * bs + i % bs;
  *num_cached = (int64_t)matched.size() * bs;
  return pa::clear_error();
}

int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int64_t n,
                       int32_t* tables, int max_blocks_per_seq, int32_t* context_lens) {
  if (!bm) return pa::set_error(PA_EINVAL, "null block manager");
  if (n < 0 || max_blocks_per_seq < 1) return pa::set_error(PA_EINVAL, "bad sizes");
  if (n > 0 && (!seq_ids || !tables || !context_lens)) return pa::set_error(PA_EINVAL, "null pointer argument");
  for (int64_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pa::set_error(PA_EINVAL, "unknown sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.frames.size() > max_blocks_per_seq)
      return pa::set_error(PA_ERANGE, "sequence %lld has %zu blocks > max_blocks_per_seq %d",
                           (long long)seq_ids[i], it->second.frames.size(), max_blocks_per_seq);
    if (it->second.len > INT32_MAX) return pa::set_error(PA_ERANGE, "sequence too long");
  }
  for (int64_t i = 0; i < n; ++i) {
    const pa_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + (size_t)i * max_blocks_per_seq;
    const size_t k = s.frames.size();
    std::copy(s.frames.begin(), s.frames.end(), row);
    std::fill(row + k, row + max_blocks_per_seq, -1);
    context_lens[i] = (int32_t)s.len;
  }
  return pa::clear_error();
}

}  // extern "C"
