// Host-side KV block manager (include/pa_blocks.h).
//
// The KV cache is managed like virtual memory ("vLLM Project Update" talk,
// PagedAttention recap): each sequence owns a table of physical block ids;
// blocks carry reference counts so that sequences can share them (a fork
// shares every block, a write into a shared block first takes a private copy);
// full blocks whose KV is written can be registered in a prefix cache (the
// talk's prefix-caching update) and are then found by later sequences whose
// prompt starts with the same tokens.
//
// The prefix cache is a trie over blocks of tokens: node = (parent node, the
// block's token ids), so a node stands for one exact token prefix and no hash
// collision can map two different prefixes to one block.  A node may hold one
// cached physical block.  Nodes are reference counted by the sequences whose
// written blocks pass through them, by their children and by their cached
// block; node ids are never reused.  A node whose block was evicted stays
// while something refers to it, so the trie always answers for exact token
// prefixes.  Lookups walk from the root and stop at the first node without a
// cached block.
//
// Released cached blocks (reference count 0) stay cached in a
// least-recently-released list and are only taken when no free block is left.
#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_blocks.h"

namespace {

struct NodeKey {
  int64_t parent;
  std::vector<int32_t> tokens;
  bool operator==(const NodeKey& o) const { return parent == o.parent && tokens == o.tokens; }
};

struct NodeKeyHash {
  size_t operator()(const NodeKey& k) const {
    // 64-bit FNV-1a over the parent id and the token ids (equality decides)
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](uint64_t v) {
      for (int i = 0; i < 8; ++i) {
        h ^= (v >> (8 * i)) & 0xff;
        h *= 1099511628211ull;
      }
    };
    mix((uint64_t)k.parent);
    for (int32_t t : k.tokens) mix((uint32_t)t);
    return (size_t)h;
  }
};

struct Node {
  NodeKey key;
  int32_t block = -1;  // the cached physical block of this prefix, or -1
  int64_t refs = 0;    // sequences through it + children + (block >= 0)
};

struct Seq {
  std::vector<int32_t> blocks;       // device blocks (resident)
  std::vector<int32_t> host_blocks;  // host blocks (swapped out)
  std::vector<int32_t> tokens;       // token ids (prefix caching only)
  std::vector<int64_t> nodes;        // trie node of each leading written block
  int32_t len = 0;
  bool resident = true;
};

}  // namespace

struct pa_block_manager {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  bool caching = false;

  std::vector<int32_t> refs;           // per device block
  std::vector<int64_t> node_of_block;  // trie node caching the block, or 0
  std::vector<int32_t> free_list;      // blocks with refs 0 and no cached prefix
  // cached blocks with refs 0, oldest release first: a doubly linked list
  // through per-block links (so that releasing never allocates)
  std::vector<int32_t> lru_prev, lru_next;
  int32_t lru_head = -1, lru_tail = -1;
  int64_t lru_count = 0;
  std::vector<int32_t> host_free;

  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int64_t, Node> nodes;  // id >= 1; 0 is the root
  std::unordered_map<NodeKey, int64_t, NodeKeyHash> children;
  int64_t next_node = 1;

  int64_t allocatable() const { return (int64_t)free_list.size() + lru_count; }

  void lru_push_back(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    ++lru_count;
  }

  void lru_remove(int32_t b) {
    if (lru_prev[b] >= 0) lru_next[lru_prev[b]] = lru_next[b]; else lru_head = lru_next[b];
    if (lru_next[b] >= 0) lru_prev[lru_next[b]] = lru_prev[b]; else lru_tail = lru_prev[b];
    --lru_count;
  }

  void unref_node(int64_t id) {
    while (id != 0) {
      auto it = nodes.find(id);
      if (--it->second.refs > 0) return;
      const int64_t parent = it->second.key.parent;
      children.erase(it->second.key);
      nodes.erase(it);
      id = parent;  // the child's reference on its parent goes with it
    }
  }

  // One free block with refs = 1: a never-cached one if any, else the least
  // recently released cached block (its prefix leaves the cache).
  int32_t take_block() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.back();
      free_list.pop_back();
    } else {
      b = lru_head;
      lru_remove(b);
      const int64_t node = node_of_block[b];
      nodes.find(node)->second.block = -1;
      node_of_block[b] = 0;
      unref_node(node);
    }
    refs[b] = 1;
    return b;
  }

  void release_block(int32_t b) {
    if (--refs[b] > 0) return;
    if (node_of_block[b] != 0) {
      lru_push_back(b);
    } else {
      free_list.push_back(b);
    }
  }

  // Drop a resident sequence's device blocks (last block first, so that the
  // prompt's first blocks are the last of them to be evicted) and its nodes.
  void release_device(Seq& s) {
    for (auto it = s.blocks.rbegin(); it != s.blocks.rend(); ++it) release_block(*it);
    s.blocks.clear();
    for (auto it = s.nodes.rbegin(); it != s.nodes.rend(); ++it) unref_node(*it);
    s.nodes.clear();
  }

  NodeKey key_of(int64_t parent, const Seq& s, int32_t blk) const {
    const auto first = s.tokens.begin() + (int64_t)blk * block_size;
    return NodeKey{parent, std::vector<int32_t>(first, first + block_size)};
  }
};

extern "C" {

int pa_bm_create(int64_t num_blocks, int32_t block_size, int64_t num_host_blocks, uint32_t flags,
                 pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  if (num_blocks < 1 || num_blocks > 0x7fffffffLL || block_size < 1 || num_host_blocks < 0 ||
      num_host_blocks > 0x7fffffffLL || (flags & ~PA_BM_PREFIX_CACHING))
    return PA_ERR_SHAPE;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_CAPACITY;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->caching = (flags & PA_BM_PREFIX_CACHING) != 0;
    bm->refs.assign(num_blocks, 0);
    bm->node_of_block.assign(num_blocks, 0);
    bm->lru_prev.assign(num_blocks, -1);
    bm->lru_next.assign(num_blocks, -1);
    bm->free_list.resize(num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) bm->free_list[i] = (int32_t)(num_blocks - 1 - i);
    bm->host_free.resize(num_host_blocks);
    for (int64_t i = 0; i < num_host_blocks; ++i)
      bm->host_free[i] = (int32_t)(num_host_blocks - 1 - i);
  } catch (...) {
    delete bm;
    return PA_ERR_CAPACITY;
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                       int32_t num_tokens, int32_t* num_cached_tokens) {
  if (!bm) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (bm->caching && num_tokens > 0 && !tokens) return PA_ERR_NULL;
  if (bm->seqs.count(seq_id)) return PA_ERR_SEQUENCE;
  const int32_t bs = bm->block_size;
  const int64_t n_blocks = ((int64_t)num_tokens + bs - 1) / bs;

  // Everything that allocates happens before any state changes, so that an
  // allocation failure leaves the manager as it was.
  std::vector<int64_t> hit_nodes;
  int64_t revived = 0;  // hits on released cached blocks (they leave the LRU)
  Seq* t = nullptr;
  try {
    Seq s;
    s.len = num_tokens;
    if (bm->caching) s.tokens.assign(tokens, tokens + num_tokens);
    // the cached leading blocks: walk the trie while each prefix has a block
    if (bm->caching) {
      int64_t parent = 0;
      for (int32_t i = 0; i < num_tokens / bs; ++i) {
        auto c = bm->children.find(bm->key_of(parent, s, i));
        if (c == bm->children.end()) break;
        const int32_t b = bm->nodes.find(c->second)->second.block;
        if (b < 0) break;
        hit_nodes.push_back(c->second);
        if (bm->refs[b] == 0) ++revived;
        parent = c->second;
      }
    }
    if (n_blocks - (int64_t)hit_nodes.size() > bm->allocatable() - revived)
      return PA_ERR_CAPACITY;
    s.blocks.reserve(n_blocks);
    s.nodes.reserve(hit_nodes.size());
    t = &bm->seqs.emplace(seq_id, std::move(s)).first->second;
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  for (int64_t id : hit_nodes) {
    Node& nd = bm->nodes.find(id)->second;
    const int32_t b = nd.block;
    if (bm->refs[b] == 0) bm->lru_remove(b);
    ++bm->refs[b];
    ++nd.refs;
    t->blocks.push_back(b);
    t->nodes.push_back(id);
  }
  while ((int64_t)t->blocks.size() < n_blocks) t->blocks.push_back(bm->take_block());
  if (num_cached_tokens) *num_cached_tokens = (int32_t)hit_nodes.size() * bs;
  return PA_OK;
}

int pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens, int32_t n,
                 int64_t* slots, int32_t* copies, int32_t* num_copies) {
  if (!bm || !num_copies) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) {
    *num_copies = 0;
    return PA_OK;
  }
  if (!seq_ids || !slots || !copies || (bm->caching && !tokens)) return PA_ERR_NULL;
  const int32_t bs = bm->block_size;

  // Validate and count the blocks the batch takes (on a copy of the counts),
  // and make room for the new entries, before any state changes.
  std::vector<Seq*> ss;
  try {
    ss.resize(n);
    std::unordered_set<int64_t> seen;
    std::unordered_map<int32_t, int32_t> dropped;  // shared last blocks given up
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end() || !it->second.resident || !seen.insert(seq_ids[i]).second)
        return PA_ERR_SEQUENCE;
      Seq& s = it->second;
      if (s.len == 0x7fffffff) return PA_ERR_SHAPE;
      ss[i] = &s;
      if (s.len % bs == 0) {
        ++need;
      } else {
        const int32_t last = s.blocks.back();
        if (bm->refs[last] - dropped[last] > 1) {
          ++need;
          ++dropped[last];
        }
      }
    }
    if (need > bm->allocatable()) return PA_ERR_CAPACITY;
    for (Seq* s : ss) {
      s->blocks.reserve(s->blocks.size() + 1);
      if (bm->caching) s->tokens.reserve(s->tokens.size() + 1);
    }
  } catch (...) {
    return PA_ERR_CAPACITY;
  }

  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = *ss[i];
    const int32_t pos = s.len;
    if (pos % bs == 0) {
      s.blocks.push_back(bm->take_block());
    } else if (bm->refs[s.blocks.back()] > 1) {  // copy-on-write
      const int32_t src = s.blocks.back();
      const int32_t dst = bm->take_block();
      copies[2 * nc] = src;
      copies[2 * nc + 1] = dst;
      ++nc;
      bm->release_block(src);
      s.blocks.back() = dst;
    }
    slots[i] = (int64_t)s.blocks[pos / bs] * bs + pos % bs;
    if (bm->caching) s.tokens.push_back(tokens[i]);
    s.len = pos + 1;
  }
  *num_copies = nc;
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || !it->second.resident || bm->seqs.count(child))
    return PA_ERR_SEQUENCE;
  Seq c;
  try {
    c = it->second;
    bm->seqs.emplace(child, c);
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  for (int32_t b : c.blocks) ++bm->refs[b];
  for (int64_t id : c.nodes) ++bm->nodes.find(id)->second.refs;
  return PA_OK;
}

int pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  Seq& s = it->second;
  if (s.resident) {
    bm->release_device(s);
  } else {
    for (auto h = s.host_blocks.rbegin(); h != s.host_blocks.rend(); ++h)
      bm->host_free.push_back(*h);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_mark_computed(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || !it->second.resident) return PA_ERR_SEQUENCE;
  if (!bm->caching) return PA_OK;
  Seq& s = it->second;
  const int32_t full = s.len / bm->block_size;
  try {
    s.nodes.reserve(full);
    for (int32_t i = (int32_t)s.nodes.size(); i < full; ++i) {
      const int64_t parent = i ? s.nodes[i - 1] : 0;
      NodeKey key = bm->key_of(parent, s, i);
      auto c = bm->children.find(key);
      int64_t id;
      if (c == bm->children.end()) {
        id = bm->next_node;
        Node fresh;
        fresh.key = key;
        bm->nodes.emplace(id, std::move(fresh));
        try {
          bm->children.emplace(std::move(key), id);
        } catch (...) {
          bm->nodes.erase(id);
          throw;
        }
        ++bm->next_node;
        if (parent) ++bm->nodes.find(parent)->second.refs;  // the child's reference
      } else {
        id = c->second;
      }
      Node& nd = bm->nodes.find(id)->second;
      const int32_t b = s.blocks[i];
      if (nd.block < 0 && bm->node_of_block[b] == 0) {  // this prefix gets its block
        nd.block = b;
        bm->node_of_block[b] = id;
        ++nd.refs;
      }
      ++nd.refs;  // this sequence's reference
      s.nodes.push_back(id);
    }
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  return PA_OK;
}

int pa_bm_slots(const pa_block_manager* bm, int64_t seq_id, int32_t start, int32_t n,
                int64_t* slots) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || !it->second.resident) return PA_ERR_SEQUENCE;
  const Seq& s = it->second;
  if (start < 0 || n < 0 || (int64_t)start + n > s.len) return PA_ERR_SHAPE;
  if (n > 0 && !slots) return PA_ERR_NULL;
  const int32_t bs = bm->block_size;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pos = start + i;
    slots[i] = (int64_t)s.blocks[pos / bs] * bs + pos % bs;
  }
  return PA_OK;
}

int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                       int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0 || max_blocks_per_seq < 1) return PA_ERR_SHAPE;
  if (n > 0 && (!seq_ids || !block_tables || !context_lens)) return PA_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || !it->second.resident) return PA_ERR_SEQUENCE;
    if ((int64_t)it->second.blocks.size() > max_blocks_per_seq) return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    const int32_t nb = (int32_t)s.blocks.size();
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + nb, row + max_blocks_per_seq, -1);
    context_lens[i] = s.len;
  }
  return PA_OK;
}

int pa_bm_swap_out(pa_block_manager* bm, int64_t seq_id, int32_t* pairs, int32_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || !it->second.resident) return PA_ERR_SEQUENCE;
  Seq& s = it->second;
  const int32_t nb = (int32_t)s.blocks.size();
  if (nb > 0 && !pairs) return PA_ERR_NULL;
  if ((int64_t)nb > (int64_t)bm->host_free.size()) return PA_ERR_CAPACITY;
  try {
    s.host_blocks.reserve(nb);
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t h = bm->host_free.back();
    bm->host_free.pop_back();
    pairs[2 * j] = s.blocks[j];
    pairs[2 * j + 1] = h;
    s.host_blocks.push_back(h);
  }
  bm->release_device(s);
  s.resident = false;
  *num_pairs = nb;
  return PA_OK;
}

int pa_bm_swap_in(pa_block_manager* bm, int64_t seq_id, int32_t* pairs, int32_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || it->second.resident) return PA_ERR_SEQUENCE;
  Seq& s = it->second;
  const int32_t nb = (int32_t)s.host_blocks.size();
  if (nb > 0 && !pairs) return PA_ERR_NULL;
  if (nb > bm->allocatable()) return PA_ERR_CAPACITY;
  try {
    s.blocks.reserve(nb);
  } catch (...) {
    return PA_ERR_CAPACITY;
  }
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t b = bm->take_block();
    pairs[2 * j] = s.host_blocks[j];
    pairs[2 * j + 1] = b;
    s.blocks.push_back(b);
  }
  for (auto h = s.host_blocks.rbegin(); h != s.host_blocks.rend(); ++h)
    bm->host_free.push_back(*h);
  s.host_blocks.clear();
  s.resident = true;
  *num_pairs = nb;
  return PA_OK;
}

int pa_bm_num_free_blocks(const pa_block_manager* bm, int64_t* num_free) {
  if (!bm || !num_free) return PA_ERR_NULL;
  *num_free = bm->allocatable();
  return PA_OK;
}

int pa_bm_num_free_host_blocks(const pa_block_manager* bm, int64_t* num_free) {
  if (!bm || !num_free) return PA_ERR_NULL;
  *num_free = (int64_t)bm->host_free.size();
  return PA_OK;
}

int pa_bm_seq_info(const pa_block_manager* bm, int64_t seq_id, int32_t* length,
                   int32_t* resident) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  if (length) *length = it->second.len;
  if (resident) *resident = it->second.resident ? 1 : 0;
  return PA_OK;
}

int pa_bm_ref_count(const pa_block_manager* bm, int32_t block, int32_t* refs) {
  if (!bm || !refs) return PA_ERR_NULL;
  if (block < 0 || block >= bm->num_blocks) return PA_ERR_SHAPE;
  *refs = bm->refs[block];
  return PA_OK;
}

}  // extern "C"
