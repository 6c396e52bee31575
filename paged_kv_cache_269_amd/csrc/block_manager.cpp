// Host KV-cache block manager: the allocator the decode path's block tables
// come from.  Declarations and the meaning of every argument:
// include/pagedattn_blocks.h.
//
// Rules (vLLM manual (doramagic.ai), "KVCacheManager -- cache block
// management", "sharing mechanism", "cache allocation strategy"): free
// blocks in a deque, taken from the front ceil(tokens / block_size) at a time
// and returned to the back; shared blocks carry a reference count and return
// only when it reaches zero; a request that grows past its last block gets
// one more from the front.  An allocation that does not fit fails before it
// takes anything.
#include "pagedattn.h"
#include "pagedattn_blocks.h"

#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

struct pa_block_manager {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_blocks;
  std::vector<int32_t> refcount;
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  bool take(int64_t n, std::vector<int32_t>& out) {
    if (n > (int64_t)free_blocks.size()) return false;
    for (int64_t i = 0; i < n; ++i) {
      const int32_t b = free_blocks.front();
      free_blocks.pop_front();
      refcount[b] = 1;
      out.push_back(b);
    }
    return true;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return nullptr;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->refcount.assign((size_t)num_blocks, 0);
    for (int64_t b = 0; b < num_blocks; ++b) m->free_blocks.push_back((int32_t)b);
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int pa_bm_allocate(pa_block_manager* m, int64_t request_id, int64_t num_tokens) {
  if (!m) return PA_ERR_NULL;
  if (num_tokens < 0 || m->seqs.count(request_id)) return PA_ERR_RANGE;
  const int64_t need = (num_tokens + m->block_size - 1) / m->block_size;
  if (need > (int64_t)m->free_blocks.size()) return PA_ERR_EXHAUSTED;
  try {
    pa_block_manager::Seq s;
    s.len = num_tokens;
    m->take(need, s.blocks);
    m->seqs.emplace(request_id, std::move(s));
  } catch (...) {
    return PA_ERR_EXHAUSTED;
  }
  return PA_OK;
}

int pa_bm_share(pa_block_manager* m, int64_t src_id, int64_t dst_id, int64_t num_blocks) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(src_id);
  if (it == m->seqs.end() || m->seqs.count(dst_id) || num_blocks < 0 ||
      num_blocks * m->block_size > it->second.len)
    return PA_ERR_RANGE;
  try {
    pa_block_manager::Seq s;
    s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + num_blocks);
    s.len = num_blocks * m->block_size;
    for (int32_t b : s.blocks) ++m->refcount[b];
    m->seqs.emplace(dst_id, std::move(s));
  } catch (...) {
    return PA_ERR_EXHAUSTED;
  }
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* m, int64_t src_id, int64_t dst_id) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(src_id);
  if (it == m->seqs.end() || m->seqs.count(dst_id)) return PA_ERR_RANGE;
  try {
    pa_block_manager::Seq s = it->second;
    for (int32_t b : s.blocks) ++m->refcount[b];
    m->seqs.emplace(dst_id, std::move(s));
  } catch (...) {
    return PA_ERR_EXHAUSTED;
  }
  return PA_OK;
}

namespace {

// Blocks one append to `s` takes: a new block at a block boundary, or a
// private copy of a last block that other requests still map (`extra_refs`
// of those references already given up earlier in the same batch).
int blocks_needed(const pa_block_manager* m, const pa_block_manager::Seq& s, int extra_refs) {
  if (s.len % m->block_size == 0) return 1;
  return m->refcount[s.blocks.back()] - extra_refs > 1 ? 1 : 0;
}

int append_one(pa_block_manager* m, pa_block_manager::Seq& s, int64_t* slot, int32_t* copy_pair) {
  copy_pair[0] = copy_pair[1] = -1;
  try {
    if (s.len % m->block_size == 0) {
      if (!m->take(1, s.blocks)) return PA_ERR_EXHAUSTED;
    } else if (m->refcount[s.blocks.back()] > 1) {
      // copy-on-write: the token would land in a block other requests map
      std::vector<int32_t> fresh;
      if (!m->take(1, fresh)) return PA_ERR_EXHAUSTED;
      const int32_t old = s.blocks.back();
      --m->refcount[old];
      s.blocks.back() = fresh[0];
      copy_pair[0] = old;
      copy_pair[1] = fresh[0];
    }
  } catch (...) {
    return PA_ERR_EXHAUSTED;
  }
  const int64_t t = s.len++;
  *slot = (int64_t)s.blocks[t / m->block_size] * m->block_size + t % m->block_size;
  return PA_OK;
}

}  // namespace

int pa_bm_append(pa_block_manager* m, int64_t request_id, int64_t* slot, int32_t* copy_pair) {
  if (!m || !slot || !copy_pair) return PA_ERR_NULL;
  auto it = m->seqs.find(request_id);
  if (it == m->seqs.end()) return PA_ERR_RANGE;
  return append_one(m, it->second, slot, copy_pair);
}

int pa_bm_append_batch(pa_block_manager* m, const int64_t* request_ids, int32_t n,
                       int64_t* slots, int32_t* copy_pairs, int32_t* num_copies) {
  if (!m) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (!num_copies) return PA_ERR_NULL;
  *num_copies = 0;
  if (n == 0) return PA_OK;
  if (!request_ids || !slots || !copy_pairs) return PA_ERR_NULL;
  // Check everything first -- known, distinct ids and enough free blocks,
  // the copies included, in batch order -- then no append fails half-way.
  int64_t need = 0;
  try {
    std::unordered_map<int64_t, int> seen;
    std::unordered_map<int32_t, int> given_up;  // references dropped by earlier copies
    seen.reserve((size_t)n * 2);
    for (int32_t i = 0; i < n; ++i) {
      auto it = m->seqs.find(request_ids[i]);
      if (it == m->seqs.end() || !seen.emplace(request_ids[i], 1).second) return PA_ERR_RANGE;
      const pa_block_manager::Seq& s = it->second;
      const int32_t last = s.blocks.empty() ? -1 : s.blocks.back();
      const int extra = last >= 0 && given_up.count(last) ? given_up[last] : 0;
      const int k = blocks_needed(m, s, extra);
      need += k;
      if (k && s.len % m->block_size != 0) ++given_up[last];
    }
  } catch (...) {
    return PA_ERR_EXHAUSTED;
  }
  if (need > (int64_t)m->free_blocks.size()) return PA_ERR_EXHAUSTED;
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t pair[2];
    const int rc = append_one(m, m->seqs.find(request_ids[i])->second, &slots[i], pair);
    if (rc != PA_OK) return rc;  // not reached: checked above
    if (pair[0] >= 0) {
      copy_pairs[2 * nc] = pair[0];
      copy_pairs[2 * nc + 1] = pair[1];
      ++nc;
    }
  }
  *num_copies = nc;
  return PA_OK;
}

int pa_bm_free(pa_block_manager* m, int64_t request_id) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(request_id);
  if (it == m->seqs.end()) return PA_OK;
  for (int32_t b : it->second.blocks)
    if (--m->refcount[b] == 0) m->free_blocks.push_back(b);
  m->seqs.erase(it);
  return PA_OK;
}

int64_t pa_bm_num_free(const pa_block_manager* m) {
  return m ? (int64_t)m->free_blocks.size() : -1;
}

int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t request_id) {
  if (!m) return -1;
  auto it = m->seqs.find(request_id);
  return it == m->seqs.end() ? -1 : it->second.len;
}

int pa_bm_block_tables(const pa_block_manager* m, const int64_t* request_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t pad, int32_t* block_tables,
                       int32_t* context_lens) {
  if (!m) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!request_ids || !block_tables || !context_lens) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = m->seqs.find(request_ids[i]);
    if (it == m->seqs.end() || (int64_t)it->second.blocks.size() > max_blocks_per_seq ||
        it->second.len > INT32_MAX)
      return PA_ERR_RANGE;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pa_block_manager::Seq& s = m->seqs.find(request_ids[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    const int32_t n = (int32_t)s.blocks.size();
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < n ? s.blocks[j] : pad;
    context_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

int pa_bm_free_blocks(const pa_block_manager* m, int32_t* out, int64_t capacity) {
  if (!m) return PA_ERR_NULL;
  if (capacity < (int64_t)m->free_blocks.size()) return PA_ERR_SHAPE;
  if (!out && !m->free_blocks.empty()) return PA_ERR_NULL;
  int64_t i = 0;
  for (int32_t b : m->free_blocks) out[i++] = b;
  return PA_OK;
}

}  // extern "C"
