// Host block manager: physical KV-cache blocks with reference counts, per-
// sequence block tables, prefix sharing with copy on write (page
// "Nano-vLLM-Ascend", section 2.1, Block / BlockTable; page "vLLM-Ascend ...",
// section 4, block sharing for long contexts).  Plain C++; every public call
// takes the manager's mutex and changes nothing when it fails.
#include <cstdint>
#include <deque>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_internal.h"

using pa::fail;
using pa::ok;

struct pa_block_manager {
  int64_t num_blocks;
  int block_size;
  std::vector<int32_t> free_stack;  // top = back(): the next block handed out
  std::vector<int32_t> refs;        // reference count per physical block
  struct Seq {
    int64_t tokens = 0;
    std::vector<int32_t> blocks;  // logical block j -> physical block
  };
  std::unordered_map<int64_t, Seq> seqs;
  std::deque<std::pair<int64_t, int64_t>> copies;  // queued copy-on-write pairs
  std::mutex mu;

  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }

  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refs[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refs[b] == 0) free_stack.push_back(b);
  }
};

namespace {

bool bad_count(int64_t n) { return n < 0; }

// Blocks `append` of n tokens needs from the pool, copy on write included.
int64_t append_need(const pa_block_manager& m, const pa_block_manager::Seq& s, int64_t n) {
  if (n == 0) return 0;
  int64_t need = m.blocks_for(s.tokens + n) - (int64_t)s.blocks.size();
  if (s.tokens % m.block_size != 0 && m.refs[s.blocks.back()] > 1) need += 1;
  return need;
}

}  // namespace

extern "C" {

int pa_bm_create(int64_t num_blocks, int block_size, pa_block_manager** out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "pa_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || num_blocks > INT32_MAX || block_size < 1)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks %lld or block_size %d out of range",
                (long long)num_blocks, block_size);
  pa_block_manager* m = new (std::nothrow) pa_block_manager();
  if (!m) return fail(PA_ERR_INVALID_ARG, "pa_bm_create: out of host memory");
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->refs.assign((size_t)num_blocks, 0);
  m->free_stack.resize((size_t)num_blocks);
  for (int64_t i = 0; i < num_blocks; ++i) m->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
  *out = m;
  return ok();
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add(pa_block_manager* bm, int64_t seq, int64_t num_tokens, int64_t* slots) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_add: manager is NULL");
  if (bad_count(num_tokens) || (num_tokens > 0 && !slots))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_add: bad token count or NULL slots");
  std::lock_guard<std::mutex> lk(bm->mu);
  if (bm->seqs.count(seq)) return fail(PA_ERR_INVALID_ARG, "pa_bm_add: sequence %lld exists", (long long)seq);
  const int64_t need = bm->blocks_for(num_tokens);
  if (need > (int64_t)bm->free_stack.size())
    return fail(PA_ERR_NO_BLOCKS, "pa_bm_add: %lld blocks needed, %zu free", (long long)need,
                bm->free_stack.size());
  pa_block_manager::Seq s;
  s.tokens = num_tokens;
  s.blocks.reserve((size_t)need);
  for (int64_t j = 0; j < need; ++j) s.blocks.push_back(bm->take());
  for (int64_t t = 0; t < num_tokens; ++t)
    slots[t] = (int64_t)s.blocks[(size_t)(t / bm->block_size)] * bm->block_size + t % bm->block_size;
  bm->seqs.emplace(seq, std::move(s));
  return ok();
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child, int64_t num_tokens) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: manager is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: unknown parent %lld", (long long)parent);
  if (bm->seqs.count(child)) return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: sequence %lld exists", (long long)child);
  if (num_tokens < 0 || num_tokens > it->second.tokens)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: %lld tokens of a %lld-token parent",
                (long long)num_tokens, (long long)it->second.tokens);
  pa_block_manager::Seq s;
  s.tokens = num_tokens;
  const int64_t nb = bm->blocks_for(num_tokens);
  s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + nb);
  for (int32_t b : s.blocks) ++bm->refs[b];
  bm->seqs.emplace(child, std::move(s));
  return ok();
}

int pa_bm_append(pa_block_manager* bm, int64_t seq, int64_t n, int64_t* slots) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_append: manager is NULL");
  if (bad_count(n) || (n > 0 && !slots))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_append: bad token count or NULL slots");
  std::lock_guard<std::mutex> lk(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID_ARG, "pa_bm_append: unknown sequence %lld", (long long)seq);
  pa_block_manager::Seq& s = it->second;
  const int64_t need = append_need(*bm, s, n);
  if (need > (int64_t)bm->free_stack.size())
    return fail(PA_ERR_NO_BLOCKS, "pa_bm_append: %lld blocks needed, %zu free", (long long)need,
                bm->free_stack.size());
  if (n == 0) return ok();
  const int bs = bm->block_size;
  if (s.tokens % bs != 0 && bm->refs[s.blocks.back()] > 1) {  // copy on write
    const int32_t shared = s.blocks.back();
    const int32_t mine = bm->take();
    bm->release(shared);
    s.blocks.back() = mine;
    bm->copies.emplace_back(shared, mine);
  }
  for (int64_t k = 0; k < n; ++k) {
    const int64_t t = s.tokens + k;
    if (t / bs == (int64_t)s.blocks.size()) s.blocks.push_back(bm->take());
    slots[k] = (int64_t)s.blocks[(size_t)(t / bs)] * bs + t % bs;
  }
  s.tokens += n;
  return ok();
}

int pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_free: manager is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID_ARG, "pa_bm_free: unknown sequence %lld", (long long)seq);
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return ok();
}

int pa_bm_tables(pa_block_manager* bm, const int64_t* seqs, int num_seqs, int max_blocks_per_seq,
                 int32_t* block_tables, int32_t* context_lens) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_tables: manager is NULL");
  if (num_seqs < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_tables: negative size");
  if (num_seqs == 0) return ok();
  if (!seqs || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_tables: NULL array");
  std::lock_guard<std::mutex> lk(bm->mu);
  for (int i = 0; i < num_seqs; ++i) {  // validate everything before writing
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_INVALID_ARG, "pa_bm_tables: unknown sequence %lld", (long long)seqs[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_tables: sequence %lld holds %zu blocks > %d",
                  (long long)seqs[i], it->second.blocks.size(), max_blocks_per_seq);
    if (it->second.tokens > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_tables: sequence %lld too long", (long long)seqs[i]);
  }
  for (int i = 0; i < num_seqs; ++i) {
    const pa_block_manager::Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    for (int j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int)s.blocks.size() ? s.blocks[(size_t)j] : -1;
    context_lens[i] = (int32_t)s.tokens;
  }
  return ok();
}

int64_t pa_bm_take_copies(pa_block_manager* bm, int64_t* src, int64_t* dst, int64_t capacity) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_take_copies: manager is NULL");
  if (capacity < 0 || (capacity > 0 && (!src || !dst)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_take_copies: bad capacity or NULL array");
  std::lock_guard<std::mutex> lk(bm->mu);
  int64_t k = 0;
  while (k < capacity && !bm->copies.empty()) {
    src[k] = bm->copies.front().first;
    dst[k] = bm->copies.front().second;
    bm->copies.pop_front();
    ++k;
  }
  ok();
  return k;
}

int64_t pa_bm_num_free(pa_block_manager* bm) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_num_free: manager is NULL");
  std::lock_guard<std::mutex> lk(bm->mu);
  return (int64_t)bm->free_stack.size();
}

int64_t pa_bm_num_tokens(pa_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lk(bm->mu);
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.tokens;
}

int pa_bm_ref_count(pa_block_manager* bm, int64_t block) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lk(bm->mu);
  return block < 0 || block >= bm->num_blocks ? -1 : bm->refs[(size_t)block];
}

int64_t pa_bm_num_seqs(pa_block_manager* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lk(bm->mu);
  return (int64_t)bm->seqs.size();
}

}  // extern "C"
