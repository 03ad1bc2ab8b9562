// scheduler.cpp -- host-side block allocator and continuous-batching
// scheduler: the control plane that produces the block tables, lengths and
// query counts the kernels consume.
//
// The nano-vLLM guide announcement names both pieces: ch. 4 "PagedAttention"
// (a block allocator hands out fixed-size KV pages as sequences grow, so a
// sequence never holds more than one partly filled page, where reserving each
// request's maximum up front lets fragmentation waste 60-80% of the memory)
// and ch. 5 "The Scheduler" (continuous batching: requests join and leave the
// running batch at every step instead of waiting for a whole batch to
// finish).  The paper-digest page lists continuous batching among tiny-vLLM's
// core mechanics.  The pages print no algorithm for either, so this file
// takes the plain reading:
//
//  * Allocator: a LIFO free list of physical block ids.  A sequence owns the
//    blocks of its table in logical order and gets a new one only when its
//    next token would not fit.
//  * Step: every running sequence first, oldest first (one token for a
//    sequence that is decoding, the next chunk for one still in prefill),
//    then waiting requests in arrival order while the batch, the step's token
//    budget and the free blocks allow.  Prompts longer than the remaining
//    budget are processed in chunks over several steps (each chunk attends
//    to the sequence's cached tokens, the prefill kernel's history case).
//  * Preemption by recomputation: when a running sequence needs a block and
//    none is free, the most recently arrived running sequence that is not yet
//    in this step's batch gives up all its blocks and goes back to the
//    waiting queue; when it is admitted again it recomputes its prompt and
//    the tokens it had generated.  A waiting request never preempts, and a
//    step that preempted admits no waiting request.
//  * Static batching (for comparison): a new batch is admitted only when the
//    previous one has finished completely.
//  * Sharing (guide ch. 7 "Prefix Caching"): a block may sit in several
//    tables and carries a count of them; it returns to the free list when
//    the last one lets go.  A request may name a live sequence whose first
//    prefix_len tokens (whole blocks) equal its own: when it is admitted it
//    takes those blocks instead of computing them.  A fork starts a new
//    sequence from a decoding one with all of its blocks shared (several
//    samples of one prompt).  Copy on write: before a sequence stores a token
//    into a block that another table also holds, it gets a fresh block and
//    the step lists a (source, destination) block copy, to run before the
//    step's appends.
//
// A step is planned and the sequences advance as if it ran: after its chunk
// a sequence that has caught up with its length samples one more token, and
// one that reaches its token limit finishes; its blocks return to the free
// list after the whole step is planned, so no block is handed to two
// sequences within one step.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

struct pkv_scheduler {
  struct Seq {
    int64_t id = 0;
    int64_t arrival = 0;
    int64_t prefix_owner = -1;  // live sequence to share the first prefix_len tokens with
    int32_t prefix_len = 0;
    int32_t prompt_len = 0, max_new = 0;
    int32_t generated = 0;  // tokens sampled so far
    int32_t computed = 0;   // tokens whose K/V are in the cache
    std::vector<int32_t> blocks;
    int32_t length() const { return prompt_len + generated; }
  };

  int32_t num_blocks, block_size, max_blocks_per_seq, max_batch, max_step_tokens;
  bool static_batching;
  int64_t next_arrival = 0;
  std::vector<int32_t> free_list;
  std::vector<int32_t> ref;  // tables holding each block
  std::vector<int32_t> copy_src, copy_dst;  // this step's copies on write
  std::unordered_map<int64_t, Seq> seqs;
  std::deque<int64_t> waiting;   // arrival order
  std::vector<int64_t> running;  // arrival order
  std::vector<int64_t> last_finished, last_preempted;
  int64_t stats[PKV_SCHED_STATS] = {};

  pkv_scheduler(int32_t n, int32_t bs, int32_t maxb, int32_t batch, int32_t tokens, bool st)
      : num_blocks(n), block_size(bs), max_blocks_per_seq(maxb), max_batch(batch),
        max_step_tokens(tokens), static_batching(st) {
    free_list.reserve(n);
    for (int32_t b = n - 1; b >= 0; --b) free_list.push_back(b);  // block 0 handed out first
    ref.assign(n, 0);
  }

  int32_t blocks_for(int32_t tokens) const { return (tokens + block_size - 1) / block_size; }

  void release(Seq& s) {
    for (auto it = s.blocks.rbegin(); it != s.blocks.rend(); ++it)
      if (--ref[*it] == 0) free_list.push_back(*it);
    s.blocks.clear();
    s.computed = 0;
  }

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    return b;
  }

  // The next token goes into a partly filled block that another table holds.
  bool shared_tail(const Seq& s) const {
    if (s.computed % block_size == 0) return false;
    const int32_t j = s.computed / block_size;
    return j < (int32_t)s.blocks.size() && ref[s.blocks[j]] > 1;
  }

  // Make s's table cover `tokens` tokens, with a private copy of a shared
  // tail block first; false (and no change) if the free list is short.
  bool grow(Seq& s, int32_t tokens) {
    const bool cow = shared_tail(s);
    const int32_t need = blocks_for(tokens) - (int32_t)s.blocks.size() + (cow ? 1 : 0);
    if (need <= 0) return true;
    if ((int32_t)free_list.size() < need) return false;
    if (cow) {
      const int32_t j = s.computed / block_size;
      const int32_t fresh = take();
      copy_src.push_back(s.blocks[j]);
      copy_dst.push_back(fresh);
      --ref[s.blocks[j]];
      s.blocks[j] = fresh;
      ++stats[14];
    }
    while ((int32_t)s.blocks.size() < blocks_for(tokens)) s.blocks.push_back(take());
    return true;
  }

  // On admission: take the whole blocks of the prefix this request shares
  // with a live sequence, if that sequence still holds them computed.
  void share_prefix(Seq& q) {
    if (q.prefix_owner < 0 || q.computed != 0 || !q.blocks.empty()) return;
    auto it = seqs.find(q.prefix_owner);
    if (it == seqs.end()) return;
    const Seq& o = it->second;
    const int32_t nb = q.prefix_len / block_size;
    if (o.computed < q.prefix_len || (int32_t)o.blocks.size() < nb) return;
    for (int32_t j = 0; j < nb; ++j) {
      q.blocks.push_back(o.blocks[j]);
      ++ref[o.blocks[j]];
    }
    q.computed = q.prefix_len;
    stats[15] += q.prefix_len;
  }

  void requeue(int64_t id) {
    // keep the waiting queue in arrival order
    const int64_t arr = seqs[id].arrival;
    auto pos = std::find_if(waiting.begin(), waiting.end(),
                            [&](int64_t w) { return seqs[w].arrival > arr; });
    waiting.insert(pos, id);
  }
};

extern "C" {

pkv_scheduler* pkv_sched_create(int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t max_batch,
                                int32_t max_step_tokens, int32_t static_batching) {
  if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || max_batch <= 0 ||
      max_step_tokens <= 0)
    return nullptr;
  return new (std::nothrow) pkv_scheduler(num_blocks, block_size, max_blocks_per_seq, max_batch,
                                          max_step_tokens, static_batching != 0);
}

void pkv_sched_destroy(pkv_scheduler* s) { delete s; }

int pkv_sched_add_request(pkv_scheduler* s, int64_t id, int32_t prompt_len,
                          int32_t max_new_tokens) {
  if (!s || prompt_len <= 0 || max_new_tokens <= 0) return PKV_ERR_INVALID_ARG;
  if (s->seqs.count(id)) return PKV_ERR_INVALID_ARG;
  // the longest the sequence gets: prompt plus every sampled token but the last
  const int64_t longest = (int64_t)prompt_len + max_new_tokens - 1;
  const int64_t blocks = (longest + s->block_size - 1) / s->block_size;
  if (blocks > s->max_blocks_per_seq || blocks > s->num_blocks) return PKV_ERR_UNSUPPORTED;
  pkv_scheduler::Seq q;
  q.id = id;
  q.arrival = s->next_arrival++;
  q.prompt_len = prompt_len;
  q.max_new = max_new_tokens;
  s->seqs.emplace(id, std::move(q));
  s->waiting.push_back(id);
  return PKV_OK;
}

int pkv_sched_add_request_prefix(pkv_scheduler* s, int64_t id, int32_t prompt_len,
                                 int32_t max_new_tokens, int64_t prefix_owner,
                                 int32_t prefix_len) {
  if (!s || prefix_len <= 0 || prefix_len % s->block_size != 0 || prefix_len >= prompt_len ||
      prefix_owner == id)
    return PKV_ERR_INVALID_ARG;
  const int rc = pkv_sched_add_request(s, id, prompt_len, max_new_tokens);
  if (rc != PKV_OK) return rc;
  auto& q = s->seqs[id];
  q.prefix_owner = prefix_owner;
  q.prefix_len = prefix_len;
  return PKV_OK;
}

int pkv_sched_fork(pkv_scheduler* s, int64_t parent_id, int64_t child_id, int32_t extra_tokens) {
  if (!s || extra_tokens <= 0 || s->seqs.count(child_id) || !s->seqs.count(parent_id))
    return PKV_ERR_INVALID_ARG;
  const auto& par = s->seqs[parent_id];
  const bool running =
      std::find(s->running.begin(), s->running.end(), parent_id) != s->running.end();
  // the parent must be decoding: every token but its latest sample cached
  if (!running || par.generated == 0 || par.computed != par.length() - 1)
    return PKV_ERR_INVALID_ARG;
  pkv_scheduler::Seq c;
  c.id = child_id;
  c.arrival = s->next_arrival++;
  c.prompt_len = par.prompt_len;
  c.generated = par.generated;  // same history; its latest sample is its own
  c.max_new = par.generated + extra_tokens;
  const int64_t longest = (int64_t)c.prompt_len + c.max_new - 1;
  if ((longest + s->block_size - 1) / s->block_size > s->max_blocks_per_seq)
    return PKV_ERR_UNSUPPORTED;
  c.computed = par.computed;
  c.blocks = par.blocks;
  for (int32_t b : c.blocks) ++s->ref[b];
  s->seqs.emplace(child_id, std::move(c));
  s->running.push_back(child_id);  // the newest sequence
  return PKV_OK;
}

int32_t pkv_sched_copies(const pkv_scheduler* s, int32_t* src, int32_t* dst, int32_t max_pairs) {
  if (!s) return PKV_ERR_INVALID_ARG;
  const int32_t n = (int32_t)s->copy_src.size();
  for (int32_t k = 0; k < n && k < max_pairs; ++k) {
    if (src) src[k] = s->copy_src[k];
    if (dst) dst[k] = s->copy_dst[k];
  }
  return n;
}

int pkv_sched_step(pkv_scheduler* s, int64_t* seq_ids, int32_t* q_lens, int32_t* context_lens,
                   int32_t* cu_q_lens, int32_t* block_tables) {
  if (!s || !seq_ids || !q_lens || !context_lens || !cu_q_lens || !block_tables)
    return PKV_ERR_INVALID_ARG;
  s->last_finished.clear();
  s->last_preempted.clear();
  s->copy_src.clear();
  s->copy_dst.clear();
  struct Entry {
    int64_t id;
    int32_t q;
  };
  std::vector<Entry> batch;
  int32_t budget = s->max_step_tokens;

  // 1. running sequences, oldest first; preempt from the newest when short
  std::vector<int64_t> kept;
  for (size_t k = 0; k < s->running.size(); ++k) {
    const int64_t id = s->running[k];
    auto& q = s->seqs[id];
    if ((int32_t)batch.size() == s->max_batch || budget == 0) {
      kept.push_back(id);
      continue;
    }
    const int32_t chunk = std::min(q.length() - q.computed, budget);
    bool ok = s->grow(q, q.computed + chunk);
    while (!ok) {
      // newest running sequence not yet scheduled in this step
      const int64_t victim = s->running.back();
      auto& v = s->seqs[victim];
      s->release(v);
      s->running.pop_back();
      s->requeue(victim);
      s->last_preempted.push_back(victim);
      ++s->stats[4];
      if (victim == id) break;  // it gave up its own blocks
      ok = s->grow(q, q.computed + chunk);
    }
    if (!ok) break;  // this sequence was the newest: nothing after it is left
    batch.push_back({id, chunk});
    budget -= chunk;
    kept.push_back(id);
  }
  // running now holds the sequences not preempted, in arrival order
  s->running.erase(std::remove_if(s->running.begin(), s->running.end(),
                                  [&](int64_t id) {
                                    return std::find(kept.begin(), kept.end(), id) == kept.end();
                                  }),
                   s->running.end());

  // 2. waiting requests in arrival order.  Continuous batching admits while
  //    the batch, the budget and the free blocks allow.  Static batching
  //    admits only into an empty running set, up to max_batch requests at
  //    once; those the budget cannot start now start on later steps (as
  //    running sequences), and nothing more is admitted until all finish.
  //    A step that had to preempt admits nothing: memory is short.
  if (!s->last_preempted.empty()) {
    // no admission
  } else if (!s->static_batching) {
    while (!s->waiting.empty() && (int32_t)batch.size() < s->max_batch && budget > 0) {
      const int64_t id = s->waiting.front();
      auto& q = s->seqs[id];
      s->share_prefix(q);
      const int32_t chunk = std::min(q.length() - q.computed, budget);
      if (!s->grow(q, q.computed + chunk)) {
        s->release(q);  // a waiting request holds no blocks
        break;
      }
      s->waiting.pop_front();
      s->running.push_back(id);
      batch.push_back({id, chunk});
      budget -= chunk;
    }
  } else if (s->running.empty()) {
    while (!s->waiting.empty() && (int32_t)s->running.size() < s->max_batch) {
      const int64_t id = s->waiting.front();
      auto& q = s->seqs[id];
      s->share_prefix(q);
      const int32_t chunk = std::min(q.length() - q.computed, budget);
      if (chunk > 0 && !s->grow(q, q.computed + chunk)) {
        s->release(q);  // a waiting request holds no blocks
        break;
      }
      s->waiting.pop_front();
      s->running.push_back(id);
      if (chunk > 0) {
        batch.push_back({id, chunk});
        budget -= chunk;
      }
    }
  }

  // 3. write the batch, then advance every scheduled sequence
  const int32_t B = (int32_t)batch.size();
  cu_q_lens[0] = 0;
  std::vector<int64_t> done;
  for (int32_t b = 0; b < B; ++b) {
    auto& q = s->seqs[batch[b].id];
    q.computed += batch[b].q;
    seq_ids[b] = q.id;
    q_lens[b] = batch[b].q;
    context_lens[b] = q.computed;
    cu_q_lens[b + 1] = cu_q_lens[b] + batch[b].q;
    int32_t* row = block_tables + (int64_t)b * s->max_blocks_per_seq;
    for (int32_t j = 0; j < s->max_blocks_per_seq; ++j)
      row[j] = j < (int32_t)q.blocks.size() ? q.blocks[j] : -1;
    const bool prefill = q.computed - batch[b].q < q.prompt_len;
    s->stats[prefill ? 2 : 3] += batch[b].q;
    if (q.computed == q.length()) {  // caught up: the model samples a token
      if (++q.generated == q.max_new) done.push_back(q.id);
    }
  }
  s->stats[0] += 1;
  s->stats[1] += cu_q_lens[B];
  s->stats[13] += B;
  // memory held during this step, by everything in the running set
  for (int64_t id : s->running) {
    const auto& q = s->seqs[id];
    s->stats[9] += q.computed;
    s->stats[10] += (int64_t)q.blocks.size() * s->block_size;
    s->stats[11] += q.prompt_len + q.max_new - 1;
    s->stats[12] += (int64_t)s->max_blocks_per_seq * s->block_size;
  }
  for (int64_t id : done) {
    auto& q = s->seqs[id];
    s->release(q);
    s->running.erase(std::find(s->running.begin(), s->running.end(), id));
    s->last_finished.push_back(id);
    s->seqs.erase(id);
    ++s->stats[5];
  }
  return B;
}

int32_t pkv_sched_events(const pkv_scheduler* s, int32_t which, int64_t* ids, int32_t max_ids) {
  if (!s) return PKV_ERR_INVALID_ARG;
  const auto& v = which == 0 ? s->last_finished : s->last_preempted;
  if (which != 0 && which != 1) return PKV_ERR_INVALID_ARG;
  const int32_t n = (int32_t)v.size();
  if (ids)
    for (int32_t k = 0; k < n && k < max_ids; ++k) ids[k] = v[k];
  return n;
}

int pkv_sched_stats(const pkv_scheduler* s, int64_t* out) {
  if (!s || !out) return PKV_ERR_INVALID_ARG;
  std::memcpy(out, s->stats, sizeof s->stats);
  out[6] = (int64_t)s->free_list.size();
  out[7] = (int64_t)s->running.size();
  out[8] = (int64_t)s->waiting.size();
  return PKV_OK;
}

}  // extern "C"
