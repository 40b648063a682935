// Host-side manager of the paged KV cache: which pages of the pool hold which
// user's history, with least-recently-used eviction when the pool runs out.
//
// The pages describe the cache as a paged table on the GPU with lookup,
// allocate, append and evict operations, and reuse of a user's cached prefix
// across requests (page "recomendador-generativo-hstu-dynamo-triton",
// section "Como o recomendador generativo HSTU reutiliza o histórico"; "Deploying
// an HSTU Generative Recommender with NVIDIA Dynamo-Triton", section
// "Technical Stack and Performance Gains"). This file is the bookkeeping half:
// the K/V/timestamp bytes live in the device page pools that hstu_kv_append
// writes and the cached attention reads; here only page ids move.
//
// State: a user (64-bit id) owns a slot = one row of the page table, its
// cached length and the ordered list of its pages (a prefix of the row: the
// committed pages, then those of a reservation not yet committed). Free pages
// form a stack.
// Every lookup, and every user of a reserve in batch order, stamps the slot
// with the next value of a logical clock; eviction takes the smallest stamp
// among users not pinned by the current request.
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/hstu.h"

struct hstu_page_manager {
  int32_t num_pages, max_pages, max_users, page_size;
  std::vector<int32_t> table;      // [max_users, max_pages], -1 = none
  std::vector<int32_t> len;        // cached tokens per slot
  std::vector<int64_t> owner;      // user id per slot (valid when used)
  std::vector<uint8_t> used;
  std::vector<uint64_t> stamp;     // last use, logical clock
  std::vector<int32_t> free_pages; // stack
  std::vector<int32_t> free_slots; // stack
  std::unordered_map<int64_t, int32_t> slot_of;
  uint64_t clock = 0;
  int64_t evictions = 0;
  std::mutex mu;
};

namespace {

int32_t pages_for(const hstu_page_manager* m, int64_t tokens) {
  return (int32_t)((tokens + m->page_size - 1) / m->page_size);
}

void release_slot(hstu_page_manager* m, int32_t s) {
  int32_t* row = m->table.data() + (size_t)s * m->max_pages;
  for (int32_t i = 0; i < m->max_pages; ++i) {
    if (row[i] >= 0) m->free_pages.push_back(row[i]);
    row[i] = -1;
  }
  m->slot_of.erase(m->owner[s]);
  m->used[s] = 0;
  m->len[s] = 0;
  m->free_slots.push_back(s);
  ++m->evictions;
}

// least recently used slot not pinned; -1 if none
int32_t lru_victim(const hstu_page_manager* m, const std::vector<uint8_t>& pinned) {
  int32_t best = -1;
  for (int32_t s = 0; s < m->max_users; ++s)
    if (m->used[s] && !pinned[s] && (best < 0 || m->stamp[s] < m->stamp[best])) best = s;
  return best;
}

}  // namespace

extern "C" {

hstu_page_manager_t* hstu_pm_create(int32_t num_pages, int32_t max_pages_per_seq, int32_t max_users) {
  if (num_pages < 1 || max_pages_per_seq < 1 || max_users < 1) return nullptr;
  hstu_page_manager* m = new (std::nothrow) hstu_page_manager();
  if (!m) return nullptr;
  m->num_pages = num_pages;
  m->max_pages = max_pages_per_seq;
  m->max_users = max_users;
  m->page_size = 64;
  m->table.assign((size_t)max_users * max_pages_per_seq, -1);
  m->len.assign(max_users, 0);
  m->owner.assign(max_users, 0);
  m->used.assign(max_users, 0);
  m->stamp.assign(max_users, 0);
  for (int32_t p = num_pages - 1; p >= 0; --p) m->free_pages.push_back(p);  // page 0 handed out first
  for (int32_t s = max_users - 1; s >= 0; --s) m->free_slots.push_back(s);
  return m;
}

void hstu_pm_destroy(hstu_page_manager_t* m) { delete m; }

hstu_status_t hstu_pm_reserve(hstu_page_manager_t* m, int32_t batch, const int64_t* user_ids, const int32_t* n_new,
                              int32_t* cache_lens, int32_t* page_table, int32_t* evicted) {
  if (!m || batch < 0) return HSTU_ERR_INVALID_ARG;
  if (batch > 0 && (!user_ids || !n_new || !cache_lens || !page_table)) return HSTU_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(m->mu);
  const int64_t ev0 = m->evictions;
  // checks first: a request that cannot fit changes nothing
  std::vector<int32_t> slot(batch, -1);
  std::vector<uint8_t> pinned(m->max_users, 0);  // the batch's resident users are never evicted
  std::unordered_map<int64_t, int32_t> seen;
  int64_t need_new_slots = 0, pinned_slots = 0, want_pages = 0, need_pages = 0;
  for (int32_t i = 0; i < batch; ++i) {
    if (n_new[i] < 0) return HSTU_ERR_INVALID_ARG;
    if (!seen.emplace(user_ids[i], i).second) return HSTU_ERR_INVALID_ARG;  // one entry per user
    auto f = m->slot_of.find(user_ids[i]);
    const int64_t have = f == m->slot_of.end() ? 0 : m->len[f->second];
    const int32_t want = pages_for(m, have + n_new[i]);
    if (want > m->max_pages) return HSTU_ERR_UNSUPPORTED;  // history too long
    want_pages += want;
    if (f == m->slot_of.end()) {
      ++need_new_slots;
      need_pages += want;
    } else {
      slot[i] = f->second;
      pinned[f->second] = 1;
      ++pinned_slots;
      // pages of an earlier reservation that was never committed are reused
      const int32_t* row = m->table.data() + (size_t)f->second * m->max_pages;
      for (int32_t pg = 0; pg < want; ++pg) need_pages += row[pg] < 0;
    }
  }
  // after the request the batch's users hold exactly want_pages pages; every
  // other user can be evicted
  if (need_new_slots > m->max_users - pinned_slots || want_pages > m->num_pages) return HSTU_ERR_WORKSPACE;
  // from here on the request succeeds. Pages a resident user holds beyond its
  // new page count (a larger reservation that was never committed) go back to
  // the pool first.
  for (int32_t i = 0; i < batch; ++i) {
    if (slot[i] < 0) continue;
    int32_t* row = m->table.data() + (size_t)slot[i] * m->max_pages;
    for (int32_t pg = pages_for(m, (int64_t)m->len[slot[i]] + n_new[i]); pg < m->max_pages; ++pg) {
      if (row[pg] >= 0) m->free_pages.push_back(row[pg]);
      row[pg] = -1;
    }
  }
  // evict unpinned users, least recently used first, until the free slots
  // and pages cover the request
  while ((int64_t)m->free_slots.size() < need_new_slots || (int64_t)m->free_pages.size() < need_pages) {
    const int32_t v = lru_victim(m, pinned);
    if (v < 0) return HSTU_ERR_WORKSPACE;  // unreachable after the check above
    release_slot(m, v);
  }
  // assign slots and pages; the request's users count as used in batch order
  for (int32_t i = 0; i < batch; ++i) {
    int32_t s = slot[i];
    if (s < 0) {
      s = m->free_slots.back();
      m->free_slots.pop_back();
      m->used[s] = 1;
      m->owner[s] = user_ids[i];
      m->len[s] = 0;
      m->slot_of[user_ids[i]] = s;
      slot[i] = s;
    }
    m->stamp[s] = ++m->clock;
    int32_t* row = m->table.data() + (size_t)s * m->max_pages;
    const int32_t want = pages_for(m, (int64_t)m->len[s] + n_new[i]);
    for (int32_t pg = 0; pg < want; ++pg) {
      if (row[pg] >= 0) continue;  // committed, or reserved earlier and not committed
      row[pg] = m->free_pages.back();
      m->free_pages.pop_back();
    }
    cache_lens[i] = m->len[s];
    std::memcpy(page_table + (size_t)i * m->max_pages, row, sizeof(int32_t) * m->max_pages);
  }
  if (evicted) *evicted = (int32_t)(m->evictions - ev0);
  return HSTU_OK;
}

hstu_status_t hstu_pm_commit(hstu_page_manager_t* m, int32_t batch, const int64_t* user_ids, const int32_t* n_new) {
  if (!m || batch < 0 || (batch > 0 && (!user_ids || !n_new))) return HSTU_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(m->mu);
  std::unordered_set<int64_t> seen;
  for (int32_t i = 0; i < batch; ++i) {
    if (!seen.insert(user_ids[i]).second) return HSTU_ERR_INVALID_ARG;  // one entry per user
    auto f = m->slot_of.find(user_ids[i]);
    if (f == m->slot_of.end() || n_new[i] < 0) return HSTU_ERR_INVALID_ARG;
    const int32_t s = f->second;
    const int64_t after = (int64_t)m->len[s] + n_new[i];
    if (pages_for(m, after) > m->max_pages) return HSTU_ERR_INVALID_ARG;
    const int32_t* row = m->table.data() + (size_t)s * m->max_pages;
    for (int32_t pg = 0; pg < pages_for(m, after); ++pg)
      if (row[pg] < 0) return HSTU_ERR_INVALID_ARG;  // not reserved
  }
  for (int32_t i = 0; i < batch; ++i) m->len[m->slot_of[user_ids[i]]] += n_new[i];
  return HSTU_OK;
}

int32_t hstu_pm_lookup(hstu_page_manager_t* m, int64_t user_id) {
  if (!m) return -1;
  std::lock_guard<std::mutex> lock(m->mu);
  auto f = m->slot_of.find(user_id);
  if (f == m->slot_of.end()) return -1;
  m->stamp[f->second] = ++m->clock;
  return m->len[f->second];
}

hstu_status_t hstu_pm_evict(hstu_page_manager_t* m, int64_t user_id) {
  if (!m) return HSTU_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(m->mu);
  auto f = m->slot_of.find(user_id);
  if (f == m->slot_of.end()) return HSTU_ERR_INVALID_ARG;
  release_slot(m, f->second);
  return HSTU_OK;
}

hstu_status_t hstu_pm_stats(hstu_page_manager_t* m, int32_t* free_pages, int32_t* users, int64_t* evictions) {
  if (!m) return HSTU_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(m->mu);
  if (free_pages) *free_pages = (int32_t)m->free_pages.size();
  if (users) *users = (int32_t)m->slot_of.size();
  if (evictions) *evictions = m->evictions;
  return HSTU_OK;
}

}  // extern "C"
