// Host-side prefix-mode choice: for each query, whether the user history or
// the query's items is the cached prefix, and the two cache pools' contents.
//
// The Bat page (sections "The idea" and "Why it works") has a scheduler
// choose, under memory limits, which prefix each query uses so that hot,
// resident caches get reused, with user-prefix and item-prefix caches in
// separate pools.  The page leaves the policy open; this file implements one
// plain reading of it:
//   * score, per query, the prefix tokens that are hot -- resident, or
//     asked for by an earlier query and able to stay resident: user mode =
//     n_u if the user is resident or was asked for before and its blocks fit
//     the user pool; item mode = T per item that is resident or was asked
//     for before while the item pool has slots.  Item mode wins only on a
//     larger score.  The user-as-prefix policy always picks user.
//   * the chosen prefix only is cached: user pool = least recently used
//     eviction by blocks; item pool = lowest unused slot, else replace the
//     resident item (not of this query) with the fewest earlier requests,
//     then least recent use, then lowest id -- only if it was asked for
//     strictly fewer times than the newcomer.
//   * every query then counts once more for its user and each of its items.
// and the attention work the choice implies (computed prefix and suffix
// tokens, query-key pairs of the computed rows).
//
// The choice is sequential (each query sees the pools its predecessors left),
// so it runs on the host.  All state lives in one caller-owned buffer of
// fixed size (no allocation): an intrusive doubly linked LRU list over users
// and an indexed binary min-heap over the resident items keyed by
// (pinned, requests, last use, id).  The items of the query being served are
// pinned -- raised above every other key -- so the heap's top is always the
// eviction victim.  Slots are taken in order and only ever change hands
// (an eviction hands the victim's slot to the newcomer), so the lowest
// unused slot is a counter.  A query costs O(m log C) for m items and C item
// slots.
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "bat.h"

namespace {

struct Header {
  bat_sched_config cfg;
  int64_t queries;        // queries served so far (the query clock)
  int64_t validations;    // stamp of the argument check
  int64_t used_blocks;    // user-pool blocks held
  int32_t lru_head, lru_tail;
  int32_t next_free;      // lowest slot never used
  int32_t heap_size;
  // offsets (bytes from the start of the state) of the arrays, in Array order
  int64_t off[13];
  uint64_t magic;
};

// The state's arrays: per user, per item, per item slot.
enum Array {
  kUserLen, kUserPrev, kUserNext, kUserCount, kUserRes,
  kItemSlot, kItemPos, kItemCount, kItemLast, kItemStamp, kItemPin,
  kSlotItem, kHeap, kNumArrays
};
static_assert(kNumArrays == 13, "one offset per array");

constexpr uint64_t kMagic = 0x6261747363686431ull;  // "batschd1"

inline int64_t align_up(int64_t x) { return (x + 63) & ~int64_t(63); }

struct Layout {
  int64_t off[kNumArrays];
  int64_t total;
};

bool make_layout(const bat_sched_config *c, Layout &L) {
  if (!c || c->num_users < 0 || c->num_items < 0 || c->item_capacity < 0 ||
      c->user_capacity_blocks < 0 || c->item_tokens <= 0 || c->user_block <= 0 ||
      (c->policy != BAT_POLICY_USER_PREFIX && c->policy != BAT_POLICY_HOTNESS))
    return false;
  const int64_t U = c->num_users, N = c->num_items, C = c->item_capacity;
  const int64_t sizes[kNumArrays] = {U * 4, U * 4, U * 4, U * 8, U * 1,           // users
                                     N * 4, N * 4, N * 8, N * 8, N * 8, N * 1,    // items
                                     C * 4, C * 4};                               // slots
  int64_t at = align_up(sizeof(Header));
  for (int i = 0; i < kNumArrays; ++i) {
    L.off[i] = at;
    at = align_up(at + sizes[i]);
  }
  L.total = at;
  return true;
}

struct State {
  Header *h;
  int32_t *user_len, *prev, *next;
  int64_t *ucount;
  uint8_t *ures;
  int32_t *slot, *pos;
  int64_t *icount, *last, *stamp;
  uint8_t *pin;
  int32_t *slot_item, *heap;

  explicit State(void *base) {
    uint8_t *b = static_cast<uint8_t *>(base);
    h = reinterpret_cast<Header *>(b);
    user_len = reinterpret_cast<int32_t *>(b + h->off[kUserLen]);
    prev = reinterpret_cast<int32_t *>(b + h->off[kUserPrev]);
    next = reinterpret_cast<int32_t *>(b + h->off[kUserNext]);
    ucount = reinterpret_cast<int64_t *>(b + h->off[kUserCount]);
    ures = b + h->off[kUserRes];
    slot = reinterpret_cast<int32_t *>(b + h->off[kItemSlot]);
    pos = reinterpret_cast<int32_t *>(b + h->off[kItemPos]);
    icount = reinterpret_cast<int64_t *>(b + h->off[kItemCount]);
    last = reinterpret_cast<int64_t *>(b + h->off[kItemLast]);
    stamp = reinterpret_cast<int64_t *>(b + h->off[kItemStamp]);
    pin = b + h->off[kItemPin];
    slot_item = reinterpret_cast<int32_t *>(b + h->off[kSlotItem]);
    heap = reinterpret_cast<int32_t *>(b + h->off[kHeap]);
  }

  // ---- user pool: LRU list, head = most recent ----
  int64_t blocks(int32_t n) const { return (int64_t(n) + h->cfg.user_block - 1) / h->cfg.user_block; }
  void unlink(int32_t u) {
    const int32_t p = prev[u], n = next[u];
    if (p >= 0) next[p] = n; else h->lru_head = n;
    if (n >= 0) prev[n] = p; else h->lru_tail = p;
  }
  void push_front(int32_t u) {
    prev[u] = -1;
    next[u] = h->lru_head;
    if (h->lru_head >= 0) prev[h->lru_head] = u; else h->lru_tail = u;
    h->lru_head = u;
  }

  // ---- item pool: indexed min-heap of resident items ----
  bool less(int32_t a, int32_t b) const {
    if (pin[a] != pin[b]) return pin[a] < pin[b];
    if (icount[a] != icount[b]) return icount[a] < icount[b];
    if (last[a] != last[b]) return last[a] < last[b];
    return a < b;
  }
  void place(int32_t i, int32_t at) {
    heap[at] = i;
    pos[i] = at;
  }
  void sift_up(int32_t at) {
    const int32_t x = heap[at];
    while (at > 0) {
      const int32_t p = (at - 1) >> 1;
      if (!less(x, heap[p])) break;
      place(heap[p], at);
      at = p;
    }
    place(x, at);
  }
  void sift_down(int32_t at) {
    const int32_t x = heap[at], n = h->heap_size;
    for (;;) {
      int32_t c = 2 * at + 1;
      if (c >= n) break;
      if (c + 1 < n && less(heap[c + 1], heap[c])) ++c;
      if (!less(heap[c], x)) break;
      place(heap[c], at);
      at = c;
    }
    place(x, at);
  }
  void fix(int32_t i) {  // after any change of i's key
    sift_up(pos[i]);
    sift_down(pos[i]);
  }
  void heap_push(int32_t i) {
    place(i, h->heap_size++);
    sift_up(pos[i]);
  }
  void heap_pop_top() {
    const int32_t top = heap[0];
    pos[top] = -1;
    if (--h->heap_size > 0) {
      place(heap[h->heap_size], 0);
      sift_down(0);
    }
  }
};

}  // namespace

extern "C" {

size_t bat_sched_state_size(const bat_sched_config *cfg) {
  Layout L;
  return make_layout(cfg, L) ? static_cast<size_t>(L.total) : 0;
}

bat_status bat_sched_init(const bat_sched_config *cfg, const int32_t *user_len, void *state,
                          size_t state_bytes) {
  Layout L;
  if (!make_layout(cfg, L) || !state || (cfg->num_users > 0 && !user_len))
    return BAT_ERR_INVALID_ARG;
  if (state_bytes < static_cast<size_t>(L.total)) return BAT_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(state) % 8) return BAT_ERR_INVALID_ARG;
  for (int32_t u = 0; u < cfg->num_users; ++u)
    if (user_len[u] < 0) return BAT_ERR_INVALID_ARG;
  std::memset(state, 0, static_cast<size_t>(L.total));
  Header *h = static_cast<Header *>(state);
  h->cfg = *cfg;
  h->lru_head = h->lru_tail = -1;
  for (int i = 0; i < kNumArrays; ++i) h->off[i] = L.off[i];
  h->magic = kMagic;
  State s(state);
  for (int32_t u = 0; u < cfg->num_users; ++u) {
    s.user_len[u] = user_len[u];
    s.prev[u] = s.next[u] = -1;
  }
  for (int32_t i = 0; i < cfg->num_items; ++i) {
    s.slot[i] = -1;
    s.pos[i] = -1;
    s.stamp[i] = -1;
  }
  for (int32_t k = 0; k < cfg->item_capacity; ++k) s.slot_item[k] = -1;
  return BAT_OK;
}

bat_status bat_sched_step(void *state, int32_t R, int32_t m, const int32_t *user,
                          const int32_t *items, uint8_t *mode, uint8_t *user_hit,
                          int32_t *item_hits, int64_t *prefix_tokens, int64_t *suffix_tokens,
                          int64_t *pairs, int32_t *item_slot) {
  if (!state || R < 0 || m < 0) return BAT_ERR_INVALID_ARG;
  if (static_cast<Header *>(state)->magic != kMagic) return BAT_ERR_INVALID_ARG;
  if (R == 0) return BAT_OK;
  if (!user || (m > 0 && !items)) return BAT_ERR_INVALID_ARG;
  State s(state);
  Header &h = *s.h;
  const bat_sched_config &c = h.cfg;
  // every id in range and a query's items distinct, before any state changes
  for (int32_t r = 0; r < R; ++r) {
    if (user[r] < 0 || user[r] >= c.num_users) return BAT_ERR_INVALID_ARG;
    const int64_t v = h.validations++;
    for (int32_t j = 0; j < m; ++j) {
      const int32_t i = items[int64_t(r) * m + j];
      if (i < 0 || i >= c.num_items || s.stamp[i] == v) return BAT_ERR_INVALID_ARG;
      s.stamp[i] = v;
    }
  }
  const int64_t T = c.item_tokens, mT = int64_t(m) * T;

  for (int32_t r = 0; r < R; ++r) {
    const int64_t q = h.queries++;
    const int32_t u = user[r];
    const int64_t n_u = s.user_len[u];
    const int32_t *its = items + int64_t(r) * m;
    const bool fits = s.blocks(s.user_len[u]) <= c.user_capacity_blocks;
    // 1) reuse now
    const bool u_hit = s.ures[u] != 0;
    int32_t hits = 0;
    for (int32_t j = 0; j < m; ++j) hits += s.slot[its[j]] >= 0;
    // 2) choice
    bool item_mode = false;
    if (c.policy == BAT_POLICY_HOTNESS) {
      const int64_t s_user = (u_hit || (fits && s.ucount[u] > 0)) ? n_u : 0;
      int64_t s_item = 0;
      for (int32_t j = 0; j < m; ++j) {
        const int32_t i = its[j];
        if (s.slot[i] >= 0) s_item += T;
        else if (c.item_capacity > 0 && s.icount[i] > 0) s_item += T;
      }
      item_mode = s_item > s_user;
    }
    int32_t *out_slot = item_slot ? item_slot + int64_t(r) * m : nullptr;
    if (out_slot)
      for (int32_t j = 0; j < m; ++j) out_slot[j] = -1;
    // 3) cache update and accounting
    int64_t pre, suf, pr;
    if (!item_mode) {
      if (u_hit) {
        s.unlink(u);
        s.push_front(u);
      } else if (fits) {
        const int64_t b = s.blocks(s.user_len[u]);
        while (h.used_blocks + b > c.user_capacity_blocks) {
          const int32_t v = h.lru_tail;
          s.unlink(v);
          s.ures[v] = 0;
          h.used_blocks -= s.blocks(s.user_len[v]);
        }
        s.push_front(u);
        s.ures[u] = 1;
        h.used_blocks += b;
      }
      pre = u_hit ? 0 : n_u;
      suf = mT;
      pr = (u_hit ? 0 : n_u * n_u) + mT * (n_u + mT);
    } else {
      // hits: used now, pinned while this query admits its missing items
      for (int32_t j = 0; j < m; ++j) {
        const int32_t i = its[j];
        if (s.slot[i] < 0) continue;
        s.last[i] = q;
        s.pin[i] = 1;
        s.fix(i);
        if (out_slot) out_slot[j] = s.slot[i];
      }
      for (int32_t j = 0; j < m; ++j) {
        const int32_t i = its[j];
        if (s.slot[i] >= 0) continue;  // a hit (admitted items are other ids)
        int32_t k;
        if (h.next_free < c.item_capacity) {
          k = h.next_free++;
        } else {
          if (h.heap_size == 0) continue;
          const int32_t v = s.heap[0];
          if (s.pin[v] || !(s.icount[v] < s.icount[i])) continue;
          k = s.slot[v];
          s.heap_pop_top();
          s.slot[v] = -1;
        }
        s.slot_item[k] = i;
        s.slot[i] = k;
        s.last[i] = q;
        s.pin[i] = 1;
        s.heap_push(i);
        if (out_slot) out_slot[j] = k;
      }
      pre = T * (m - hits);
      suf = n_u;
      pr = int64_t(m - hits) * T * T + n_u * (n_u + mT);
    }
    // 4) hotness; unpin this query's resident items
    s.ucount[u] += 1;
    for (int32_t j = 0; j < m; ++j) {
      const int32_t i = its[j];
      s.icount[i] += 1;
      if (s.slot[i] >= 0) {
        s.pin[i] = 0;
        s.fix(i);
      }
    }
    if (mode) mode[r] = item_mode ? BAT_PREFIX_ITEM : BAT_PREFIX_USER;
    if (user_hit) user_hit[r] = u_hit;
    if (item_hits) item_hits[r] = hits;
    if (prefix_tokens) prefix_tokens[r] = pre;
    if (suffix_tokens) suffix_tokens[r] = suf;
    if (pairs) pairs[r] = pr;
  }
  return BAT_OK;
}

bat_status bat_sched_pools(const void *state, int32_t *resident_users, int32_t *n_resident_users,
                           int32_t *slot_item) {
  if (!state || static_cast<const Header *>(state)->magic != kMagic) return BAT_ERR_INVALID_ARG;
  State s(const_cast<void *>(state));
  int32_t n = 0;
  for (int32_t u = s.h->lru_head; u >= 0; u = s.next[u]) {
    if (resident_users) resident_users[n] = u;
    ++n;
  }
  if (n_resident_users) *n_resident_users = n;
  if (slot_item)
    for (int32_t k = 0; k < s.h->cfg.item_capacity; ++k) slot_item[k] = s.slot_item[k];
  return BAT_OK;
}

}  // extern "C"
