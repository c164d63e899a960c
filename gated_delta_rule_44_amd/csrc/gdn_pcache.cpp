// Prefix-state cache of the GDN layer (host bookkeeping; "qev_fast/statecache.py" page, StateCache).
//
// A checkpoint is the state and conv tail after the first `pos` tokens of some earlier row, kept in one
// slot of a caller-owned pool of state records. A new row looks for the deepest checkpoint whose tokens
// it shares (it may start from there instead of from zero), and leaves checkpoints at the chunk ends
// the page places: the multiples of `stride`, p - tail and p, rounded down to `align`, with no chunk
// longer than `max_chunk`, where p is the row's checkpointable prefix. Checkpoints are evicted least
// recently used first once there are more than the pool's slots; using one as a starting point
// refreshes it. Only the recurrent state is cached: the attention K / V the page also keeps belongs to
// another layer. This file plans and books; the GPU work (restore, chunked prefill, snapshots) is the
// caller's, on one stream, in the plan's order.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <list>
#include <map>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "gdn.h"

struct gdn_pcache {
  struct Ckpt {
    int64_t group;
    int pos;
    int slot;
    std::list<int64_t>::iterator lru;  // position in the use order
  };
  struct Group {
    std::vector<int32_t> ids;          // the prefix tokens of the row that made it
    std::vector<int64_t> ckpts;        // its checkpoints, in position order (evicted ones included)
    int live = 0;                      // of which still cached; the group goes with its last one
  };
  int slots, stride, tail, align, max_chunk, min_prefix;
  std::map<int64_t, Group> groups;            // rows with a live checkpoint, by creation number
  int64_t groups_made = 0;
  std::unordered_map<int64_t, Ckpt> ckpts;    // live checkpoints by number
  std::list<int64_t> lru;                     // least recently used first
  std::vector<int> free_slots;
  int64_t made = 0;
  int64_t stats[GDN_PCACHE_NSTATS] = {};
};

namespace {

int down(const gdn_pcache* c, int x) { return c->align > 0 ? x - x % c->align : x; }

// chunk ends from position c0 for a prefix of p tokens (the page's _bounds)
std::vector<int> bounds_of(const gdn_pcache* c, int c0, int p) {
  const int e = down(c, p);
  std::set<int> b;
  if (c->stride > 0)
    for (long k = c->stride; k < e; k += c->stride)
      if (k > c0) b.insert((int)k);
  if (c->tail > 0 && down(c, p - c->tail) > c0) b.insert(down(c, p - c->tail));
  if (e > c0) b.insert(e);
  std::vector<int> out;
  long s = c0;
  for (int x : b) {
    while (x - s > c->max_chunk) {
      s += c->max_chunk;
      out.push_back((int)s);
    }
    out.push_back(x);
    s = x;
  }
  return out;
}

}  // namespace

extern "C" {

int gdn_pcache_create(int slots, int stride, int tail, int align, int max_chunk, int min_prefix, gdn_pcache** out) {
  if (!out) return GDN_EINVAL;
  *out = nullptr;
  if (slots < 0 || stride < 0 || tail < 0 || align < 0 || max_chunk <= 0 || min_prefix < 0) return GDN_EINVAL;
  gdn_pcache* c = new (std::nothrow) gdn_pcache;
  if (!c) return GDN_EINVAL;
  c->slots = slots; c->stride = stride; c->tail = tail; c->align = align;
  c->max_chunk = max_chunk; c->min_prefix = min_prefix;
  for (int s = slots - 1; s >= 0; --s) c->free_slots.push_back(s);
  *out = c;
  return GDN_OK;
}

void gdn_pcache_destroy(gdn_pcache* c) { delete c; }

int gdn_pcache_row(gdn_pcache* c, const int32_t* ids, int n, int p_state, int cap, int32_t* info, int32_t* bounds,
                   int32_t* snap_slot, int64_t* ckpt) {
  if (!c || !info || (n > 0 && !ids) || n < 0 || p_state < 0 || cap < 0) return GDN_EINVAL;
  const int p = down(c, std::min(p_state, n));
  if (p < c->min_prefix || p == 0) {  // too short to checkpoint: the plain path
    c->stats[GDN_PCACHE_PLAIN]++;
    c->stats[GDN_PCACHE_TOKENS_COMPUTED] += n;
    info[0] = -1; info[1] = 0; info[2] = p; info[3] = 0;
    if (ckpt) ckpt[0] = -1;
    return 0;
  }
  // the deepest usable checkpoint (the first one found among equals)
  int64_t best = -1;
  int best_pos = -1;
  for (const auto& kv : c->groups) {
    const gdn_pcache::Group& g = kv.second;
    const int m = std::min((int)g.ids.size(), p);
    if (m == 0 || g.ids[0] != ids[0]) continue;
    int lcp = 0;
    while (lcp < m && g.ids[lcp] == ids[lcp]) ++lcp;
    for (int64_t num : g.ckpts) {
      auto it = c->ckpts.find(num);
      if (it == c->ckpts.end() || it->second.pos > lcp) continue;
      if (it->second.pos > best_pos || (it->second.pos == best_pos && num < best)) {  // ties: made first
        best = num;
        best_pos = it->second.pos;
      }
    }
  }
  const int c0 = best >= 0 ? best_pos : 0;
  // the chunk ends come from the unrounded prefix length (p - tail is rounded after the subtraction)
  const std::vector<int> bs = c0 < p ? bounds_of(c, c0, std::min(p_state, n)) : std::vector<int>();
  if ((int)bs.size() > cap) return GDN_EINVAL;  // nothing booked: the caller retries with room
  if (!bs.empty() && (!bounds || !snap_slot)) return GDN_EINVAL;

  c->stats[GDN_PCACHE_ROWS]++;
  c->stats[c0 == p ? GDN_PCACHE_HITS : c0 > 0 ? GDN_PCACHE_PARTIAL : GDN_PCACHE_COLD]++;
  c->stats[GDN_PCACHE_TOKENS_REUSED] += c0;
  c->stats[GDN_PCACHE_TOKENS_COMPUTED] += n - c0;
  int restore_slot = -1;
  if (best >= 0) {
    gdn_pcache::Ckpt& k = c->ckpts[best];
    restore_slot = k.slot;
    c->lru.splice(c->lru.end(), c->lru, k.lru);  // most recently used
  }
  std::vector<int64_t> fresh;
  if (!bs.empty()) {
    const int64_t gid = c->groups_made++;
    gdn_pcache::Group& g = c->groups[gid];
    g.ids.assign(ids, ids + p);
    g.live = (int)bs.size();
    for (int b : bs) {
      const int64_t num = c->made++;
      g.ckpts.push_back(num);
      c->lru.push_back(num);
      gdn_pcache::Ckpt k;
      k.group = gid;
      k.pos = b;
      k.slot = -1;
      k.lru = std::prev(c->lru.end());
      c->ckpts.emplace(num, k);
      fresh.push_back(num);
      c->stats[GDN_PCACHE_CKPTS_MADE]++;
    }
  }
  // evict down to the pool's size, least recently used first; a new checkpoint evicted here was never
  // stored, the others free their slot
  while ((long)c->ckpts.size() > c->slots) {
    const int64_t num = c->lru.front();
    c->lru.pop_front();
    auto it = c->ckpts.find(num);
    if (it->second.slot >= 0) c->free_slots.push_back(it->second.slot);
    auto g = c->groups.find(it->second.group);
    if (--g->second.live == 0) c->groups.erase(g);  // no checkpoint of that row is left
    c->ckpts.erase(it);
    c->stats[GDN_PCACHE_EVICTED]++;
  }
  c->stats[GDN_PCACHE_ROWS_KEPT] = (int64_t)c->groups.size();
  for (size_t i = 0; i < fresh.size(); ++i) {
    auto it = c->ckpts.find(fresh[i]);
    if (it != c->ckpts.end()) {
      it->second.slot = c->free_slots.back();
      c->free_slots.pop_back();
    }
    bounds[i] = bs[i];
    snap_slot[i] = it != c->ckpts.end() ? it->second.slot : -1;
    if (ckpt) ckpt[1 + i] = it != c->ckpts.end() ? fresh[i] : -1;
  }
  info[0] = restore_slot; info[1] = c0; info[2] = p; info[3] = (int)bs.size();
  if (ckpt) ckpt[0] = best;
  return (int)bs.size();
}

int gdn_pcache_stats(const gdn_pcache* c, int64_t* stats) {
  if (!c || !stats) return GDN_EINVAL;
  memcpy(stats, c->stats, sizeof(c->stats));
  return GDN_OK;
}

int gdn_pcache_alive(const gdn_pcache* c, int cap, int64_t* nums) {
  if (!c || cap < 0 || (cap > 0 && !nums)) return GDN_EINVAL;
  std::vector<int64_t> v;
  v.reserve(c->ckpts.size());
  for (const auto& kv : c->ckpts) v.push_back(kv.first);
  std::sort(v.begin(), v.end());
  for (int i = 0; i < cap && i < (int)v.size(); ++i) nums[i] = v[i];
  return (int)v.size();
}

}  // extern "C"
