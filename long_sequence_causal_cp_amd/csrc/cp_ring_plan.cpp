// Host-only planning of the one-GPU ring replay (see cp_ring_plan.h).
#include "cp_ring_plan.h"

#include <stdint.h>

#include <algorithm>
#include <cstdio>

namespace cpplan {

cp_status_t check_chunks(const cp_chunks_t* t, const char* name, std::string* err) {
  char buf[256];
  auto bad = [&](cp_status_t st) {
    if (err) *err = buf;
    return st;
  };
  if (!t) {
    snprintf(buf, sizeof(buf), "%s is NULL", name);
    return bad(CP_ERR_INVALID);
  }
  if (t->n_chunks < 1 || t->n_chunks > CP_MAX_CHUNKS) {
    snprintf(buf, sizeof(buf), "%s.n_chunks = %d, must be in [1, %d]", name, (int)t->n_chunks, CP_MAX_CHUNKS);
    return bad(CP_ERR_INVALID);
  }
  if (t->chunk_len <= 0 || t->chunk_len % 64 != 0) {
    snprintf(buf, sizeof(buf), "%s.chunk_len = %d, must be a positive multiple of 64", name, (int)t->chunk_len);
    return bad(CP_ERR_INVALID);
  }
  for (int i = 0; i < t->n_chunks; ++i) {
    if (t->start[i] < 0 || t->start[i] > (int64_t)INT32_MAX - t->chunk_len) {
      snprintf(buf, sizeof(buf), "%s.start[%d] = %lld out of range [0, 2^31 - chunk_len]", name, i,
               (long long)t->start[i]);
      return bad(CP_ERR_INVALID);
    }
    for (int j = 0; j < i; ++j)
      if (t->start[i] < t->start[j] + t->chunk_len && t->start[j] < t->start[i] + t->chunk_len) {
        snprintf(buf, sizeof(buf), "%s: chunks %d and %d overlap", name, j, i);
        return bad(CP_ERR_INVALID);
      }
  }
  return CP_OK;
}

long long chunk_pairs(long long qs, long long lq, long long ks, long long lk) {
  // query at position p sees min(max(p - ks + 1, 0), lk) keys; with x = p - ks + 1
  // running over [a, b], the sum is S(b) - S(a - 1), S(n) = sum_{x=1..n} min(x, lk)
  auto S = [lk](long long n) -> long long {
    if (n <= 0) return 0;
    if (n <= lk) return n * (n + 1) / 2;
    return lk * (lk + 1) / 2 + (n - lk) * lk;
  };
  const long long a = qs - ks + 1, b = qs - ks + lq;
  return S(b) - S(a - 1);
}

long long pairs_for_chunk(const cp_chunks_t* q, int c, const cp_chunks_t* kv) {
  long long p = 0;
  for (int j = 0; j < kv->n_chunks; ++j) p += chunk_pairs(q->start[c], q->chunk_len, kv->start[j], kv->chunk_len);
  return p;
}

void zigzag_table(int cp_size, int r, int chunk_len, cp_chunks_t* t) {
  *t = cp_chunks_t{};
  t->n_chunks = 2;
  t->chunk_len = chunk_len;
  t->start[0] = (int64_t)r * chunk_len;                    // chunk r
  t->start[1] = (2 * (int64_t)cp_size - 1 - r) * chunk_len;  // chunk 2N-1-r
}

void plan_ring_fwd(const cp_chunks_t* q, const cp_chunks_t* kv_steps, int n_steps, int max_steps_per_launch,
                   FwdPlan* plan) {
  *plan = FwdPlan{};
  const int nkv = kv_steps[0].n_chunks;
  const int per = std::max(1, std::min(max_steps_per_launch, CP_MAX_CHUNKS / nkv));
  plan->steps_per_launch = per;

  // launches: step 0 alone, then the rest in the fewest groups of <= per steps,
  // smaller groups first (a later group is never smaller, so its staging fits
  // under the launch before it)
  std::vector<FwdLaunch>& L = plan->launches;
  L.emplace_back();
  L[0].first_step = 0;
  L[0].count = 1;
  {
    const int rest = n_steps - 1;
    const int groups = (rest + per - 1) / per;
    for (int g = 0, j = 1; g < groups; ++g) {
      FwdLaunch l;
      l.first_step = j;
      l.count = rest / groups + (g >= groups - rest % groups ? 1 : 0);
      l.slot = g & 1;
      j += l.count;
      L.push_back(l);
    }
  }
  const int n_launch = (int)L.size();
  const int nq = q->n_chunks;

  // a query chunk's first and last launch with visible keys
  int first[CP_MAX_CHUNKS], last[CP_MAX_CHUNKS];
  for (int c = 0; c < nq; ++c) first[c] = last[c] = -1;
  for (int l = 0; l < n_launch; ++l)
    for (int c = 0; c < nq; ++c) {
      long long w = 0;
      for (int j = L[l].first_step; j < L[l].first_step + L[l].count; ++j) w += pairs_for_chunk(q, c, &kv_steps[j]);
      L[l].work[c] = w;
      if (w > 0) {
        if (first[c] < 0) first[c] = l;
        last[c] = l;
      }
    }
  for (int c = 0; c < nq; ++c)
    if (first[c] < 0) first[c] = last[c] = n_launch - 1;  // no key at all: write O = 0, LSE = -inf
  for (int l = 0; l < n_launch; ++l)
    for (int c = 0; c < nq; ++c) {
      if (l < first[c] || l > last[c] || (L[l].work[c] == 0 && l != last[c] && l != first[c])) continue;
      L[l].active[L[l].n_active++] = c;
      L[l].flags[c] = (l == first[c] ? 0 : kMerge) | (l == last[c] ? kFinalize : kWriteO);
    }

  // stream operations
  const int ev_entry = 0, ev_done = 1;
  auto staged = [&](int l) { return 2 + l; };
  auto released = [&](int l) { return 2 + n_launch + l; };
  plan->n_events = 2 + 2 * n_launch;
  std::vector<Op>& ops = plan->ops;
  auto stage = [&](int l) {
    if (l >= 3) ops.push_back({OpKind::Wait, kCopy, released(l - 2), -1});  // slot last read by launch l-2
    ops.push_back({OpKind::Stage, kCopy, -1, l});
    ops.push_back({OpKind::Record, kCopy, staged(l), -1});
  };
  ops.push_back({OpKind::Record, kCompute, ev_entry, -1});
  ops.push_back({OpKind::Wait, kCopy, ev_entry, -1});
  for (int l = 1; l < n_launch && l <= 2; ++l) stage(l);
  for (int l = 0; l < n_launch; ++l) {
    if (l >= 1) ops.push_back({OpKind::Wait, kCompute, staged(l), -1});
    ops.push_back({OpKind::Launch, kCompute, -1, l});
    if (l + 2 < n_launch) {
      // launch l + 2 reuses the slot launch l reads
      if (l >= 1) ops.push_back({OpKind::Record, kCompute, released(l), -1});
      if (l + 2 >= 3) stage(l + 2);
    }
  }
  ops.push_back({OpKind::Record, kCopy, ev_done, -1});
  ops.push_back({OpKind::Wait, kCompute, ev_done, -1});
}

void plan_ring_bwd(int n_steps, BwdPlan* plan) {
  *plan = BwdPlan{};
  const int ev_entry = 0, ev_done = 1;
  auto received = [&](int j) { return 2 + j; };
  auto computed = [&](int j) { return 2 + n_steps + j; };
  plan->n_events = 2 + 2 * n_steps;
  std::vector<Op>& ops = plan->ops;
  auto receive = [&](int j) {
    ops.push_back({OpKind::Receive, kCopy, -1, j});
    ops.push_back({OpKind::Record, kCopy, received(j), -1});
  };
  ops.push_back({OpKind::Record, kCompute, ev_entry, -1});
  ops.push_back({OpKind::Wait, kCopy, ev_entry, -1});
  for (int j = 1; j < n_steps && j <= 2; ++j) receive(j);
  ops.push_back({OpKind::Delta, kCompute, -1, -1});
  for (int j = 0; j < n_steps; ++j) {
    if (j > 0) ops.push_back({OpKind::Wait, kCompute, received(j), -1});
    ops.push_back({OpKind::Kernels, kCompute, -1, j});
    if (j == 0) continue;  // the rank's own block: its dK/dV are written in place
    // send of step j: the updated partial sums leave the slot; step j + 2's
    // receive into the same slot follows it on the copy stream
    ops.push_back({OpKind::Record, kCompute, computed(j), -1});
    ops.push_back({OpKind::Wait, kCopy, computed(j), -1});
    ops.push_back({OpKind::Send, kCopy, -1, j});
    if (j + 2 < n_steps) receive(j + 2);
  }
  ops.push_back({OpKind::Record, kCopy, ev_done, -1});
  ops.push_back({OpKind::Wait, kCompute, ev_done, -1});
}

}  // namespace cpplan
