// CPU check of the ring drivers' host planning, built with address and
// undefined-behaviour sanitizers (tests/test_ring_plan_sanitized.py).
//
// It drives the pure-host planning code of the library (chunk-table checks,
// visible-pair counts, zigzag tables, and the forward and backward ring
// plans) over 1..64 ring steps, 1..8 chunks per table, ragged and
// non-zigzag tables and every steps-per-launch limit, and checks:
//   - each plan covers every ring step once, in ring order, with at most the
//     allowed steps and key chunks per launch;
//   - each query chunk is written by its first launch with visible keys,
//     merged afterwards and finalised by its last; work counts equal a
//     brute-force count of visible pairs;
//   - the happens-before order of the plan's stream operations (program
//     order on each stream, plus record -> wait edges) orders every pair of
//     conflicting accesses to a staging slot or a travelling gradient buffer,
//     every read sees the write it is meant to see, every copy follows the
//     call's entry and precedes its return (the double buffering of the
//     pages' context-parallel loop: the transfer for a later step may fill a
//     buffer only after the step that used it is done);
//   - planted mistakes in copies of a plan (a dropped wait, a record moved,
//     a slot swapped) are caught by that check;
//   - the kernels' XCD-aware job order (cp_job_map.h) maps the grid one to
//     one onto (block, b*h), keeps every (b, h) on one XCD, runs a head
//     group's blocks in consecutive rounds, and splits a key-split grid into
//     pairs on one XCD; the head-group size divides an XCD's heads and fits.
// Exit status 0 when every check passes.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "../../long_sequence_causal_cp_amd/csrc/cp_job_map.h"
#include "../../long_sequence_causal_cp_amd/csrc/cp_ring_plan.h"

using namespace cpplan;

static int g_fail = 0;
static long g_checks = 0;
#define CHECK(cond, ...)                                 \
  do {                                                   \
    ++g_checks;                                          \
    if (!(cond)) {                                       \
      if (g_fail < 20) {                                 \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);               \
        std::fprintf(stderr, "\n");                      \
      }                                                  \
      ++g_fail;                                          \
    }                                                    \
  } while (0)

// ---------------------------------------------------------------- happens-before
// An access of one operation to one abstract buffer.
struct Access {
  int op;
  std::string buf;
  bool write;
  int intended_writer;  // for reads: the op whose write it must see (-1: the buffer's content on entry)
};

struct HB {
  int n = 0;
  std::vector<std::vector<uint64_t>> reach;  // reach[a] bit b: a happens before b (a != b)
  bool before(int a, int b) const { return (reach[a][b / 64] >> (b % 64)) & 1; }
};

// Happens-before closure of a plan's operations.  Returns false (with a
// message) if a wait names an event not recorded earlier in issue order.
static bool build_hb(const std::vector<Op>& ops, int n_events, HB* hb, std::string* why) {
  const int n = (int)ops.size();
  hb->n = n;
  const int W = (n + 63) / 64;
  hb->reach.assign(n, std::vector<uint64_t>(W, 0));
  std::vector<std::vector<int>> succ(n);
  int last_on[2] = {-1, -1};
  std::vector<int> recorded(n_events, -1);
  for (int i = 0; i < n; ++i) {
    const Op& o = ops[i];
    if (o.stream < 0 || o.stream > 1) {
      *why = "bad stream";
      return false;
    }
    if (last_on[o.stream] >= 0) succ[last_on[o.stream]].push_back(i);
    last_on[o.stream] = i;
    if (o.kind == OpKind::Record) {
      if (o.event < 0 || o.event >= n_events) {
        *why = "record of an event outside the plan";
        return false;
      }
      if (recorded[o.event] >= 0) {
        *why = "event recorded twice in one call";
        return false;
      }
      recorded[o.event] = i;
    } else if (o.kind == OpKind::Wait) {
      if (o.event < 0 || o.event >= n_events || recorded[o.event] < 0) {
        char b[96];
        std::snprintf(b, sizeof(b), "op %d waits for event %d before it is recorded", i, o.event);
        *why = b;
        return false;
      }
      succ[recorded[o.event]].push_back(i);
    }
  }
  // ops are in issue order and every edge goes forward, so a reverse sweep closes them
  for (int i = n - 1; i >= 0; --i)
    for (int j : succ[i]) {
      hb->reach[i][j / 64] |= uint64_t(1) << (j % 64);
      for (int w = 0; w < W; ++w) hb->reach[i][w] |= hb->reach[j][w];
    }
  return true;
}

// Race and visibility check of a list of accesses under hb.  Returns an
// empty string when ordered correctly.
static std::string check_accesses(const std::vector<Op>& ops, const HB& hb, const std::vector<Access>& acc) {
  std::map<std::string, std::vector<const Access*>> by_buf;
  for (const Access& a : acc) by_buf[a.buf].push_back(&a);
  char b[200];
  for (auto& kv : by_buf) {
    const auto& v = kv.second;
    for (size_t i = 0; i < v.size(); ++i)
      for (size_t j = i + 1; j < v.size(); ++j) {
        const Access *x = v[i], *y = v[j];
        if (!x->write && !y->write) continue;
        if (x->op == y->op) continue;
        if (!hb.before(x->op, y->op) && !hb.before(y->op, x->op)) {
          std::snprintf(b, sizeof(b), "race on %s between op %d and op %d", kv.first.c_str(), x->op, y->op);
          return b;
        }
      }
    for (const Access* r : v) {
      if (r->write) continue;
      for (const Access* w : v) {
        if (!w->write || w->op == r->op) continue;
        if (w->op == r->intended_writer) {
          if (!hb.before(w->op, r->op)) {
            std::snprintf(b, sizeof(b), "read of %s by op %d not after its write by op %d", kv.first.c_str(), r->op,
                          w->op);
            return b;
          }
        } else {
          // another write must come before the intended one, or after the read
          const bool before_intended = r->intended_writer >= 0 && hb.before(w->op, r->intended_writer);
          if (!before_intended && !hb.before(r->op, w->op)) {
            std::snprintf(b, sizeof(b), "read of %s by op %d may see op %d's write instead of op %d's",
                          kv.first.c_str(), r->op, w->op, r->intended_writer);
            return b;
          }
        }
      }
    }
  }
  // every copy-stream op after the call's entry and before its return
  int first_compute = -1, last_compute = -1;
  for (int i = 0; i < (int)ops.size(); ++i)
    if (ops[i].stream == kCompute) {
      if (first_compute < 0) first_compute = i;
      last_compute = i;
    }
  for (int i = 0; i < (int)ops.size(); ++i) {
    if (ops[i].stream != kCopy) continue;
    if (first_compute >= 0 && !hb.before(first_compute, i)) {
      std::snprintf(b, sizeof(b), "copy-stream op %d does not follow the call's entry", i);
      return b;
    }
    if (last_compute >= 0 && !hb.before(i, last_compute)) {
      std::snprintf(b, sizeof(b), "copy-stream op %d is not ordered before the call returns", i);
      return b;
    }
  }
  return "";
}

// ---------------------------------------------------------------- forward
static std::vector<Access> fwd_accesses(const FwdPlan& p) {
  std::vector<Access> acc;
  std::map<int, int> stage_op;  // launch -> its Stage op
  for (int i = 0; i < (int)p.ops.size(); ++i)
    if (p.ops[i].kind == OpKind::Stage) stage_op[p.ops[i].index] = i;
  for (int i = 0; i < (int)p.ops.size(); ++i) {
    const Op& o = p.ops[i];
    if (o.kind != OpKind::Stage && o.kind != OpKind::Launch) continue;
    const FwdLaunch& L = p.launches[o.index];
    if (L.slot < 0) continue;  // the rank's own block, read in place
    for (int k = 0; k < L.count; ++k) {
      const std::string buf = "slot" + std::to_string(L.slot) + "[" + std::to_string(k) + "]";
      if (o.kind == OpKind::Stage) acc.push_back({i, buf, true, -1});
      else acc.push_back({i, buf, false, stage_op.count(o.index) ? stage_op[o.index] : -2});
    }
  }
  return acc;
}

static std::string check_fwd_order(const FwdPlan& p) {
  HB hb;
  std::string why;
  if (!build_hb(p.ops, p.n_events, &hb, &why)) return why;
  return check_accesses(p.ops, hb, fwd_accesses(p));
}

static long long brute_pairs(const cp_chunks_t& q, int c, const cp_chunks_t& kv) {
  long long n = 0;
  for (long long i = 0; i < q.chunk_len; ++i) {
    const long long qp = q.start[c] + i;
    for (int k = 0; k < kv.n_chunks; ++k) {
      const long long lo = kv.start[k], hi = kv.start[k] + kv.chunk_len - 1;
      if (qp >= lo) n += (qp < hi ? qp : hi) - lo + 1;
    }
  }
  return n;
}

static void check_fwd_plan(const cp_chunks_t& q, const std::vector<cp_chunks_t>& kv, int per, const char* what) {
  const int n = (int)kv.size();
  FwdPlan p;
  plan_ring_fwd(&q, kv.data(), n, per, &p);
  const int nkv = kv[0].n_chunks;
  // coverage: step 0 alone, then consecutive groups
  CHECK(!p.launches.empty() && p.launches[0].first_step == 0 && p.launches[0].count == 1 && p.launches[0].slot == -1,
        "%s: launch 0 is not step 0 in place", what);
  int next = 0, prev_count = 0;
  for (size_t l = 0; l < p.launches.size(); ++l) {
    const FwdLaunch& L = p.launches[l];
    CHECK(L.first_step == next, "%s: launch %zu starts at step %d, expected %d", what, l, L.first_step, next);
    CHECK(L.count >= 1 && L.count <= p.steps_per_launch, "%s: launch %zu covers %d steps", what, l, L.count);
    CHECK(L.count * nkv <= CP_MAX_CHUNKS, "%s: launch %zu holds %d key chunks", what, l, L.count * nkv);
    if (l >= 1) {
      CHECK(L.slot == (int)((l - 1) & 1), "%s: launch %zu in slot %d", what, l, L.slot);
      if (l >= 2) CHECK(L.count >= prev_count, "%s: launch %zu smaller than the one before", what, l);
      prev_count = L.count;
    }
    next += L.count;
  }
  CHECK(next == n, "%s: launches cover %d of %d steps", what, next, n);
  // groups: the fewest possible
  const int per_eff = p.steps_per_launch;
  CHECK((int)p.launches.size() - 1 == (n - 1 + per_eff - 1) / per_eff, "%s: %zu launches", what, p.launches.size());
  // flags and work
  for (int c = 0; c < q.n_chunks; ++c) {
    long long total = 0;
    for (int j = 0; j < n; ++j) total += brute_pairs(q, c, kv[j]);
    long long sum = 0;
    int first = -1, last = -1;
    for (size_t l = 0; l < p.launches.size(); ++l) {
      const FwdLaunch& L = p.launches[l];
      long long w = 0;
      for (int j = L.first_step; j < L.first_step + L.count; ++j) w += brute_pairs(q, c, kv[j]);
      CHECK(L.work[c] == w, "%s: launch %zu chunk %d work %lld, brute force %lld", what, l, c, L.work[c], w);
      sum += L.work[c];
      bool active = false;
      for (int i = 0; i < L.n_active; ++i) active = active || L.active[i] == c;
      if (active) {
        if (first < 0) first = (int)l;
        last = (int)l;
      } else {
        CHECK(w == 0, "%s: launch %zu skips chunk %d with %lld visible pairs", what, l, c, w);
      }
    }
    CHECK(sum == total, "%s: chunk %d work %lld vs %lld", what, c, sum, total);
    CHECK(first >= 0, "%s: chunk %d never computed", what, c);
    if (first < 0) continue;
    for (int l = first; l <= last; ++l) {
      const FwdLaunch& L = p.launches[l];
      bool active = false;
      for (int i = 0; i < L.n_active; ++i) active = active || L.active[i] == c;
      if (!active) continue;
      const int f = L.flags[c];
      CHECK(((f & kMerge) != 0) == (l != first), "%s: chunk %d launch %d merge flag", what, c, l);
      CHECK(((f & kFinalize) != 0) == (l == last), "%s: chunk %d launch %d finalize flag", what, c, l);
      CHECK(((f & kWriteO) != 0) == (l != last), "%s: chunk %d launch %d write-O flag", what, c, l);
    }
    if (total == 0) CHECK(first == last && first == (int)p.launches.size() - 1, "%s: empty chunk %d", what, c);
  }
  for (const FwdLaunch& L : p.launches) {
    std::set<int> seen;
    for (int i = 0; i < L.n_active; ++i) {
      CHECK(L.active[i] >= 0 && L.active[i] < q.n_chunks, "%s: active chunk out of range", what);
      CHECK(seen.insert(L.active[i]).second, "%s: chunk listed twice", what);
    }
  }
  const std::string why = check_fwd_order(p);
  CHECK(why.empty(), "%s: %s", what, why.c_str());

  // planted mistakes in copies of the plan must be caught (only when a
  // slot is reused, i.e. from five launches on, or read at all)
  if (p.launches.size() >= 2) {
    // a launch that does not wait for its staging
    FwdPlan m = p;
    for (size_t i = 0; i < m.ops.size(); ++i)
      if (m.ops[i].kind == OpKind::Wait && m.ops[i].stream == kCompute && i + 1 < m.ops.size() &&
          m.ops[i + 1].kind == OpKind::Launch) {
        m.ops.erase(m.ops.begin() + i);
        break;
      }
    CHECK(!check_fwd_order(m).empty(), "%s: a launch without its staged wait passed", what);
  }
  if (p.launches.size() >= 4) {
    // staging into a slot before the launch that last read it has released it
    FwdPlan m = p;
    for (size_t i = 0; i < m.ops.size(); ++i)
      if (m.ops[i].kind == OpKind::Wait && m.ops[i].stream == kCopy && m.ops[i].event != 0) {
        m.ops.erase(m.ops.begin() + i);
        break;
      }
    CHECK(!check_fwd_order(m).empty(), "%s: a staging copy without the release wait passed", what);
    // the release recorded before the launch instead of after it
    m = p;
    for (size_t i = 1; i < m.ops.size(); ++i)
      if (m.ops[i].kind == OpKind::Record && m.ops[i].stream == kCompute && m.ops[i - 1].kind == OpKind::Launch) {
        std::swap(m.ops[i], m.ops[i - 1]);
        break;
      }
    CHECK(!check_fwd_order(m).empty(), "%s: a release recorded before its launch passed", what);
  }
  if (p.launches.size() >= 3) {
    // two consecutive launches in the same slot
    FwdPlan m = p;
    m.launches[2].slot = m.launches[1].slot;
    CHECK(!check_fwd_order(m).empty(), "%s: consecutive launches sharing a slot passed", what);
  }
}

// ---------------------------------------------------------------- backward
static std::vector<Access> bwd_accesses(const BwdPlan& p, const std::vector<bool>& adds) {
  std::vector<Access> acc;
  std::map<int, int> recv_op, kern_op;
  for (int i = 0; i < (int)p.ops.size(); ++i) {
    if (p.ops[i].kind == OpKind::Receive) recv_op[p.ops[i].index] = i;
    if (p.ops[i].kind == OpKind::Kernels) kern_op[p.ops[i].index] = i;
  }
  auto get = [](std::map<int, int>& m, int j) { return m.count(j) ? m[j] : -2; };
  for (int i = 0; i < (int)p.ops.size(); ++i) {
    const Op& o = p.ops[i];
    const int j = o.index;
    const std::string s = std::to_string((j - 1) & 1);
    const std::string kv = "slot" + s + ".kv", g = "slot" + s + ".grad", c = "caller.grad" + std::to_string(j);
    switch (o.kind) {
      case OpKind::Receive:
        acc.push_back({i, kv, true, -1});
        if (adds[j]) {
          acc.push_back({i, c, false, -1});  // the partial sums as they arrived
          acc.push_back({i, g, true, -1});
        }
        break;
      case OpKind::Kernels:
        if (j == 0) {
          acc.push_back({i, c, true, -1});
          if (adds[0]) acc.push_back({i, c, false, -1});
        } else {
          acc.push_back({i, kv, false, get(recv_op, j)});
          if (adds[j]) acc.push_back({i, g, false, get(recv_op, j)});
          acc.push_back({i, g, true, -1});
        }
        break;
      case OpKind::Send:
        acc.push_back({i, g, false, get(kern_op, j)});
        acc.push_back({i, c, true, -1});
        break;
      default:
        break;
    }
  }
  return acc;
}

static std::string check_bwd_order(const BwdPlan& p, const std::vector<bool>& adds) {
  HB hb;
  std::string why;
  if (!build_hb(p.ops, p.n_events, &hb, &why)) return why;
  return check_accesses(p.ops, hb, bwd_accesses(p, adds));
}

static void check_bwd_plan(int n, const std::vector<bool>& adds, const char* what) {
  BwdPlan p;
  plan_ring_bwd(n, &p);
  std::vector<int> kern(n, 0), recv(n, 0), send(n, 0);
  int delta_at = -1, first_kern = -1;
  for (int i = 0; i < (int)p.ops.size(); ++i) {
    const Op& o = p.ops[i];
    if (o.kind == OpKind::Kernels) {
      CHECK(o.index >= 0 && o.index < n, "%s: kernels of step %d", what, o.index);
      if (o.index >= 0 && o.index < n) {
        CHECK(o.index == 0 || kern[o.index - 1] == 1, "%s: step %d computed out of ring order", what, o.index);
        kern[o.index]++;
      }
      if (first_kern < 0) first_kern = i;
    }
    if (o.kind == OpKind::Receive && o.index > 0 && o.index < n) recv[o.index]++;
    if (o.kind == OpKind::Send && o.index > 0 && o.index < n) send[o.index]++;
    if (o.kind == OpKind::Delta) delta_at = i;
  }
  for (int j = 0; j < n; ++j) {
    CHECK(kern[j] == 1, "%s: step %d computed %d times", what, j, kern[j]);
    CHECK(recv[j] == (j > 0), "%s: step %d received %d times", what, j, recv[j]);
    CHECK(send[j] == (j > 0), "%s: step %d sent %d times", what, j, send[j]);
  }
  CHECK(delta_at >= 0 && delta_at < first_kern, "%s: Delta not before the first kernels", what);
  const std::string why = check_bwd_order(p, adds);
  CHECK(why.empty(), "%s: %s", what, why.c_str());
  if (n >= 2) {
    BwdPlan m = p;  // kernels that do not wait for their receive
    for (size_t i = 0; i < m.ops.size(); ++i)
      if (m.ops[i].kind == OpKind::Wait && m.ops[i].stream == kCompute && i + 1 < m.ops.size() &&
          m.ops[i + 1].kind == OpKind::Kernels) {
        m.ops.erase(m.ops.begin() + i);
        break;
      }
    CHECK(!check_bwd_order(m, adds).empty(), "%s: kernels without their receive wait passed", what);
    m = p;  // a send that does not wait for the kernels
    for (size_t i = 0; i < m.ops.size(); ++i)
      if (m.ops[i].kind == OpKind::Wait && m.ops[i].stream == kCopy && m.ops[i].event != 0) {
        m.ops.erase(m.ops.begin() + i);
        break;
      }
    CHECK(!check_bwd_order(m, adds).empty(), "%s: a send without the kernels' wait passed", what);
  }
  // step j+2's receive issued before step j's send: with partial sums to
  // receive it overwrites the slot's sums before they are sent (without, it
  // writes only K/V, which step j has finished reading, and is harmless)
  for (size_t i = 0; i + 1 < p.ops.size(); ++i)
    if (p.ops[i].kind == OpKind::Send && p.ops[i + 1].kind == OpKind::Receive && adds[p.ops[i + 1].index]) {
      BwdPlan m = p;
      std::swap(m.ops[i], m.ops[i + 1]);
      CHECK(!check_bwd_order(m, adds).empty(), "%s: a receive overtaking the send of its slot passed", what);
      break;
    }
}

// ---------------------------------------------------------------- tables
static void check_tables() {
  std::string err;
  cp_chunks_t t{};
  CHECK(check_chunks(nullptr, "t", &err) == CP_ERR_INVALID && !err.empty(), "NULL table accepted");
  t.n_chunks = 0;
  t.chunk_len = 64;
  CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "0 chunks accepted");
  t.n_chunks = CP_MAX_CHUNKS + 1;
  CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "9 chunks accepted");
  for (int len : {0, -64, 32, 96, 65}) {
    t = cp_chunks_t{};
    t.n_chunks = 1;
    t.chunk_len = len;
    CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "chunk_len %d accepted", len);
  }
  t = cp_chunks_t{};
  t.n_chunks = 2;
  t.chunk_len = 64;
  t.start[0] = 0;
  t.start[1] = 63;
  CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "overlapping chunks accepted");
  t.start[1] = 64;
  CHECK(check_chunks(&t, "t", &err) == CP_OK, "adjacent chunks rejected: %s", err.c_str());
  t.start[1] = -1;
  CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "negative start accepted");
  t.start[1] = (int64_t)INT32_MAX - 63;
  CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "start past 2^31 - len accepted");
  t.start[1] = (int64_t)INT32_MAX - 64;
  CHECK(check_chunks(&t, "t", &err) == CP_OK, "last valid start rejected: %s", err.c_str());
  t.start[1] = INT64_MAX;
  CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "huge start accepted");
  t.start[1] = INT64_MIN;
  CHECK(check_chunks(&t, "t", &err) == CP_ERR_INVALID, "INT64_MIN start accepted");
  t.chunk_len = INT32_MAX - (INT32_MAX % 64);
  t.n_chunks = 1;
  t.start[0] = 0;
  CHECK(check_chunks(&t, "t", &err) == CP_OK, "largest chunk rejected: %s", err.c_str());
  // pair counts at the extremes of valid tables, against the closed forms
  const long long L = t.chunk_len;
  CHECK(chunk_pairs(0, L, 0, L) == L * (L + 1) / 2, "diagonal pairs");
  CHECK(chunk_pairs(L, 64, 0, L) == 64 * L, "full pairs");
  CHECK(chunk_pairs(0, 64, L, 64) == 0, "future pairs");
  // zigzag tables
  for (int N : {1, 2, 3, 8, 64, 1000})
    for (int r = 0; r < N; r += (N > 8 ? 97 : 1)) {
      zigzag_table(N, r, 64, &t);
      CHECK(t.n_chunks == 2 && t.start[0] == 64LL * r && t.start[1] == 64LL * (2 * N - 1 - r), "zigzag N=%d r=%d",
            N, r);
      CHECK(check_chunks(&t, "zigzag", &err) == CP_OK, "zigzag table N=%d r=%d rejected", N, r);
    }
}

// ---------------------------------------------------------------- job order
static void check_job_map() {
  using cpattn::heads_per_group;
  using cpattn::split_job;
  using cpattn::xcd_job;
  const int bhs[] = {1, 2, 3, 8, 12, 16, 24, 32, 64, 72, 128, 256};
  const int nrbs[] = {1, 2, 3, 4, 8, 16, 32};
  const long long slotss[] = {16, 32, 64, 128};
  for (int BH : bhs)
    for (int nrb : nrbs)
      for (long long slots : slotss) {
        const int hpx = BH % 8 == 0 ? BH / 8 : 0;
        const int hpg = hpx > 0 ? heads_per_group(hpx, nrb, slots) : 0;
        if (hpx > 0) {
          CHECK(hpg >= 1 && hpx % hpg == 0, "heads_per_group %d of %d", hpg, hpx);
          CHECK(hpg == 1 || hpg * (long long)nrb <= slots, "group of %d heads x %d blocks over %lld", hpg, nrb, slots);
          for (int d = hpg + 1; d <= hpx; ++d)
            CHECK(hpx % d != 0 || d * (long long)nrb > slots, "a larger group (%d) fits", d);
        }
        const int grid = nrb * BH;
        std::vector<int> seen(grid, 0), xcd_of(BH, -1);
        bool ok = true;
        for (int job = 0; job < grid; ++job) {
          int blk = -1, bh = -1;
          xcd_job(job, BH, hpx, hpg, nrb, blk, bh);
          if (blk < 0 || blk >= nrb || bh < 0 || bh >= BH) {
            ok = false;
            break;
          }
          ++seen[blk * BH + bh];
          if (hpx > 0) {
            if (xcd_of[bh] < 0) xcd_of[bh] = job & 7;
            ok = ok && xcd_of[bh] == (job & 7);
            // the heads of a group occupy consecutive jobs of their XCD
            ok = ok && ((job >> 3) / (hpg * nrb)) == (bh - (job & 7) * hpx) / hpg;
          }
        }
        for (int i = 0; ok && i < grid; ++i) ok = seen[i] == 1;
        CHECK(ok, "xcd_job BH=%d blocks=%d slots=%lld: not one to one, or a head off its XCD or group", BH, nrb,
              slots);
        // key split: the doubled grid pairs up on one job, both halves on one XCD
        std::vector<int> halves(2 * grid, 0);
        bool sok = true;
        for (int w = 0; w < 2 * grid; ++w) {
          int job = -1, ks = -1;
          split_job(w, hpx, job, ks);
          if (job < 0 || job >= grid || ks < 0 || ks > 1) {
            sok = false;
            break;
          }
          ++halves[2 * job + ks];
          if (hpx > 0) sok = sok && (w & 7) == (job & 7);
        }
        for (int i = 0; sok && i < 2 * grid; ++i) sok = halves[i] == 1;
        CHECK(sok, "split_job BH=%d blocks=%d: not one to one or halves on different XCDs", BH, nrb);
      }
}

int main() {
  check_tables();
  check_job_map();
  // zigzag rings: every size up to the driver's limit, first, middle and last rank
  for (int N = 1; N <= CP_MAX_STEPS; ++N) {
    std::set<int> ranks = {0, N / 2, N - 1};
    for (int r : ranks)
      for (int per = 1; per <= 4; ++per) {
        cp_chunks_t q;
        zigzag_table(N, r, 64, &q);
        std::vector<cp_chunks_t> kv(N);
        for (int j = 0; j < N; ++j) zigzag_table(N, ((r - j) % N + N) % N, 64, &kv[j]);
        char what[64];
        std::snprintf(what, sizeof(what), "zigzag N=%d r=%d per=%d", N, r, per);
        check_fwd_plan(q, kv, per, what);
      }
  }
  // odd tables: 1..8 chunks, chunk lengths 64..256, random disjoint starts,
  // tables that repeat across steps, keys past or before every query
  std::mt19937_64 rng(12345);
  for (int trial = 0; trial < 400; ++trial) {
    const int nq = 1 + (int)(rng() % 8), nkv = 1 + (int)(rng() % 8);
    const int lq = 64 * (1 + (int)(rng() % 4)), lk = 64 * (1 + (int)(rng() % 4));
    const int n = 1 + (int)(rng() % 12);
    auto table = [&](int nc, int len) {
      cp_chunks_t t{};
      t.n_chunks = nc;
      t.chunk_len = len;
      std::vector<int> slots(24);
      for (int i = 0; i < 24; ++i) slots[i] = i;
      std::shuffle(slots.begin(), slots.end(), rng);
      for (int i = 0; i < nc; ++i) t.start[i] = (int64_t)slots[i] * 256 + (int64_t)(rng() % 3) * 64 * (len < 192);
      return t;
    };
    cp_chunks_t q = table(nq, lq);
    std::string err;
    if (check_chunks(&q, "q", &err) != CP_OK) continue;
    std::vector<cp_chunks_t> kv;
    bool ok = true;
    for (int j = 0; j < n; ++j) {
      kv.push_back(table(nkv, lk));
      ok = ok && check_chunks(&kv.back(), "kv", &err) == CP_OK;
    }
    if (!ok) continue;
    for (int per = 1; per <= 4; ++per) {
      char what[96];
      std::snprintf(what, sizeof(what), "odd trial %d nq=%d nkv=%d n=%d per=%d", trial, nq, nkv, n, per);
      check_fwd_plan(q, kv, per, what);
    }
  }
  // backward rings: the ring's own pattern (step 0 writes, later steps add),
  // every step adding, none adding, and random patterns
  for (int n = 1; n <= CP_MAX_STEPS; ++n) {
    std::vector<std::vector<bool>> pats;
    std::vector<bool> ring(n, true);
    ring[0] = false;
    pats.push_back(ring);
    pats.push_back(std::vector<bool>(n, true));
    pats.push_back(std::vector<bool>(n, false));
    for (int k = 0; k < 2; ++k) {
      std::vector<bool> a(n);
      for (int j = 0; j < n; ++j) a[j] = rng() & 1;
      pats.push_back(a);
    }
    for (size_t k = 0; k < pats.size(); ++k) {
      char what[64];
      std::snprintf(what, sizeof(what), "backward n=%d pattern %zu", n, k);
      check_bwd_plan(n, pats[k], what);
    }
  }
  std::printf("ring plan checks: %ld passed, %d failed\n", g_checks - g_fail, g_fail);
  return g_fail == 0 ? 0 : 1;
}
