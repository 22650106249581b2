// C ABI of the causal ring-attention library: argument checks, per-step work
// planning, the one-GPU ring replay (staging slots, side stream, events) and
// kernel timing.  See include/cp_attn.h for the contract of each entry point.
//
// Sources (web pages, cited by title and section):
//   [MLM] "Megatron-LM源码解析：Context Parallel如何革新长序列训练", section 5
//         (double-buffered loop of cp_size+1 iterations: while step i computes
//         on buffer i%2, the transfer for step i+1 fills the other buffer on
//         its own stream) and section 3 (the context-parallel work runs on a
//         dedicated stream).
//   [RAF] "如何用Context并行加速大模型训练？手把手教你配置RingAttention+FlashAttention",
//         section 3 (ring order: step j uses the block of rank (rank - j) mod N)
//         and section 5, item 1 (2N zigzag chunks).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/cp_attn.h"
#include "cp_attn_internal.h"
#include "cp_attn_fp8.h"
#include "cp_attn_ring.h"
#include "cp_ring_plan.h"

using cpattn::StepArgs;
using cpattn::kSplitMaxBlocks;
using cpattn::kSplitRows;

static_assert(cpplan::kMerge == cpattn::kFlagMerge && cpplan::kFinalize == cpattn::kFlagFinalize &&
                  cpplan::kWriteO == cpattn::kFlagWriteO,
              "plan flags are the step kernels' flags");
static_assert(cpplan::kMerge == CP_PLAN_MERGE && cpplan::kFinalize == CP_PLAN_FINALIZE &&
                  cpplan::kWriteO == CP_PLAN_WRITE_O,
              "the published plan flags are the planner's");

// Most ring steps one step-kernel launch of cp_ring_attn_fwd covers; a
// staging slot holds this many K/V blocks.
constexpr int kStepsPerLaunch = cpattn::kMaxStepsPerLaunch;
// Longest delay cp_test_set_delays accepts.
constexpr int kMaxTestDelayUs = 100000;

namespace {

thread_local std::string g_last_error;

cp_status_t fail(cp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cp_status_t hip_fail(hipError_t e, const char* what) {
  return fail(CP_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

cp_status_t check_chunks(const cp_chunks_t* t, const char* name) {
  std::string err;
  const cp_status_t st = cpplan::check_chunks(t, name, &err);
  if (st != CP_OK) return fail(st, "%s", err.c_str());
  return CP_OK;
}

cp_status_t check_common(int B, int H, int D, float scale) {
  if (B < 1 || H < 1) return fail(CP_ERR_INVALID, "B = %d and H = %d must be >= 1", B, H);
  if ((long long)B * H > (1LL << 24)) return fail(CP_ERR_INVALID, "B*H = %lld too large", (long long)B * H);
  if (D != 64 && D != 128) return fail(CP_ERR_UNSUPPORTED, "head dim D = %d not built (64 or 128)", D);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(CP_ERR_INVALID, "softmax_scale = %g must be finite and > 0", (double)scale);
  return CP_OK;
}

using cpplan::pairs_for_chunk;

// Append the chunks of one [BH, Skv, D] K/V block (table `kvc`) to a launch.
void add_kv_block(StepArgs& a, const void* k, const void* v, const cp_chunks_t* kvc) {
  for (int i = 0; i < kvc->n_chunks; ++i, ++a.n_kv_chunks) {
    const size_t off = (size_t)i * kvc->chunk_len * (size_t)a.D;
    a.kc[a.n_kv_chunks] = static_cast<const uint16_t*>(k) + off;
    a.vc[a.n_kv_chunks] = static_cast<const uint16_t*>(v) + off;
    a.kv_start[a.n_kv_chunks] = (int)kvc->start[i];
  }
}

// Fill the launch arguments shared by every step for one K/V block; flags
// and order are set by the caller, further blocks added by add_kv_block.
void base_args(StepArgs& a, const void* q, const void* k, const void* v, float* o, float* lse, void* out,
               int B, int H, int D, const cp_chunks_t* qc, const cp_chunks_t* kvc, float scale) {
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.o_run = o;
  a.lse_run = lse;
  a.out = static_cast<uint16_t*>(out);
  a.BH = B * H;
  a.D = D;
  a.Sq = qc->n_chunks * qc->chunk_len;
  a.Skv = kvc->n_chunks * kvc->chunk_len;
  a.q_chunk_len = qc->chunk_len;
  a.kv_chunk_len = kvc->chunk_len;
  for (int i = 0; i < qc->n_chunks; ++i) a.q_start[i] = (int)qc->start[i];
  add_kv_block(a, k, v, kvc);
  a.rb_per_chunk = qc->chunk_len / cpattn::step_block_rows(qc->chunk_len);
  a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
  a.heads_per_group = a.heads_per_xcd;
  a.scale_log2 = scale * 1.4426950408889634f;
}

// Order the active query chunks heaviest first so long-running workgroups start early.
void set_order(StepArgs& a, const std::vector<int>& active, const std::vector<long long>& work) {
  std::vector<int> idx(active);
  std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return work[x] > work[y]; });
  a.n_order = (int)idx.size();
  for (int i = 0; i < a.n_order; ++i) a.order[i] = idx[i];
}

// ---------------- kernel timing ----------------
struct Profiler {
  std::mutex mu;
  bool enabled = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  std::vector<const char*> names;  // per used entry: the launched kernel (static string), or null
  size_t used = 0;
};
Profiler& profiler() {
  static Profiler p;
  return p;
}
constexpr size_t kMaxTimed = 4096;

// Run one kernel launch, `launch(stream, &name)`, bracketed by two timing
// events while profiling is enabled; the name it reports is kept with them.
template <class Launch>
hipError_t timed(hipStream_t s, Launch&& launch) {
  Profiler& p = profiler();
  long slot = -1;
  std::pair<hipEvent_t, hipEvent_t> evs{};
  {
    std::lock_guard<std::mutex> lk(p.mu);
    if (p.enabled && p.used < kMaxTimed) {
      if (p.used == p.ev.size()) {
        hipEvent_t e0, e1;
        // device-scope release: the timed kernels only need ordering on the GPU
        hipError_t e = hipEventCreateWithFlags(&e0, hipEventReleaseToDevice);
        if (e != hipSuccess) return e;
        e = hipEventCreateWithFlags(&e1, hipEventReleaseToDevice);
        if (e != hipSuccess) return e;
        p.ev.emplace_back(e0, e1);
        p.names.push_back(nullptr);
      }
      slot = (long)p.used++;
      evs = p.ev[slot];
    }
  }
  hipError_t e;
  if (slot >= 0 && (e = hipEventRecord(evs.first, s)) != hipSuccess) return e;
  const char* name = nullptr;
  e = launch(s, &name);
  if (e != hipSuccess) return e;
  if (slot >= 0) {
    {
      std::lock_guard<std::mutex> lk(p.mu);
      p.names[slot] = name;
    }
    if ((e = hipEventRecord(evs.second, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_step_timed(const StepArgs& a, int D, hipStream_t s) {
  return timed(s, [&](hipStream_t st, const char** nm) { return cpattn::launch_step(a, D, st, nm); });
}

// Launch arguments of the two backward kernels for one K/V block.
cpattn::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* d_out, const float* lse,
                         const float* delta, float* dq, float* dk, float* dv, int B, int H, int D,
                         const cp_chunks_t* qc, const cp_chunks_t* kvc, float scale, int mode) {
  cpattn::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.dout = static_cast<const uint16_t*>(d_out);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.BH = B * H;
  a.D = D;
  a.Sq = qc->n_chunks * qc->chunk_len;
  a.Skv = kvc->n_chunks * kvc->chunk_len;
  a.q_chunk_len = qc->chunk_len;
  a.kv_chunk_len = kvc->chunk_len;
  a.n_q_chunks = qc->n_chunks;
  a.n_kv_chunks = kvc->n_chunks;
  for (int i = 0; i < a.n_q_chunks; ++i) a.q_start[i] = (int)qc->start[i];
  for (int i = 0; i < a.n_kv_chunks; ++i) a.kv_start[i] = (int)kvc->start[i];
  a.accumulate = mode;
  a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
  a.heads_per_group = a.heads_per_xcd;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  return a;
}

// Both backward kernels of one block (dq rows, then dk/dv rows), each timed.
hipError_t launch_bwd_pair(const cpattn::BwdArgs& a, hipStream_t stream) {
  hipError_t e = timed(stream, [&](hipStream_t s, const char** nm) { return cpattn::launch_bwd_dq(a, s, nm); });
  if (e != hipSuccess) return e;
  return timed(stream, [&](hipStream_t s, const char** nm) { return cpattn::launch_bwd_dkdv(a, s, nm); });
}

// ---------------- ring-driver event pool (per device) ----------------
std::mutex g_pool_mu;
std::map<int, std::vector<hipEvent_t>> g_pools;

cp_status_t get_events(int n, std::vector<hipEvent_t>& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_pool_mu);
  auto& pool = g_pools[dev];
  while ((int)pool.size() < n) {
    hipEvent_t ev;
    // ordering between two streams of one device needs no system-scope fence
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    pool.push_back(ev);
  }
  out.assign(pool.begin(), pool.begin() + n);
  return CP_OK;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------- test hook: bounded delays inside a ring replay ----------------
// While set (cp_test_set_delays), every kernel launch of a ring driver is
// preceded on the compute stream by a spin of compute_us microseconds, and
// every staging copy on the copy stream by one of copy_us: a launch then
// reads its slot late while the copies run ahead, or a copy lands late, so a
// missing wait would change the result.
std::mutex g_delay_mu;
int g_delay_us[2] = {0, 0};  // [compute, copy]

hipError_t test_delay(int stream_kind, hipStream_t s) {
  int us;
  {
    std::lock_guard<std::mutex> lk(g_delay_mu);
    us = g_delay_us[stream_kind];
  }
  return us > 0 ? cpattn::launch_delay(us, s) : hipSuccess;
}

// ---------------- ring replay shared by the bf16 and fp8 forwards ----------------
// One launch of a ring forward: the steps it covers, the base of each step's
// K and V block (the caller's for step 0, a staging slot after it), the query
// chunks it computes with their merge/finalize flags, and their work.
struct RingLaunch {
  int first_step = 0, count = 0;
  const void* k[kStepsPerLaunch] = {};
  const void* v[kStepsPerLaunch] = {};
  std::vector<int> active;
  int flags[CP_MAX_CHUNKS] = {};
  std::vector<long long> work;
};

// Execute the forward ring plan (cpplan::plan_ring_fwd: step 0 on the
// caller's block, then groups of at most `per` steps, double-buffered
// staging slots on copy_stream).  `slots` holds the two slots, K blocks then
// V blocks (kv_bytes each, 256-byte aligned): K slot 0 [0, per), K slot 1
// [per, 2 per), V slot 0 [2 per, 3 per), V slot 1 [3 per, 4 per) in blocks,
// so a slot's blocks are adjacent.  `launch(rl)` enqueues the kernel of one
// launch on `stream`.
template <class Launch>
cp_status_t ring_replay(const cp_chunks_t* q_chunks, const void* const* k_steps, const void* const* v_steps,
                        const cp_chunks_t* kv_chunks_steps, int n_steps, int per, size_t kv_bytes,
                        unsigned char* slots, hipStream_t stream, hipStream_t copy_stream, Launch&& launch) {
  cp_status_t st;
  cpplan::FwdPlan plan;
  cpplan::plan_ring_fwd(q_chunks, kv_chunks_steps, n_steps, per, &plan);
  const size_t kv_slot = round256(kv_bytes);
  auto slot_k = [&](int slot, int i) -> void* { return slots + (size_t)(per * slot + i) * kv_slot; };
  auto slot_v = [&](int slot, int i) -> void* { return slots + (size_t)(2 * per + per * slot + i) * kv_slot; };

  std::vector<hipEvent_t> ev;
  if ((st = get_events(plan.n_events, ev)) != CP_OK) return st;
  hipError_t e;
#define HIP_TRY(call, what)                                   \
  do {                                                        \
    if ((e = (call)) != hipSuccess) return hip_fail(e, what); \
  } while (0)
  for (const cpplan::Op& op : plan.ops) {
    const hipStream_t s = op.stream == cpplan::kCompute ? stream : copy_stream;
    switch (op.kind) {
      case cpplan::OpKind::Record:
        HIP_TRY(hipEventRecord(ev[op.event], s), "hipEventRecord");
        break;
      case cpplan::OpKind::Wait:
        HIP_TRY(hipStreamWaitEvent(s, ev[op.event], 0), "hipStreamWaitEvent");
        break;
      case cpplan::OpKind::Stage: {
        const cpplan::FwdLaunch& L = plan.launches[op.index];
        HIP_TRY(test_delay(op.stream, s), "delay kernel launch");
        for (int i = 0; i < L.count; ++i) {
          const int j = L.first_step + i;
          HIP_TRY(cpattn::launch_stage_copy(k_steps[j], slot_k(L.slot, i), v_steps[j], slot_v(L.slot, i), kv_bytes, s),
                  "staging copy launch");
        }
        break;
      }
      case cpplan::OpKind::Launch: {
        const cpplan::FwdLaunch& L = plan.launches[op.index];
        RingLaunch rl;
        rl.first_step = L.first_step;
        rl.count = L.count;
        for (int i = 0; i < L.count; ++i) {
          rl.k[i] = L.slot < 0 ? k_steps[0] : slot_k(L.slot, i);
          rl.v[i] = L.slot < 0 ? v_steps[0] : slot_v(L.slot, i);
        }
        rl.active.assign(L.active, L.active + L.n_active);
        for (int c = 0; c < CP_MAX_CHUNKS; ++c) rl.flags[c] = L.flags[c];
        rl.work.assign(L.work, L.work + CP_MAX_CHUNKS);
        if (op.index > 0) HIP_TRY(test_delay(op.stream, s), "delay kernel launch");
        HIP_TRY(launch(rl), "step kernel launch");
        break;
      }
      default:
        return fail(CP_ERR_INVALID, "internal: backward operation in a forward plan");
    }
  }
#undef HIP_TRY
  return CP_OK;
}

}  // namespace

extern "C" {

const char* cp_last_error(void) { return g_last_error.c_str(); }

int cp_version(void) { return 100; }

cp_status_t cp_zigzag_chunks(int cp_size, int rank, int chunk_len, int step, cp_chunks_t* q_chunks,
                             cp_chunks_t* kv_chunks) {
  if (cp_size < 1) return fail(CP_ERR_INVALID, "cp_size = %d must be >= 1", cp_size);
  if (rank < 0 || rank >= cp_size) return fail(CP_ERR_INVALID, "rank = %d outside [0, %d)", rank, cp_size);
  if (step < 0 || step >= cp_size) return fail(CP_ERR_INVALID, "step = %d outside [0, %d)", step, cp_size);
  if (chunk_len <= 0) return fail(CP_ERR_INVALID, "chunk_len = %d must be > 0", chunk_len);
  if (2 * (int64_t)cp_size * chunk_len > (int64_t)INT32_MAX)
    return fail(CP_ERR_INVALID, "sequence of 2 * %d chunks of %d tokens exceeds 2^31 - 1 positions", cp_size, chunk_len);
  if (q_chunks) cpplan::zigzag_table(cp_size, rank, chunk_len, q_chunks);
  if (kv_chunks) cpplan::zigzag_table(cp_size, ((rank - step) % cp_size + cp_size) % cp_size, chunk_len, kv_chunks);
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_attn_step_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                             void* out_bf16_or_null, int B, int H, int D, const cp_chunks_t* q_chunks,
                             const cp_chunks_t* kv_chunks, float softmax_scale, int mode, hipStream_t stream) {
  cp_status_t st = check_common(B, H, D, softmax_scale);
  if (st != CP_OK) return st;
  if ((st = check_chunks(q_chunks, "q_chunks")) != CP_OK) return st;
  if ((st = check_chunks(kv_chunks, "kv_chunks")) != CP_OK) return st;
  if (mode != CP_STEP_WRITE && mode != CP_STEP_MERGE) return fail(CP_ERR_INVALID, "mode = %d unknown", mode);
  if (!q || !k || !v || !o || !lse) return fail(CP_ERR_INVALID, "q, k, v, o and lse must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(out_bf16_or_null, 16))
    return fail(CP_ERR_INVALID, "q, k, v, o, out must be 16-byte aligned and lse 4-byte aligned");
  const size_t BH = (size_t)B * H;
  const size_t Sq = (size_t)q_chunks->n_chunks * q_chunks->chunk_len;
  const size_t Skv = (size_t)kv_chunks->n_chunks * kv_chunks->chunk_len;
  const size_t qb = BH * Sq * D * 2, kvb = BH * Skv * D * 2, ob = BH * Sq * D * 4, lb = BH * Sq * 4;
  const void* ins[3] = {q, k, v};
  const size_t insz[3] = {qb, kvb, kvb};
  for (int i = 0; i < 3; ++i)
    if (overlaps(ins[i], insz[i], o, ob) || overlaps(ins[i], insz[i], lse, lb) ||
        overlaps(ins[i], insz[i], out_bf16_or_null, qb))
      return fail(CP_ERR_INVALID, "inputs must not alias o, lse or out");
  if (overlaps(o, ob, lse, lb) || overlaps(o, ob, out_bf16_or_null, qb) || overlaps(lse, lb, out_bf16_or_null, qb))
    return fail(CP_ERR_INVALID, "o, lse and out must not overlap");

  StepArgs a;
  base_args(a, q, k, v, o, lse, out_bf16_or_null, B, H, D, q_chunks, kv_chunks, softmax_scale);
  std::vector<int> active;
  std::vector<long long> work(CP_MAX_CHUNKS, 0);
  for (int c = 0; c < q_chunks->n_chunks; ++c) {
    work[c] = pairs_for_chunk(q_chunks, c, kv_chunks);
    const bool needed = (mode == CP_STEP_WRITE) || work[c] > 0 || out_bf16_or_null != nullptr;
    if (needed) active.push_back(c);
    a.flags[c] = (mode == CP_STEP_MERGE ? cpattn::kFlagMerge : 0) | cpattn::kFlagWriteO |
                 (out_bf16_or_null ? cpattn::kFlagFinalize : 0);
  }
  set_order(a, active, work);
  hipError_t e = launch_step_timed(a, D, stream);
  if (e != hipSuccess) return hip_fail(e, "step kernel launch");
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_attn_step_fwd_fp8(const void* q, const void* k, const void* vt, float* o, float* lse,
                                 void* out_bf16_or_null, int B, int H, int D, const cp_chunks_t* q_chunks,
                                 const cp_chunks_t* kv_chunks, float softmax_scale, float q_scale, float k_scale,
                                 float v_scale, int mode, hipStream_t stream) {
  cp_status_t st = check_common(B, H, D, softmax_scale);
  if (st != CP_OK) return st;
  if ((st = check_chunks(q_chunks, "q_chunks")) != CP_OK) return st;
  if ((st = check_chunks(kv_chunks, "kv_chunks")) != CP_OK) return st;
  if (D != 128) return fail(CP_ERR_UNSUPPORTED, "fp8 step: head dim D = %d not built (128)", D);
  if (q_chunks->chunk_len % cpattn::kFp8RowQuantum != 0)
    return fail(CP_ERR_UNSUPPORTED, "fp8 step: q chunk_len = %d must be a multiple of %d", q_chunks->chunk_len,
                cpattn::kFp8RowQuantum);
  const float sc[3] = {q_scale, k_scale, v_scale};
  for (float x : sc)
    if (!std::isfinite(x) || !(x > 0.f)) return fail(CP_ERR_INVALID, "fp8 step: scales must be finite and > 0");
  if (mode != CP_STEP_WRITE && mode != CP_STEP_MERGE) return fail(CP_ERR_INVALID, "mode = %d unknown", mode);
  if (!q || !k || !vt || !o || !lse) return fail(CP_ERR_INVALID, "q, k, vt, o and lse must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vt, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(out_bf16_or_null, 16))
    return fail(CP_ERR_INVALID, "q, k, vt, o, out must be 16-byte aligned and lse 4-byte aligned");
  const size_t BH = (size_t)B * H;
  const size_t Sq = (size_t)q_chunks->n_chunks * q_chunks->chunk_len;
  const size_t Skv = (size_t)kv_chunks->n_chunks * kv_chunks->chunk_len;
  const size_t qb = BH * Sq * D, kvb = BH * Skv * D, ob = BH * Sq * D * 4, lb = BH * Sq * 4, outb = BH * Sq * D * 2;
  const void* ins[3] = {q, k, vt};
  const size_t insz[3] = {qb, kvb, kvb};
  for (int i = 0; i < 3; ++i)
    if (overlaps(ins[i], insz[i], o, ob) || overlaps(ins[i], insz[i], lse, lb) ||
        overlaps(ins[i], insz[i], out_bf16_or_null, outb))
      return fail(CP_ERR_INVALID, "inputs must not alias o, lse or out");
  if (overlaps(o, ob, lse, lb) || overlaps(o, ob, out_bf16_or_null, outb) || overlaps(lse, lb, out_bf16_or_null, outb))
    return fail(CP_ERR_INVALID, "o, lse and out must not overlap");

  cpattn::Fp8StepArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint8_t*>(q);
  a.o = o;
  a.lse = lse;
  a.out = static_cast<uint16_t*>(out_bf16_or_null);
  a.BH = (int)BH;
  a.Sq = (int)Sq;
  a.Skv = (int)Skv;
  a.q_chunk_len = q_chunks->chunk_len;
  a.kv_chunk_len = kv_chunks->chunk_len;
  a.n_kv_chunks = kv_chunks->n_chunks;
  for (int i = 0; i < q_chunks->n_chunks; ++i) a.q_start[i] = (int)q_chunks->start[i];
  for (int i = 0; i < kv_chunks->n_chunks; ++i) {
    a.kc[i] = static_cast<const uint8_t*>(k) + (size_t)i * kv_chunks->chunk_len * D;
    a.vtc[i] = static_cast<const uint8_t*>(vt) + (size_t)i * kv_chunks->chunk_len;
    a.kv_start[i] = (int)kv_chunks->start[i];
  }
  a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
  a.heads_per_group = a.heads_per_xcd;
  a.scale_log2 = softmax_scale * q_scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  std::vector<int> idx;
  std::vector<long long> work(CP_MAX_CHUNKS, 0);
  for (int c = 0; c < q_chunks->n_chunks; ++c) {
    work[c] = pairs_for_chunk(q_chunks, c, kv_chunks);
    if (mode == CP_STEP_WRITE || work[c] > 0 || out_bf16_or_null) idx.push_back(c);
    a.flags[c] = (mode == CP_STEP_MERGE ? cpattn::kFlagMerge : 0) | cpattn::kFlagWriteO |
                 (out_bf16_or_null ? cpattn::kFlagFinalize : 0);
  }
  std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return work[x] > work[y]; });
  a.n_order = (int)idx.size();
  for (int i = 0; i < a.n_order; ++i) a.order[i] = idx[i];
  hipError_t e = timed(stream, [&](hipStream_t s, const char** nm) { return cpattn::launch_step_fp8(a, s, nm); });
  if (e != hipSuccess) return hip_fail(e, "fp8 step kernel launch");
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_attn_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part, int B, int H,
                          int Sq, int D, void* out_bf16_or_null, hipStream_t stream) {
  if (B < 1 || H < 1 || Sq < 0) return fail(CP_ERR_INVALID, "B, H must be >= 1 and Sq >= 0");
  if (D < 4 || D % 4 != 0) return fail(CP_ERR_INVALID, "D = %d must be a positive multiple of 4", D);
  if (Sq == 0) {  // nothing to merge; the pointers of empty tensors may be NULL
    g_last_error.clear();
    return CP_OK;
  }
  if (!o_acc || !lse_acc || !o_part || !lse_part) return fail(CP_ERR_INVALID, "NULL operand");
  if (!aligned(o_acc, 16) || !aligned(o_part, 16) || !aligned(out_bf16_or_null, 8) || !aligned(lse_acc, 4) ||
      !aligned(lse_part, 4))
    return fail(CP_ERR_INVALID, "o_acc/o_part must be 16-byte, out 8-byte, lse 4-byte aligned");
  const int64_t rows = (int64_t)B * H * Sq;
  const size_t ob = (size_t)rows * D * 4, lb = (size_t)rows * 4;
  if (overlaps(o_acc, ob, o_part, ob) || overlaps(lse_acc, lb, lse_part, lb) || overlaps(o_acc, ob, lse_acc, lb) ||
      overlaps(o_acc, ob, lse_part, lb) || overlaps(lse_acc, lb, o_part, ob) ||
      overlaps(out_bf16_or_null, (size_t)rows * D * 2, o_acc, ob) ||
      overlaps(out_bf16_or_null, (size_t)rows * D * 2, o_part, ob))
    return fail(CP_ERR_INVALID, "merge operands must not overlap");
  hipError_t e = cpattn::launch_merge(o_acc, lse_acc, o_part, lse_part, static_cast<uint16_t*>(out_bf16_or_null),
                                      rows, D, stream);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_attn_bwd_delta(const void* out, const void* d_out, float* delta, int B, int H, int Sq, int D,
                              hipStream_t stream) {
  if (B < 1 || H < 1 || Sq < 0) return fail(CP_ERR_INVALID, "B, H must be >= 1 and Sq >= 0");
  if ((long long)B * H > (1LL << 24)) return fail(CP_ERR_INVALID, "B*H = %lld too large", (long long)B * H);
  if (D != 64 && D != 128) return fail(CP_ERR_UNSUPPORTED, "head dim D = %d not built (64 or 128)", D);
  if (Sq == 0) {  // nothing to compute; the pointers of empty tensors may be NULL
    g_last_error.clear();
    return CP_OK;
  }
  if (!out || !d_out || !delta) return fail(CP_ERR_INVALID, "out, d_out and delta must be non-NULL");
  if (!aligned(out, 16) || !aligned(d_out, 16) || !aligned(delta, 4))
    return fail(CP_ERR_INVALID, "out, d_out must be 16-byte aligned and delta 4-byte aligned");
  const int64_t rows = (int64_t)B * H * Sq;
  const size_t xb = (size_t)rows * D * 2, db = (size_t)rows * 4;
  if (overlaps(delta, db, out, xb) || overlaps(delta, db, d_out, xb))
    return fail(CP_ERR_INVALID, "delta must not overlap out or d_out");
  hipError_t e = cpattn::launch_bwd_delta(static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(d_out),
                                          delta, rows, D, stream);
  if (e != hipSuccess) return hip_fail(e, "delta kernel launch");
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_attn_step_bwd(const void* q, const void* k, const void* v, const void* d_out, const float* lse,
                             const float* delta, float* dq, float* dk, float* dv, int B, int H, int D,
                             const cp_chunks_t* q_chunks, const cp_chunks_t* kv_chunks, float softmax_scale, int mode,
                             hipStream_t stream) {
  cp_status_t st = check_common(B, H, D, softmax_scale);
  if (st != CP_OK) return st;
  if ((st = check_chunks(q_chunks, "q_chunks")) != CP_OK) return st;
  if ((st = check_chunks(kv_chunks, "kv_chunks")) != CP_OK) return st;
  if (mode & ~(CP_BWD_DQ_ACCUMULATE | CP_BWD_DKV_ACCUMULATE)) return fail(CP_ERR_INVALID, "mode = %d unknown", mode);
  if (!q || !k || !v || !d_out || !lse || !delta || !dq || !dk || !dv)
    return fail(CP_ERR_INVALID, "every tensor argument must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_out, 16) || !aligned(dq, 16) ||
      !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return fail(CP_ERR_INVALID, "q, k, v, d_out, dq, dk, dv must be 16-byte aligned and lse, delta 4-byte aligned");
  const size_t BH = (size_t)B * H;
  const size_t Sq = (size_t)q_chunks->n_chunks * q_chunks->chunk_len;
  const size_t Skv = (size_t)kv_chunks->n_chunks * kv_chunks->chunk_len;
  const size_t qb = BH * Sq * D * 2, kvb = BH * Skv * D * 2, lb = BH * Sq * 4;
  const size_t dqb = BH * Sq * D * 4, dkb = BH * Skv * D * 4;
  const void* ins[6] = {q, k, v, d_out, lse, delta};
  const size_t insz[6] = {qb, kvb, kvb, qb, lb, lb};
  const void* outs[3] = {dq, dk, dv};
  const size_t outsz[3] = {dqb, dkb, dkb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return fail(CP_ERR_INVALID, "dq, dk, dv must not alias an input");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return fail(CP_ERR_INVALID, "dq, dk and dv must not overlap");
  }

  const cpattn::BwdArgs a = bwd_args(q, k, v, d_out, lse, delta, dq, dk, dv, B, H, D, q_chunks, kv_chunks,
                                     softmax_scale, mode);
  hipError_t e = launch_bwd_pair(a, stream);
  if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  g_last_error.clear();
  return CP_OK;
}

size_t cp_ring_attn_workspace_bytes(int B, int H, int Skv, int D, int Sq) {
  return cpattn::ring_fwd_workspace_bytes(B, H, Skv, D, Sq, kStepsPerLaunch);
}

}  // extern "C"

namespace cpattn {

// Rows of the key-split partial buffers of a ring workspace.
size_t split_rows(int B, int H, int Sq) { return std::min((size_t)kSplitRows, (size_t)B * H * Sq); }

size_t ring_fwd_workspace_bytes(int B, int H, int Skv, int D, int Sq, int steps_per_launch) {
  if (B <= 0 || H <= 0 || Skv <= 0 || D <= 0 || Sq <= 0 || steps_per_launch <= 0) return 0;
  const size_t kv = round256((size_t)B * H * Skv * D * 2);
  const size_t o = round256((size_t)B * H * Sq * D * 4);
  const size_t R = split_rows(B, H, Sq);
  const size_t split = round256(2 * R * D * 4) + round256(2 * R * 4) + round256((size_t)kSplitMaxBlocks * 4);
  return 4 * (size_t)steps_per_launch * kv + o + split;
}

cp_status_t ring_fwd(const void* q, const cp_chunks_t* q_chunks, const void* const* k_steps,
                     const void* const* v_steps, const cp_chunks_t* kv_chunks_steps, int n_steps, void* out, float* lse,
                     int B, int H, int D, float softmax_scale, void* workspace, size_t workspace_bytes,
                     int steps_per_launch, hipStream_t stream, hipStream_t copy_stream) {
  cp_status_t st = check_common(B, H, D, softmax_scale);
  if (st != CP_OK) return st;
  if (n_steps < 1 || n_steps > CP_MAX_STEPS)
    return fail(CP_ERR_INVALID, "n_steps = %d outside [1, %d]", n_steps, CP_MAX_STEPS);
  if (steps_per_launch < 1 || steps_per_launch > kStepsPerLaunch)
    return fail(CP_ERR_INVALID, "internal: %d steps per launch", steps_per_launch);
  if ((st = check_chunks(q_chunks, "q_chunks")) != CP_OK) return st;
  if (!k_steps || !v_steps || !kv_chunks_steps) return fail(CP_ERR_INVALID, "k_steps, v_steps, kv_chunks_steps NULL");
  for (int j = 0; j < n_steps; ++j) {
    char name[48];
    snprintf(name, sizeof(name), "kv_chunks_steps[%d]", j);
    if ((st = check_chunks(&kv_chunks_steps[j], name)) != CP_OK) return st;
    if (kv_chunks_steps[j].n_chunks != kv_chunks_steps[0].n_chunks ||
        kv_chunks_steps[j].chunk_len != kv_chunks_steps[0].chunk_len)
      return fail(CP_ERR_INVALID, "every step's K/V table must have the same n_chunks and chunk_len");
    if (!k_steps[j] || !v_steps[j] || !aligned(k_steps[j], 16) || !aligned(v_steps[j], 16))
      return fail(CP_ERR_INVALID, "k_steps[%d] / v_steps[%d] NULL or not 16-byte aligned", j, j);
  }
  if (!q || !out || !lse) return fail(CP_ERR_INVALID, "q, out and lse must be non-NULL");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return fail(CP_ERR_INVALID, "q, out must be 16-byte aligned and lse 4-byte aligned");
  if (!workspace || !aligned(workspace, 256)) return fail(CP_ERR_INVALID, "workspace NULL or not 256-byte aligned");
  if (!copy_stream && stream)
    return fail(CP_ERR_INVALID, "copy_stream is NULL (pass stream itself to run the copies in order)");
  const int Sq = q_chunks->n_chunks * q_chunks->chunk_len;
  const int Skv = kv_chunks_steps[0].n_chunks * kv_chunks_steps[0].chunk_len;
  const size_t need = ring_fwd_workspace_bytes(B, H, Skv, D, Sq, steps_per_launch);
  if (workspace_bytes < need)
    return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const size_t BH = (size_t)B * H;
  const size_t kv_bytes = BH * Skv * D * 2, q_bytes = BH * Sq * D * 2, lse_bytes = BH * Sq * 4;
  // no operand may overlap the workspace or the outputs
  const void* outs[3] = {workspace, out, lse};
  const size_t outsz[3] = {need, q_bytes, lse_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(q, q_bytes, outs[i], outsz[i])) return fail(CP_ERR_INVALID, "q overlaps an output or the workspace");
    for (int j = 0; j < n_steps; ++j)
      if (overlaps(k_steps[j], kv_bytes, outs[i], outsz[i]) || overlaps(v_steps[j], kv_bytes, outs[i], outsz[i]))
        return fail(CP_ERR_INVALID, "K/V of step %d overlaps an output or the workspace", j);
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j]))
        return fail(CP_ERR_INVALID, "out, lse and workspace must not overlap");
  }

  // workspace: staging slots, running O, key-split partials (O, LSE) and counters
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  unsigned char* p = ws + 4 * (size_t)steps_per_launch * round256(kv_bytes);
  float* o_run = reinterpret_cast<float*>(p);
  p += round256(BH * Sq * D * 4);
  const size_t R = split_rows(B, H, Sq);
  float* part_o = reinterpret_cast<float*>(p);
  p += round256(2 * R * D * 4);
  float* part_lse = reinterpret_cast<float*>(p);
  p += round256(2 * R * 4);
  unsigned* part_cnt = reinterpret_cast<unsigned*>(p);
  st = ring_replay(q_chunks, k_steps, v_steps, kv_chunks_steps, n_steps, steps_per_launch, kv_bytes, ws, stream,
                   copy_stream,
                   [&](const RingLaunch& rl) -> hipError_t {
                       StepArgs a;
                       base_args(a, q, rl.k[0], rl.v[0], o_run, lse, out, B, H, D, q_chunks,
                                 &kv_chunks_steps[rl.first_step], softmax_scale);
                       a.part_o = part_o;
                       a.part_lse = part_lse;
                       a.part_cnt = part_cnt;
                       a.part_rows = (int)R;
                       // the ring's first launch clears the key-split counters
                       a.cnt_to_clear = rl.first_step == 0 ? part_cnt : nullptr;
                       for (int i = 1; i < rl.count; ++i)
                         add_kv_block(a, rl.k[i], rl.v[i], &kv_chunks_steps[rl.first_step + i]);
                       for (int c : rl.active) a.flags[c] = rl.flags[c] | cpattn::kFlagLaneO;
                       set_order(a, rl.active, rl.work);
                       return launch_step_timed(a, D, stream);
                     });
  if (st == CP_OK) g_last_error.clear();
  return st;
}

cp_status_t fail_status(cp_status_t st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace cpattn

extern "C" {

cp_status_t cp_ring_attn_fwd(const void* q, const cp_chunks_t* q_chunks, const void* const* k_steps,
                             const void* const* v_steps, const cp_chunks_t* kv_chunks_steps, int n_steps, void* out,
                             float* lse, int B, int H, int D, float softmax_scale, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, hipStream_t copy_stream) {
  return cpattn::ring_fwd(q, q_chunks, k_steps, v_steps, kv_chunks_steps, n_steps, out, lse, B, H, D, softmax_scale,
                          workspace, workspace_bytes, kStepsPerLaunch, stream, copy_stream);
}

cp_status_t cp_ring_attn_fwd_plan(const cp_chunks_t* q_chunks, const cp_chunks_t* kv_chunks_steps, int n_steps,
                                  int max_launches, int* n_launches, int* first_step, int* step_count,
                                  int* chunk_flags) {
  cp_status_t st;
  if (n_steps < 1 || n_steps > CP_MAX_STEPS)
    return fail(CP_ERR_INVALID, "n_steps = %d outside [1, %d]", n_steps, CP_MAX_STEPS);
  if ((st = check_chunks(q_chunks, "q_chunks")) != CP_OK) return st;
  if (!kv_chunks_steps) return fail(CP_ERR_INVALID, "kv_chunks_steps is NULL");
  for (int j = 0; j < n_steps; ++j) {
    char name[48];
    snprintf(name, sizeof(name), "kv_chunks_steps[%d]", j);
    if ((st = check_chunks(&kv_chunks_steps[j], name)) != CP_OK) return st;
    if (kv_chunks_steps[j].n_chunks != kv_chunks_steps[0].n_chunks ||
        kv_chunks_steps[j].chunk_len != kv_chunks_steps[0].chunk_len)
      return fail(CP_ERR_INVALID, "every step's K/V table must have the same n_chunks and chunk_len");
  }
  if (!n_launches) return fail(CP_ERR_INVALID, "n_launches is NULL");
  cpplan::FwdPlan plan;
  cpplan::plan_ring_fwd(q_chunks, kv_chunks_steps, n_steps, kStepsPerLaunch, &plan);
  const int n = (int)plan.launches.size();
  *n_launches = n;
  for (int l = 0; l < n && l < max_launches; ++l) {
    const cpplan::FwdLaunch& L = plan.launches[l];
    if (first_step) first_step[l] = L.first_step;
    if (step_count) step_count[l] = L.count;
    if (chunk_flags)
      for (int c = 0; c < CP_MAX_CHUNKS; ++c) {
        bool active = false;
        for (int i = 0; i < L.n_active; ++i) active = active || L.active[i] == c;
        chunk_flags[l * CP_MAX_CHUNKS + c] = active ? (L.flags[c] | CP_PLAN_ACTIVE) : 0;
      }
  }
  g_last_error.clear();
  return CP_OK;
}

size_t cp_ring_attn_fwd_fp8_workspace_bytes(int B, int H, int Skv, int D, int Sq) {
  if (B <= 0 || H <= 0 || Skv <= 0 || D <= 0 || Sq <= 0) return 0;
  const size_t kv = round256((size_t)B * H * Skv * D);
  const size_t o = round256((size_t)B * H * Sq * D * 4);
  return 4 * kStepsPerLaunch * kv + o;
}

cp_status_t cp_ring_attn_fwd_fp8(const void* q, const cp_chunks_t* q_chunks, const void* const* k_steps,
                                 const void* const* vt_steps, const cp_chunks_t* kv_chunks_steps, int n_steps,
                                 void* out, float* lse, int B, int H, int D, float softmax_scale, float q_scale,
                                 float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, hipStream_t copy_stream) {
  cp_status_t st = check_common(B, H, D, softmax_scale);
  if (st != CP_OK) return st;
  if (D != 128) return fail(CP_ERR_UNSUPPORTED, "fp8 ring: head dim D = %d not built (128)", D);
  if (n_steps < 1 || n_steps > CP_MAX_STEPS)
    return fail(CP_ERR_INVALID, "n_steps = %d outside [1, %d]", n_steps, CP_MAX_STEPS);
  if ((st = check_chunks(q_chunks, "q_chunks")) != CP_OK) return st;
  if (q_chunks->chunk_len % cpattn::kFp8RowQuantum != 0)
    return fail(CP_ERR_UNSUPPORTED, "fp8 ring: q chunk_len = %d must be a multiple of %d", q_chunks->chunk_len,
                cpattn::kFp8RowQuantum);
  const float sc[3] = {q_scale, k_scale, v_scale};
  for (float x : sc)
    if (!std::isfinite(x) || !(x > 0.f)) return fail(CP_ERR_INVALID, "fp8 ring: scales must be finite and > 0");
  if (!k_steps || !vt_steps || !kv_chunks_steps) return fail(CP_ERR_INVALID, "k_steps, vt_steps, kv_chunks_steps NULL");
  for (int j = 0; j < n_steps; ++j) {
    char name[48];
    snprintf(name, sizeof(name), "kv_chunks_steps[%d]", j);
    if ((st = check_chunks(&kv_chunks_steps[j], name)) != CP_OK) return st;
    if (kv_chunks_steps[j].n_chunks != kv_chunks_steps[0].n_chunks ||
        kv_chunks_steps[j].chunk_len != kv_chunks_steps[0].chunk_len)
      return fail(CP_ERR_INVALID, "every step's K/V table must have the same n_chunks and chunk_len");
    if (!k_steps[j] || !vt_steps[j] || !aligned(k_steps[j], 16) || !aligned(vt_steps[j], 16))
      return fail(CP_ERR_INVALID, "k_steps[%d] / vt_steps[%d] NULL or not 16-byte aligned", j, j);
  }
  if (!q || !out || !lse) return fail(CP_ERR_INVALID, "q, out and lse must be non-NULL");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return fail(CP_ERR_INVALID, "q, out must be 16-byte aligned and lse 4-byte aligned");
  if (!workspace || !aligned(workspace, 256)) return fail(CP_ERR_INVALID, "workspace NULL or not 256-byte aligned");
  if (!copy_stream && stream)
    return fail(CP_ERR_INVALID, "copy_stream is NULL (pass stream itself to run the copies in order)");
  const int Sq = q_chunks->n_chunks * q_chunks->chunk_len;
  const int Skv = kv_chunks_steps[0].n_chunks * kv_chunks_steps[0].chunk_len;
  const size_t need = cp_ring_attn_fwd_fp8_workspace_bytes(B, H, Skv, D, Sq);
  if (workspace_bytes < need)
    return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const size_t BH = (size_t)B * H;
  const size_t kv_bytes = BH * Skv * D, q_bytes = BH * Sq * D, out_bytes = BH * Sq * D * 2, lse_bytes = BH * Sq * 4;
  const void* outs[3] = {workspace, out, lse};
  const size_t outsz[3] = {need, out_bytes, lse_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(q, q_bytes, outs[i], outsz[i])) return fail(CP_ERR_INVALID, "q overlaps an output or the workspace");
    for (int j = 0; j < n_steps; ++j)
      if (overlaps(k_steps[j], kv_bytes, outs[i], outsz[i]) || overlaps(vt_steps[j], kv_bytes, outs[i], outsz[i]))
        return fail(CP_ERR_INVALID, "K/V of step %d overlaps an output or the workspace", j);
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j]))
        return fail(CP_ERR_INVALID, "out, lse and workspace must not overlap");
  }

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* o_run = reinterpret_cast<float*>(ws + 4 * kStepsPerLaunch * round256(kv_bytes));
  st = ring_replay(q_chunks, k_steps, vt_steps, kv_chunks_steps, n_steps, kStepsPerLaunch, kv_bytes, ws, stream,
                   copy_stream,
                   [&](const RingLaunch& rl) -> hipError_t {
                     cpattn::Fp8StepArgs a;
                     std::memset(&a, 0, sizeof(a));
                     a.q = static_cast<const uint8_t*>(q);
                     a.o = o_run;
                     a.lse = lse;
                     a.out = static_cast<uint16_t*>(out);
                     a.BH = (int)BH;
                     a.Sq = Sq;
                     a.Skv = Skv;
                     a.q_chunk_len = q_chunks->chunk_len;
                     a.kv_chunk_len = kv_chunks_steps[0].chunk_len;
                     for (int i = 0; i < q_chunks->n_chunks; ++i) a.q_start[i] = (int)q_chunks->start[i];
                     for (int i = 0; i < rl.count; ++i) {
                       const cp_chunks_t& t = kv_chunks_steps[rl.first_step + i];
                       for (int c = 0; c < t.n_chunks; ++c, ++a.n_kv_chunks) {
                         a.kc[a.n_kv_chunks] = static_cast<const uint8_t*>(rl.k[i]) + (size_t)c * t.chunk_len * D;
                         a.vtc[a.n_kv_chunks] = static_cast<const uint8_t*>(rl.v[i]) + (size_t)c * t.chunk_len;
                         a.kv_start[a.n_kv_chunks] = (int)t.start[c];
                       }
                     }
                     a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
                     a.heads_per_group = a.heads_per_xcd;
                     a.scale_log2 = softmax_scale * q_scale * k_scale * 1.4426950408889634f;
                     a.v_scale = v_scale;
                     std::vector<int> idx(rl.active);
                     std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return rl.work[x] > rl.work[y]; });
                     a.n_order = (int)idx.size();
                     for (int i = 0; i < a.n_order; ++i) {
                       a.order[i] = idx[i];
                       a.flags[idx[i]] = rl.flags[idx[i]];
                     }
                     return timed(stream, [&](hipStream_t s, const char** nm) { return cpattn::launch_step_fp8(a, s, nm); });
                   });
  if (st == CP_OK) g_last_error.clear();
  return st;
}

size_t cp_ring_attn_bwd_workspace_bytes(int B, int H, int Skv, int D, int Sq) {
  if (B <= 0 || H <= 0 || Skv <= 0 || D <= 0 || Sq <= 0) return 0;
  const size_t kv = round256((size_t)B * H * Skv * D * 2);
  const size_t g = round256((size_t)B * H * Skv * D * 4);
  const size_t delta = round256((size_t)B * H * Sq * 4);
  return delta + 2 * (2 * kv + 2 * g);
}

cp_status_t cp_ring_attn_bwd(const void* q, const cp_chunks_t* q_chunks, const void* d_out, const void* out,
                             const float* lse, const void* const* k_steps, const void* const* v_steps,
                             const cp_chunks_t* kv_chunks_steps, int n_steps, float* const* dk_steps,
                             float* const* dv_steps, const int* dkv_accumulate, float* dq, int B, int H, int D,
                             float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream,
                             hipStream_t copy_stream) {
  cp_status_t st = check_common(B, H, D, softmax_scale);
  if (st != CP_OK) return st;
  if (n_steps < 1 || n_steps > CP_MAX_STEPS)
    return fail(CP_ERR_INVALID, "n_steps = %d outside [1, %d]", n_steps, CP_MAX_STEPS);
  if ((st = check_chunks(q_chunks, "q_chunks")) != CP_OK) return st;
  if (!k_steps || !v_steps || !kv_chunks_steps || !dk_steps || !dv_steps)
    return fail(CP_ERR_INVALID, "k_steps, v_steps, kv_chunks_steps, dk_steps, dv_steps must be non-NULL");
  for (int j = 0; j < n_steps; ++j) {
    char name[48];
    snprintf(name, sizeof(name), "kv_chunks_steps[%d]", j);
    if ((st = check_chunks(&kv_chunks_steps[j], name)) != CP_OK) return st;
    if (kv_chunks_steps[j].n_chunks != kv_chunks_steps[0].n_chunks ||
        kv_chunks_steps[j].chunk_len != kv_chunks_steps[0].chunk_len)
      return fail(CP_ERR_INVALID, "every step's K/V table must have the same n_chunks and chunk_len");
    if (!k_steps[j] || !v_steps[j] || !dk_steps[j] || !dv_steps[j] || !aligned(k_steps[j], 16) ||
        !aligned(v_steps[j], 16) || !aligned(dk_steps[j], 16) || !aligned(dv_steps[j], 16))
      return fail(CP_ERR_INVALID, "step %d: K, V, dK or dV NULL or not 16-byte aligned", j);
  }
  if (!q || !d_out || !out || !lse || !dq) return fail(CP_ERR_INVALID, "q, d_out, out, lse and dq must be non-NULL");
  if (!aligned(q, 16) || !aligned(d_out, 16) || !aligned(out, 16) || !aligned(dq, 16) || !aligned(lse, 4))
    return fail(CP_ERR_INVALID, "q, d_out, out, dq must be 16-byte aligned and lse 4-byte aligned");
  if (!workspace || !aligned(workspace, 256)) return fail(CP_ERR_INVALID, "workspace NULL or not 256-byte aligned");
  if (!copy_stream && stream)
    return fail(CP_ERR_INVALID, "copy_stream is NULL (pass stream itself to run the copies in order)");
  const int Sq = q_chunks->n_chunks * q_chunks->chunk_len;
  const int Skv = kv_chunks_steps[0].n_chunks * kv_chunks_steps[0].chunk_len;
  const size_t need = cp_ring_attn_bwd_workspace_bytes(B, H, Skv, D, Sq);
  if (workspace_bytes < need)
    return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const size_t BH = (size_t)B * H;
  const size_t kv_bytes = BH * Skv * D * 2, g_bytes = BH * Skv * D * 4;
  const size_t q_bytes = BH * Sq * D * 2, dq_bytes = BH * Sq * D * 4, lse_bytes = BH * Sq * 4;
  // outputs (dq, every dK/dV, the workspace) must not overlap each other or any input
  std::vector<std::pair<const void*, size_t>> ins = {{q, q_bytes}, {d_out, q_bytes}, {out, q_bytes}, {lse, lse_bytes}};
  std::vector<std::pair<const void*, size_t>> outs = {{workspace, need}, {dq, dq_bytes}};
  for (int j = 0; j < n_steps; ++j) {
    ins.emplace_back(k_steps[j], kv_bytes);
    ins.emplace_back(v_steps[j], kv_bytes);
    outs.emplace_back(dk_steps[j], g_bytes);
    outs.emplace_back(dv_steps[j], g_bytes);
  }
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const auto& in : ins)
      if (overlaps(outs[i].first, outs[i].second, in.first, in.second))
        return fail(CP_ERR_INVALID, "dq, dK/dV buffers and workspace must not overlap an input");
    for (size_t k = i + 1; k < outs.size(); ++k)
      if (overlaps(outs[i].first, outs[i].second, outs[k].first, outs[k].second))
        return fail(CP_ERR_INVALID, "dq, the dK/dV buffers of every step and the workspace must not overlap");
  }

  // workspace: Delta, then two slots of (K, V, dK, dV); step j >= 1 uses slot (j - 1) % 2
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* delta = reinterpret_cast<float*>(ws);
  unsigned char* slots = ws + round256(lse_bytes);
  const size_t kv_r = round256(kv_bytes), g_r = round256(g_bytes);
  const size_t slot_bytes = 2 * kv_r + 2 * g_r;
  auto slot_k = [&](int j) -> void* { return slots + (size_t)((j - 1) & 1) * slot_bytes; };
  auto slot_v = [&](int j) -> void* { return slots + (size_t)((j - 1) & 1) * slot_bytes + kv_r; };
  auto slot_dk = [&](int j) -> float* {
    return reinterpret_cast<float*>(slots + (size_t)((j - 1) & 1) * slot_bytes + 2 * kv_r);
  };
  auto slot_dv = [&](int j) -> float* {
    return reinterpret_cast<float*>(slots + (size_t)((j - 1) & 1) * slot_bytes + 2 * kv_r + g_r);
  };
  auto adds = [&](int j) { return dkv_accumulate ? dkv_accumulate[j] != 0 : j > 0; };

  cpplan::BwdPlan plan;
  cpplan::plan_ring_bwd(n_steps, &plan);
  std::vector<hipEvent_t> ev;
  if ((st = get_events(plan.n_events, ev)) != CP_OK) return st;
  hipError_t e;
#define HIP_TRY(call, what)                                   \
  do {                                                        \
    if ((e = (call)) != hipSuccess) return hip_fail(e, what); \
  } while (0)
  for (const cpplan::Op& op : plan.ops) {
    const hipStream_t s = op.stream == cpplan::kCompute ? stream : copy_stream;
    const int j = op.index;
    switch (op.kind) {
      case cpplan::OpKind::Record:
        HIP_TRY(hipEventRecord(ev[op.event], s), "hipEventRecord");
        break;
      case cpplan::OpKind::Wait:
        HIP_TRY(hipStreamWaitEvent(s, ev[op.event], 0), "hipStreamWaitEvent");
        break;
      case cpplan::OpKind::Receive:  // the block, and the partial sums it carries
        HIP_TRY(test_delay(op.stream, s), "delay kernel launch");
        HIP_TRY(cpattn::launch_stage_copy(k_steps[j], slot_k(j), v_steps[j], slot_v(j), kv_bytes, s),
                "staging copy launch");
        if (adds(j))
          HIP_TRY(cpattn::launch_stage_copy(dk_steps[j], slot_dk(j), dv_steps[j], slot_dv(j), g_bytes, s),
                  "staging copy launch");
        break;
      case cpplan::OpKind::Delta:
        HIP_TRY(cpattn::launch_bwd_delta(static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(d_out),
                                         delta, (int64_t)BH * Sq, D, s),
                "delta kernel launch");
        break;
      case cpplan::OpKind::Kernels: {
        const int mode = (j > 0 ? CP_BWD_DQ_ACCUMULATE : 0) | (adds(j) ? CP_BWD_DKV_ACCUMULATE : 0);
        cpattn::BwdArgs a;
        if (j == 0) {  // the rank's own block, in place
          a = bwd_args(q, k_steps[0], v_steps[0], d_out, lse, delta, dq, dk_steps[0], dv_steps[0], B, H, D, q_chunks,
                       &kv_chunks_steps[0], softmax_scale, mode);
        } else {
          HIP_TRY(test_delay(op.stream, s), "delay kernel launch");
          a = bwd_args(q, slot_k(j), slot_v(j), d_out, lse, delta, dq, slot_dk(j), slot_dv(j), B, H, D, q_chunks,
                       &kv_chunks_steps[j], softmax_scale, mode);
        }
        HIP_TRY(launch_bwd_pair(a, s), "backward kernel launch");
        break;
      }
      case cpplan::OpKind::Send:  // the updated partial sums leave the slot
        HIP_TRY(test_delay(op.stream, s), "delay kernel launch");
        HIP_TRY(cpattn::launch_stage_copy(slot_dk(j), dk_steps[j], slot_dv(j), dv_steps[j], g_bytes, s),
                "staging copy launch");
        break;
      default:
        return fail(CP_ERR_INVALID, "internal: forward operation in a backward plan");
    }
  }
#undef HIP_TRY
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_test_set_delays(int compute_us, int copy_us) {
  if (compute_us < 0 || copy_us < 0 || compute_us > kMaxTestDelayUs || copy_us > kMaxTestDelayUs)
    return fail(CP_ERR_INVALID, "delays must be in [0, %d] microseconds", kMaxTestDelayUs);
  std::lock_guard<std::mutex> lk(g_delay_mu);
  g_delay_us[cpplan::kCompute] = compute_us;
  g_delay_us[cpplan::kCopy] = copy_us;
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_profile_enable(int enable) {
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  p.enabled = enable != 0;
  p.used = 0;
  return CP_OK;
}

cp_status_t cp_profile_read_named(float* kernel_ms, const char** kernel_names, int max_entries, int* n_entries) {
  Profiler& p = profiler();
  std::lock_guard<std::mutex> lk(p.mu);
  int n = 0;
  for (size_t i = 0; i < p.used; ++i) {
    hipError_t e = hipEventSynchronize(p.ev[i].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    if (n < max_entries) {
      if (kernel_ms) {
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, p.ev[i].first, p.ev[i].second);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        kernel_ms[n] = ms;
      }
      if (kernel_names) kernel_names[n] = p.names[i] ? p.names[i] : "";
      ++n;
    }
  }
  if (n_entries) *n_entries = n;
  p.used = 0;
  g_last_error.clear();
  return CP_OK;
}

cp_status_t cp_profile_read(float* kernel_ms, int max_entries, int* n_entries) {
  return cp_profile_read_named(kernel_ms, nullptr, max_entries, n_entries);
}

}  // extern "C"
