// gfx950 kernels for one context-parallel rank's share of causal ring attention.
//
// Sources (web pages, cited by title and section):
//   [MLM] "Megatron-LM源码解析：Context Parallel如何革新长序列训练", sections 3 and 5
//         (per-step fused attention inside the context-parallel loop; the causal
//         triangle wastes about half of the work; HBM round trips are the
//         other cost).
//   [RAF] "如何用Context并行加速大模型训练？手把手教你配置RingAttention+FlashAttention",
//         section 3 (per-step FlashAttention over the received K/V block, mask
//         from the blocks' absolute offsets) and section 5 (zigzag chunks).
//
// Step kernel.  One workgroup owns BM = 32*NW consecutive query rows of one
// (batch, head) inside one query chunk; each wave owns 32 of them.  K and V
// tiles of 64 keys are staged HBM -> LDS by direct-to-LDS 16-byte loads,
// double buffered, one barrier per tile.  Per 32-key sub-tile a wave computes
// the transposed score block S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so
// that every lane holds one query's scores; the causal mask and the
// exponentials are then lane-local.  The exponentials are taken against the
// running maximum as it stands; only when a lane's sum shows that some
// probability outgrew the lazy-rescale bound (and on a row's first
// sub-tile) is the row maximum formed (one v_permlane32_swap across the two
// halves of the row) and the sub-tile redone.  P^T feeds the second MFMA
// directly from registers; V^T comes from the row-major V tile through the
// gfx950 LDS transpose read (ds_read_b64_tr_b16).  The epilogue normalises,
// forms the natural-log LSE and merges into the running fp32 result by
// log-sum-exp rescaling, optionally writing the bf16 output.
#include "cp_attn_internal.h"
#include "cp_attn_tile.h"

#include <math.h>

#include <type_traits>

namespace cpattn {
namespace {

// Lazy rescaling.  A lane's 16 exponentials of a sub-tile, taken against the
// row maximum as it stands, are accepted while their sum is at most
// kSumLimit, so every accepted p is at most 2^8 (exact headroom in fp32, and
// the same relative rounding in bf16).  A larger sum (inf or NaN while a row
// has no maximum yet) sends the wave to the slow path, which raises each
// row's maximum to the sub-tile's, rescales the output and redoes the
// sub-tile.
constexpr float kSumLimit = 256.0f;

// Buffer-resource word 3 of a raw byte buffer, and the cache-policy argument
// of the buffer load/store builtins that makes an access device-coherent
// (scope bit SC1).
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kDeviceCoherent = 16;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

// max / sum with the partner lane (lane ^ 32): v_permlane32_swap returns each
// lane's own value and its partner's, in some order.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Each wave runs a software pipeline over 32-key sub-tiles u (two per
// 64-key LDS tile): sub-iteration u computes the exponentials of sub-tile u
// while its MFMAs are QK^T of sub-tile u+1 and PV of sub-tile u-1, neither of
// which depends on that sub-iteration's VALU work, so the two streams
// interleave freely.
template <int D, int NW, bool kSplit>
__device__ __forceinline__ void step_body(const StepArgs& a) {
  constexpr int BM = 32 * NW;
  constexpr int NS = D / 16;   // k-steps of the QK^T MFMA
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int TB = kTileKeys * D * 2;
  // two K and two V tile buffers, separate objects so that the compiler can
  // tell the direct-to-LDS writes of one buffer from the reads of another
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int lq = lane & 31;

  if constexpr (!kSplit) {
    if (a.cnt_to_clear != nullptr && blockIdx.x == 0)
      for (int i = threadIdx.x; i < kSplitMaxBlocks; i += blockDim.x) a.cnt_to_clear[i] = 0u;
  }

  // ---- which (row block, batch*head) this workgroup owns ----
  // With a key split (kSplit) two workgroups share a row block, each over
  // half of its key tiles; `ks` says which half.  The pair keeps the same
  // job number modulo 8, so both halves run on one XCD.
  int job = blockIdx.x, ks = 0;
  if constexpr (kSplit) split_job(blockIdx.x, a.heads_per_xcd, job, ks);
  // the row block's index (heaviest first, see below) and (b, h)
  int rb_idx, bh;
  xcd_job(job, a.BH, a.heads_per_xcd, a.heads_per_group, a.n_order * a.rb_per_chunk, rb_idx, bh);
  const int oi = rb_idx / a.rb_per_chunk;
  const int rbi = a.rb_per_chunk - 1 - rb_idx % a.rb_per_chunk;  // later rows (more keys) first
  const int qc = a.order[oi];
  const int flags = a.flags[qc];
  const int q_local0 = qc * a.q_chunk_len + rbi * BM;
  const int q_pos0 = a.q_start[qc] + rbi * BM;
  const int q_posmax = q_pos0 + BM - 1;
  const int qw_local = q_local0 + wave * 32;
  const int qw_pos = q_pos0 + wave_u * 32;
  const size_t bh_q = (size_t)bh * a.Sq;
  const size_t bh_kv = (size_t)bh * a.Skv;

  // visible tiles per K/V chunk for this workgroup (key position <= q_posmax)
  const int tiles_per_chunk = a.kv_chunk_len / kTileKeys;
  int n_vis[kMaxChunks];
  int T = 0;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int nv = 0;
    if (c < a.n_kv_chunks && q_posmax >= a.kv_start[c]) {
      nv = (q_posmax - a.kv_start[c]) / kTileKeys + 1;
      nv = nv < tiles_per_chunk ? nv : tiles_per_chunk;
    }
    n_vis[c] = nv;
    T += nv;
  }
  // Tiles are visited chunk by chunk.  A cursor names one tile: its chunk,
  // how many visible tiles of that chunk remain from it, its absolute key
  // position and its first K and V rows (every chunk has its own base, so a
  // launch can span several ring steps' blocks).  The chunk table is only
  // read with constant indices, so it stays in scalar registers.
  int kv_start[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) kv_start[c] = a.kv_start[c];
  struct Cursor {
    int c, left, kpos;
    const uint16_t* kp;  // the tile's first K row
    const uint16_t* vp;  // and V row
  };
  // first visible tile of a chunk after chunk `after` (c = kMaxChunks if none)
  auto chunk_after = [&](int after) {
    Cursor t{kMaxChunks, 0, 0, a.kc[0], a.vc[0]};
#pragma unroll
    for (int c = kMaxChunks - 1; c >= 0; --c)
      if (c > after && n_vis[c] > 0) t = Cursor{c, n_vis[c], kv_start[c], a.kc[c] + bh_kv * D, a.vc[c] + bh_kv * D};
    return t;
  };
  auto next_tile = [&](Cursor t) {
    t.left -= 1;
    t.kpos += kTileKeys;
    t.kp += kTileKeys * D;
    t.vp += kTileKeys * D;
    if (t.left <= 0) t = chunk_after(t.c);  // rare: chunk boundary
    return t;
  };
  const TileLoad<D, NW> k_loader(true, wave_u, lane), v_loader(false, wave_u, lane);
  auto load_k = [&](const Cursor& t, unsigned char* buf) { k_loader(t.kp, buf, wave_u); };
  auto load_v = [&](const Cursor& t, unsigned char* buf) { v_loader(t.vp, buf, wave_u); };

  // Q^T fragments: lane holds Q[row lq][16s + 8g .. +8]
  bf16x8 qf[NS];
  {
    const uint16_t* qrow = a.q + (bh_q + qw_local + lq) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = neg_inf();  // running max, log2-scaled units
  float l_lane = 0.f;       // this lane's share of the row sum

  // per-lane constant parts of the LDS reads
  const int k_base = k_lds_off(lq, 0, g);
  const int j16 = lane & 15;
  const int G = lane >> 4;
  const int tr_row = 4 * g + (j16 >> 2);  // + 16t (+8)
  const int tr_swz = v_swz<D>(tr_row);
  const int tr_colbyte = 8 * (j16 & 1);
  int tr_off[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    tr_off[db] = tr_row * (D * 2) + (((4 * db + 2 * (G & 1) + ((j16 & 3) >> 1)) ^ tr_swz) << 4) + tr_colbyte;

  // S^T of one 32-key sub-tile: K rows [32h, 32h+32) of the tile in `kb`
  auto qk_sub = [&](const unsigned char* kb, int h) {
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + k_base + st * 2048 + h * 1024);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s, 0, 0, 0);
    }
    return s;
  };

  // Exponentials of one sub-tile against the shift `negm` (minus the row's
  // reference maximum): P(u) in bf16 and this lane's share of its row sum,
  // summed in fp32 before rounding.
  auto exps = [&](const f32x16& s_cur, bf16x8 (&p_cur)[2], float negm) {
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[8 * t + e], a.scale_log2, negm));
        lsum += p;
        p_cur[t][e] = (__bf16)p;
      }
    return lsum;
  };

  // The branch-free body of sub-iteration u.
  //   exp:  16 exponentials per lane of s_cur (scores of sub-tile u) against
  //         the running maximum as it stands, packed to bf16 into p_cur, and
  //         their row sum (returned in lsum);
  //   QK:   s_nxt = K Q^T of sub-tile u+1, rows [32 hn, +32) of `kn` (kQK);
  //   PV:   O^T += V^T P^T of sub-tile u-1, rows [32 hp, +32) of `vp` (kPV).
  // Returns true in a lane whose exponentials must be redone with a new
  // maximum: its sum exceeds kSumLimit (inf or NaN while the row has no
  // maximum yet, m_run = -inf).
  auto body = [&](const f32x16& s_cur, f32x16& s_nxt, bf16x8 (&p_cur)[2], const bf16x8 (&p_prev)[2],
                  const unsigned char* kn, int hn, const unsigned char* vp, int hp, float& lsum, auto exp_tag,
                  auto qk_tag, auto pv_tag) {
    constexpr bool kExp = decltype(exp_tag)::value;
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPV = decltype(pv_tag)::value;
    // MFMA stream: QK^T and PV alternate so that consecutive MFMAs never
    // share an accumulator
    if constexpr (kQK) s_nxt = f32x16{};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if constexpr (kQK) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kn + k_base + i * 2048 + hn * 1024);
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i], s_nxt, 0, 0, 0);
      }
      if constexpr (kPV) {
        if (i < 2 * NDB) {
          const int t = i / NDB, db = i % NDB;
          const unsigned char* base = vp + (32 * hp + 16 * t) * (D * 2) + tr_off[db];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, base));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, base + 8 * (D * 2)));
          const bf16x8 af = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, p_prev[t], oacc[db], 0, 0, 0);
        }
      }
    }
    if constexpr (!kExp) return false;
    // VALU stream.  -m_run is +inf while the row has no maximum: every p is
    // then inf (or NaN where masked) and the test below fails.
    lsum = exps(s_cur, p_cur, -m_run);
    // use the packed P here: otherwise the compiler sinks the conversions
    // past the slow-path branch, out of the MFMA stream
    asm volatile("" ::"v"(p_cur[0]), "v"(p_cur[1]));
    // interleave: each MFMA followed by its share of LDS reads and three
    // VALU instructions; the remaining VALU work (about a fifth) follows the
    // last MFMA.  Three per MFMA measured about 3% faster than four, and
    // faster than two or than alternating three and four.
    constexpr int kMfma = (kQK ? NS : 0) + (kPV ? 2 * NDB : 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    return !(lsum <= kSumLimit);
  };

  auto mask = [&](f32x16& s, int kpos) {
    const int qpos = qw_pos + lq;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kp = kpos + 8 * (r >> 2) + 4 * g + (r & 3);
      if (kp > qpos) s[r] = neg_inf();
    }
  };
  // Sub-iteration u: mask S(u) (first key at kpos) if it crosses this wave's
  // diagonal and run the body.  Rarely (on a row's first sub-tile, and when
  // the scores outgrow the running maximum) the slow path raises every row
  // maximum of the wave to its sub-tile maximum, rescales the output (PV(u-1)
  // is in by then) and redoes the exponentials.
  auto sub = [&](int kpos, f32x16& s_cur, f32x16& s_nxt, bf16x8 (&p_cur)[2], const bf16x8 (&p_prev)[2],
                 const unsigned char* kn, int hn, const unsigned char* vp, int hp, auto exp_tag, auto qk_tag,
                 auto pv_tag) {
    constexpr bool kExp = decltype(exp_tag)::value;
    if constexpr (kExp) {
      if (kpos + 31 > qw_pos) mask(s_cur, kpos);
    }
    float lsum = 0.f;
    const bool redo = body(s_cur, s_nxt, p_cur, p_prev, kn, hn, vp, hp, lsum, exp_tag, qk_tag, pv_tag);
    if constexpr (kExp) {
      float alpha = 1.f;
      if (__any(redo)) {
        float mx = neg_inf();
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
        mx = xhalf_max(mx) * a.scale_log2;
        const float m_new = fmaxf(m_run, mx);
        alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        lsum = exps(s_cur, p_cur, (m_run == neg_inf()) ? 0.f : -m_run);
        if (__any(alpha != 1.f)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
      }
      l_lane = __builtin_fmaf(l_lane, alpha, lsum);
    }
  };
  // Cursors at pair n: tm = tile n, tv = tile n+1, tk = tile n+2.
  Cursor tm = chunk_after(-1);
  if constexpr (kSplit) {
    // the first half of the visible tiles, or the rest
    const int half = (T + 1) >> 1;
    if (ks == 1)
      for (int i = 0; i < half; ++i) tm = next_tile(tm);
    T = ks == 0 ? half : T - half;
  }
  Cursor tv = next_tile(tm);
  Cursor tk = next_tile(tv);
  // Top of tile pair n: K(n+1) and V(n) have landed and every wave is done
  // with K(n) and V(n-1); start loading K(n+2) and V(n+1) into those buffers.
  auto barrier_and_prefetch = [&](int n, unsigned char* k_dst, unsigned char* v_dst) {
    wait_vmem_all();
    __syncthreads();
    if (n + 2 < T) load_k(tk, k_dst);
    if (n + 1 < T) load_v(tv, v_dst);
  };
  auto advance = [&]() {
    tm = tv;
    tv = tk;
    tk = next_tile(tk);
  };

  // Sub-tile u is half (u & 1) of tile u >> 1; K(t) and V(t) live in buffer
  // t & 1.  Sub-iteration u uses registers sa/pa for S(u)/P(u) when u is
  // even and sb/pb when u is odd.  Tile pair n holds sub-iterations 2n+1
  // (QK^T of tile n+1 half 0, PV of tile n half 0) and 2n+2 (halves 1).
  using Yes = std::true_type;
  using No = std::false_type;
  if (T > 0) {
    load_k(tm, lds_k0);
    if (T > 1) load_k(tv, lds_k1);
    load_v(tm, lds_v0);
    wait_vmem_all();
    __syncthreads();
    f32x16 sa, sb;
    bf16x8 pa[2], pb[2];
    sa = qk_sub(lds_k0, 0);
    sub(tm.kpos, sa, sb, pa, pb, lds_k0, 1, lds_v0, 0, Yes{}, Yes{}, No{});
    int n = 0;
    // full pairs n = 0 .. T-2, two per trip (even n, then odd n)
    for (; n + 2 < T; n += 2) {
      barrier_and_prefetch(n, lds_k0, lds_v1);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k1, 0, lds_v0, 0, Yes{}, Yes{}, Yes{});
      sub(tv.kpos, sa, sb, pa, pb, lds_k1, 1, lds_v0, 1, Yes{}, Yes{}, Yes{});
      advance();
      barrier_and_prefetch(n + 1, lds_k1, lds_v0);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k0, 0, lds_v1, 0, Yes{}, Yes{}, Yes{});
      sub(tv.kpos, sa, sb, pa, pb, lds_k0, 1, lds_v1, 1, Yes{}, Yes{}, Yes{});
      advance();
    }
    if (n + 1 < T) {
      // n = T-2 (even): one more full pair, then the tail pair T-1 (odd, V in v1)
      barrier_and_prefetch(n, lds_k0, lds_v1);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k1, 0, lds_v0, 0, Yes{}, Yes{}, Yes{});
      sub(tv.kpos, sa, sb, pa, pb, lds_k1, 1, lds_v0, 1, Yes{}, Yes{}, Yes{});
      advance();
      barrier_and_prefetch(n + 1, lds_k1, lds_v0);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k0, 0, lds_v1, 0, Yes{}, No{}, Yes{});
      sub(0, sa, sb, pa, pb, lds_k0, 0, lds_v1, 1, No{}, No{}, Yes{});
    } else {
      // n = T-1 (even): the tail pair, V in v0
      barrier_and_prefetch(n, lds_k1, lds_v1);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k1, 0, lds_v0, 0, Yes{}, No{}, Yes{});
      sub(0, sa, sb, pa, pb, lds_k1, 0, lds_v0, 1, No{}, No{}, Yes{});
    }
  }

  // ---- epilogue: normalise, LSE, merge, write ----
  const float l = xhalf_sum(l_lane);
  const float lse_j = (l > 0.f) ? (m_run + __log2f(l)) * kLn2 : neg_inf();
  const float inv_l = (l > 0.f) ? 1.f / l : 0.f;
  const size_t row = bh_q + qw_local + lq;
  // This launch's partial for the row: oacc * inv_l with log-sum-exp lse_c,
  // or, with a key split, the two halves' normalised partials p0, p1 merged
  // as w0 * p0 + w1 * p1.
  float lse_c = lse_j, w0 = 0.f, w1 = 0.f;
  // key split: the halves' partial outputs and LSE, and the other half's offset
  const size_t slot_rows = (size_t)a.part_rows;
  const __amdgpu_buffer_rsrc_t po =
      __builtin_amdgcn_make_buffer_rsrc(a.part_o, 0, (int)(2 * slot_rows * D * sizeof(float)), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t pl =
      __builtin_amdgcn_make_buffer_rsrc(a.part_lse, 0, (int)(2 * slot_rows * sizeof(float)), kBufferRsrcWord3);
  int oth_off = 0;
  if constexpr (kSplit) {
    // Both halves write their normalised partial (lane order) and LSE to
    // their own slot and count in on the row block's counter; the second to
    // arrive merges the two and goes on, the first is done.  Nothing waits
    // on the other half.  The partials go through device-coherent accesses
    // (write-through stores, loads that do not hit a stale cached copy), so
    // no cache-wide write-back or invalidate is needed: the stores have
    // completed before the count, and the count is a device-scope atomic.
    // The merge uses the partials in the halves' order (the arriving half's
    // own values equal what it stored), so the result does not depend on
    // which half arrives last.
    const size_t prow0 = (size_t)job * BM + 32 * wave;  // the wave's first slot row
    const int my_o = (int)((((size_t)ks * slot_rows + prow0) * D + lane * 4) * sizeof(float));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        f32x4 o;
        o[0] = oacc[db][4 * rr + 0] * inv_l;
        o[1] = oacc[db][4 * rr + 1] * inv_l;
        o[2] = oacc[db][4 * rr + 2] * inv_l;
        o[3] = oacc[db][4 * rr + 3] * inv_l;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), po, my_o + (4 * db + rr) * 256 * 4, 0,
                                               kDeviceCoherent);
      }
    if (g == 0)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse_j), pl,
                                            (int)(((size_t)ks * slot_rows + prow0 + lq) * sizeof(float)), 0,
                                            kDeviceCoherent);
    // Wait until this wave's stores have completed (a device-scope release
    // fence would also write back and invalidate the whole L2, which the
    // write-through stores do not need): s_waitcnt vmcnt(0).
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    __shared__ unsigned arrived;
    if (threadIdx.x == 0)
      arrived = __hip_atomic_fetch_add(&a.part_cnt[job], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived == 0) return;  // the other half merges
    if (threadIdx.x == 0)  // ready for the next launch
      __hip_atomic_store(&a.part_cnt[job], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int ot = ks ^ 1;
    const int ot_o = (int)((((size_t)ot * slot_rows + prow0) * D + lane * 4) * sizeof(float));
    const float l_other = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        pl, (int)(((size_t)ot * slot_rows + prow0 + lq) * sizeof(float)), 0, kDeviceCoherent));
    oth_off = ot_o;
    const float l0 = ks == 0 ? lse_j : l_other, l1 = ks == 0 ? l_other : lse_j;
    if (l0 == neg_inf()) {
      w1 = (l1 == neg_inf()) ? 0.f : 1.f;
      lse_c = l1;
    } else if (l1 == neg_inf()) {
      w0 = 1.f;
      lse_c = l0;
    } else {
      const float x2 = l0 * kLog2e, y2 = l1 * kLog2e;
      const float mm = fmaxf(x2, y2);
      const float L2 = mm + __log2f(exp2f(x2 - mm) + exp2f(y2 - mm));
      w0 = exp2f(x2 - L2);
      w1 = exp2f(y2 - L2);
      lse_c = L2 * kLn2;
    }
  }
  // merge with the running result of earlier launches
  float w_prev = 0.f, w_cur = 1.f, lse_new = lse_c;
  if (flags & kFlagMerge) {
    const float lp = a.lse_run[row];
    if (lp != neg_inf()) {
      if (lse_c == neg_inf()) {
        w_prev = 1.f;
        w_cur = 0.f;
        lse_new = lp;
      } else {
        const float x2 = lp * kLog2e, y2 = lse_c * kLog2e;
        const float mm = fmaxf(x2, y2);
        const float L2 = mm + __log2f(exp2f(x2 - mm) + exp2f(y2 - mm));
        w_prev = exp2f(x2 - L2);
        w_cur = exp2f(y2 - L2);
        lse_new = L2 * kLn2;
      }
    }
  }
  const float w_self = w_cur * inv_l;
  if (g == 0) a.lse_run[row] = lse_new;
  const bool write_o = (flags & kFlagWriteO) != 0;
  const bool finalize = (flags & kFlagFinalize) != 0;
  // The running O of this wave's 32 rows occupies the 32 x D floats at
  // o_run + (bh_q + qw_local) D.  In row-major order a lane's 16-byte piece
  // (d0 .. d0+3 of row lq) lands 32 rows apart from its neighbours' pieces;
  // in lane order (kFlagLaneO, the ring driver's private workspace) piece k
  // of lane L is the 16 bytes at float (64 k + L) 4 of the block, so each
  // wave load or store covers one contiguous KiB.
  // Either way piece k = 4 db + rr sits at o_base + k * o_stride.
  const bool lane_order = (flags & kFlagLaneO) != 0;
  float* const o_base = a.o_run + (bh_q + qw_local) * D + (lane_order ? lane * 4 : lq * D + 4 * g);
  const int o_stride = lane_order ? 256 : 8;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d0 = 32 * db + 8 * rr + 4 * g;
      float* const o_ptr = o_base + (4 * db + rr) * o_stride;
      f32x4 o;
      if constexpr (kSplit) {
        f32x4 own, oth = __builtin_bit_cast(
                       f32x4, __builtin_amdgcn_raw_buffer_load_b128(po, oth_off + (4 * db + rr) * 256 * 4, 0,
                                                                    kDeviceCoherent));
        own[0] = oacc[db][4 * rr + 0] * inv_l;
        own[1] = oacc[db][4 * rr + 1] * inv_l;
        own[2] = oacc[db][4 * rr + 2] * inv_l;
        own[3] = oacc[db][4 * rr + 3] * inv_l;
        const f32x4 p0 = ks == 0 ? own : oth, p1 = ks == 0 ? oth : own;
        o = (p0 * w0 + p1 * w1) * w_cur;
      } else {
        o[0] = oacc[db][4 * rr + 0] * w_self;
        o[1] = oacc[db][4 * rr + 1] * w_self;
        o[2] = oacc[db][4 * rr + 2] * w_self;
        o[3] = oacc[db][4 * rr + 3] * w_self;
      }
      if (w_prev != 0.f) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(o_ptr);
        o += w_prev * prev;
      }
      if (write_o) *reinterpret_cast<f32x4*>(o_ptr) = o;
      if (finalize) {
        bf16x4 h;
        h[0] = (__bf16)o[0];
        h[1] = (__bf16)o[1];
        h[2] = (__bf16)o[2];
        h[3] = (__bf16)o[3];
        *reinterpret_cast<bf16x4*>(a.out + row * D + d0) = h;
      }
    }
}

// Entry points.  Eight-wave workgroups (256 rows) run two waves per SIMD and
// are held to 248 VGPRs, so that 16 registers per SIMD stay free for the
// waves of a concurrent staging copy on the copy stream; the smaller shapes
// (chunk lengths that are not multiples of 256) run one wave per SIMD.
template <int D>
__global__ void __launch_bounds__(512, 1) __attribute__((amdgpu_num_vgpr(124))) step_kernel_256(const StepArgs a) {
  step_body<D, 8, false>(a);
}
// The same with each row block's key tiles split over two workgroups: for
// grids of 256-row blocks that would leave compute units idle and hold no
// diagonal chunk pair.  The halves' partials meet in the workspace and the
// second to finish merges them.
template <int D>
__global__ void __launch_bounds__(512, 1) __attribute__((amdgpu_num_vgpr(124))) step_kernel_256s(const StepArgs a) {
  step_body<D, 8, true>(a);
}
// 128-row workgroups held to the same register budget, two per CU: for grids
// of 256-row workgroups that would leave compute units idle, and for chunk
// lengths that are multiples of 128 but not of 256.
template <int D>
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_num_vgpr(124))) step_kernel_128(const StepArgs a) {
  step_body<D, 4, false>(a);
}
// The same with the key split (grids with a diagonal chunk pair whose
// 128-row workgroups would hold at most one wave per SIMD).
template <int D>
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_num_vgpr(124))) step_kernel_128s(const StepArgs a) {
  step_body<D, 4, true>(a);
}
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 1) step_kernel_small(const StepArgs a) {
  step_body<D, NW, false>(a);
}

// ---- standalone log-sum-exp merge, HBM-bound elementwise pass ----
__global__ void __launch_bounds__(256) merge_kernel(float* o_acc, float* lse_acc, const float* o_part,
                                                    const float* lse_part, uint16_t* out, int64_t rows,
                                                    int D) {
  const int D4 = D / 4;
  const int tpr = D4 < 256 ? D4 : 256;
  const int rpb = 256 / tpr;
  const int r_in = threadIdx.x / tpr;
  const int j = threadIdx.x % tpr;
  for (int64_t base = (int64_t)blockIdx.x * rpb; base < rows; base += (int64_t)gridDim.x * rpb) {
    const int64_t row = base + r_in;
    const bool active = r_in < rpb && row < rows;
    float wa = 0.f, wb = 0.f, L = neg_inf();
    if (active) {
      const float la = lse_acc[row], lb = lse_part[row];
      if (la == neg_inf()) {
        if (lb != neg_inf()) { wb = 1.f; L = lb; }
      } else if (lb == neg_inf()) {
        wa = 1.f;
        L = la;
      } else {
        const float x2 = la * kLog2e, y2 = lb * kLog2e;
        const float mm = fmaxf(x2, y2);
        const float L2 = mm + __log2f(exp2f(x2 - mm) + exp2f(y2 - mm));
        wa = exp2f(x2 - L2);
        wb = exp2f(y2 - L2);
        L = L2 * kLn2;
      }
    }
    __syncthreads();  // every read of lse_acc in this block precedes the writes
    if (active) {
      for (int d4 = j; d4 < D4; d4 += tpr) {
        const int64_t off = row * D + 4 * d4;
        f32x4 x = *reinterpret_cast<const f32x4*>(o_acc + off);
        const f32x4 y = *reinterpret_cast<const f32x4*>(o_part + off);
        f32x4 o;
        o[0] = (wa != 0.f ? wa * x[0] : 0.f) + (wb != 0.f ? wb * y[0] : 0.f);
        o[1] = (wa != 0.f ? wa * x[1] : 0.f) + (wb != 0.f ? wb * y[1] : 0.f);
        o[2] = (wa != 0.f ? wa * x[2] : 0.f) + (wb != 0.f ? wb * y[2] : 0.f);
        o[3] = (wa != 0.f ? wa * x[3] : 0.f) + (wb != 0.f ? wb * y[3] : 0.f);
        *reinterpret_cast<f32x4*>(o_acc + off) = o;
        if (out) {
          bf16x4 h;
          h[0] = (__bf16)o[0];
          h[1] = (__bf16)o[1];
          h[2] = (__bf16)o[2];
          h[3] = (__bf16)o[3];
          *reinterpret_cast<bf16x4*>(out + off) = h;
        }
      }
      if (j == 0) lse_acc[row] = L;
    }
  }
}

// ---- staging copy of one ring step's K and V blocks (the stand-in for the
// peer-to-peer receive), run on the copy stream beside a step kernel ----
// One wave per SIMD and at most 16 VGPRs, so that it fits next to the 8-wave
// step workgroup (248 VGPRs per wave) on every CU; the waves raise their
// issue priority because they mostly wait on memory, and without it the
// older step waves would starve them.  K is copied first, then V, in 16-byte
// chunks; every lane keeps two chunks in flight.  Loads and stores are
// nontemporal, so the streamed block does not displace the step kernel's
// K/V tiles from L2.
__device__ __forceinline__ void copy_range(const u32x4* __restrict__ src, u32x4* __restrict__ dst, unsigned n,
                                           unsigned i, unsigned stride) {
  for (; i + stride < n; i += 2 * stride) {
    const u32x4 x = __builtin_nontemporal_load(&src[i]);
    const u32x4 y = __builtin_nontemporal_load(&src[i + stride]);
    __builtin_nontemporal_store(x, &dst[i]);
    __builtin_nontemporal_store(y, &dst[i + stride]);
  }
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}
__global__ void __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(8)))
    stage_copy_kernel(const u32x4* __restrict__ k_src, u32x4* __restrict__ k_dst, const u32x4* __restrict__ v_src,
                      u32x4* __restrict__ v_dst, unsigned n16) {
  __builtin_amdgcn_s_setprio(3);
  const unsigned stride = gridDim.x * blockDim.x;
  const unsigned i = blockIdx.x * blockDim.x + threadIdx.x;
  copy_range(k_src, k_dst, n16, i, stride);
  copy_range(v_src, v_dst, n16, i, stride);
}

// ---- bounded spin for the stream-ordering tests: one wave waits `ticks` of
// the constant 100 MHz clock, sleeping between reads ----
__global__ void __launch_bounds__(64) delay_kernel(long long ticks) {
  const long long t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(32);
}

}  // namespace

__global__ void __launch_bounds__(256) zero_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_delay(int us, hipStream_t stream) {
  if (us <= 0) return hipSuccess;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, stream, 100LL * us);
  return hipGetLastError();
}

int step_block_rows(int q_chunk_len) {
  return (q_chunk_len % 256 == 0) ? 256 : (q_chunk_len % 128 == 0) ? 128 : 64;
}

namespace {
int device_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      return cus;
    return 256;
  }();
  return n;
}
}  // namespace

hipError_t launch_step(const StepArgs& args, int D, hipStream_t stream, const char** name) {
  StepArgs a = args;
  int bm = step_block_rows(a.q_chunk_len);
  // Every row's result is the same whatever the row-block size (a row block
  // only decides which tiles are staged; tiles past a row are masked to exact
  // zeros), so the launch picks it: 256-row blocks unless their grid would
  // leave compute units idle, or would give each unit exactly one block of a
  // launch that holds a diagonal chunk pair (its blocks' work then ranges from
  // a few tiles to twice the mean, and 128-row blocks, two per unit, let the
  // light ones finish beside the heavy ones).
  bool diag = false;
  for (int i = 0; i < a.n_order; ++i)
    for (int k = 0; k < a.n_kv_chunks; ++k) diag = diag || a.q_start[a.order[i]] == a.kv_start[k];
  // Key split (needs the caller's partial buffers: the ring driver's
  // workspace): each row block's key tiles are split over two workgroups
  // whose partials are merged by log-sum-exp.  Taken for a 256-row grid
  // without a diagonal pair that would leave compute units idle (its halves
  // then keep the eight-wave blocks), and for a 128-row grid that holds fewer
  // than two workgroups per compute unit.
  const long long g256 = (long long)a.n_order * (a.q_chunk_len / 256) * a.BH;
  const auto split_fits = [&](long long grid_rows) {
    return a.part_rows > 0 && grid_rows <= a.part_rows;
  };
  bool split = false;
  if (bm == 256 && !diag && g256 < device_cus() && g256 <= kSplitMaxBlocks && split_fits(g256 * 256))
    split = true;
  else if (bm == 256 && (g256 < device_cus() || (diag && g256 <= device_cus())))
    bm = 128;
  a.rb_per_chunk = a.q_chunk_len / bm;
  const long long grid = (long long)a.n_order * a.rb_per_chunk * a.BH;
  if (name) *name = nullptr;
  if (grid <= 0)  // nothing to launch; counters this launch was to clear are cleared all the same
    return a.cnt_to_clear != nullptr ? launch_zero_u32(a.cnt_to_clear, kSplitMaxBlocks, stream) : hipSuccess;
  if (bm == 128 && grid < 2LL * device_cus() && grid <= kSplitMaxBlocks && split_fits(grid * 128)) split = true;
  // Heads per group: the most heads (a divisor of an XCD's share) whose row
  // blocks fit in what one XCD runs at once (one 256-row or two 128-row
  // workgroups per CU, two workgroups per row block with the key split), so
  // that a head's row blocks run together and share its K/V tiles in the
  // L2.  A launch with a diagonal chunk pair, whose row blocks' work differs,
  // allows twice that: heaviest-first order then spans two rounds of
  // workgroups, which keeps the tail short.
  if (a.heads_per_xcd > 0) {
    const long long rb_per_head = (long long)a.n_order * a.rb_per_chunk * (split ? 2 : 1);
    const long long slots = (long long)(device_cus() / 8) * (bm == 256 ? 1 : 2) * (diag ? 2 : 1);
    a.heads_per_group = heads_per_group(a.heads_per_xcd, rb_per_head, slots);
  }
  if (split && a.cnt_to_clear != nullptr) {
    const hipError_t e = launch_zero_u32(a.cnt_to_clear, kSplitMaxBlocks, stream);
    if (e != hipSuccess) return e;
    a.cnt_to_clear = nullptr;
  }
  const dim3 g((unsigned)(split ? 2 * grid : grid)), blk((unsigned)(2 * bm));  // one wave per 32 rows
  const char* n;
  if (D == 128) {
    if (bm == 256 && split) { hipLaunchKernelGGL((step_kernel_256s<128>), g, blk, 0, stream, a); n = "step_kernel_256s<128>"; }
    else if (bm == 256) { hipLaunchKernelGGL((step_kernel_256<128>), g, blk, 0, stream, a); n = "step_kernel_256<128>"; }
    else if (split) { hipLaunchKernelGGL((step_kernel_128s<128>), g, blk, 0, stream, a); n = "step_kernel_128s<128>"; }
    else if (bm == 128) { hipLaunchKernelGGL((step_kernel_128<128>), g, blk, 0, stream, a); n = "step_kernel_128<128>"; }
    else { hipLaunchKernelGGL((step_kernel_small<128, 2>), g, blk, 0, stream, a); n = "step_kernel_small<128, 2>"; }
  } else {
    if (bm == 256 && split) { hipLaunchKernelGGL((step_kernel_256s<64>), g, blk, 0, stream, a); n = "step_kernel_256s<64>"; }
    else if (bm == 256) { hipLaunchKernelGGL((step_kernel_256<64>), g, blk, 0, stream, a); n = "step_kernel_256<64>"; }
    else if (split) { hipLaunchKernelGGL((step_kernel_128s<64>), g, blk, 0, stream, a); n = "step_kernel_128s<64>"; }
    else if (bm == 128) { hipLaunchKernelGGL((step_kernel_128<64>), g, blk, 0, stream, a); n = "step_kernel_128<64>"; }
    else { hipLaunchKernelGGL((step_kernel_small<64, 2>), g, blk, 0, stream, a); n = "step_kernel_small<64, 2>"; }
  }
  if (name) *name = n;
  return hipGetLastError();
}

hipError_t launch_stage_copy(const void* k_src, void* k_dst, const void* v_src, void* v_dst, size_t bytes,
                             hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0 || bytes / 16 > 0x7fffffffull) return hipErrorInvalidValue;
  const unsigned n16 = (unsigned)(bytes / 16);
  unsigned blocks = (n16 + 255) / 256;
  if (blocks > 256) blocks = 256;  // one workgroup per CU
  hipLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(k_src),
                     static_cast<u32x4*>(k_dst), static_cast<const u32x4*>(v_src), static_cast<u32x4*>(v_dst), n16);
  return hipGetLastError();
}

hipError_t launch_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                        uint16_t* out, int64_t rows, int D, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int D4 = D / 4;
  const int tpr = D4 < 256 ? D4 : 256;
  const int rpb = 256 / tpr;
  long long blocks = (rows + rpb - 1) / rpb;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o_acc, lse_acc, o_part,
                     lse_part, out, rows, D);
  return hipGetLastError();
}

}  // namespace cpattn
