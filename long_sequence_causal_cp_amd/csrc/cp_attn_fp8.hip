// gfx950 fp8 (e4m3) kernel for one context-parallel ring step: the same
// causal step as the bf16 step kernel (online softmax over 64-key tiles,
// fused log-sum-exp merge), with Q, K and V in fp8 and the probabilities
// rounded to fp8 for the PV product.
//
// Sources (web pages, cited by title and section):
//   [MLM] "Megatron-LM源码解析：Context Parallel如何革新长序列训练", section 4
//         (FP8 used together with context parallelism) and section 5
//         (per-step fused attention inside the context-parallel loop).
//   [RAF] "如何用Context并行加速大模型训练？手把手教你配置RingAttention+FlashAttention",
//         section 3 (per-step attention over one received K/V block, mask
//         from the blocks' absolute offsets).
//
// Values: Q, K, V hold e4m3 codes with per-tensor dequantisation factors;
// q_scale * k_scale is folded into the softmax scale and v_scale into the
// output.  Products use v_mfma_f32_32x32x16_fp8_fp8 (eight codes per lane, in
// the lane layout of the bf16 32x32x16 product) with fp32 accumulation.
//
// Per 32-key sub-tile a wave forms S^T = K Q^T (one query per lane pair, as in
// the bf16 kernel), the exponentials against the lazily kept row maximum
// (every accepted p <= 2^8, inside e4m3's range of 448), packs P to e4m3, and
// adds O^T += V^T P^T.  The score layout gives lane (query, half g) the keys
// {4g..4g+3, 8+4g..8+4g+3} of each 16-key step; one v_permlane32_swap per
// step hands the partner lane's group across, so that the P operand holds
// keys 8g..8g+7 and V^T is read along its rows in natural key order.
//
// LDS: a K tile is 64 keys x 128 bytes, its 16-byte chunk c of row r stored
// at chunk c ^ ((r >> 1) & 7); a V^T tile is 128 rows (d) x 64 bytes (keys),
// chunk c of row d at c ^ ((d >> 2) & 3).  Both are filled by direct-to-LDS
// 16-byte loads, one instruction per wave per tile, and read with 8-byte
// loads at most two lanes to a bank.
#include "cp_attn_fp8.h"
#include "cp_attn_tile.h"

#include <type_traits>

namespace cpattn {
namespace {

typedef unsigned long long u64;

constexpr int kD8 = 128;          // head dimension of the fp8 kernel
constexpr int kNW8 = 8;           // waves per workgroup, 32 rows each
constexpr int kTB8 = kTileKeys * kD8;  // bytes of one K or V^T tile
constexpr float kSumLimit8 = 256.0f;

__device__ __forceinline__ float half_max8(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum8(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// P^T operand of one 16-key step from the 8 probabilities p[0..7] of that
// step (keys 4g + {0..3} then 8 + 4g + {0..3}), packed to e4m3.
__device__ __forceinline__ u64 pack_p(float p0, float p1, float p2, float p3, float p4, float p5, float p6,
                                      float p7) {
  int x0 = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
  x0 = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x0, true);
  int x1 = __builtin_amdgcn_cvt_pk_fp8_f32(p4, p5, 0, false);
  x1 = __builtin_amdgcn_cvt_pk_fp8_f32(p6, p7, x1, true);
  // upper half-wave of x0 <-> lower half-wave of x1
  auto r = __builtin_amdgcn_permlane32_swap((unsigned)x0, (unsigned)x1, false, false);
  return (u64)r[0] | ((u64)r[1] << 32);
}

__device__ __forceinline__ void fp8_step_body(const Fp8StepArgs& a) {
  constexpr int D = kD8;
  constexpr int NW = kNW8;
  constexpr int BM = 32 * NW;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TB = kTB8;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[TB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int lq = lane & 31;

  const int job = blockIdx.x;
  int rb_idx, bh;
  if (a.heads_per_xcd > 0) {
    const int x = job & 7, kk = job >> 3;
    rb_idx = kk / a.heads_per_xcd;
    bh = x * a.heads_per_xcd + kk % a.heads_per_xcd;
  } else {
    rb_idx = job / a.BH;
    bh = job % a.BH;
  }
  const int oi = rb_idx / a.rb_per_chunk;
  const int rbi = a.rb_per_chunk - 1 - rb_idx % a.rb_per_chunk;
  const int qc = a.order[oi];
  const int flags = a.flags[qc];
  const int q_local0 = qc * a.q_chunk_len + rbi * BM;
  const int q_pos0 = a.q_start[qc] + rbi * BM;
  const int q_posmax = q_pos0 + BM - 1;
  const int qw_local = q_local0 + wave * 32;
  const int qw_pos = q_pos0 + wave_u * 32;
  const size_t bh_q = (size_t)bh * a.Sq;
  const size_t bh_kv = (size_t)bh * a.Skv;

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
  int kv_start[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) kv_start[c] = a.kv_start[c];
  struct Cursor {
    int c, left, kpos;
    const uint8_t* kp;  // the tile's first K row
    const uint8_t* vp;  // the tile's first V^T column (row 0)
  };
  auto chunk_after = [&](int after) {
    Cursor t{kMaxChunks, 0, 0, a.kc[0], a.vtc[0]};
#pragma unroll
    for (int c = kMaxChunks - 1; c >= 0; --c)
      if (c > after && n_vis[c] > 0) t = Cursor{c, n_vis[c], kv_start[c], a.kc[c] + bh_kv * D, a.vtc[c] + bh_kv * D};
    return t;
  };
  auto next_tile = [&](Cursor t) {
    t.left -= 1;
    t.kpos += kTileKeys;
    t.kp += kTileKeys * D;
    t.vp += kTileKeys;
    if (t.left <= 0) t = chunk_after(t.c);
    return t;
  };
  // this wave's direct-to-LDS instruction of each tile writes LDS bytes
  // [1024 wave, +1024): lane i the 16 bytes at 1024 wave + 16 i
  unsigned k_ld, v_ld;
  {
    const int r = 8 * wave_u + lane / 8, pc = lane % 8;
    k_ld = (unsigned)(r * D + 16 * (pc ^ ((r >> 1) & 7)));
    const int dr = 16 * wave_u + lane / 4, pv = lane % 4;
    v_ld = (unsigned)(dr * a.Skv + 16 * (pv ^ ((dr >> 2) & 3)));
  }
  auto load_k = [&](const Cursor& t, unsigned char* buf) { global_to_lds_16(t.kp, k_ld, buf + 1024 * wave_u); };
  auto load_v = [&](const Cursor& t, unsigned char* buf) { global_to_lds_16(t.vp, v_ld, buf + 1024 * wave_u); };

  // Q^T fragments: lane holds Q[row lq][16 s + 8 g .. + 8]
  u64 qf[NS];
  {
    const uint8_t* qrow = a.q + (bh_q + qw_local + lq) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const u64*>(qrow + 16 * s);
  }
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = neg_inf();
  float l_lane = 0.f;

  // per-lane LDS read offsets: K rows (key lq of a sub-tile, d 16 st + 8 g),
  // V^T rows (d 32 db + lq, keys 32 h + 16 t + 8 g)
  int kro[NS];
  {
    const int kx = (lq >> 1) & 7;
#pragma unroll
    for (int st = 0; st < NS; ++st) kro[st] = lq * D + 8 * g + 16 * (st ^ kx);
  }
  int vro[4];
  {
    const int vx = (lq >> 2) & 3;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) vro[ht] = lq * kTileKeys + 8 * g + 16 * (ht ^ vx);
  }

  auto kread = [&](const unsigned char* kb, int h, int st) {
    return *reinterpret_cast<const u64*>(kb + kro[st] + h * 32 * D);
  };
  auto vread = [&](const unsigned char* vb, int h, int t, int db) {
    return *reinterpret_cast<const u64*>(vb + vro[2 * h + t] + db * 32 * kTileKeys);
  };
  auto qk_sub = [&](const unsigned char* kb, int h) {
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < NS; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8((long)kread(kb, h, st), (long)qf[st], s, 0, 0, 0);
    return s;
  };
  auto exps = [&](const f32x16& s_cur, u64 (&p_cur)[2], float negm) {
    float e[16];
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], a.scale_log2, negm));
      lsum += e[r];
    }
    p_cur[0] = pack_p(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    p_cur[1] = pack_p(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    return lsum;
  };
  auto body = [&](const f32x16& s_cur, f32x16& s_nxt, u64 (&p_cur)[2], const u64 (&p_prev)[2],
                  const unsigned char* kn, int hn, const unsigned char* vp, int hp, float& lsum, auto exp_tag,
                  auto qk_tag, auto pv_tag) {
    constexpr bool kExp = decltype(exp_tag)::value;
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPV = decltype(pv_tag)::value;
    if constexpr (kQK) s_nxt = f32x16{};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if constexpr (kQK)
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8((long)kread(kn, hn, i), (long)qf[i], s_nxt, 0, 0, 0);
      if constexpr (kPV) {
        if (i < 2 * NDB) {
          const int t = i / NDB, db = i % NDB;
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8((long)vread(vp, hp, t, db), (long)p_prev[t],
                                                                 oacc[db], 0, 0, 0);
        }
      }
    }
    if constexpr (!kExp) return false;
    lsum = exps(s_cur, p_cur, -m_run);
    asm volatile("" ::"v"(p_cur[0]), "v"(p_cur[1]));
    constexpr int kMfma = (kQK ? NS : 0) + (kPV ? 2 * NDB : 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    return !(lsum <= kSumLimit8);
  };
  auto mask = [&](f32x16& s, int kpos) {
    const int qpos = qw_pos + lq;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kp = kpos + 8 * (r >> 2) + 4 * g + (r & 3);
      if (kp > qpos) s[r] = neg_inf();
    }
  };
  auto sub = [&](int kpos, f32x16& s_cur, f32x16& s_nxt, u64 (&p_cur)[2], const u64 (&p_prev)[2],
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
        mx = half_max8(mx) * a.scale_log2;
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
  Cursor tm = chunk_after(-1);
  Cursor tv = next_tile(tm);
  Cursor tk = next_tile(tv);
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
  using Yes = std::true_type;
  using No = std::false_type;
  if (T > 0) {
    load_k(tm, lds_k0);
    if (T > 1) load_k(tv, lds_k1);
    load_v(tm, lds_v0);
    wait_vmem_all();
    __syncthreads();
    f32x16 sa, sb;
    u64 pa[2], pb[2];
    sa = qk_sub(lds_k0, 0);
    sub(tm.kpos, sa, sb, pa, pb, lds_k0, 1, lds_v0, 0, Yes{}, Yes{}, No{});
    int n = 0;
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
      barrier_and_prefetch(n, lds_k0, lds_v1);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k1, 0, lds_v0, 0, Yes{}, Yes{}, Yes{});
      sub(tv.kpos, sa, sb, pa, pb, lds_k1, 1, lds_v0, 1, Yes{}, Yes{}, Yes{});
      advance();
      barrier_and_prefetch(n + 1, lds_k1, lds_v0);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k0, 0, lds_v1, 0, Yes{}, No{}, Yes{});
      sub(0, sa, sb, pa, pb, lds_k0, 0, lds_v1, 1, No{}, No{}, Yes{});
    } else {
      barrier_and_prefetch(n, lds_k1, lds_v1);
      sub(tm.kpos + 32, sb, sa, pb, pa, lds_k1, 0, lds_v0, 0, Yes{}, No{}, Yes{});
      sub(0, sa, sb, pa, pb, lds_k1, 0, lds_v0, 1, No{}, No{}, Yes{});
    }
  }

  // ---- epilogue: normalise (with V's dequantisation factor), LSE, merge, write ----
  const float l = half_sum8(l_lane);
  const float lse_j = (l > 0.f) ? (m_run + __log2f(l)) * kLn2 : neg_inf();
  const float inv_l = (l > 0.f) ? a.v_scale / l : 0.f;
  const size_t row = bh_q + qw_local + lq;
  float w_prev = 0.f, w_cur = inv_l, lse_new = lse_j;
  if (flags & kFlagMerge) {
    const float lp = a.lse[row];
    if (lp != neg_inf()) {
      if (lse_j == neg_inf()) {
        w_prev = 1.f;
        w_cur = 0.f;
        lse_new = lp;
      } else {
        const float x2 = lp * kLog2e, y2 = lse_j * kLog2e;
        const float mm = fmaxf(x2, y2);
        const float L2 = mm + __log2f(exp2f(x2 - mm) + exp2f(y2 - mm));
        w_prev = exp2f(x2 - L2);
        w_cur = exp2f(y2 - L2) * inv_l;
        lse_new = L2 * kLn2;
      }
    }
  }
  if (g == 0) a.lse[row] = lse_new;
  const bool write_o = (flags & kFlagWriteO) != 0;
  const bool finalize = (flags & kFlagFinalize) != 0;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d0 = 32 * db + 8 * rr + 4 * g;
      float* const o_ptr = a.o + row * D + d0;
      f32x4 o;
      o[0] = oacc[db][4 * rr + 0] * w_cur;
      o[1] = oacc[db][4 * rr + 1] * w_cur;
      o[2] = oacc[db][4 * rr + 2] * w_cur;
      o[3] = oacc[db][4 * rr + 3] * w_cur;
      if (w_prev != 0.f) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(o_ptr);
        o += w_prev * prev;
      }
      if (write_o) *reinterpret_cast<f32x4*>(o_ptr) = o;
      if (finalize) {
        bf16x4 hh;
        hh[0] = (__bf16)o[0];
        hh[1] = (__bf16)o[1];
        hh[2] = (__bf16)o[2];
        hh[3] = (__bf16)o[3];
        *reinterpret_cast<bf16x4*>(a.out + row * D + d0) = hh;
      }
    }
}

__global__ void __launch_bounds__(512, 1) __attribute__((amdgpu_num_vgpr(124))) fp8_step_kernel(const Fp8StepArgs a) {
  fp8_step_body(a);
}

}  // namespace

hipError_t launch_step_fp8(const Fp8StepArgs& a, hipStream_t stream) {
  const long long grid = (long long)a.n_order * a.rb_per_chunk * a.BH;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_step_kernel, dim3((unsigned)grid), dim3(64 * kNW8), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cpattn
