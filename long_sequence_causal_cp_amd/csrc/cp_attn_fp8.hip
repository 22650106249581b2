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
// output.  Products use gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// block scales (twice the rate of the 32x32x16 fp8 product) and fp32
// accumulation.  Lane l holds row l % 32 of either operand and its k-indices
// 32 (l / 32) .. + 31, 32 codes in eight dwords.
//
// Per 64-key tile a wave forms S^T = K Q^T for its 32 queries (two 32x32
// accumulators, keys 0-31 and 32-63), the exponentials against the lazily
// kept row maximum (every accepted p <= 2^8, inside e4m3's range of 448),
// packs P to e4m3 and adds O^T += V^T P^T, k = the tile's 64 keys.  The
// score layout gives lane (query, half g) the keys 8i + 4g + {0..3} of each
// 32-key half; one v_permlane32_swap per i hands the partner's group across,
// so that half 0 holds keys 0-31 and half 1 keys 32-63 in natural order, as
// the PV product takes them.
//
// Software pipeline: while a wave exponentiates tile u, its MFMAs are
// S(u+1) and O += V(u-1) P(u-1).  When a tile's row maximum rises past the
// lazy bound (rare after the first tile), its scores are formed again from
// K(u), which stays resident in one of three K buffers for that purpose, so
// that S(u) need not stay live across the exponentials.
//
// LDS: a K tile is 64 keys x 128 bytes, its 16-byte chunk c of row r stored
// at chunk c ^ ((r >> 1) & 7); a V^T tile is 128 rows (d) x 64 bytes (keys),
// chunk c of row d at c ^ ((d >> 2) & 3).  Both are filled by direct-to-LDS
// 16-byte loads, one instruction per wave per tile, and read with 16-byte
// loads that touch every bank once per 16 lanes.
#include "cp_attn_fp8.h"
#include "cp_attn_tile.h"

#include <type_traits>

namespace cpattn {
namespace {


constexpr int kD8 = 128;          // head dimension of the fp8 kernel
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

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int NW>
__device__ __forceinline__ void fp8_step_body(const Fp8StepArgs& a) {
  constexpr int D = kD8;
  constexpr int BM = 32 * NW;
  constexpr int LPW = 8 / NW;  // direct-to-LDS instructions per wave per K or V^T tile (8 KiB)
  constexpr int NK = D / 64;   // k-steps of the QK^T product
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int TB = kTB8;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k2[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[TB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[TB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int lq = lane & 31;

  const int job = blockIdx.x;
  int rb_idx, bh;
  xcd_job(job, a.BH, a.heads_per_xcd, a.heads_per_group, a.n_order * a.rb_per_chunk, rb_idx, bh);
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
  // direct-to-LDS instruction i of this wave fills 1-KiB block b = wave + NW i
  // of each tile: lane l the 16 bytes at 1024 b + 16 l
  unsigned k_ld[LPW], v_ld[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int b = wave_u + NW * i;
    const int r = 8 * b + lane / 8, pc = lane % 8;
    k_ld[i] = (unsigned)(r * D + 16 * (pc ^ ((r >> 1) & 7)));
    const int dr = 16 * b + lane / 4, pv = lane % 4;
    v_ld[i] = (unsigned)(dr * a.Skv + 16 * (pv ^ ((dr >> 2) & 3)));
  }
  auto load_k = [&](const Cursor& t, unsigned char* buf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) global_to_lds_16(t.kp, k_ld[i], buf + 1024 * (wave_u + NW * i));
  };
  auto load_v = [&](const Cursor& t, unsigned char* buf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) global_to_lds_16(t.vp, v_ld[i], buf + 1024 * (wave_u + NW * i));
  };

  // Q^T fragments: lane holds Q[row lq][64 ks + 32 g .. + 32]
  i32x8 qreg[NK];
  {
    const uint8_t* qrow = a.q + (bh_q + qw_local + lq) * D + 32 * g;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) qreg[ks] = *reinterpret_cast<const i32x8*>(qrow + 64 * ks);
  }
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = neg_inf();
  float l_lane = 0.f;

  // LDS read offsets: K row (32 j + lq), bytes 64 ks + 32 g + 16 h; V^T row
  // (32 db + lq), bytes (keys) 32 g + 16 h
  int kro[NK][2], vro[2];
  {
    const int kx = (lq >> 1) & 7, vx = (lq >> 2) & 3;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) kro[ks][h] = lq * D + 16 * ((4 * ks + 2 * g + h) ^ kx);
#pragma unroll
    for (int h = 0; h < 2; ++h) vro[h] = lq * kTileKeys + 16 * ((2 * g + h) ^ vx);
  }
  auto kfrag = [&](const unsigned char* kb, int j, int ks) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(kb + kro[ks][0] + j * 32 * D);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(kb + kro[ks][1] + j * 32 * D);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto qfrag = [&](int ks) { return qreg[ks]; };
  auto vfrag = [&](const unsigned char* vb, int db) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(vb + vro[0] + db * 32 * kTileKeys);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(vb + vro[1] + db * 32 * kTileKeys);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // operand formats 0 (e4m3) for both, block scales 127 (2^0 in E8M0)
  auto mm = [](const i32x8& x, const i32x8& y, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 127, 0, 127);
  };
  using SS = f32x16[2];
  auto qk = [&](const unsigned char* kb, SS& s) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const i32x8 qf = qfrag(ks);
      s[0] = mm(kfrag(kb, 0, ks), qf, s[0]);
      s[1] = mm(kfrag(kb, 1, ks), qf, s[1]);
    }
  };
  // exponentials of the tile's 64 keys against -negm, their lane sum, and
  // the P^T operand (half g: keys 32 g + 0..31)
  auto exps = [&](const SS& s, i32x8& p, float negm) {
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float e0[4], e1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][4 * i + r], a.scale_log2, negm));
        e1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1][4 * i + r], a.scale_log2, negm));
        lsum += e0[r] + e1[r];
      }
      int x0 = __builtin_amdgcn_cvt_pk_fp8_f32(e0[0], e0[1], __float_as_int(e0[0]), false);
      x0 = __builtin_amdgcn_cvt_pk_fp8_f32(e0[2], e0[3], x0, true);
      int x1 = __builtin_amdgcn_cvt_pk_fp8_f32(e1[0], e1[1], __float_as_int(e1[0]), false);
      x1 = __builtin_amdgcn_cvt_pk_fp8_f32(e1[2], e1[3], x1, true);
      auto r = __builtin_amdgcn_permlane32_swap((unsigned)x0, (unsigned)x1, false, false);
      p[2 * i] = (int)r[0];
      p[2 * i + 1] = (int)r[1];
    }
    return lsum;
  };
  auto body = [&](const SS& s_cur, SS& s_nxt, i32x8& p_cur, const i32x8& p_prev, const unsigned char* kn,
                  const unsigned char* vp, float& lsum, auto exp_tag, auto qk_tag, auto pv_tag) {
    constexpr bool kExp = decltype(exp_tag)::value;
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPV = decltype(pv_tag)::value;
    if constexpr (kQK) {
      s_nxt[0] = f32x16{};
      s_nxt[1] = f32x16{};
    }
    i32x8 qf;
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      if constexpr (kQK) {
        const int j = i & 1, ks = i >> 1;
        if (j == 0) qf = qfrag(ks);
        s_nxt[j] = mm(kfrag(kn, j, ks), qf, s_nxt[j]);
      }
      if constexpr (kPV) oacc[i] = mm(vfrag(vp, i), p_prev, oacc[i]);
    }
    if constexpr (!kExp) return false;
    lsum = exps(s_cur, p_cur, -m_run);
    // keeps the packing of P(u) inside this sub-iteration's interleaved VALU stream
    asm volatile("" ::"v"(p_cur));
    constexpr int kMfma = (kQK ? 2 * NK : 0) + (kPV ? NDB : 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    return !(lsum <= kSumLimit8);
  };
  auto mask = [&](SS& s, int kpos) {
    const int qpos = qw_pos + lq;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = kpos + 32 * j + 8 * (r >> 2) + 4 * g + (r & 3);
        if (kp > qpos) s[j][r] = neg_inf();
      }
  };
  auto sub = [&](int kpos, SS& s_cur, SS& s_nxt, i32x8& p_cur, const i32x8& p_prev, const unsigned char* kc,
                 const unsigned char* kn, const unsigned char* vp, auto exp_tag, auto qk_tag, auto pv_tag) {
    constexpr bool kExp = decltype(exp_tag)::value;
    const bool diag = kpos + 63 > qw_pos;
    if constexpr (kExp) {
      if (diag) mask(s_cur, kpos);
    }
    float lsum = 0.f;
    const bool redo = body(s_cur, s_nxt, p_cur, p_prev, kn, vp, lsum, exp_tag, qk_tag, pv_tag);
    if constexpr (kExp) {
      float alpha = 1.f;
      if (__any(redo)) {
        // the scores of tile u again (K(u) stays resident until the next sub-iteration)
        SS s;
        qk(kc, s);
        if (diag) mask(s, kpos);
        float mx = neg_inf();
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
        mx = half_max8(mx) * a.scale_log2;
        const float m_new = fmaxf(m_run, mx);
        alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        lsum = exps(s, p_cur, (m_run == neg_inf()) ? 0.f : -m_run);
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
  // Tile u: K(u) in one of three K buffers (kb_c; kb_n holds K(u+1), kb_f
  // receives K(u+2)), V(u) in V buffer u & 1.  Sub-iteration u forms P(u)
  // while its MFMAs are S(u+1) and O += V(u-1) P(u-1); K(u) stays resident
  // through it, for the rare recomputation of S(u).  At its top every wave is
  // done with K(u-1) and V(u-2); K(u+1) and V(u-1) have landed; load K(u+2)
  // and V(u) into those buffers.
  Cursor tc = chunk_after(-1);  // tile u
  Cursor tn = next_tile(tc);    // tile u+1
  Cursor tnn = next_tile(tn);   // tile u+2
  unsigned char* kb_c = lds_k0;
  unsigned char* kb_n = lds_k1;
  unsigned char* kb_f = lds_k2;
  auto barrier_and_prefetch = [&](int u) {
    wait_vmem_all();
    __syncthreads();
    if (u + 2 < T) load_k(tnn, kb_f);
    if (u >= 1) load_v(tc, (u & 1) ? lds_v1 : lds_v0);
  };
  auto advance = [&]() {
    tc = tn;
    tn = tnn;
    tnn = next_tile(tnn);
    unsigned char* const t = kb_c;
    kb_c = kb_n;
    kb_n = kb_f;
    kb_f = t;
  };
  using Yes = std::true_type;
  using No = std::false_type;
  if (T > 0) {
    load_k(tc, lds_k0);
    if (T > 1) load_k(tn, lds_k1);
    load_v(tc, lds_v0);
    wait_vmem_all();
    __syncthreads();
    SS sa, sb;
    i32x8 pa, pb;
    float dummy = 0.f;  // the row-sum output of the PV-only drain calls
    qk(lds_k0, sa);
    barrier_and_prefetch(0);
    // each branch ends with the drain: O += V(T-1) P(T-1), once V(T-1) has landed
    if (T == 1) {
      sub(tc.kpos, sa, sb, pa, pb, kb_c, kb_n, lds_v0, Yes{}, No{}, No{});
      wait_vmem_all();
      __syncthreads();
      body(sb, sa, pb, pa, kb_n, lds_v0, dummy, No{}, No{}, Yes{});
    } else {
      sub(tc.kpos, sa, sb, pa, pb, kb_c, kb_n, lds_v0, Yes{}, Yes{}, No{});
      advance();
      int u = 1;
      // u odd: S(u) in sb, S(u+1) into sa; u even: the other way round
      for (; u + 2 < T; u += 2) {
        barrier_and_prefetch(u);
        sub(tc.kpos, sb, sa, pb, pa, kb_c, kb_n, lds_v0, Yes{}, Yes{}, Yes{});
        advance();
        barrier_and_prefetch(u + 1);
        sub(tc.kpos, sa, sb, pa, pb, kb_c, kb_n, lds_v1, Yes{}, Yes{}, Yes{});
        advance();
      }
      if (u + 1 < T) {
        // u = T-2 (odd): one full sub-iteration, then the last tile (even)
        barrier_and_prefetch(u);
        sub(tc.kpos, sb, sa, pb, pa, kb_c, kb_n, lds_v0, Yes{}, Yes{}, Yes{});
        advance();
        barrier_and_prefetch(u + 1);
        sub(tc.kpos, sa, sb, pa, pb, kb_c, kb_n, lds_v1, Yes{}, No{}, Yes{});
        wait_vmem_all();
        __syncthreads();
        body(sb, sa, pb, pa, kb_n, lds_v0, dummy, No{}, No{}, Yes{});
      } else {
        // u = T-1 (odd): the last tile
        barrier_and_prefetch(u);
        sub(tc.kpos, sb, sa, pb, pa, kb_c, kb_n, lds_v0, Yes{}, No{}, Yes{});
        wait_vmem_all();
        __syncthreads();
        body(sa, sb, pa, pb, kb_n, lds_v1, dummy, No{}, No{}, Yes{});
      }
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

// Eight waves (256 rows), two per SIMD, held to 248 VGPRs like the bf16 step
// kernel, so that registers stay free for the waves of a concurrent staging
// copy on the copy stream.
__global__ void __launch_bounds__(512, 1) __attribute__((amdgpu_num_vgpr(124))) fp8_step_kernel(const Fp8StepArgs a) {
  fp8_step_body<8>(a);
}
// Four waves (128 rows), two workgroups per CU under the same register budget:
// for grids of 256-row workgroups that would leave compute units idle, and for
// query chunk lengths that are multiples of 128 but not of 256.
__global__ void __launch_bounds__(256, 2) __attribute__((amdgpu_num_vgpr(124)))
fp8_step_kernel_128(const Fp8StepArgs a) {
  fp8_step_body<4>(a);
}

int fp8_device_cus() {
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

hipError_t launch_step_fp8(const Fp8StepArgs& args, hipStream_t stream, const char** name) {
  // A row's result does not depend on the row-block size (a block only decides
  // which tiles it stages; keys past a row are masked), so the launch picks it:
  // 256-row blocks unless their grid would leave compute units idle, or would
  // give each unit exactly one block of a launch that holds a diagonal chunk
  // pair (block work then ranges from a few tiles to twice the mean; two
  // 128-row blocks per unit let the light ones finish beside the heavy ones).
  Fp8StepArgs a = args;
  int bm = (a.q_chunk_len % 256 == 0) ? 256 : 128;
  bool diag = false;
  for (int i = 0; i < a.n_order; ++i)
    for (int k = 0; k < a.n_kv_chunks; ++k) diag = diag || a.q_start[a.order[i]] == a.kv_start[k];
  const long long g256 = (long long)a.n_order * (a.q_chunk_len / 256) * a.BH;
  if (bm == 256 && (g256 < fp8_device_cus() || (diag && g256 <= fp8_device_cus()))) bm = 128;
  a.rb_per_chunk = a.q_chunk_len / bm;
  const long long grid = (long long)a.n_order * a.rb_per_chunk * a.BH;
  if (name) *name = nullptr;
  if (grid <= 0) return hipSuccess;
  // heads per group of the XCD-aware order, as for the bf16 step kernel
  if (a.heads_per_xcd > 0)
    a.heads_per_group = heads_per_group(a.heads_per_xcd, (long long)a.n_order * a.rb_per_chunk,
                                        (long long)(fp8_device_cus() / 8) * (bm == 256 ? 1 : 2) * (diag ? 2 : 1));
  if (bm == 256)
    hipLaunchKernelGGL(fp8_step_kernel, dim3((unsigned)grid), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(fp8_step_kernel_128, dim3((unsigned)grid), dim3(256), 0, stream, a);
  if (name) *name = bm == 256 ? "fp8_step_kernel" : "fp8_step_kernel_128";
  return hipGetLastError();
}

}  // namespace cpattn
