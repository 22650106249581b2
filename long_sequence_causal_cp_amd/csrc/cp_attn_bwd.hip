// gfx950 kernels for the backward pass of one ring step of causal attention.
//
// Sources (web pages, cited by title and section):
//   [MLM] "Megatron-LM源码解析：Context Parallel如何革新长序列训练", section 2
//         (the backward pass mirrors the forward: the K/V gradients go back
//         along the path the blocks came) and section 5 (forward and backward
//         of one autograd function around the per-step attention).
//   [RAF] "如何用Context并行加速大模型训练？手把手教你配置RingAttention+FlashAttention",
//         section 3 (per-step attention over one received K/V block, mask
//         from the blocks' absolute offsets).
//
// The gradients are those of softmax attention over the visible keys,
// recomputing the probabilities from the forward's saved log-sum-exp:
//   P = exp(tau q.k - LSE),  dV = P^T dO,  dP = dO V^T,
//   Delta = rowsum(dO * O),  dS = P (dP - Delta),
//   dQ = tau dS K,  dK = tau dS^T Q.
// Every term for one key needs only that key and the queries' complete
// forward results, so one K/V block's contribution is separable: its dQ part
// adds to the query rows' gradient, and its dK, dV are that block's rows.
//
// Two kernels, each owning its output rows (no atomics, deterministic):
//   * dq kernel (query-stationary): a wave holds 32 query rows, one per lane
//     pair, like the forward step kernel; per 32-key sub-tile it forms
//     S^T = K Q^T and dP^T = V dO^T by MFMA, then dS^T lane-locally, and
//     accumulates dQ^T += K^T dS^T with K^T read through the LDS transpose
//     read.
//   * dk/dv kernel (key-stationary): a wave holds 32 keys, K and V rows in
//     registers; per 32-query sub-tile it forms S = Q K^T and dP = dO V^T,
//     then P and dS with the per-query LSE and Delta staged in LDS, and
//     accumulates dV^T += dO^T P and dK^T += Q^T dS.
// Tiles of 64 rows are staged HBM -> LDS by the direct-to-LDS loads of the
// forward, double buffered, in both LDS layouts where a tile is read both
// as rows and transposed.
#include "cp_attn_internal.h"
#include "cp_attn_tile.h"

namespace cpattn {
namespace {


// Per-lane byte offsets of the transposed (ds_read_b64_tr_b16) reads of a
// V-layout tile: for 32-row block db of D, the A operand X^T[d][row] of one
// 16-row k-step.
template <int D>
struct TrOffsets {
  static constexpr int NDB = D / 32;
  int off[NDB];
  __device__ __forceinline__ explicit TrOffsets(int lane) {
    const int g = lane >> 5, j16 = lane & 15, G = lane >> 4;
    const int tr_row = 4 * g + (j16 >> 2);
    const int swz = v_swz<D>(tr_row);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      off[db] = tr_row * (D * 2) + (((4 * db + 2 * (G & 1) + ((j16 & 3) >> 1)) ^ swz) << 4) + 8 * (j16 & 1);
  }
  // A operand X^T[32 db + lane row][rows 16 t .. 16 t + 15 of sub-tile h] of
  // the V-layout tile at `tile`
  __device__ __forceinline__ bf16x8 read(const unsigned char* tile, int h, int t, int db) const {
    const unsigned char* base = tile + (32 * h + 16 * t) * (D * 2) + off[db];
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, base + 8 * (D * 2)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Write (or add) a lane's share of a 32 x D transposed accumulator X^T (lane
// column = row lq of X) to row-major fp32 rows at `row_ptr` (row lq), times
// `scale`.
template <int D>
__device__ __forceinline__ void store_rows(float* row_ptr, const f32x16 (&acc)[D / 32], float scale, bool add,
                                           int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float* p = row_ptr + 32 * db + 8 * rr + 4 * g;
      f32x4 o;
      o[0] = acc[db][4 * rr + 0] * scale;
      o[1] = acc[db][4 * rr + 1] * scale;
      o[2] = acc[db][4 * rr + 2] * scale;
      o[3] = acc[db][4 * rr + 3] * scale;
      if (add) o += *reinterpret_cast<const f32x4*>(p);
      *reinterpret_cast<f32x4*>(p) = o;
    }
}

// log2-domain shift for a row's probabilities: -LSE log2(e), and -inf for a
// row without any visible key (LSE = -inf), whose probabilities are all 0.
__device__ __forceinline__ float neg_lse2(float lse) { return lse == neg_inf() ? neg_inf() : -lse * kLog2e; }

// ---------------------------------------------------------------- dq kernel
template <int D, int NW>
__device__ __forceinline__ void dq_body(const BwdArgs& a) {
  constexpr int BM = 32 * NW;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TB = kTileKeys * D * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k[2 * TB];   // K, K layout (rows)
  __shared__ __attribute__((aligned(1024))) unsigned char lds_kt[2 * TB];  // K, V layout (transposed reads)
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v[2 * TB];   // V, K layout (rows)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int lq = lane & 31;

  int rb_idx, bh;
  xcd_job(blockIdx.x, a.BH, a.heads_per_xcd, a.heads_per_group, a.Sq / BM, rb_idx, bh);
  const int rb = a.Sq / BM - 1 - rb_idx;  // later rows (more keys) first
  const int q_local0 = rb * BM;
  const int qc = q_local0 / a.q_chunk_len;
  const int q_pos0 = a.q_start[qc] + (q_local0 - qc * a.q_chunk_len);
  const int q_posmax = q_pos0 + BM - 1;
  const int qw_pos = q_pos0 + 32 * wave_u;
  const size_t row = (size_t)bh * a.Sq + q_local0 + 32 * wave + lq;
  const size_t bh_kv = (size_t)bh * a.Skv;

  // visible 64-key tiles per K/V chunk (first key <= q_posmax)
  const int tiles_per_chunk = a.kv_chunk_len / kTileKeys;
  int n_vis[kMaxChunks], kv_start[kMaxChunks];
  int T = 0;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    kv_start[c] = a.kv_start[c];
    int nv = 0;
    if (c < a.n_kv_chunks && q_posmax >= kv_start[c]) {
      nv = (q_posmax - kv_start[c]) / kTileKeys + 1;
      nv = nv < tiles_per_chunk ? nv : tiles_per_chunk;
    }
    n_vis[c] = nv;
    T += nv;
  }
  struct Cursor {
    int c, left, kpos;
    const uint16_t* kp;  // the tile's first K row
    const uint16_t* vp;  // and V row
  };
  auto chunk_after = [&](int after) {
    Cursor t{kMaxChunks, 0, 0, a.k, a.v};
#pragma unroll
    for (int c = kMaxChunks - 1; c >= 0; --c)
      if (c > after && n_vis[c] > 0) {
        const size_t off = (bh_kv + (size_t)c * a.kv_chunk_len) * D;
        t = Cursor{c, n_vis[c], kv_start[c], a.k + off, a.v + off};
      }
    return t;
  };
  auto next_tile = [&](Cursor t) {
    t.left -= 1;
    t.kpos += kTileKeys;
    t.kp += kTileKeys * D;
    t.vp += kTileKeys * D;
    if (t.left <= 0) t = chunk_after(t.c);
    return t;
  };
  const TileLoad<D, NW> rows_loader(true, wave_u, lane), tr_loader(false, wave_u, lane);
  auto load = [&](const Cursor& t, int buf) {
    rows_loader(t.kp, lds_k + buf * TB, wave_u);
    tr_loader(t.kp, lds_kt + buf * TB, wave_u);
    rows_loader(t.vp, lds_v + buf * TB, wave_u);
  };

  // Q^T and dO^T fragments: lane holds X[row lq][16 s + 8 g .. + 8]
  bf16x8 qf[NS], of[NS];
  {
    const uint16_t* qrow = a.q + row * D + 8 * g;
    const uint16_t* orow = a.dout + row * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
      of[s] = *reinterpret_cast<const bf16x8*>(orow + 16 * s);
    }
  }
  const float nl2 = neg_lse2(a.lse[row]);
  const float dl = a.delta[row];

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  const int k_base = k_lds_off(lq, 0, g);
  const TrOffsets<D> tr(lane);

  // one 32-key sub-tile h of the tile in buffer `buf`, first key at kpos
  auto sub = [&](int buf, int h, int kpos) {
    if (kpos > qw_pos + 31) return;  // every key after every row of this wave
    const unsigned char* kb = lds_k + buf * TB;
    const unsigned char* vb = lds_v + buf * TB;
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + k_base + st * 2048 + h * 1024);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s, 0, 0, 0);
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vb + k_base + st * 2048 + h * 1024);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, of[st], dp, 0, 0, 0);
    }
    // element r: key kpos + 8 (r >> 2) + 4 g + (r & 3), query qw_pos + lq
    if (kpos + 31 > qw_pos) {
      const int qpos = qw_pos + lq;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kpos + 8 * (r >> 2) + 4 * g + (r & 3) > qpos) s[r] = neg_inf();
    }
    bf16x8 ds[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * t + e], a.scale_log2, nl2));
        ds[t][e] = (__bf16)(p * (dp[8 * t + e] - dl));
      }
    const unsigned char* ktb = lds_kt + buf * TB;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr.read(ktb, h, t, db), ds[t], acc[db], 0, 0, 0);
  };

  Cursor cur = chunk_after(-1);
  if (T > 0) load(cur, 0);
  for (int n = 0; n < T; ++n) {
    // tile n has landed in buffer n & 1; every wave is done with buffer (n + 1) & 1
    wait_vmem_all();
    __syncthreads();
    const Cursor nxt = next_tile(cur);
    if (n + 1 < T) load(nxt, (n + 1) & 1);
    sub(n & 1, 0, cur.kpos);
    sub(n & 1, 1, cur.kpos + 32);
    cur = nxt;
  }
  // adding a part that no key contributes to would rewrite the rows unchanged
  const bool add_q = (a.accumulate & 1) != 0;
  if (T > 0 || !add_q) store_rows<D>(a.dq + row * D, acc, a.scale, add_q, g);
}

// ------------------------------------------------------------ dk/dv kernel
template <int D, int NW>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a) {
  constexpr int BN = 32 * NW;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TB = kTileKeys * D * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_q[2 * TB];   // Q, K layout (rows)
  __shared__ __attribute__((aligned(1024))) unsigned char lds_qt[2 * TB];  // Q, V layout (transposed reads)
  __shared__ __attribute__((aligned(1024))) unsigned char lds_o[2 * TB];   // dO, K layout
  __shared__ __attribute__((aligned(1024))) unsigned char lds_ot[2 * TB];  // dO, V layout
  __shared__ __attribute__((aligned(16))) float lds_nl2[2][kTileKeys];     // -LSE log2(e) per query
  __shared__ __attribute__((aligned(16))) float lds_dl[2][kTileKeys];      // Delta per query

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 5;
  const int lq = lane & 31;

  int kb_idx, bh;
  xcd_job(blockIdx.x, a.BH, a.heads_per_xcd, a.heads_per_group, a.Skv / BN, kb_idx, bh);
  const int k_local0 = kb_idx * BN;  // earlier keys (more queries) first
  const int kc = k_local0 / a.kv_chunk_len;
  const int k_pos0 = a.kv_start[kc] + (k_local0 - kc * a.kv_chunk_len);
  const int kw_pos = k_pos0 + 32 * wave_u;
  const size_t krow = (size_t)bh * a.Skv + k_local0 + 32 * wave + lq;
  const size_t bh_q = (size_t)bh * a.Sq;

  // visible 64-query tiles per query chunk (last query >= k_pos0)
  const int tiles_per_chunk = a.q_chunk_len / kTileKeys;
  int n_vis[kMaxChunks], first[kMaxChunks], q_start[kMaxChunks];
  int T = 0;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    q_start[c] = a.q_start[c];
    int f = 0, nv = 0;
    if (c < a.n_q_chunks) {
      const int x = k_pos0 - q_start[c] - (kTileKeys - 1);
      f = x <= 0 ? 0 : (x + kTileKeys - 1) / kTileKeys;
      nv = tiles_per_chunk - f;
      nv = nv > 0 ? nv : 0;
    }
    first[c] = f;
    n_vis[c] = nv;
    T += nv;
  }
  struct Cursor {
    int c, left, qpos, qrow;  // chunk, tiles left in it, first query's position and local row
  };
  auto chunk_after = [&](int after) {
    Cursor t{kMaxChunks, 0, 0, 0};
#pragma unroll
    for (int c = kMaxChunks - 1; c >= 0; --c)
      if (c > after && n_vis[c] > 0)
        t = Cursor{c, n_vis[c], q_start[c] + kTileKeys * first[c], c * a.q_chunk_len + kTileKeys * first[c]};
    return t;
  };
  auto next_tile = [&](Cursor t) {
    t.left -= 1;
    t.qpos += kTileKeys;
    t.qrow += kTileKeys;
    if (t.left <= 0) t = chunk_after(t.c);
    return t;
  };
  const TileLoad<D, NW> rows_loader(true, wave_u, lane), tr_loader(false, wave_u, lane);
  auto load = [&](const Cursor& t, int buf) {
    const size_t off = (bh_q + t.qrow) * D;
    rows_loader(a.q + off, lds_q + buf * TB, wave_u);
    tr_loader(a.q + off, lds_qt + buf * TB, wave_u);
    rows_loader(a.dout + off, lds_o + buf * TB, wave_u);
    tr_loader(a.dout + off, lds_ot + buf * TB, wave_u);
  };

  // K^T and V^T fragments: lane holds X[key lq][16 s + 8 g .. + 8]
  bf16x8 kf[NS], vf[NS];
  {
    const uint16_t* kr = a.k + krow * D + 8 * g;
    const uint16_t* vr = a.v + krow * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8*>(kr + 16 * s);
      vf[s] = *reinterpret_cast<const bf16x8*>(vr + 16 * s);
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const int k_base = k_lds_off(lq, 0, g);
  const TrOffsets<D> tr(lane);

  // one 32-query sub-tile h of the tile in buffer `buf`, first query at qpos
  auto sub = [&](int buf, int h, int qpos) {
    if (qpos + 31 < kw_pos) return;  // every query before every key of this wave
    const unsigned char* qb = lds_q + buf * TB;
    const unsigned char* ob = lds_o + buf * TB;
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qb + k_base + st * 2048 + h * 1024);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[st], s, 0, 0, 0);
    }
    // dP after S (not interleaved): fewer operand reads in flight at once
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bf16x8 oa = *reinterpret_cast<const bf16x8*>(ob + k_base + st * 2048 + h * 1024);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[st], dp, 0, 0, 0);
    }
    // element r: query qpos + 8 (r >> 2) + 4 g + (r & 3), key kw_pos + lq
    if (qpos < kw_pos + 31) {
      const int kpos = kw_pos + lq;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kpos > qpos + 8 * (r >> 2) + 4 * g + (r & 3)) s[r] = neg_inf();
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int qi = 32 * h + 8 * rq + 4 * g;
      const f32x4 nl = *reinterpret_cast<const f32x4*>(&lds_nl2[buf][qi]);
      const f32x4 dl = *reinterpret_cast<const f32x4*>(&lds_dl[buf][qi]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rq + i;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, nl[i]));
        pb[r >> 3][r & 7] = (__bf16)p;
        dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl[i]));
      }
    }
    const unsigned char* qtb = lds_qt + buf * TB;
    const unsigned char* otb = lds_ot + buf * TB;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr.read(otb, h, t, db), pb[t], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr.read(qtb, h, t, db), dsb[t], dk[db], 0, 0, 0);
      }
  };

  // per-query statistics of a tile: wave 0 fetches them into registers and
  // writes them to LDS once the buffer they go to is free
  float st_nl2 = 0.f, st_dl = 0.f;
  auto fetch_stats = [&](const Cursor& t) {
    const size_t r = bh_q + t.qrow + lane;
    st_nl2 = neg_lse2(a.lse[r]);
    st_dl = a.delta[r];
  };
  auto put_stats = [&](int buf) {
    lds_nl2[buf][lane] = st_nl2;
    lds_dl[buf][lane] = st_dl;
  };

  Cursor cur = chunk_after(-1);
  if (T > 0) {
    load(cur, 0);
    if (wave == 0) {
      fetch_stats(cur);
      put_stats(0);
    }
  }
  for (int n = 0; n < T; ++n) {
    // tile n (and its statistics) are in buffer n & 1; every wave is done
    // with buffer (n + 1) & 1
    wait_vmem_all();
    __syncthreads();
    const Cursor nxt = next_tile(cur);
    const bool more = n + 1 < T;
    if (more) {
      load(nxt, (n + 1) & 1);
      if (wave == 0) fetch_stats(nxt);
    }
    sub(n & 1, 0, cur.qpos);
    sub(n & 1, 1, cur.qpos + 32);
    if (more && wave == 0) put_stats((n + 1) & 1);
    cur = nxt;
  }
  const bool add = (a.accumulate & 2) != 0;
  if (T == 0 && add) return;  // no query sees these keys: the partial sums stay as they are
  store_rows<D>(a.dk + krow * D, dk, a.scale, add, g);
  store_rows<D>(a.dv + krow * D, dv, 1.f, add, g);
}

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 1) bwd_dq_kernel(const BwdArgs a) {
  dq_body<D, NW>(a);
}
// Two waves per SIMD at 256 keys per workgroup (8 waves): the register budget
// is then 256 per lane, which the dk and dv accumulators (128) and the
// stationary K and V fragments (64) nearly fill.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(const BwdArgs a) {
  dkdv_body<D, NW>(a);
}

// delta[r] = sum_d dout[r][d] out[r][d]: D/8 lanes per row, 16 bytes each,
// fp32 products and sums; HBM-bound.
__global__ void __launch_bounds__(256) bwd_delta_kernel(const uint16_t* __restrict__ out,
                                                        const uint16_t* __restrict__ dout, float* __restrict__ delta,
                                                        int64_t rows, int D) {
  const int tpr = D / 8;
  const int rpb = 256 / tpr;
  const int r_in = threadIdx.x / tpr, j = threadIdx.x % tpr;
  for (int64_t base = (int64_t)blockIdx.x * rpb; base < rows; base += (int64_t)gridDim.x * rpb) {
    const int64_t r = base + r_in;
    float s = 0.f;
    if (r < rows) {
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(out + r * D + 8 * j);
      const bf16x8 d = *reinterpret_cast<const bf16x8*>(dout + r * D + 8 * j);
#pragma unroll
      for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)o[e], (float)d[e], s);
    }
    // sum over the row's tpr consecutive lanes (tpr divides 64)
    for (int w = tpr / 2; w > 0; w >>= 1) s += __shfl_xor(s, w);
    if (r < rows && j == 0) delta[r] = s;
  }
}

}  // namespace

int bwd_dq_rows(int q_chunk_len) {
  return (q_chunk_len % 256 == 0) ? 256 : (q_chunk_len % 128 == 0) ? 128 : 64;
}
int bwd_dkdv_keys(int kv_chunk_len) { return (kv_chunk_len % 256 == 0) ? 256 : (kv_chunk_len % 128 == 0) ? 128 : 64; }

namespace {
int bwd_device_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      return cus;
    return 256;
  }();
  return n;
}

// Whether the block holds a diagonal chunk pair (a query chunk at a key
// chunk's position).
bool bwd_diag(const BwdArgs& a) {
  bool diag = false;
  for (int i = 0; i < a.n_q_chunks; ++i)
    for (int k = 0; k < a.n_kv_chunks; ++k) diag = diag || a.q_start[i] == a.kv_start[k];
  return diag;
}
// Heads per group of the XCD-aware job order: a head's blocks run together
// (one workgroup per CU), twice as many where block work differs (diagonal).
int bwd_heads_per_group(const BwdArgs& a, long long blocks_per_head) {
  if (a.heads_per_xcd <= 0) return 0;
  return heads_per_group(a.heads_per_xcd, blocks_per_head, (long long)(bwd_device_cus() / 8) * (bwd_diag(a) ? 2 : 1));
}
}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& args, hipStream_t stream, const char** name) {
  BwdArgs a = args;
  // The grid covers every query row of the rank, and in a ring step past the
  // first the rows of one chunk see no key (their workgroups end at once).  Where
  // a grid of 256-row workgroups holds at most one per compute unit, 128-row
  // ones spread the busy rows over twice as many units.  A row's dQ does not
  // depend on the choice: its wave sums the same key tiles in the same order,
  // and the tiles a larger block adds are masked to exact zeros.
  int bm = bwd_dq_rows(a.q_chunk_len);
  if (bm == 256 && (long long)a.BH * (a.Sq / 256) <= bwd_device_cus()) bm = 128;
  const long long grid = (long long)a.BH * (a.Sq / bm);
  if (name) *name = nullptr;
  if (grid <= 0) return hipSuccess;
  a.heads_per_group = bwd_heads_per_group(a, a.Sq / bm);
  const dim3 g((unsigned)grid), blk((unsigned)(2 * bm));  // one wave per 32 rows
  const char* n;
  if (a.D == 128) {
    if (bm == 256) { hipLaunchKernelGGL((bwd_dq_kernel<128, 8>), g, blk, 0, stream, a); n = "bwd_dq_kernel<128, 8>"; }
    else if (bm == 128) { hipLaunchKernelGGL((bwd_dq_kernel<128, 4>), g, blk, 0, stream, a); n = "bwd_dq_kernel<128, 4>"; }
    else { hipLaunchKernelGGL((bwd_dq_kernel<128, 2>), g, blk, 0, stream, a); n = "bwd_dq_kernel<128, 2>"; }
  } else {
    if (bm == 256) { hipLaunchKernelGGL((bwd_dq_kernel<64, 8>), g, blk, 0, stream, a); n = "bwd_dq_kernel<64, 8>"; }
    else if (bm == 128) { hipLaunchKernelGGL((bwd_dq_kernel<64, 4>), g, blk, 0, stream, a); n = "bwd_dq_kernel<64, 4>"; }
    else { hipLaunchKernelGGL((bwd_dq_kernel<64, 2>), g, blk, 0, stream, a); n = "bwd_dq_kernel<64, 2>"; }
  }
  if (name) *name = n;
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& args, hipStream_t stream, const char** name) {
  BwdArgs a = args;
  // In a step that holds a diagonal chunk pair, a grid of 256-key workgroups
  // with at most one per compute unit has blocks whose work ranges from a few
  // query tiles to twice the mean, and with fewer blocks than units it also
  // leaves units idle; 128-key blocks, two per unit, let the light ones finish
  // beside the heavy ones and spread the work over more units.  A key's dK, dV
  // are the same either way (its wave sums the same query tiles in order).
  int bn = bwd_dkdv_keys(a.kv_chunk_len);
  const bool diag = bwd_diag(a);
  if (bn == 256 && diag && (long long)a.BH * (a.Skv / 256) <= bwd_device_cus()) bn = 128;
  const long long grid = (long long)a.BH * (a.Skv / bn);
  if (name) *name = nullptr;
  if (grid <= 0) return hipSuccess;
  a.heads_per_group = bwd_heads_per_group(a, a.Skv / bn);
  const dim3 g((unsigned)grid), blk((unsigned)(2 * bn));  // one wave per 32 keys
  const char* n;
  if (a.D == 128) {
    if (bn == 256) { hipLaunchKernelGGL((bwd_dkdv_kernel<128, 8>), g, blk, 0, stream, a); n = "bwd_dkdv_kernel<128, 8>"; }
    else if (bn == 128) { hipLaunchKernelGGL((bwd_dkdv_kernel<128, 4>), g, blk, 0, stream, a); n = "bwd_dkdv_kernel<128, 4>"; }
    else { hipLaunchKernelGGL((bwd_dkdv_kernel<128, 2>), g, blk, 0, stream, a); n = "bwd_dkdv_kernel<128, 2>"; }
  } else {
    if (bn == 256) { hipLaunchKernelGGL((bwd_dkdv_kernel<64, 8>), g, blk, 0, stream, a); n = "bwd_dkdv_kernel<64, 8>"; }
    else if (bn == 128) { hipLaunchKernelGGL((bwd_dkdv_kernel<64, 4>), g, blk, 0, stream, a); n = "bwd_dkdv_kernel<64, 4>"; }
    else { hipLaunchKernelGGL((bwd_dkdv_kernel<64, 2>), g, blk, 0, stream, a); n = "bwd_dkdv_kernel<64, 2>"; }
  }
  if (name) *name = n;
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const uint16_t* out, const uint16_t* dout, float* delta, int64_t rows, int D,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int rpb = 256 / (D / 8);
  long long blocks = (rows + rpb - 1) / rpb;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, dout, delta, rows, D);
  return hipGetLastError();
}

}  // namespace cpattn
