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
// tiles of 64 keys are staged HBM -> registers -> LDS (16-byte loads, double
// buffered, one barrier per tile).  Per tile a wave computes the transposed
// score block S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so that every lane
// holds one query's scores; the causal mask, the row maximum and the
// exponentials are then lane-local, with one cross-half exchange
// (v_permlane32_swap) per tile.  P^T feeds the second MFMA directly from
// registers; V^T comes from the row-major V tile through the gfx950 LDS
// transpose read (ds_read_b64_tr_b16).  The epilogue divides by the row sum,
// forms the natural-log LSE and merges into the running fp32 result by
// log-sum-exp rescaling, optionally writing the bf16 output.
#include "cp_attn_internal.h"

#include <math.h>

#include <type_traits>

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A row's stored maximum is only raised when a tile exceeds it by more than
// 2^8 in probability scale; smaller excesses leave p <= 256, exact in fp32.
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

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

// LDS layouts of one 64-key tile, row-major [key][d] bf16, 16-byte chunks
// XOR-swizzled so that the MFMA operand reads hit distinct banks.
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * (D * 2) + ((c ^ (r & (D / 8 - 1))) << 4);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int v_off(int r, int c) {
  return r * (D * 2) + ((c ^ v_swz<D>(r)) << 4);
}

// Four-wave workgroups are built for two waves per SIMD (at most 256 VGPRs),
// so two workgroups share a CU and one's softmax overlaps the other's MFMAs.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) step_kernel(const StepArgs a) {
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int NC = D / 8;    // 16-byte chunks per row
  constexpr int NS = D / 16;   // k-steps of the QK^T MFMA
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int TB = kTileKeys * D * 2;
  constexpr int CPT = kTileKeys * NC / NT;  // chunks per thread per tile
  static_assert(CPT * NT == kTileKeys * NC, "tile load must divide evenly");
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int lq = lane & 31;

  // ---- which (row block, batch*head) this workgroup owns ----
  const int job = blockIdx.x;
  int rb_idx, bh;
  if (a.heads_per_xcd > 0) {
    // workgroups are dealt to the 8 XCDs round-robin: keep each head's row
    // blocks on one XCD so its K/V tiles are shared through that XCD's L2
    const int x = job & 7, kk = job >> 3;
    rb_idx = kk / a.heads_per_xcd;
    bh = x * a.heads_per_xcd + kk % a.heads_per_xcd;
  } else {
    rb_idx = job / a.BH;
    bh = job % a.BH;
  }
  const int oi = rb_idx / a.rb_per_chunk;
  const int rbi = a.rb_per_chunk - 1 - rb_idx % a.rb_per_chunk;  // later rows (more keys) first
  const int qc = a.order[oi];
  const int flags = a.flags[qc];
  const int q_local0 = qc * a.q_chunk_len + rbi * BM;
  const int q_pos0 = a.q_start[qc] + rbi * BM;
  const int q_posmax = q_pos0 + BM - 1;
  const int qw_local = q_local0 + wave * 32;
  const int qw_pos = q_pos0 + wave * 32;
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
  auto tile_at = [&](int it, int& krow, int& kpos) {
    int c = 0;
#pragma unroll
    for (int cc = 0; cc < kMaxChunks - 1; ++cc)
      if (c == cc && it >= n_vis[cc]) { it -= n_vis[cc]; c = cc + 1; }
    krow = c * a.kv_chunk_len + it * kTileKeys;
    kpos = a.kv_start[c] + it * kTileKeys;
  };

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
  const int j16 = lane & 15;
  const int G = lane >> 4;
  const int tr_row = 4 * g + (j16 >> 2);               // + 16t (+8)
  const int tr_swz = v_swz<D>(tr_row);
  const int tr_colbyte = 8 * (j16 & 1);
  int tr_chunk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) tr_chunk[db] = 4 * db + 2 * (G & 1) + ((j16 & 3) >> 1);

  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int it) {
    int krow, kpos;
    tile_at(it, krow, kpos);
    const uint16_t* kb = a.k + (bh_kv + krow) * D;
    const uint16_t* vb = a.v + (bh_kv + krow) * D;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / NC, c = idx % NC;
      kreg[i] = *reinterpret_cast<const u32x4*>(kb + r * D + 8 * c);
      vreg[i] = *reinterpret_cast<const u32x4*>(vb + r * D + 8 * c);
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* kl = lds + buf * 2 * TB;
    unsigned char* vl = kl + TB;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / NC, c = idx % NC;
      *reinterpret_cast<u32x4*>(kl + k_off<D>(r, c)) = kreg[i];
      *reinterpret_cast<u32x4*>(vl + v_off<D>(r, c)) = vreg[i];
    }
  };

  auto compute_tile = [&](int buf, int kpos, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const unsigned char* kl = lds + buf * 2 * TB;
    const unsigned char* vl = kl + TB;
    // S^T = K Q^T over two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const int r = 32 * kb + lq;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + k_off<D>(r, 2 * s + g));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kb], 0, 0, 0);
      }
    }
    if constexpr (kMasked) {
      const int qpos = qw_pos + lq;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kp = kpos + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          if (kp > qpos) sacc[kb][r] = neg_inf();
        }
    }
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = xhalf_max(mx) * a.scale_log2;
    const bool need = mx > m_run + kRescaleThreshold;
    if (__any(need)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_lane *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float negm = (m_run == neg_inf()) ? 0.f : -m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], a.scale_log2, negm));
        sacc[kb][r] = p;
        l_lane += p;
      }
    // O^T += V^T P^T, four k-steps of 16 keys
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[t >> 1][8 * (t & 1) + e];
      const int row1 = 16 * t + tr_row;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int cb = ((tr_chunk[db] ^ tr_swz) << 4) + tr_colbyte;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vl + row1 * (D * 2) + cb));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vl + (row1 + 8) * (D * 2) + cb));
        const bf16x8 af = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb, oacc[db], 0, 0, 0);
      }
    }
  };

  if (T > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < T; ++it) {
      const int buf = it & 1;
      if (it + 1 < T) load_tile(it + 1);
      int krow, kpos;
      tile_at(it, krow, kpos);
      if (kpos <= qw_pos + 31) {  // this wave sees at least one key of the tile
        if (kpos + kTileKeys - 1 > qw_pos)
          compute_tile(buf, kpos, std::true_type{});
        else
          compute_tile(buf, kpos, std::false_type{});
      }
      if (it + 1 < T) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: normalise, LSE, merge, write ----
  const float l = xhalf_sum(l_lane);
  const float lse_j = (l > 0.f) ? (m_run + __log2f(l)) * kLn2 : neg_inf();
  const float inv_l = (l > 0.f) ? 1.f / l : 0.f;
  const size_t row = bh_q + qw_local + lq;
  float w_prev = 0.f, w_cur = inv_l, lse_new = lse_j;
  if (flags & kFlagMerge) {
    const float lp = a.lse_run[row];
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
  if (g == 0) a.lse_run[row] = lse_new;
  const bool write_o = (flags & kFlagWriteO) != 0;
  const bool finalize = (flags & kFlagFinalize) != 0;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d0 = 32 * db + 8 * rr + 4 * g;
      f32x4 o;
      o[0] = oacc[db][4 * rr + 0] * w_cur;
      o[1] = oacc[db][4 * rr + 1] * w_cur;
      o[2] = oacc[db][4 * rr + 2] * w_cur;
      o[3] = oacc[db][4 * rr + 3] * w_cur;
      if (w_prev != 0.f) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(a.o_run + row * D + d0);
        o += w_prev * prev;
      }
      if (write_o) *reinterpret_cast<f32x4*>(a.o_run + row * D + d0) = o;
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

}  // namespace

int step_block_rows(int q_chunk_len) { return (q_chunk_len % 128 == 0) ? 128 : 64; }

hipError_t launch_step(const StepArgs& a, int D, hipStream_t stream) {
  const int bm = step_block_rows(a.q_chunk_len);
  const long long grid = (long long)a.n_order * a.rb_per_chunk * a.BH;
  if (grid <= 0) return hipSuccess;
  if (D == 128 && bm == 128)
    hipLaunchKernelGGL((step_kernel<128, 4>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL((step_kernel<128, 2>), dim3((unsigned)grid), dim3(128), 0, stream, a);
  else if (bm == 128)
    hipLaunchKernelGGL((step_kernel<64, 4>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((step_kernel<64, 2>), dim3((unsigned)grid), dim3(128), 0, stream, a);
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
