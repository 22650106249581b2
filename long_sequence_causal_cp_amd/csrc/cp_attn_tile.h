// Device helpers shared by the forward and backward attention kernels:
// vector types, the two LDS tile layouts of a 64-row bf16 tile and the
// direct-to-LDS tile loader.  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cp_job_map.h"

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
__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// LDS layout of a K tile (64 keys x D): D/16 column blocks of 16 d-values;
// block st holds the 64 rows at 32 B each, and a row's two 16-B halves are
// swapped when bits 2 and 3 of the row differ.  The QK^T operand read of lane
// (row r, half g) in block st is then one base address plus the immediate
// st*2048, and any 8 (or 16) consecutive lanes hit distinct 16-B bank groups.
__device__ __forceinline__ int k_half_swap(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
__device__ __forceinline__ int k_lds_off(int r, int st, int g) {
  return st * 2048 + r * 32 + ((g ^ k_half_swap(r)) << 4);
}
// LDS layout of a V tile: row-major [key][d] bf16, 16-byte chunks XOR-swizzled
// by the row so that the transposed reads hit distinct banks.
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

// One direct-to-LDS load: each lane fetches the 16 bytes at `base` +
// `voff` (`base` wave-uniform, in SGPRs; `voff` this lane's byte offset);
// lane i's bytes land at LDS address `lds_dst` + 16 i (`lds_dst`
// wave-uniform, in M0).  With a scalar base and a precomputed offset no
// vector address arithmetic is spent per load.  Issued as inline assembly so
// that the compiler's LDS-counter bookkeeping is not made conservative by
// it: with a compiler-visible LDS DMA in flight every ds_read wait becomes
// lgkmcnt(0).  Completion is tracked by hand instead: wait_vmem_all() before
// the barrier that publishes the tile.  No other code in this file uses M0.
__device__ __forceinline__ void global_to_lds_16(const void* base, unsigned voff, unsigned char* lds_dst) {
  const unsigned m0 = (unsigned)(uintptr_t)LDS_PTR(void, lds_dst);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0) : "memory");
}

// Global -> LDS copy of one 64-key tile with the direct-to-LDS load: every
// wave instruction j writes LDS bytes [1024 j, 1024 j + 1024), lane i the 16
// bytes at 1024 j + 16 i, so each layout is produced by choosing which global
// 16-B chunk lane i fetches.  Wave w issues instructions j = i NW + w.
template <int D, int NW>
struct TileLoad {
  static constexpr int NC = D / 8;     // 16-B chunks per row = 1 KiB blocks per tile
  static constexpr int LPW = NC / NW;  // load instructions per wave per tile
  static_assert(LPW * NW == NC, "tile load must divide evenly");
  unsigned off[LPW];  // byte offset, from the tile's first row, of this lane's chunk

  __device__ __forceinline__ TileLoad(bool is_k, int wave_u, int lane) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = i * NW + wave_u;
      int r, c;
      if (is_k) {
        r = 32 * (j & 1) + (lane >> 1);
        c = 2 * (j >> 1) + ((lane & 1) ^ k_half_swap(r));
      } else {
        const int slot = j * 64 + lane;
        r = slot / NC;
        c = (slot % NC) ^ v_swz<D>(r);
      }
      off[i] = (unsigned)(r * D + 8 * c) * 2u;
    }
  }
  __device__ __forceinline__ void operator()(const uint16_t* tile, unsigned char* lds_buf, int wave_u) const {
#pragma unroll
    for (int i = 0; i < LPW; ++i) global_to_lds_16(tile, off[i], lds_buf + (i * NW + wave_u) * 1024);
  }
};

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0): every global load this wave issued, including the
  // direct-to-LDS ones, has landed
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace
}  // namespace cpattn
