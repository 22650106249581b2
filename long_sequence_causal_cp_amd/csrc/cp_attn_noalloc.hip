// cp_ring_attn_fwd_noalloc: the forward ring of cp_ring_attn_fwd for callers
// that cannot allocate device memory (code under graph capture, tight serving
// loops).  Its workspace (two staging slots and the fp32 running output) is
// a static device array of this file, `scratch`, of kNoAllocScratchBytes; each
// GPU the library runs on holds its own copy until the process ends.
//
// Host code never uses the array's name as an address: on a device's first
// call the library looks up that device's copy with hipGetSymbolAddress (with
// the device current) and keeps the pointer per device; the kernels receive
// that pointer like any workspace.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "cp_attn_ring.h"

constexpr size_t kNoAllocScratchBytes = 64ull << 20;  // 64 MiB per device

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> its copy of `scratch`

// This device's copy of the scratch array, looked up once per device.
cp_status_t scratch_for_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return cpattn::fail_status(CP_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return CP_OK;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr)
    return cpattn::fail_status(CP_ERR_HIP, "hipGetSymbolAddress of the no-allocation scratch array failed");
  g_scratch_ptr[dev] = p;
  *ptr = p;
  return CP_OK;
}

}  // namespace

extern "C" {

size_t cp_ring_attn_fwd_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

cp_status_t cp_ring_attn_fwd_noalloc(const void* q, const cp_chunks_t* q_chunks, const void* const* k_steps,
                                     const void* const* v_steps, const cp_chunks_t* kv_chunks_steps, int n_steps,
                                     void* out, float* lse, int B, int H, int D, float softmax_scale,
                                     hipStream_t stream, hipStream_t copy_stream) {
  if (!q_chunks || !kv_chunks_steps || n_steps < 1 || B < 1 || H < 1 || D < 1)
    return cpattn::fail_status(CP_ERR_INVALID, "q_chunks, kv_chunks_steps, n_steps, B, H or D invalid");
  if (q_chunks->n_chunks < 1 || q_chunks->chunk_len < 1 || kv_chunks_steps[0].n_chunks < 1 ||
      kv_chunks_steps[0].chunk_len < 1)
    return cpattn::fail_status(CP_ERR_INVALID, "empty chunk table");
  const long long sq = (long long)q_chunks->n_chunks * q_chunks->chunk_len;
  const long long skv = (long long)kv_chunks_steps[0].n_chunks * kv_chunks_steps[0].chunk_len;
  if (sq > (1LL << 30) || skv > (1LL << 30))
    return cpattn::fail_status(CP_ERR_INVALID, "local sequence too long");
  // the launch grouping of cp_ring_attn_fwd if its workspace fits, else fewer
  // ring steps per launch (smaller staging slots)
  int per = cpattn::kMaxStepsPerLaunch;
  while (per > 1 && cpattn::ring_fwd_workspace_bytes(B, H, (int)skv, D, (int)sq, per) > kNoAllocScratchBytes) --per;
  const size_t need = cpattn::ring_fwd_workspace_bytes(B, H, (int)skv, D, (int)sq, per);
  if (need == 0 || need > kNoAllocScratchBytes)
    return cpattn::fail_status(CP_ERR_WORKSPACE,
                               "share too large for the no-allocation scratch (one ring step per launch needs more "
                               "than its 64 MiB); use cp_ring_attn_fwd with a workspace");
  void* ws = nullptr;
  cp_status_t st = scratch_for_current_device(&ws);
  if (st != CP_OK) return st;
  return cpattn::ring_fwd(q, q_chunks, k_steps, v_steps, kv_chunks_steps, n_steps, out, lse, B, H, D, softmax_scale,
                          ws, kNoAllocScratchBytes, per, stream, copy_stream);
}

}  // extern "C"
