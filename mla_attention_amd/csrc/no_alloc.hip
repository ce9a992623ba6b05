// no_alloc.hip -- grouped-query decode attention for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): zl_decode_attn_gqa with its workspace (the
// fp32 partials of split sequences) taken from a fixed array in device memory
// instead of a caller buffer.
//
// `scratch` is a file-scope device array; every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code its
// name is only a stand-in, so its device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and only that address
// is ever passed on.  The workspace needs no initialisation (every worker
// writes its partial slots before the merge reads them, and the merge finds
// them by rule), so nothing is cleared between calls.  Calls that overlap in time on one GPU
// share the array and race; calls on one stream are ordered.
#include <hip/hip_runtime.h>

#include <mutex>

#include "zl_attn.h"

static constexpr size_t kScratchBytes = (size_t)16 << 20;  // 16 MiB per GPU
static constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// The current device's copy of `scratch` (looked up on its first use).
zl_status_t device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ZL_ERR_HIP;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ZL_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return ZL_OK;
}

}  // namespace

extern "C" {

zl_status_t zl_decode_attn_gqa_no_alloc(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* cu_seqlens, int batch, int num_q_heads, int num_kv_heads,
                                        int head_dim, int max_seqlen_k, float softmax_scale, int dtype,
                                        void* out, float* lse, zl_stream_t stream) {
  const size_t need =
      zl_decode_attn_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_seqlen_k, dtype);
  // need == 0: the sizes are invalid; the plain call reports which status,
  // before any HIP call and without touching a workspace.
  if (need == 0) return zl_decode_attn_gqa(q, k_cache, v_cache, cu_seqlens, batch, num_q_heads, num_kv_heads,
                                           head_dim, max_seqlen_k, softmax_scale, dtype, out, lse, nullptr, 0,
                                           stream);
  if (need > kScratchBytes) return ZL_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const zl_status_t st = device_scratch(&ws);
  if (st != ZL_OK) return st;
  return zl_decode_attn_gqa(q, k_cache, v_cache, cu_seqlens, batch, num_q_heads, num_kv_heads, head_dim,
                            max_seqlen_k, softmax_scale, dtype, out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"
