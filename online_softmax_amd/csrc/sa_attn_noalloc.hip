// libsa_attn: the allocation-free decode entry point (sa_attn_decode_noalloc)
// for callers that cannot allocate device memory.
//
// It is sa_attn_decode (split and merge kernels, launched by launch_decode in
// sa_attn.hip) with the decode's partial results held in a fixed scratch array
// of this library instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/sa_attn.h"
#include "host_logic.hpp"
#include "launch.hpp"

namespace sa {
namespace {

// The scratch: each GPU holds its own copy from the library's load until the
// process ends, and every call on a GPU shares it, so calls on one GPU that
// may overlap (different streams with no ordering between them) race.
// Nothing in it needs clearing: each call's split kernel writes every partial
// result that its merge kernel reads.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The device address of the current GPU's scratch, looked up once per device
// with that device current (in host code the array's name is only a stand-in,
// not a device address).
int scratch_address(void** out) {
  static std::once_flag flags[kMaxDevices];
  static void* ptrs[kMaxDevices];
  static hipError_t errs[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_HIP, "device index %d out of range", dev);
  std::call_once(flags[dev], [dev] { errs[dev] = hipGetSymbolAddress(&ptrs[dev], HIP_SYMBOL(scratch)); });
  if (errs[dev] != hipSuccess)
    return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(errs[dev]));
  if (!ptrs[dev]) return fail(SA_ERR_HIP, "the scratch has no device address");
  *out = ptrs[dev];
  return SA_OK;
}

}  // namespace
}  // namespace sa

extern "C" {

int sa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                           int B, int S_k, int H_q, int H_kv, int D, float scale,
                           const uint8_t* key_padding_mask, const float* alibi_slopes, int dtype,
                           sa_stream_t stream) {
  using namespace sa;
  clear_error();
  DecodeShape shp{q, k_cache, v_cache, out, lse, B, S_k, H_q, H_kv, D, scale,
                  key_padding_mask, alibi_slopes, dtype, nullptr, 0};
  bool noop = false;
  int st = check_decode_need(shp, 0, &noop);  // the arguments (the scratch is checked below)
  if (st != SA_OK || noop) return st;
  int cus = 0;
  st = num_cus(&cus);
  if (st != SA_OK) return st;
  const int splits = decode_num_splits(B, S_k, H_q, H_kv, cus);
  const int64_t need = decode_layout(B, H_q, splits, D).bytes;
  if (need > (int64_t)kNoAllocScratchBytes)
    return fail(SA_ERR_UNSUPPORTED,
                "this decode needs %lld bytes of partial results, more than the %zu bytes of the "
                "library's scratch (use sa_attn_decode with a workspace)",
                (long long)need, kNoAllocScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SA_OK) return st;
  shp.workspace = ws;
  shp.workspace_bytes = kNoAllocScratchBytes;
  st = check_decode_need(shp, (size_t)need, &noop);  // outputs and inputs against the scratch
  if (st != SA_OK || noop) return st;
  return launch_decode(shp, splits, ws, stream);
}

}  // extern "C"
