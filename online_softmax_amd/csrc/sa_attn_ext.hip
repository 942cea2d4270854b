// libsa_attn: the extended forward's C ABI entry point and launches.
//
// Host code around the extended mode of the prefill kernel (prefill.hpp:
// additive float bias and Philox dropout): validate (host_logic.cpp, no HIP
// call), pick the template instance for {dtype, D, causal, mask, ALiBi},
// launch on the caller's stream.  Without a bias and without dropout the
// call is the plain forward's.  Causal dropout without ALiBi runs the
// two-group layout (eight waves over a 128-row block at two waves per SIMD,
// as the plain causal forward), where another wave's matrix work covers the
// generator's; everything else runs workgroups of four waves at one wave per
// SIMD, whose registers leave room for the bias tile loaded a step ahead.
// Same-process timing on the [1, 4096, 16, 128] causal workload (us, four
// waves -> two groups): dropout 0.1 151 -> 126, with a [4096, 4096] bias
// 194 -> 177; a bias alone 153 -> 159 (so it keeps four waves).
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/sa_attn.h"
#include "host_logic.hpp"
#include "launch.hpp"
#include "prefill.hpp"

namespace sa {
namespace {

template <class T, int D, bool C, bool M, bool A>
void launch_ext(const FwdArgs& args, hipStream_t st) {
  if constexpr (C && !A) {
    if (args.drop_thr != 0u) {
      hipLaunchKernelGGL((fwd_kernel<T, D, C, M, A, 8, false, true, 2>), dim3(args.nitems), dim3(512), 0, st, args);
      return;
    }
  }
  hipLaunchKernelGGL((fwd_kernel<T, D, C, M, A, 4, false, true>), dim3(args.nitems), dim3(256), 0, st, args);
}

template <class T, int D>
void dispatch_ext(const FwdArgs& args, bool causal, bool mask, bool alibi, hipStream_t st) {
  const int key = (causal ? 4 : 0) | (mask ? 2 : 0) | (alibi ? 1 : 0);
  switch (key) {
    case 0: launch_ext<T, D, false, false, false>(args, st); break;
    case 1: launch_ext<T, D, false, false, true>(args, st); break;
    case 2: launch_ext<T, D, false, true, false>(args, st); break;
    case 3: launch_ext<T, D, false, true, true>(args, st); break;
    case 4: launch_ext<T, D, true, false, false>(args, st); break;
    case 5: launch_ext<T, D, true, false, true>(args, st); break;
    case 6: launch_ext<T, D, true, true, false>(args, st); break;
    default: launch_ext<T, D, true, true, true>(args, st); break;
  }
}

}  // namespace
}  // namespace sa

extern "C" {

int sa_attn_fwd_ext(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int S_q, int S_k, int H_q, int H_kv, int D, float scale, int causal,
                    const uint8_t* key_padding_mask, const float* alibi_slopes,
                    const float* attn_bias, int64_t bias_stride_b, int64_t bias_stride_h,
                    int64_t bias_stride_q, double dropout_p, uint64_t seed, uint32_t offset,
                    int dtype, sa_stream_t stream) {
  using namespace sa;
  clear_error();
  FwdShape shp{q, k, v, out, lse, B, S_q, S_k, H_q, H_kv, D, scale, causal,
               key_padding_mask, alibi_slopes, dtype};
  ExtShape ext{attn_bias, bias_stride_b, bias_stride_h, bias_stride_q, dropout_p};
  bool noop = false;
  int st = check_ext(shp, ext, &noop);
  if (st != SA_OK || noop) return st;
  // Neither a bias nor dropout: the plain forward computes exactly this.
  if (attn_bias == nullptr && dropout_p == 0.0)
    return sa_attn_fwd(q, k, v, out, lse, B, S_q, S_k, H_q, H_kv, D, scale, causal, key_padding_mask,
                       alibi_slopes, dtype, stream);

  FwdArgs args;
  args.q = (const uint16_t*)q;
  args.k = (const uint16_t*)k;
  args.v = (const uint16_t*)v;
  args.out = (uint16_t*)out;
  args.lse = lse;
  args.mask = key_padding_mask;
  args.slopes = alibi_slopes;
  args.B = B; args.S_q = S_q; args.S_k = S_k; args.H_q = H_q; args.H_kv = H_kv;
  args.G = H_q / H_kv;
  args.scale2 = scale * kLog2e;
  args.alibi2 = 1.0f / std::fabs(scale);
  args.nmb = (S_q + 127) / 128;
  args.nitems = B * H_q * args.nmb;
  args.block_mask = nullptr;
  args.nkb = 0;
  args.bias = attn_bias;
  args.bias_sb = bias_stride_b;
  args.bias_sh = bias_stride_h;
  args.bias_sq = bias_stride_q;
  args.drop_thr = drop_threshold(dropout_p);
  args.drop_scale = (float)(1.0 / (1.0 - dropout_p));
  args.seed_lo = (uint32_t)seed;
  args.seed_hi = (uint32_t)(seed >> 32);
  args.drop_offset = offset;
  const bool c = causal != 0, m = key_padding_mask != nullptr, al = alibi_slopes != nullptr;
  hipStream_t hs = (hipStream_t)stream;
  if (dtype == SA_F16) {
    if (D == 64) dispatch_ext<F16, 64>(args, c, m, al, hs);
    else dispatch_ext<F16, 128>(args, c, m, al, hs);
  } else {
    if (D == 64) dispatch_ext<BF16, 64>(args, c, m, al, hs);
    else dispatch_ext<BF16, 128>(args, c, m, al, hs);
  }
  return launched("extended attention forward");
}

}  // extern "C"
