// libsa_attn: the backward's C ABI entry points, kernel selection and launches.
//
// Host code around the kernels of backward.hpp: validate (host_logic.cpp, no
// HIP call), pick the template instance for {dtype, D, causal, mask, ALiBi},
// launch the dq kernel (which also forms each row's Di and base-2 lse for the
// next kernel) and the dk/dv kernel on the caller's stream.  This file is compiled on its own, with MFMA results kept
// in ordinary vector registers: the dk/dv kernel holds both gradient blocks
// and its key/value rows live across the whole sweep, and letting the
// compiler place MFMA results in accumulation registers made it move those
// blocks between the two register files on every query tile.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/sa_attn.h"
#include "backward.hpp"
#include "host_logic.hpp"
#include "launch.hpp"

namespace sa {
namespace {

template <class T, int D, bool C, bool M, bool A>
void launch_bwd_main(const BwdArgs& args, hipStream_t st) {
  const int ndq = args.B * args.H_q * args.nqb, ndk = args.B * args.H_kv * args.nkb;
  if (ndq > 0) hipLaunchKernelGGL((bwd_dq_kernel<T, D, C, M, A>), dim3(ndq), dim3(256), 0, st, args);
  if (ndk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, C, M, A>), dim3(ndk), dim3(256), 0, st, args);
}

template <class T, int D>
void dispatch_bwd(const BwdArgs& args, bool causal, bool mask, bool alibi, hipStream_t st) {
  const int key = (causal ? 4 : 0) | (mask ? 2 : 0) | (alibi ? 1 : 0);
  switch (key) {
    case 0: launch_bwd_main<T, D, false, false, false>(args, st); break;
    case 1: launch_bwd_main<T, D, false, false, true>(args, st); break;
    case 2: launch_bwd_main<T, D, false, true, false>(args, st); break;
    case 3: launch_bwd_main<T, D, false, true, true>(args, st); break;
    case 4: launch_bwd_main<T, D, true, false, false>(args, st); break;
    case 5: launch_bwd_main<T, D, true, false, true>(args, st); break;
    case 6: launch_bwd_main<T, D, true, true, false>(args, st); break;
    default: launch_bwd_main<T, D, true, true, true>(args, st); break;
  }
}

}  // namespace
}  // namespace sa

extern "C" {

size_t sa_attn_bwd_workspace_size(int B, int H_q, int S_q) { return sa::bwd_workspace_size(B, H_q, S_q); }

int sa_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int S_q, int S_k, int H_q,
                int H_kv, int D, float scale, int causal, const uint8_t* key_padding_mask,
                const float* alibi_slopes, int dtype, void* workspace, size_t workspace_bytes,
                sa_stream_t stream) {
  using namespace sa;
  clear_error();
  BwdShape shp{q, k, v, out, dout, lse, dq, dk, dv, B, S_q, S_k, H_q, H_kv, D, scale, causal,
               key_padding_mask, alibi_slopes, dtype, workspace, workspace_bytes};
  bool noop = false;
  int st = check_bwd(shp, &noop);
  if (st != SA_OK || noop) return st;

  BwdArgs args;
  args.q = (const uint16_t*)q;
  args.k = (const uint16_t*)k;
  args.v = (const uint16_t*)v;
  args.out = (const uint16_t*)out;
  args.dout = (const uint16_t*)dout;
  args.lse = lse;
  args.dq = (uint16_t*)dq;
  args.dk = (uint16_t*)dk;
  args.dv = (uint16_t*)dv;
  args.mask = key_padding_mask;
  args.slopes = alibi_slopes;
  args.ld = (float2*)workspace;
  args.B = B; args.S_q = S_q; args.S_k = S_k; args.H_q = H_q; args.H_kv = H_kv;
  args.G = H_q / H_kv;
  args.scale = scale;
  args.scale2 = std::fabs(scale) * kLog2e;
  args.alibi2 = scale != 0.f ? 1.0f / std::fabs(scale) : 0.f;
  args.nqb = (S_q + 127) / 128;
  args.nkb = (S_k + 127) / 128;
  int cus = 0;
  st = num_cus(&cus);
  if (st != SA_OK) return st;
  args.pair_ncu = fwd_pair_ncu(B * H_q * args.nqb, args.nqb, causal != 0, 4, cus);
  args.pair_ncu_kv = fwd_pair_ncu(B * H_kv * args.nkb, args.nkb, causal != 0, 4, cus);
  const bool c = causal != 0, m = key_padding_mask != nullptr, al = alibi_slopes != nullptr;
  hipStream_t hs = (hipStream_t)stream;
  if (dtype == SA_F16) {
    if (D == 64) dispatch_bwd<F16, 64>(args, c, m, al, hs);
    else dispatch_bwd<F16, 128>(args, c, m, al, hs);
  } else {
    if (D == 64) dispatch_bwd<BF16, 64>(args, c, m, al, hs);
    else dispatch_bwd<BF16, 128>(args, c, m, al, hs);
  }
  return launched("attention backward");
}

}  // extern "C"
