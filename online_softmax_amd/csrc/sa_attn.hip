// libsa_attn: C ABI entry points, kernel selection and launches.
//
// Everything here is host code around the kernels of prefill.hpp and
// decode.hpp (the backward's entry points are in sa_attn_bwd.hip): validate (host_logic.cpp, no HIP call), pick the template
// instance for {dtype, D, causal, mask, ALiBi}, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/sa_attn.h"
#include "decode.hpp"
#include "host_logic.hpp"
#include "launch.hpp"
#include "prefill.hpp"

namespace sa {
namespace {

// nw = 8: 256-row blocks of eight waves.  nw = 4: 128-row blocks, run by
// four waves, or under the causal rule by eight waves in two groups.  The
// two-group kernel replaced four-wave grids with a heavy and a light causal
// block paired on each CU; same-process A/B: [1,4096,16,128] causal
// 89.7-90.2 -> 86.9-88.2 us, [2,1024,8,64] causal with padding 18.7-19.1 ->
// 17.0-17.3 us (with ALiBi 19.7 -> 18.5 us), [1,8192,8,128] causal ALiBi with
// padding 169-174 -> 154-160 us.
template <class T, int D, bool C, bool M, bool A>
void launch_fwd(const FwdArgs& args, int nw, int pgrid, hipStream_t st) {
  if (nw == 8) {
    if (pgrid > 0)
      hipLaunchKernelGGL((fwd_kernel<T, D, C, M, A, 8, false, false, 1, true>), dim3(pgrid), dim3(512), 0, st, args);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, C, M, A, 8>), dim3(args.nitems), dim3(512), 0, st, args);
  } else if constexpr (C) {
    if (pgrid > 0)
      hipLaunchKernelGGL((fwd_kernel<T, D, C, M, A, 8, false, false, 2, true>), dim3(pgrid), dim3(512), 0, st, args);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, C, M, A, 8, false, false, 2>), dim3(args.nitems), dim3(512), 0, st, args);
  } else {
    hipLaunchKernelGGL((fwd_kernel<T, D, C, M, A, 4>), dim3(args.nitems), dim3(256), 0, st, args);
  }
}

template <class T, int D>
void dispatch_fwd(const FwdArgs& args, bool causal, bool mask, bool alibi, int nw, int grid, hipStream_t st) {
  const int key = (causal ? 4 : 0) | (mask ? 2 : 0) | (alibi ? 1 : 0);
  switch (key) {
    case 0: launch_fwd<T, D, false, false, false>(args, nw, grid, st); break;
    case 1: launch_fwd<T, D, false, false, true>(args, nw, grid, st); break;
    case 2: launch_fwd<T, D, false, true, false>(args, nw, grid, st); break;
    case 3: launch_fwd<T, D, false, true, true>(args, nw, grid, st); break;
    case 4: launch_fwd<T, D, true, false, false>(args, nw, grid, st); break;
    case 5: launch_fwd<T, D, true, false, true>(args, nw, grid, st); break;
    case 6: launch_fwd<T, D, true, true, false>(args, nw, grid, st); break;
    default: launch_fwd<T, D, true, true, true>(args, nw, grid, st); break;
  }
}

template <class T, int D>
void dispatch_decode(const DecArgs& args, const MergeArgs& margs, int nwg, bool mask, bool alibi,
                     hipStream_t st) {
  const int key = (mask ? 2 : 0) | (alibi ? 1 : 0);
  switch (key) {
    case 0: hipLaunchKernelGGL((decode_kernel<T, D, false, false>), dim3(nwg), dim3(256), 0, st, args); break;
    case 1: hipLaunchKernelGGL((decode_kernel<T, D, false, true>), dim3(nwg), dim3(256), 0, st, args); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, D, true, false>), dim3(nwg), dim3(256), 0, st, args); break;
    default: hipLaunchKernelGGL((decode_kernel<T, D, true, true>), dim3(nwg), dim3(256), 0, st, args); break;
  }
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(args.B * args.H_q * (D / 16)), dim3(256), 0, st, margs);
}

template <class T, int D>
void dispatch_decode_fused(const DecArgs& args, int nwg, bool mask, bool alibi, hipStream_t st) {
  const int key = (mask ? 2 : 0) | (alibi ? 1 : 0);
  switch (key) {
    case 0: hipLaunchKernelGGL((decode_kernel<T, D, false, false, true>), dim3(nwg), dim3(256), 0, st, args); break;
    case 1: hipLaunchKernelGGL((decode_kernel<T, D, false, true, true>), dim3(nwg), dim3(256), 0, st, args); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, D, true, false, true>), dim3(nwg), dim3(256), 0, st, args); break;
    default: hipLaunchKernelGGL((decode_kernel<T, D, true, true, true>), dim3(nwg), dim3(256), 0, st, args); break;
  }
}

}  // namespace

// Split and merge launches of a validated decode over `splits` splits, with
// its partial results in `workspace` (decode_layout(B, H_q, splits, D)).
int launch_decode(const DecodeShape& s, int splits, void* workspace, sa_stream_t stream) {
  const int G = s.H_q / s.H_kv;
  const int n_hg = (G + kDecodeHeadGroup - 1) / kDecodeHeadGroup;
  const int chunk = decode_chunk(s.S_k, splits);
  const int64_t nwg = (int64_t)s.B * s.H_kv * n_hg * splits;
  if (nwg > INT32_MAX || (int64_t)s.B * s.H_q * (s.D / 16) > INT32_MAX)
    return fail(SA_ERR_INVALID_ARG, "too many decode workgroups");
  if (!decode_offsets_fit(chunk, s.H_kv, s.D))
    return fail(SA_ERR_INVALID_ARG, "one decode split would span 4 GiB or more of k_cache");

  const DecodeLayout lay = decode_layout(s.B, s.H_q, splits, s.D);
  DecArgs args;
  args.q = (const uint16_t*)s.q;
  args.k = (const uint16_t*)s.k;
  args.v = (const uint16_t*)s.v;
  args.mask = s.mask;
  args.slopes = s.slopes;
  args.out = (uint16_t*)s.out;
  args.lse = const_cast<float*>(s.lse);
  args.ws_o = (float*)((char*)workspace + lay.o_offset);
  args.ws_lse = (float*)((char*)workspace + lay.lse_offset);
  args.B = s.B; args.S_k = s.S_k; args.H_q = s.H_q; args.H_kv = s.H_kv; args.G = G;
  args.n_hg = n_hg; args.splits = splits; args.chunk = chunk;
  args.scale2 = s.scale * kLog2e;
  args.alibi2 = s.scale != 0.f ? 1.0f / std::fabs(s.scale) : 0.f;
  args.arrive = nullptr;

  MergeArgs margs;
  margs.ws_o = args.ws_o;
  margs.ws_lse = args.ws_lse;
  margs.out = (uint16_t*)s.out;
  margs.lse = const_cast<float*>(s.lse);
  margs.splits = splits;

  const bool m = s.mask != nullptr, al = s.slopes != nullptr;
  hipStream_t hs = (hipStream_t)stream;
  if (s.dtype == SA_F16) {
    if (s.D == 64) dispatch_decode<F16, 64>(args, margs, (int)nwg, m, al, hs);
    else dispatch_decode<F16, 128>(args, margs, (int)nwg, m, al, hs);
  } else {
    if (s.D == 64) dispatch_decode<BF16, 64>(args, margs, (int)nwg, m, al, hs);
    else dispatch_decode<BF16, 128>(args, margs, (int)nwg, m, al, hs);
  }
  return launched("decode");
}

}  // namespace sa

extern "C" {

int sa_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int S_q,
                int S_k, int H_q, int H_kv, int D, float scale, int causal,
                const uint8_t* key_padding_mask, const float* alibi_slopes, int dtype,
                sa_stream_t stream) {
  using namespace sa;
  clear_error();
  FwdShape shp{q, k, v, out, lse, B, S_q, S_k, H_q, H_kv, D, scale, causal,
               key_padding_mask, alibi_slopes, dtype};
  bool noop = false;
  int st = check_fwd(shp, &noop);
  if (st != SA_OK || noop) return st;

  int cus = 0;
  st = num_cus(&cus);
  if (st != SA_OK) return st;
  const int nw = fwd_waves(B, S_q, H_q, causal != 0, cus);

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
  args.nmb = (S_q + 32 * nw - 1) / (32 * nw);
  args.nitems = B * H_q * args.nmb;
  args.block_mask = nullptr;
  args.nkb = 0;
  const int grid = fwd_persistent_grid(B * H_q, args.nmb, causal != 0, nw, cus);
  const bool c = causal != 0, m = key_padding_mask != nullptr, al = alibi_slopes != nullptr;
  hipStream_t hs = (hipStream_t)stream;
  if (dtype == SA_F16) {
    if (D == 64) dispatch_fwd<F16, 64>(args, c, m, al, nw, grid, hs);
    else dispatch_fwd<F16, 128>(args, c, m, al, nw, grid, hs);
  } else {
    if (D == 64) dispatch_fwd<BF16, 64>(args, c, m, al, nw, grid, hs);
    else dispatch_fwd<BF16, 128>(args, c, m, al, nw, grid, hs);
  }
  return launched("attention forward");
}

size_t sa_attn_decode_workspace_size(int B, int H_q, int S_k, int D) {
  return sa::decode_workspace_size(B, H_q, S_k, D);
}

int sa_attn_decode_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu) {
  return sa::decode_num_splits(B, S_k, H_q, H_kv, num_cu);
}

int sa_attn_decode_fused_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu) {
  return sa::decode_fused_num_splits(B, S_k, H_q, H_kv, num_cu);
}

int sa_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                   int B, int S_k, int H_q, int H_kv, int D, float scale,
                   const uint8_t* key_padding_mask, const float* alibi_slopes, int dtype,
                   void* workspace, size_t workspace_bytes, sa_stream_t stream) {
  using namespace sa;
  clear_error();
  DecodeShape shp{q, k_cache, v_cache, out, lse, B, S_k, H_q, H_kv, D, scale,
                  key_padding_mask, alibi_slopes, dtype, workspace, workspace_bytes};
  bool noop = false;
  int st = check_decode(shp, &noop);
  if (st != SA_OK || noop) return st;
  int cus = 0;
  st = num_cus(&cus);
  if (st != SA_OK) return st;
  return launch_decode(shp, decode_num_splits(B, S_k, H_q, H_kv, cus), workspace, stream);
}

size_t sa_attn_decode_fused_workspace_size(int B, int H_q, int S_k, int D) {
  return sa::decode_fused_workspace_size(B, H_q, S_k, D);
}

int sa_attn_decode_fused(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                         int B, int S_k, int H_q, int H_kv, int D, float scale,
                         const uint8_t* key_padding_mask, const float* alibi_slopes, int dtype,
                         void* workspace, size_t workspace_bytes, sa_stream_t stream) {
  using namespace sa;
  clear_error();
  DecodeShape shp{q, k_cache, v_cache, out, lse, B, S_k, H_q, H_kv, D, scale,
                  key_padding_mask, alibi_slopes, dtype, workspace, workspace_bytes};
  bool noop = false;
  int st = check_decode_fused(shp, &noop);
  if (st != SA_OK || noop) return st;
  int cus = 0;
  st = num_cus(&cus);
  if (st != SA_OK) return st;
  const int G = H_q / H_kv;
  const int n_hg = (G + kDecodeHeadGroup - 1) / kDecodeHeadGroup;
  const int splits = decode_fused_num_splits(B, S_k, H_q, H_kv, cus);
  const int chunk = decode_chunk(S_k, splits);
  const int64_t groups = (int64_t)B * H_kv * n_hg;
  if (groups > kDecodeMaxGroups)
    return fail(SA_ERR_UNSUPPORTED, "%lld head groups exceed the %d arrival counters of the workspace "
                "(use sa_attn_decode)", (long long)groups, kDecodeMaxGroups);
  const int64_t nwg = groups * splits;
  if (nwg > INT32_MAX) return fail(SA_ERR_INVALID_ARG, "too many decode workgroups");
  if (!decode_offsets_fit(chunk, H_kv, D))
    return fail(SA_ERR_INVALID_ARG, "one decode split would span 4 GiB or more of k_cache");
  const DecodeLayout lay = decode_layout(B, H_q, splits, D);
  if (lay.lse_offset >= ((int64_t)1 << 32))
    return fail(SA_ERR_UNSUPPORTED, "partial outputs of 4 GiB or more (use sa_attn_decode)");

  char* ws = (char*)workspace + kDecodeArriveBytes;
  DecArgs args;
  args.q = (const uint16_t*)q;
  args.k = (const uint16_t*)k_cache;
  args.v = (const uint16_t*)v_cache;
  args.mask = key_padding_mask;
  args.slopes = alibi_slopes;
  args.out = (uint16_t*)out;
  args.lse = lse;
  args.ws_o = (float*)(ws + lay.o_offset);
  args.ws_lse = (float*)(ws + lay.lse_offset);
  args.B = B; args.S_k = S_k; args.H_q = H_q; args.H_kv = H_kv; args.G = G;
  args.n_hg = n_hg; args.splits = splits; args.chunk = chunk;
  args.scale2 = scale * kLog2e;
  args.alibi2 = scale != 0.f ? 1.0f / std::fabs(scale) : 0.f;
  args.arrive = (unsigned*)workspace;
  const bool m = key_padding_mask != nullptr, al = alibi_slopes != nullptr;
  hipStream_t hs = (hipStream_t)stream;
  if (dtype == SA_F16) {
    if (D == 64) dispatch_decode_fused<F16, 64>(args, (int)nwg, m, al, hs);
    else dispatch_decode_fused<F16, 128>(args, (int)nwg, m, al, hs);
  } else {
    if (D == 64) dispatch_decode_fused<BF16, 64>(args, (int)nwg, m, al, hs);
    else dispatch_decode_fused<BF16, 128>(args, (int)nwg, m, al, hs);
  }
  return launched("single-kernel decode");
}

const char* sa_status_string(int status) { return sa::status_string(status); }

const char* sa_last_error(void) { return sa::last_error(); }

}  // extern "C"
