// Host-side argument checking, decode split sizing and error reporting.
#include "host_logic.hpp"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "../../include/sa_attn.h"

namespace sa {

namespace {
thread_local char g_err[512] = "";

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Product of non-negative ints in int64 with an overflow guard.
bool mul_ok(int64_t* acc, int64_t v) {
  if (v < 0) return false;
  if (v != 0 && *acc > INT64_C(0x3fffffffffffffff) / v) return false;
  *acc *= v;
  return true;
}

int check_common(int dtype, int D, int B, int S_k, int H_q, int H_kv, float scale) {
  if (dtype != SA_F16 && dtype != SA_BF16)
    return fail(SA_ERR_UNSUPPORTED, "dtype %d is not SA_F16 (0) or SA_BF16 (1)", dtype);
  if (D != 64 && D != 128)
    return fail(SA_ERR_UNSUPPORTED, "head dimension D=%d is not supported (64 or 128)", D);
  if (B < 0 || S_k < 0)
    return fail(SA_ERR_INVALID_ARG, "negative size (B=%d, S_k=%d)", B, S_k);
  if (H_q < 1 || H_kv < 1)
    return fail(SA_ERR_INVALID_ARG, "head counts must be positive (H_q=%d, H_kv=%d)", H_q, H_kv);
  if (H_q % H_kv != 0)
    return fail(SA_ERR_INVALID_ARG, "H_q=%d is not a multiple of H_kv=%d", H_q, H_kv);
  if (!std::isfinite(scale))
    return fail(SA_ERR_INVALID_ARG, "scale is not finite");
  return SA_OK;
}
}  // namespace

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = '\0'; }
const char* last_error() { return g_err; }

const char* status_string(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    default: return "unknown sa_status";
  }
}

int check_fwd(const FwdShape& s, bool* noop) {
  *noop = false;
  int st = check_common(s.dtype, s.D, s.B, s.S_k, s.H_q, s.H_kv, s.scale);
  if (st != SA_OK) return st;
  if (s.S_q < 0) return fail(SA_ERR_INVALID_ARG, "negative S_q=%d", s.S_q);
  if (s.causal != 0 && s.causal != 1) return fail(SA_ERR_INVALID_ARG, "causal must be 0 or 1");
  // The kernels add a bias in units of 1 / |scale|, which must be finite.
  if (s.slopes && !std::isfinite(1.0f / std::fabs(s.scale)))
    return fail(SA_ERR_INVALID_ARG, "scale must be nonzero (1/|scale| finite) when ALiBi slopes are given");
  if (s.B == 0 || s.S_q == 0) { *noop = true; return SA_OK; }
  int64_t nq = 1, nk = 1;
  if (!mul_ok(&nq, s.B) || !mul_ok(&nq, s.S_q) || !mul_ok(&nq, s.H_q) || !mul_ok(&nq, s.D) ||
      !mul_ok(&nk, s.B) || !mul_ok(&nk, s.S_k) || !mul_ok(&nk, s.H_kv) || !mul_ok(&nk, s.D))
    return fail(SA_ERR_INVALID_ARG, "tensor sizes overflow");
  // Workgroups: B * H_q * ceil(S_q / 128) must fit a 1-D grid.
  int64_t items = (int64_t)s.B * s.H_q * ((s.S_q + 127) / 128);
  // One key/value tile (64 rows) must be addressable by a 32-bit buffer range.
  if ((int64_t)64 * s.H_kv * s.D * 2 >= (INT64_C(1) << 32))
    return fail(SA_ERR_UNSUPPORTED, "H_kv * D too large for the tile copies");
  if (items > INT32_MAX) return fail(SA_ERR_INVALID_ARG, "too many query blocks (%lld)", (long long)items);
  if (!s.q || !s.out) return fail(SA_ERR_INVALID_ARG, "q and out must not be NULL");
  if (s.S_k > 0 && (!s.k || !s.v)) return fail(SA_ERR_INVALID_ARG, "k and v must not be NULL when S_k > 0");
  if (!aligned(s.q, 16) || !aligned(s.out, 16) || (s.k && !aligned(s.k, 16)) || (s.v && !aligned(s.v, 16)))
    return fail(SA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (s.lse && !aligned(s.lse, 4)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (s.slopes && !aligned(s.slopes, 4)) return fail(SA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
  const size_t qb = (size_t)nq * 2, kb = (size_t)nk * 2;
  const size_t lb = (size_t)s.B * s.H_q * s.S_q * 4;
  const size_t mb = (size_t)s.B * s.S_k, sb = (size_t)s.H_q * 4;
  const void* ins[5] = {s.q, s.k, s.v, s.mask, s.slopes};
  const size_t insz[5] = {qb, kb, kb, mb, sb};
  for (int i = 0; i < 5; ++i) {
    if (overlap(s.out, qb, ins[i], insz[i]) || overlap(s.lse, s.lse ? lb : 0, ins[i], insz[i]))
      return fail(SA_ERR_INVALID_ARG, "out/lse overlap an input");
  }
  if (overlap(s.out, qb, s.lse, s.lse ? lb : 0)) return fail(SA_ERR_INVALID_ARG, "out and lse overlap");
  return SA_OK;
}

int check_block_sparse(const FwdShape& s, const uint8_t* block_mask, bool* noop) {
  int st = check_fwd(s, noop);
  if (st != SA_OK || *noop) return st;
  if (s.S_k > 64 * kSparseMaxTiles)
    return fail(SA_ERR_UNSUPPORTED, "block-sparse forward supports S_k up to %d (got %d)",
                64 * kSparseMaxTiles, s.S_k);
  if (s.S_k == 0) return SA_OK;  // no keys: the block mask is not read
  if (!block_mask) return fail(SA_ERR_INVALID_ARG, "block_mask must not be NULL when S_k > 0");
  int64_t nb = 1;
  if (!mul_ok(&nb, s.B) || !mul_ok(&nb, s.H_q) || !mul_ok(&nb, (s.S_q + kSparseBlock - 1) / kSparseBlock) ||
      !mul_ok(&nb, (s.S_k + kSparseBlock - 1) / kSparseBlock))
    return fail(SA_ERR_INVALID_ARG, "block mask size overflows");
  const size_t qb = (size_t)s.B * s.S_q * s.H_q * s.D * 2, lb = (size_t)s.B * s.H_q * s.S_q * 4;
  if (overlap(s.out, qb, block_mask, (size_t)nb) || overlap(s.lse, s.lse ? lb : 0, block_mask, (size_t)nb))
    return fail(SA_ERR_INVALID_ARG, "out/lse overlap the block mask");
  return SA_OK;
}

uint32_t drop_threshold(double p) {
  const double t = std::floor(p * 65536.0);
  return t >= 65535.0 ? 0xFFFFu : t <= 0.0 ? 0u : (uint32_t)t;
}

int check_ext(const FwdShape& s, const ExtShape& e, bool* noop) {
  if (!(e.dropout_p >= 0.0 && e.dropout_p < 1.0))
    return fail(SA_ERR_INVALID_ARG, "dropout_p must be in [0, 1) (got %g)", e.dropout_p);
  if (e.bias && !std::isfinite(1.0f / std::fabs(s.scale)))
    return fail(SA_ERR_INVALID_ARG, "scale must be nonzero (1/|scale| finite) when attn_bias is given");
  int st = check_fwd(s, noop);
  if (st != SA_OK || *noop || !e.bias || s.S_k == 0) return st;
  if (e.sb < 0 || e.sh < 0 || e.sq < 0 || e.sb % 4 || e.sh % 4 || e.sq % 4)
    return fail(SA_ERR_INVALID_ARG, "bias strides must be non-negative multiples of 4 elements");
  if (!aligned(e.bias, 16)) return fail(SA_ERR_INVALID_ARG, "attn_bias must be 16-byte aligned");
  // Elements up to the last one read: (B-1) sb + (H_q-1) sh + (S_q-1) sq + S_k.
  int64_t ext = s.S_k, t;
  const int64_t terms[3][2] = {{s.B - 1, e.sb}, {s.H_q - 1, e.sh}, {s.S_q - 1, e.sq}};
  for (const auto& tm : terms) {
    t = tm[0];
    if (!mul_ok(&t, tm[1]) || ext > INT64_MAX - t) return fail(SA_ERR_INVALID_ARG, "bias extent overflows");
    ext += t;
  }
  if (ext > INT64_MAX / 4) return fail(SA_ERR_INVALID_ARG, "bias extent overflows");
  const size_t bb = (size_t)ext * 4;
  const size_t qb = (size_t)s.B * s.S_q * s.H_q * s.D * 2, lb = (size_t)s.B * s.H_q * s.S_q * 4;
  if (overlap(s.out, qb, e.bias, bb) || overlap(s.lse, s.lse ? lb : 0, e.bias, bb))
    return fail(SA_ERR_INVALID_ARG, "out/lse overlap attn_bias");
  return SA_OK;
}

int decode_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu) {
  if (B <= 0 || S_k <= 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv) return 1;
  const int G = H_q / H_kv;
  const int64_t groups = (int64_t)B * H_kv * ((G + kDecodeHeadGroup - 1) / kDecodeHeadGroup);
  const int max_splits = (int)std::min<int64_t>(kDecodeMaxSplits, (S_k + kDecodeStepKeys - 1) / kDecodeStepKeys);
  // Aim for one four-wave workgroup per compute unit.  On 32K-key caches
  // (14:2 heads, D = 64) at batch 1, 2 and 4 this was 1-12 % faster than two
  // per CU with half the keys each, whose partial results also double the
  // merge's reads; a target of 1.5 per CU gave splits of 1.5 rounds and was
  // slower than both.
  const int64_t target = (int64_t)(num_cu > 0 ? num_cu : 1);
  int64_t splits = (target + groups - 1) / groups;
  if (splits < 1) splits = 1;
  if (splits > max_splits) splits = max_splits;
  // Round to whole steps per split, then drop splits that would be empty.
  const int chunk = decode_chunk(S_k, (int)splits);
  return (S_k + chunk - 1) / chunk;
}

int decode_fused_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu) {
  const int splits = std::min(decode_num_splits(B, S_k, H_q, H_kv, num_cu), kDecodeFusedMaxSplits);
  const int chunk = decode_chunk(S_k, splits);
  return (S_k + chunk - 1) / chunk;
}

int fwd_waves(int B, int S_q, int H_q, bool causal, int num_cu) {
  const int64_t wg8 = (int64_t)B * H_q * ((S_q + 255) / 256);
  const int64_t need = (int64_t)(num_cu > 0 ? num_cu : 1) * (causal ? 4 : 1);
  return wg8 >= need ? 8 : 4;
}

int fwd_pair_ncu(int nitems, int nmb, bool causal, int nw, int num_cu) {
  if (!causal || nw != 4 || num_cu <= 0 || nmb <= 0 || nmb % 2) return 0;
  return (int64_t)nitems == 2 * (int64_t)num_cu ? num_cu : 0;
}

int fwd_persistent_grid(int bh, int nmb, bool causal, int nw, int num_cu) {
  if (num_cu <= 0 || bh <= 0 || nmb <= 0 || !(nw == 8 || causal)) return 0;
  const int64_t units = (int64_t)bh * (causal ? (nmb + 1) / 2 : nmb);
  return units >= 2 * (int64_t)num_cu ? num_cu : 0;
}

int decode_chunk(int S_k, int splits) {
  if (splits < 1) splits = 1;
  int per = (S_k + splits - 1) / splits;
  int steps = (per + kDecodeStepKeys - 1) / kDecodeStepKeys;
  if (steps < 1) steps = 1;
  return steps * kDecodeStepKeys;
}

DecodeLayout decode_layout(int B, int H_q, int splits, int D) {
  // Partial outputs [B, H_q, splits, D], then the partial lse
  // [B, H_q, splits] from the next 256-byte boundary.
  DecodeLayout l;
  const int64_t n = (int64_t)B * H_q * splits;
  l.o_offset = 0;
  l.lse_offset = (n * D * 4 + 255) / 256 * 256;
  l.bytes = l.lse_offset + n * 4;
  return l;
}

bool decode_offsets_fit(int chunk, int H_kv, int D) {
  // Byte offsets inside one split (including the rows past its end that a
  // workgroup's last round addresses and reads as zero) are 32-bit.
  return ((int64_t)chunk + kDecodeRoundKeys) * H_kv * D * 2 < ((int64_t)1 << 32);
}

size_t decode_workspace_size(int B, int H_q, int S_k, int D) {
  if (B < 0 || H_q < 0 || S_k < 0 || D < 0) return 0;
  int64_t max_splits = std::min<int64_t>(kDecodeMaxSplits, (S_k + kDecodeStepKeys - 1) / kDecodeStepKeys);
  if (max_splits < 1) max_splits = 1;
  int64_t n = 1;
  if (!mul_ok(&n, B) || !mul_ok(&n, H_q) || !mul_ok(&n, max_splits)) return 0;
  int64_t floats = n;
  if (!mul_ok(&floats, (int64_t)D + 1)) return 0;
  if (floats > ((int64_t)1 << 60) / 4) return 0;
  return (size_t)decode_layout(B, H_q, (int)max_splits, D).bytes;
}

size_t decode_fused_workspace_size(int B, int H_q, int S_k, int D) {
  if (B < 0 || H_q < 0 || S_k < 0 || D < 0) return 0;
  const size_t n = decode_workspace_size(B, H_q, S_k, D);
  if (n == 0 && B > 0 && H_q > 0) return 0;  // overflow
  return n > SIZE_MAX - kDecodeArriveBytes ? 0 : n + kDecodeArriveBytes;
}

int check_decode_fused(const DecodeShape& s, bool* noop) {
  *noop = false;
  DecodeShape t = s;
  const int64_t ab = kDecodeArriveBytes;
  if (s.B > 0 && s.H_q > 0) {
    if (!s.workspace)
      return fail(SA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)",
                  decode_fused_workspace_size(s.B, s.H_q, s.S_k, s.D));
    if (!aligned(s.workspace, 256)) return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (s.workspace_bytes < (size_t)ab)
      return fail(SA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", s.workspace_bytes,
                  decode_fused_workspace_size(s.B, s.H_q, s.S_k, s.D));
    t.workspace = (const char*)s.workspace + ab;
    t.workspace_bytes = s.workspace_bytes - (size_t)ab;
  }
  int st = check_decode(t, noop);
  if (st != SA_OK || *noop) return st;
  const size_t qb = (size_t)s.B * s.H_q * s.D * 2, kb = (size_t)s.B * s.S_k * s.H_kv * s.D * 2;
  const size_t lb = (size_t)s.B * s.H_q * 4;
  const void* others[7] = {s.q, s.k, s.v, s.mask, s.slopes, s.out, s.lse};
  const size_t osz[7] = {qb, kb, kb, (size_t)s.B * s.S_k, (size_t)s.H_q * 4, qb, lb};
  for (int i = 0; i < 7; ++i)
    if (overlap(s.workspace, (size_t)ab, others[i], osz[i]))
      return fail(SA_ERR_INVALID_ARG, "workspace overlaps an input or output");
  return SA_OK;
}

int check_decode(const DecodeShape& s, bool* noop) {
  *noop = false;
  if (s.B > 0 && s.H_q > 0 && s.S_k >= 0 && s.D > 0 && decode_workspace_size(s.B, s.H_q, s.S_k, s.D) == 0)
    return fail(SA_ERR_INVALID_ARG, "tensor sizes overflow");
  return check_decode_need(s, decode_workspace_size(s.B, s.H_q, s.S_k, s.D), noop);
}

int check_decode_need(const DecodeShape& s, size_t need, bool* noop) {
  *noop = false;
  int st = check_common(s.dtype, s.D, s.B, s.S_k, s.H_q, s.H_kv, s.scale);
  if (st != SA_OK) return st;
  if (s.B == 0) { *noop = true; return SA_OK; }
  int64_t nk = 1;
  if (!mul_ok(&nk, s.B) || !mul_ok(&nk, s.S_k) || !mul_ok(&nk, s.H_kv) || !mul_ok(&nk, s.D))
    return fail(SA_ERR_INVALID_ARG, "tensor sizes overflow");
  if (!s.q || !s.out) return fail(SA_ERR_INVALID_ARG, "q and out must not be NULL");
  // The kernels add a bias in units of 1 / |scale|, which must be finite.
  if (s.slopes && !std::isfinite(1.0f / std::fabs(s.scale)))
    return fail(SA_ERR_INVALID_ARG, "scale must be nonzero (1/|scale| finite) when ALiBi slopes are given");
  if (s.S_k > 0 && (!s.k || !s.v)) return fail(SA_ERR_INVALID_ARG, "k_cache and v_cache must not be NULL when S_k > 0");
  if (!aligned(s.q, 16) || !aligned(s.out, 16) || (s.k && !aligned(s.k, 16)) || (s.v && !aligned(s.v, 16)))
    return fail(SA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (s.lse && !aligned(s.lse, 4)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (s.slopes && !aligned(s.slopes, 4)) return fail(SA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
  // need == 0: the argument checks only (no workspace given yet).
  if (need > 0) {
    if (!s.workspace) return fail(SA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(s.workspace, 16)) return fail(SA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (s.workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", s.workspace_bytes, need);
  }
  const size_t qb = (size_t)s.B * s.H_q * s.D * 2, kb = (size_t)nk * 2;
  const size_t lb = (size_t)s.B * s.H_q * 4;
  const void* ins[5] = {s.q, s.k, s.v, s.mask, s.slopes};
  const size_t insz[5] = {qb, kb, kb, (size_t)s.B * s.S_k, (size_t)s.H_q * 4};
  for (int i = 0; i < 5; ++i) {
    if (overlap(s.out, qb, ins[i], insz[i]) || overlap(s.lse, s.lse ? lb : 0, ins[i], insz[i]) ||
        overlap(s.workspace, need, ins[i], insz[i]))
      return fail(SA_ERR_INVALID_ARG, "out, lse or workspace overlap an input");
  }
  if (overlap(s.out, qb, s.lse, s.lse ? lb : 0) || overlap(s.workspace, need, s.out, qb) ||
      overlap(s.workspace, need, s.lse, s.lse ? lb : 0))
    return fail(SA_ERR_INVALID_ARG, "out, lse and workspace overlap each other");
  return SA_OK;
}

size_t bwd_workspace_size(int B, int H_q, int S_q) {
  if (B < 0 || H_q < 0 || S_q < 0) return 0;
  int64_t n = 8;
  if (!mul_ok(&n, B) || !mul_ok(&n, H_q) || !mul_ok(&n, S_q)) return 0;
  return (size_t)n;
}

int check_bwd(const BwdShape& s, bool* noop) {
  *noop = false;
  int st = check_common(s.dtype, s.D, s.B, s.S_k, s.H_q, s.H_kv, s.scale);
  if (st != SA_OK) return st;
  if (s.S_q < 0) return fail(SA_ERR_INVALID_ARG, "negative S_q=%d", s.S_q);
  if (s.causal != 0 && s.causal != 1) return fail(SA_ERR_INVALID_ARG, "causal must be 0 or 1");
  // The kernels add a bias in units of 1 / |scale|, which must be finite.
  if (s.slopes && !std::isfinite(1.0f / std::fabs(s.scale)))
    return fail(SA_ERR_INVALID_ARG, "scale must be nonzero (1/|scale| finite) when ALiBi slopes are given");
  // With no query rows dk and dv are zero; with no keys dq is zero: both are
  // still written.  Only an empty batch, or no rows and no keys, is a no-op.
  if (s.B == 0 || (s.S_q == 0 && s.S_k == 0)) { *noop = true; return SA_OK; }
  int64_t nq = 1, nk = 1;
  if (!mul_ok(&nq, s.B) || !mul_ok(&nq, s.S_q) || !mul_ok(&nq, s.H_q) || !mul_ok(&nq, s.D) ||
      !mul_ok(&nk, s.B) || !mul_ok(&nk, s.S_k) || !mul_ok(&nk, s.H_kv) || !mul_ok(&nk, s.D))
    return fail(SA_ERR_INVALID_ARG, "tensor sizes overflow");
  // Grids (1-D) and 32-bit buffer ranges of the tile copies.
  if ((int64_t)s.B * s.H_q * ((s.S_q + 127) / 128) > INT32_MAX ||
      (int64_t)s.B * s.H_kv * ((s.S_k + 127) / 128) > INT32_MAX ||
      ((int64_t)s.B * s.H_q * s.S_q + 255) / 256 > INT32_MAX)
    return fail(SA_ERR_INVALID_ARG, "too many rows or keys for the launch grids");
  if ((int64_t)64 * s.H_kv * s.D * 2 >= (INT64_C(1) << 32) || (int64_t)32 * s.H_q * s.D * 2 >= (INT64_C(1) << 32))
    return fail(SA_ERR_UNSUPPORTED, "H * D too large for the tile copies");
  const bool rows = s.S_q > 0, keys = s.S_k > 0;
  if (rows && (!s.q || !s.out || !s.dout || !s.lse || !s.dq))
    return fail(SA_ERR_INVALID_ARG, "q, out, dout, lse and dq must not be NULL when S_q > 0");
  if (keys && (!s.k || !s.v || !s.dk || !s.dv))
    return fail(SA_ERR_INVALID_ARG, "k, v, dk and dv must not be NULL when S_k > 0");
  const void* a16[8] = {s.q, s.k, s.v, s.out, s.dout, s.dq, s.dk, s.dv};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return fail(SA_ERR_INVALID_ARG, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (s.lse && !aligned(s.lse, 4)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (s.slopes && !aligned(s.slopes, 4)) return fail(SA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
  const size_t need = bwd_workspace_size(s.B, s.H_q, s.S_q);
  if (rows) {
    if (!s.workspace) return fail(SA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(s.workspace, 16)) return fail(SA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (s.workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", s.workspace_bytes, need);
  }
  const size_t qb = (size_t)nq * 2, kb = (size_t)nk * 2, lb = (size_t)s.B * s.H_q * s.S_q * 4;
  const void* ins[8] = {s.q, s.k, s.v, s.out, s.dout, s.lse, s.mask, s.slopes};
  const size_t insz[8] = {qb, kb, kb, qb, qb, lb, (size_t)s.B * s.S_k, (size_t)s.H_q * 4};
  const void* outs[4] = {s.dq, s.dk, s.dv, rows ? s.workspace : nullptr};
  const size_t outsz[4] = {qb, kb, kb, need};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i]))
        return fail(SA_ERR_INVALID_ARG, "dq, dk, dv or workspace overlap an input");
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlap(outs[o], outsz[o], outs[o2], outsz[o2]))
        return fail(SA_ERR_INVALID_ARG, "dq, dk, dv and workspace must not overlap");
  }
  return SA_OK;
}

}  // namespace sa
