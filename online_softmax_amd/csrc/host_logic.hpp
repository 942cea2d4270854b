// Host-side argument checking, decode split sizing and error reporting for
// libsa_attn.  Plain C++: no HIP call is made here, so every function can run
// (and is tested) on a machine without a GPU.
#pragma once
#include <cstddef>
#include <cstdint>

namespace sa {

struct FwdShape {
  const void* q; const void* k; const void* v; const void* out; const float* lse;
  int B, S_q, S_k, H_q, H_kv, D; float scale; int causal;
  const uint8_t* mask; const float* slopes; int dtype;
};

struct DecodeShape {
  const void* q; const void* k; const void* v; const void* out; const float* lse;
  int B, S_k, H_q, H_kv, D; float scale;
  const uint8_t* mask; const float* slopes; int dtype;
  const void* workspace; size_t workspace_bytes;
};

struct BwdShape {
  const void* q; const void* k; const void* v; const void* out; const void* dout; const float* lse;
  const void* dq; const void* dk; const void* dv;
  int B, S_q, S_k, H_q, H_kv, D; float scale; int causal;
  const uint8_t* mask; const float* slopes; int dtype;
  const void* workspace; size_t workspace_bytes;
};

// Keys one decode split covers at least, and most splits per (batch, KV head,
// query-head group).  A split is one workgroup of four waves.
constexpr int kDecodeStepKeys = 128;
constexpr int kDecodeMaxSplits = 256;
// Query heads one decode workgroup serves at once (the MFMA column count).
constexpr int kDecodeHeadGroup = 16;
// Most splits per head group in the single-kernel decode, where the last
// split of a group reads all of the group's partial results by itself.
constexpr int kDecodeFusedMaxSplits = 64;
// Keys a decode workgroup addresses per round (4 waves x up to 4 sub-tiles of
// 32 keys); the last round of a split may run past its end.
constexpr int kDecodeRoundKeys = 512;


// Block-sparse prefill: block size for query rows and keys (the default
// attention block of the "Stem" page, section 6), and the capacity of a
// workgroup's list of 64-key tiles, which bounds S_k at 64 * kSparseMaxTiles.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxTiles = 4096;

// Records a formatted message as the calling thread's last error and returns
// the status unchanged.
int fail(int status, const char* fmt, ...);
void clear_error();
const char* last_error();
const char* status_string(int status);

// Returns SA_OK, or an error status after recording the reason.  *noop is set
// when the call is valid but has nothing to compute.
int check_fwd(const FwdShape& s, bool* noop);
int check_decode(const DecodeShape& s, bool* noop);
// check_decode with the workspace held to `need` bytes instead of
// decode_workspace_size (need == 0: the arguments only, no workspace).
int check_decode_need(const DecodeShape& s, size_t need, bool* noop);
// The single-kernel decode: its workspace starts with kDecodeArriveBytes of
// 32-bit arrival counters, one per head group (so at most kDecodeMaxGroups
// groups), zero before the first call; the partial area follows at that
// fixed offset, whatever the shape, so calls of different shapes can share a
// workspace.  check_decode_fused checks the partial area as check_decode
// does, plus the counter area itself.
constexpr int kDecodeArriveBytes = 65536;
constexpr int kDecodeMaxGroups = kDecodeArriveBytes / 4;
int check_decode_fused(const DecodeShape& s, bool* noop);
size_t decode_fused_workspace_size(int B, int H_q, int S_k, int D);
int check_bwd(const BwdShape& s, bool* noop);
// Additive bias and dropout of the extended forward.
struct ExtShape {
  const float* bias; int64_t sb, sh, sq;  // element strides; key axis contiguous
  double dropout_p;
};
// The forward's checks plus those of the bias (alignment, strides, extent,
// overlap with out/lse) and of the dropout probability (0 <= p < 1).
int check_ext(const FwdShape& s, const ExtShape& e, bool* noop);
// 16-bit dropout values below this threshold drop: floor(p * 2^16).
uint32_t drop_threshold(double p);

// The forward's checks plus those of the block mask
// [B, H_q, ceil(S_q / kSparseBlock), ceil(S_k / kSparseBlock)].
int check_block_sparse(const FwdShape& s, const uint8_t* block_mask, bool* noop);
// Bytes of backward workspace: one float2 {lse in base 2, row dot} per
// (batch, query head, row); 0 for a negative size or on overflow.
size_t bwd_workspace_size(int B, int H_q, int S_q);

int decode_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu);
// The split count of the single-kernel decode: decode_num_splits capped at
// kDecodeFusedMaxSplits (then rounded to whole steps again).
int decode_fused_num_splits(int B, int S_k, int H_q, int H_kv, int num_cu);
// Waves per prefill workgroup (4 or 8; a workgroup owns 32 query rows per
// wave).  Eight-wave workgroups halve the key/value copy traffic per FLOP;
// they are used when there are enough of them to keep every CU busy (for
// causal work, enough to balance the unequal blocks).
int fwd_waves(int B, int S_q, int H_q, bool causal, int num_cu);
// The paired causal block mapping of the backward's dq kernel (pair_ncu):
// num_cu when a causal grid of four-wave workgroups
// (two resident per CU) has exactly two workgroups per CU and an even number
// of blocks per head, else 0.
int fwd_pair_ncu(int nitems, int nmb, bool causal, int nw, int num_cu);
// The grid of the forward's persistent schedule (one eight-wave workgroup
// per CU working through units of one (batch, head) and a complementary pair
// of causal blocks, or one block without the causal rule), or 0 for one
// block per workgroup.  Used for the eight-wave kernels (nw = 8, or causal
// with nw = 4, which runs eight waves in two groups) when there are at least
// two units per CU.
int fwd_persistent_grid(int bh, int nmb, bool causal, int nw, int num_cu);
// Keys per split for a split count (a multiple of kDecodeStepKeys).
int decode_chunk(int S_k, int splits);
size_t decode_workspace_size(int B, int H_q, int S_k, int D);

// Byte offsets of the decode workspace regions for an actual split count.
struct DecodeLayout { int64_t o_offset, lse_offset, bytes; };
DecodeLayout decode_layout(int B, int H_q, int splits, int D);
// Whether one split's key range can be addressed with 32-bit byte offsets.
bool decode_offsets_fit(int chunk, int H_kv, int D);

}  // namespace sa
