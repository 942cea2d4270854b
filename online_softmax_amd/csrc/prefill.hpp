// Prefill kernel: exact attention forward in one streaming sweep over key/value
// tiles with float32 running row maximum and row sum (online softmax), as the
// "StreamAttention: Fused Online Softmax Attention" page describes in section
// "Kernel Design (Fused Online Softmax)": per key tile, raise the running
// maximum, rescale the running numerator and denominator by
// exp(old_max - new_max), add exp(score - new_max) and its product with V;
// finish with numerator / denominator and lse = max + log(denominator).
//
// Mapping onto gfx950:
//  * a workgroup of NW waves (4 or 8) owns 32·NW query rows of one (batch,
//    head); each wave owns 32 rows and keeps their Q slice in registers;
//  * key/value tiles of 64 rows are copied from global memory straight into
//    LDS (buffer loads with the LDS destination, 16 bytes per lane) through a
//    ring of NS buffers per tensor; the buffer bounds return zeros past the
//    last key.  Iteration t issues K of tile t+NS and V of tile t+NS-1; they
//    are awaited before the barrier that closes iteration t+NS-2 (with the
//    two buffers used here, iteration t's own);
//  * LDS rows are unpadded; 16-byte chunks are placed at (chunk XOR f(row))
//    so that the K reads (16 rows, one chunk) and the transposed V reads
//    (4 consecutive rows, 4 chunks) each touch distinct banks;
//  * scores are computed transposed, S^T = K Q^T, with 32x32x16 MFMAs: the
//    accumulator then holds one query per lane (keys along the registers and
//    across the two wave halves), so row statistics are per-lane values plus
//    one exchange between the wave halves, and the probabilities already sit
//    in the B-operand layout of the next product O^T += V^T P^T;
//  * V stays row-major in LDS and is read transposed with ds_read_b64_tr_b16;
//  * with ALiBi under the causal rule the workgroup's diagonal band of tiles
//    is swept first (last tile down), then the tiles from key 0 up: every
//    wave starts on its own diagonal tile, where the largest biases sit (the
//    running maximum then settles at once), while the workgroups of a head
//    still share the tiles from key 0 in L2 (under the persistent schedule the
//    second block of a unit sweeps from its last tile down, so that the CUs
//    of one head read the same tiles at the same time); otherwise tiles go in
//    key order;
//  * software pipeline: iteration t runs S^T of the next tile on the matrix
//    cores while the vector units form the probabilities of tile t, then
//    P·V of tile t, then prepares the next tile;
//  * exponentials are base 2 on the hardware exp unit with log2(e) folded into
//    the score scale; the running maximum lives in that base-2 domain.  The
//    ALiBi bias (divided by the scale) is the initial value of the S^T
//    accumulator, so scores with and without bias share one softmax path;
//  * tiles that no rule hides any key of (the bulk of the sweep) skip the
//    masking pass; tiles on the causal diagonal, at the ragged end of the
//    keys or from the first padded key on take it.  The first padded key is
//    found once per workgroup;
//  * block-sparse mode (the execution step of the "Stem: Rethinking Causal
//    Information Flow in Sparse Attention" page, section 2.3): a workgroup
//    of 4 waves owns one block of 128 query rows and sweeps only the key
//    blocks of 128 that its row of the block mask selects; wave 0 compacts
//    the selected 64-key tiles into a list in LDS, and the sweep walks that
//    list in key order (under causal ALiBi from its last tile down, for the
//    reason given for the band order) with everything else unchanged;
//  * extended mode (the additive masks and Philox dropout of the
//    "StreamAttention" page, "Recent Updates"): an additive float32 bias is
//    loaded for each tile while the previous tile's matrix work runs and is
//    added to the scores (in accumulator units, like ALiBi) before the
//    maximum; dropout keeps or zeroes each probability by a 16-bit half of a
//    Philox4x32-10 word of its (row, key) position, after the row sum has
//    taken it;
//  * two-group mode (NG = 2, the causal forward when 128-row blocks are
//    needed to balance the CUs, and causal dropout): eight waves over one
//    128-row block in two groups of four that own the same rows and take
//    alternate tiles (each iteration stages one tile per group); at the end
//    group 1 hands its state to group 0 through LDS;
//  * persistent schedule (PERSIST, large eight-wave grids): one workgroup per
//    CU works through a list of (batch, head) units, each a complementary
//    pair of causal blocks (x and nmb - 1 - x) or one block, so that every
//    unit carries the same work and a CU never waits for a new workgroup;
//  * the reference maximum is raised only when a tile's maximum exceeds it by
//    more than kRescaleSlack (base 2): the final out = numerator / denominator
//    and lse = reference + log(denominator) are exact for any reference, and
//    the slack bounds every probability by 2^kRescaleSlack, so most tiles skip
//    rescaling the output accumulator.
#pragma once
#include "common.hpp"
#include "host_logic.hpp"

namespace sa {

constexpr float kRescaleSlack = 8.0f;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  const uint8_t* mask;
  const float* slopes;
  int B, S_q, S_k, H_q, H_kv, G;
  float scale2;  // scale * log2(e)
  float alibi2;  // log2(e) / |scale log2(e)| = 1 / |scale|: bias to accumulator units
  int nmb;       // query blocks per (batch, head)
  int nitems;    // B * H_q * nmb
  const uint8_t* block_mask;  // block-sparse mode: [B, H_q, nmb, nkb], nonzero = visit
  int nkb;                    // key blocks of kSparseBlock per row of block_mask
  // Extended mode.  Bias element (b, h, i, j) at bias[b sb + h sh + i sq + j]
  // (strides in elements, multiples of 4; NULL = none).  Dropout: a
  // probability is kept when its 16-bit Philox value is >= drop_thr (0 = no
  // generator calls: every value is); the output is scaled by drop_scale =
  // 1 / (1 - p) in the epilogue (1 without dropout).
  const float* bias;
  int64_t bias_sb, bias_sh, bias_sq;
  uint32_t drop_thr;
  float drop_scale;
  uint32_t seed_lo, seed_hi, drop_offset;
};

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds over a 128-bit counter (c0, c1, c2,
// c3) with a 64-bit key (k0, k1), the key bumped by the two Weyl constants
// between rounds; a round maps the counter to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
// hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)).
//
// The dropout counters of one lane differ only in c0 (the key quarter): c1
// (the row), c2 (batch and head) and c3 (the offset) are fixed, so the part
// of round 0 that does not involve c0, and the round keys, are computed once
// per lane (PhiloxLane) and each block runs round 0 with one product.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

// a ^ b ^ c in one instruction (the three-input bitwise operation with the
// truth table of a three-way exclusive or; the compiler leaves this chain as
// two two-input ones).
__device__ __attribute__((always_inline)) inline uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  __asm__("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

struct PhiloxLane {
  uint32_t a0, b0, c0x;     // round 0: hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), c3 ^ k1
  uint32_t k0[9], k1[9];    // keys of rounds 1 .. 9
};

__device__ __attribute__((always_inline)) inline PhiloxLane philox_lane(uint32_t c1, uint32_t c2, uint32_t c3,
                                                                       uint32_t k0, uint32_t k1) {
  PhiloxLane p;
  const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
  p.a0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
  p.b0 = (uint32_t)p1;
  p.c0x = c3 ^ k1;
#pragma unroll
  for (int r = 1; r < 10; ++r) {
    p.k0[r - 1] = k0 + (uint32_t)r * kPhiloxW0;
    p.k1[r - 1] = k1 + (uint32_t)r * kPhiloxW1;
  }
  // Keep the lane constants in vector registers (as scalars they would take
  // about twenty scalar registers the kernel does not have to spare).
  __asm__ volatile("" : "+v"(p.a0), "+v"(p.b0), "+v"(p.c0x));
#pragma unroll
  for (int r = 0; r < 9; ++r) __asm__ volatile("" : "+v"(p.k0[r]), "+v"(p.k1[r]));
  return p;
}

// The block of counter (c0, c1, c2, c3) of the lane constants L.
__device__ __attribute__((always_inline)) inline u32x4 philox4x32_10(uint32_t c0, const PhiloxLane& L) {
  const uint64_t q0 = (uint64_t)kPhiloxM0 * c0;
  uint32_t x0 = L.a0, x1 = L.b0, x2 = (uint32_t)(q0 >> 32) ^ L.c0x, x3 = (uint32_t)q0;
#pragma unroll
  for (int r = 0; r < 9; ++r) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * x0, p1 = (uint64_t)kPhiloxM1 * x2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), x1, L.k0[r]), n2 = xor3((uint32_t)(p0 >> 32), x3, L.k1[r]);
    x1 = (uint32_t)p1;
    x3 = (uint32_t)p0;
    x0 = n0;
    x2 = n2;
  }
  return (u32x4){x0, x1, x2, x3};
}

// Chunk swizzle of LDS row r (16-byte chunks, D / 8 per row).
template <int D>
__device__ inline int lds_swizzle(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// NG = 2 splits the NW waves into two groups that own the same BM = 16 NW
// query rows: group 0 takes the sweep's tiles 0, 2, 4, ... and group 1 the
// tiles 1, 3, 5, ... (each iteration stages one tile per group), and group 1's
// state joins group 0's at the end.  Eight waves then cover a 128-row block
// at two waves per SIMD, so that causal blocks of very unequal length can be
// spread over the CUs heaviest first instead of pairing them on one CU.
// The persistent schedule (PERSIST): the grid holds one workgroup per CU,
// and each works through units of its XCD's share, a unit being one (batch,
// head) and a pair of causal blocks x and nmb - 1 - x (the heavier first) --
// so that every unit carries the same work -- or one block without the
// causal rule.  The XCDs (workgroups are dealt to them round-robin) own
// contiguous ranges of units and their workgroups take the units in turn, so
// the units of one (batch, head) run at the same time on one L2.
template <bool CAUSAL>
__device__ inline int persist_upb(const FwdArgs& a) { return CAUSAL ? (a.nmb + 1) / 2 : a.nmb; }
template <bool CAUSAL>
__device__ inline int2 persist_range(const FwdArgs& a) {
  const int nunits = a.nitems / a.nmb * persist_upb<CAUSAL>(a);
  const int x = blockIdx.x & 7;
  const int u0 = x * (nunits >> 3) + min(x, nunits & 7);
  return make_int2(u0, u0 + (nunits >> 3) + (x < (nunits & 7) ? 1 : 0));
}
__device__ inline int persist_stride() {
  return ((int)gridDim.x >> 3) + ((int)(blockIdx.x & 7) < ((int)gridDim.x & 7) ? 1 : 0);
}

template <class T, int D, bool CAUSAL, bool MASK, bool ALIBI, int NW, bool SPARSE = false,
          bool EXT = false, int NG = 1, bool PERSIST = false>
__global__ __launch_bounds__(NW * 64, EXT && NG == 1 ? 1 : 2) void fwd_kernel(FwdArgs a) {
  static_assert(NG == 1 || (NG == 2 && NW == 8 && !SPARSE && !(EXT && ALIBI)), "two groups: dense eight-wave kernel only");
  static_assert(!PERSIST || (!SPARSE && !EXT), "persistent schedule: dense kernels only");
  constexpr int NWG = NW / NG;       // waves per group
  constexpr int BM = 32 * NWG;       // query rows per workgroup
  constexpr int BN = 64;             // keys per tile
  constexpr int NS = 2;  // LDS buffers per tensor
  constexpr int KK = D / 16;         // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int NI = BN * D * 2 / 1024 / NW;  // 1 KiB copies per wave per tensor per tile
  static_assert(NI >= 1, "tile too small for the copy layout");
  static_assert(!SPARSE || BM == kSparseBlock, "a block-sparse workgroup owns one query block");
  static_assert(!(SPARSE && EXT), "one mode at a time");

  __shared__ __attribute__((aligned(1024))) uint16_t Ks[NS][NG * BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[NS][NG * BN * D];
  __shared__ int Pw[MASK ? NW : 1];  // per-wave first cleared key
  __shared__ int Lw[MASK ? NW : 1];  // per-wave last kept key
  __shared__ int16_t Tl[SPARSE ? kSparseMaxTiles : 1];  // block-sparse tile list
  __shared__ int Tn;                                     // its length
  // Persistent schedule: the current unit and which of its blocks (kept in
  // LDS rather than in registers across the sweep).
  __shared__ int s_unit[2];

  if constexpr (PERSIST) {
    if (threadIdx.x == 0) {
      s_unit[0] = persist_range<CAUSAL>(a).x + (int)(blockIdx.x >> 3);
      s_unit[1] = 0;
    }
    __syncthreads();
  }
  for (;;) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int gw = NG == 1 ? 0 : w / NWG;  // this wave's group
  const int wi = w - gw * NWG;           // and its place in the group
  int bh, mb;
  bool second = false;  // persistent schedule: the unit's second (lighter) block
  if constexpr (!PERSIST) {
    const int item = xcd_contiguous(blockIdx.x, a.nitems);
    bh = item / a.nmb;
    const int mbi = item - bh * a.nmb;
    // Causal blocks are issued heaviest (last rows) first.
    mb = CAUSAL ? a.nmb - 1 - mbi : mbi;
  } else {
    const int q = __builtin_amdgcn_readfirstlane(s_unit[0]);
    const int half = __builtin_amdgcn_readfirstlane(s_unit[1]);
    if (q >= persist_range<CAUSAL>(a).y) break;
    const int upb = persist_upb<CAUSAL>(a);
    bh = q / upb;
    const int x = q - bh * upb;
    mb = CAUSAL && half == 0 ? a.nmb - 1 - x : x;
    second = CAUSAL && half != 0;
  }
  const int b = bh / a.H_q, h = bh - b * a.H_q, hk = h / a.G;
  const int m0 = mb * BM;
  const int off = a.S_k - a.S_q;  // bottom-right alignment of the causal rule
  const int qi = m0 + 32 * wi + li;
  const int ipos = qi + off;      // this row's position on the key axis

  // Extended mode: this lane's bias row and whether dropout is on.
  const bool has_bias = EXT && a.bias != nullptr;
  const bool dropping = EXT && a.drop_thr != 0u;
  // Dropout: this lane's generator constants (its row and head are fixed).
  PhiloxLane plane{};
  if constexpr (EXT) {
    if (dropping) plane = philox_lane((uint32_t)qi, (uint32_t)bh, a.drop_offset, a.seed_lo, a.seed_hi);
  }
  const float* brow_bias =
      has_bias && qi < a.S_q ? a.bias + b * a.bias_sb + h * a.bias_sh + qi * a.bias_sq : nullptr;

  int n_end = a.S_k;
  if (CAUSAL) n_end = min(n_end, m0 + BM + off);
  const int ntd = n_end > 0 ? (n_end + BN - 1) / BN : 0;  // tiles up to the last key any row may see
  int nt = ntd;                                           // tiles the sweep visits

  // The padding mask over the keys this workgroup may read (the first ntd
  // tiles): the first key it clears (S_k if none) and the last key it keeps
  // (-1 if none).  Tiles that end at or before the first cleared key need no
  // padding test, the others take the masking pass (for the usual padding, a
  // cleared tail, that is exactly the tiles holding cleared keys).  Each lane
  // checks 16 consecutive keys per round through a buffer resource that ends
  // at S_k (keys past it read as cleared), all 16 loads in flight together;
  // the extremes go over the wave by shuffles and over the waves through LDS.
  const uint8_t* mrow = MASK ? a.mask + (size_t)b * a.S_k : nullptr;
  int pad_start = a.S_k, last_kept = -1;
  auto mask_scan = [&]() {
    const auto mr = buffer_rsrc_t(mrow, (uint32_t)a.S_k);
    const int nkeys = ntd * BN;
    int first = a.S_k, last = -1;
    for (int j0 = 16 * (64 * w + lane); j0 < nkeys; j0 += 16 * 64 * NW) {
      uint32_t kept[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) kept[e] = __builtin_amdgcn_raw_buffer_load_b8(mr, (uint32_t)(j0 + e), 0, 0);
#pragma unroll
      for (int e = 15; e >= 0; --e) first = kept[e] == 0 ? min(first, j0 + e) : first;
#pragma unroll
      for (int e = 0; e < 16; ++e) last = kept[e] != 0 ? max(last, j0 + e) : last;
    }
#pragma unroll
    for (int k = 32; k > 0; k >>= 1) {
      first = min(first, __shfl_xor(first, k));
      last = max(last, __shfl_xor(last, k));
    }
    if (lane == 0) {
      Pw[w] = first;
      Lw[w] = last;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      pad_start = min(pad_start, Pw[x]);
      last_kept = max(last_kept, Lw[x]);
    }
    pad_start = __builtin_amdgcn_readfirstlane(pad_start);
    last_kept = __builtin_amdgcn_readfirstlane(last_kept);
  };
  // With ALiBi under the causal rule the sweep starts on its last tiles (see
  // the sweep order below), so it ends at the last kept key: the tiles after
  // it are cleared throughout and contribute nothing, and the first tiles
  // taken then carry the largest biases that count, so the running maximum
  // settles at once.  (Starting on cleared tiles instead, the maximum was
  // first set far from the diagonal and then raised on nearly every tile.)
  constexpr bool BAND = CAUSAL && ALIBI && !SPARSE;
  // Sweeps that start on their last tiles: the dense band order above, and
  // in block-sparse mode the whole selected list from its last tile down.
  constexpr bool DESC = CAUSAL && ALIBI;
  // The padding scan decides the sweep's first tiles here (the band below
  // the last kept key).  In block-sparse mode it runs first; in the dense
  // kernel the first tiles are copied as if nothing were cleared, together
  // with Q and the scan's own loads, and copied again in the rare case that
  // the scan moves them (the band below a cleared tail).
  constexpr bool SCAN_FIRST = MASK && DESC && SPARSE;
  constexpr bool SCAN_SPEC = MASK && DESC && !SPARSE;
  if constexpr (SCAN_FIRST) {
    mask_scan();
    nt = min(nt, last_kept >= 0 ? last_kept / BN + 1 : 0);
  }

  // Block-sparse mode: the selected tiles of this query block in key order.
  // Wave 0 takes 64 key blocks per round, one per lane; a selected block
  // contributes its one or two tiles below nt, placed by two ballots.
  if constexpr (SPARSE) {
    if (w == 0) {
      const uint8_t* brow = a.block_mask + ((size_t)bh * a.nmb + mb) * a.nkb;
      const int nkv = (nt + 1) / 2;  // key blocks holding a tile below nt
      int base = 0;
      for (int kb0 = 0; kb0 < nkv; kb0 += 64) {
        const int kbl = kb0 + lane;
        const bool sel = kbl < nkv && brow[kbl < nkv ? kbl : 0] != 0;
        const bool two = sel && 2 * kbl + 1 < nt;
        const uint64_t bs = __builtin_amdgcn_ballot_w64(sel), bt = __builtin_amdgcn_ballot_w64(two);
        const int pos = base + lanes_below(bs, lane) + lanes_below(bt, lane);
        if (sel) Tl[pos] = (int16_t)(2 * kbl);
        if (two) Tl[pos + 1] = (int16_t)(2 * kbl + 1);
        base += __builtin_popcountll(bs) + __builtin_popcountll(bt);
      }
      if (lane == 0) Tn = base;
    }
    __syncthreads();
    nt = __builtin_amdgcn_readfirstlane(Tn);
  }

  const size_t rs = (size_t)a.H_kv * D;  // key/value row stride
  const uint16_t* kb = a.k + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint16_t* vb = a.v + ((size_t)b * a.S_k * a.H_kv + hk) * D;

  // Copy u of this wave fills LDS bytes [cb KiB, cb KiB + 1 KiB) of a buffer,
  // cb = NW u + w; lane l's 16 bytes are LDS row r, position p, holding global
  // chunk p ^ f(r).
  uint32_t voff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int byte = (NW * u + w) * 1024 + 16 * lane;
    const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
    voff[u] = (uint32_t)(r * rs * 2 + 16 * (p ^ lds_swizzle<D>(r)));
  }
  auto tile_rsrc = [&](const uint16_t* base, int n0) {
    const int rows = min(BN, a.S_k - n0);
    return buffer_rsrc(base + (size_t)n0 * rs, (uint32_t)((rows - 1) * rs * 2 + 2 * D));
  };
  // Sweep order.  With ALiBi under the causal rule the workgroup's diagonal
  // band (its last BM / BN tiles) comes first, from the last tile down, and
  // then the tiles from key 0 upwards: every wave starts on its own diagonal
  // tile, where the largest biases sit, so the running maximum rarely needs
  // raising afterwards (in key order it would rise on nearly every tile for
  // the steeper slopes); and the workgroups of one head still walk the shared
  // tiles from key 0 together, which keeps them in L2.  In the two-group mode
  // the whole sweep runs from the last tile down: the groups take alternate
  // positions, so with the band first the rows of group 0 whose diagonal is
  // the band's second tile would start on key 0.  Otherwise the order is
  // plain 0 .. nt-1.
  // Under the persistent schedule the second block of a unit sweeps all its
  // tiles from the last one down.  The CUs working on the units of one head
  // reach their second blocks at different times (after first blocks of
  // different lengths); in descending order they still stand on the same
  // tile at each moment -- block x starts its descent at key block x after
  // the nmb - x key blocks of its first block, so at sweep time t every such
  // CU is at key block nmb - t -- and their reads are shared in L2.
  auto band_tiles = [&]() { return BAND ? (second ? nt : min(nt, BM / BN)) : 0; };
  int nb = band_tiles();
  auto tile_of = [&](int it) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)Tl[DESC ? nt - 1 - it : it]);
    else if constexpr (NG == 2 && BAND) return nt - 1 - it;
    else return it < nb ? nt - 1 - it : it - nb;
  };
  // Iteration t stages the tiles of sweep positions NG t .. NG t + NG - 1
  // (those below nt), the one of group j at offset j BN D of the buffer.
  int nti = (nt + NG - 1) / NG;  // iterations of the sweep
  auto issue_k = [&](int t) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      if (NG > 1 && NG * t + j >= nt) break;
      const auto r = tile_rsrc(kb, tile_of(NG * t + j) * BN);
      uint16_t* buf = Ks[t % NS] + j * BN * D;
#pragma unroll
      for (int u = 0; u < NI; ++u) load_lds16(r, buf + (NW * u + w) * 512, voff[u]);
    }
  };
  auto issue_v = [&](int t) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      if (NG > 1 && NG * t + j >= nt) break;
      const auto r = tile_rsrc(vb, tile_of(NG * t + j) * BN);
      uint16_t* buf = Vs[t % NS] + j * BN * D;
#pragma unroll
      for (int u = 0; u < NI; ++u) load_lds16(r, buf + (NW * u + w) * 512, voff[u]);
    }
  };
  // The tile this wave works on in iteration t.
  auto wtile = [&](int t) -> int { return tile_of(NG * t + gw); };

  // Prologue copies: K of iterations 0..NS-1, V of iterations 0..NS-2.
  auto prologue_copies = [&]() {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (j < nti) issue_k(j);
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
      if (j < nti) issue_v(j);
  };
  prologue_copies();

  // Q^T as the B operand: lane (row li, half g) holds q[row][16kk + 8g .. +7].
  // A negative scale is applied as |scale| on negated Q (exact in fp16/bf16),
  // so the row maximum of the raw products is the maximum of the scaled ones.
  u32x4 qreg[KK];
  const bool qvalid = qi < a.S_q;
  const uint32_t qflip = a.scale2 < 0.f ? 0x80008000u : 0u;
  const float sc2 = __builtin_fabsf(a.scale2);
  {
    const uint16_t* qp = a.q + ((size_t)(b * (size_t)a.S_q + (qvalid ? qi : 0)) * a.H_q + h) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qreg[kk] = qvalid ? *(const u32x4*)(qp + 16 * kk) : (u32x4){0, 0, 0, 0};
  }
  if constexpr (SCAN_SPEC) {
    mask_scan();
    const int ntk = min(nt, last_kept >= 0 ? last_kept / BN + 1 : 0);
    if (ntk != nt) {
      // Every copy issued so far has landed (the scan waited for its own
      // loads, which were issued after them); copy the right tiles.
      wait_vmem();
      nt = ntk;
      nb = band_tiles();
      nti = (nt + NG - 1) / NG;
      prologue_copies();
    }
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qreg[kk] ^= qflip;
    // Keep the flipped values as the loop-invariant operands (otherwise the
    // compiler re-applies the flip inside the key loop).
    __asm__ volatile("" : "+v"(qreg[kk]));
  }

  if constexpr (MASK && !DESC) mask_scan();

  float m_ref = kNegInf;  // reference maximum, base-2 domain (raised lazily)
  float l_run = 0.f;      // this lane's share of the running row sum
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};

  // ALiBi slope in accumulator units: bias / |scale| per unit distance.
  const float slope_acc = ALIBI ? a.slopes[h] * a.alibi2 : 0.f;
  const int wrow0 = m0 + 32 * wi;                      // first row of this wave
  const bool wave_active = wrow0 < a.S_q;
  const int wave_last = min(wrow0 + 31, a.S_q - 1) + off;  // furthest key the wave may see

  // Lane constants of the K reads and of the transposed V reads (see
  // lds_read_tr): row li + 32 jb, chunk 2 kk + g for K; for V, row
  // 16 ks + 8 q + tr_key, column 32 db + tr_col.
  const int ksw = lds_swizzle<D>(li);
  const int tr_key = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int vofs[2][DB];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r = 8 * q + tr_key;
      vofs[q][db] = r * D + 8 * ((4 * db + (tr_col >> 3)) ^ lds_swizzle<D>(r)) + (tr_col & 7);
    }

  // Sᵀ = K Qᵀ for the 64 keys of the tile of iteration t (register r of
  // block jb holds key n0 + 32 jb + 8 (r/4) + 4 g + r%4).  With ALiBi the accumulator starts at
  // the bias in accumulator units, -slope |ipos - key| / |scale|; under the
  // causal rule every visible key has key <= ipos, so it is linear there.
  auto init_scores = [&](const int t, const int jb, f32x16 (&s)[2]) {
    if (ALIBI) {
      const float rel = (float)(wtile(t) * BN + 4 * g - ipos);  // key - ipos at r = 0, jb = 0
      const float b0 = slope_acc * rel;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float kofs = (float)(32 * jb + 8 * (r >> 2) + (r & 3));
        s[jb][r] = CAUSAL ? fmaf(slope_acc, kofs, b0) : -slope_acc * __builtin_fabsf(rel + kofs);
      }
    } else {
      s[jb] = (f32x16){};
    }
  };
  // K fragment of Sᵀ MFMA i (k-step i/2, key block i%2).
  auto k_frag = [&](const uint16_t* kbuf, const int i) -> u32x4 {
    const int kk = i >> 1, jb = i & 1;
    return *(const u32x4*)&kbuf[(32 * jb + li) * D + 8 * ((2 * kk + g) ^ ksw)];
  };
  auto qk = [&](const int t, f32x16 (&s)[2]) {
    const uint16_t* kbuf = Ks[t % NS] + gw * BN * D;
    init_scores(t, 0, s);
    init_scores(t, 1, s);
#pragma unroll
    for (int i = 0; i < 2 * KK; ++i) s[i & 1] = T::mma(k_frag(kbuf, i), qreg[i >> 1], s[i & 1]);
  };

  // Visibility and the running-maximum update for the tile of iteration it.
  // Keys past the causal diagonal, past the end of the keys or cleared in the
  // padding mask are set to -inf in a pass that only tiles touching them take
  // (`tile_masked` is uniform over the wave).  The scale enters once, in the
  // exponent's fma, and the maximum is taken before scaling.  The reference
  // maximum is raised only when some row's tile maximum exceeds it by more
  // than the slack (rows that need no change get alpha = 1).
  auto tile_masked = [&](const int it) -> bool {
    const int t = wtile(it);
    const int n0 = t * BN;
    bool masked = n0 + BN > a.S_k || (CAUSAL && n0 + BN - 1 > wrow0 + off);
    if (MASK) masked = masked || n0 + BN > pad_start;
    return masked;
  };
  auto mask_tile = [&](const int it, f32x16 (&s)[2]) {
    const int t = wtile(it);
    const int n0 = t * BN;
    const bool pad_free = !MASK || n0 + BN <= pad_start;
    // The padding bits of the tile's 64 keys are the same for every row:
    // lane l reads the byte of key n0 + l and one ballot gathers them
    // (bit l kept).  A lane's 32 scores need the bits of key offsets
    // 4 g + 32 jb + 8 (r/4) + r%4: nibbles 0, 2, 4, 6 of each 32-bit half of
    // the ballot shifted by 4 g, packed into one word (bit 16 jb + r).
    uint32_t vis32 = ~0u;
    if (MASK && !pad_free) {
      const int kl = n0 + lane;
      const bool kept = kl < a.S_k && mrow[kl < a.S_k ? kl : 0] != 0;
      const uint64_t keep = __builtin_amdgcn_ballot_w64(kept) >> (4 * g);
      auto pick = [](uint32_t x) {
        x &= 0x0F0F0F0Fu;
        x = (x | (x >> 4)) & 0x00FF00FFu;
        return (x | (x >> 8)) & 0x0000FFFFu;
      };
      vis32 = pick((uint32_t)keep) | (pick((uint32_t)(keep >> 32)) << 16);
    }
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // Bitwise tests (no short-circuit), so that the pass is straight-line
        // selects rather than a branch per score.
        const int kj = n0 + 4 * g + 32 * jb + 8 * (r >> 2) + (r & 3);
        bool vis = kj < a.S_k;
        if (CAUSAL) vis = vis & (kj <= ipos);
        if (MASK) vis = vis & (((vis32 >> (16 * jb + r)) & 1u) != 0);
        s[jb][r] = vis ? s[jb][r] : kNegInf;
      }
  };
  // Row maximum of a tile in the base-2 domain (same value in both halves).
  auto tile_max = [&](const f32x16 (&s)[2]) -> float {
    float mx[2] = {kNegInf, kNegInf};  // two independent chains
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx[jb] = fmaxf(mx[jb], s[jb][r]);
    return max_halves(fmaxf(mx[0], mx[1])) * sc2;
  };
  auto raise_max = [&](const float tmax) {
    if (wave_any(tmax > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
  };
  // Extended mode.  Bias of the tile of iteration it, in the layout of the
  // scores (register r of block jb: key n0 + 32 jb + 8 (r/4) + 4 g + r%4,
  // four consecutive keys per quarter): eight 16-byte loads per lane, scalar
  // loads for a quarter that crosses the end of the keys, zeros past it.
  auto bias_load = [&](const int it, f32x4 (&bv)[8]) {
    const int n0 = wtile(it) * BN;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j0 = n0 + 32 * (u >> 2) + 8 * (u & 3) + 4 * g;
      if (brow_bias && j0 + 3 < a.S_k) {
        bv[u] = *(const f32x4*)(brow_bias + j0);
      } else {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (brow_bias)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + e < a.S_k) x[e] = brow_bias[j0 + e];
        bv[u] = x;
      }
    }
  };
  // Adds the bias in accumulator units (bias / |scale|, as for ALiBi).
  auto bias_add = [&](f32x16 (&s)[2], const f32x4 (&bv)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[u >> 2][4 * (u & 3) + e] = fmaf(bv[u][e], a.alibi2, s[u >> 2][4 * (u & 3) + e]);
  };
  // Dropout keep bits of the tile of iteration it: bit 16 jb + r for register
  // r of block jb.  Key j is decided by 16-bit half (j mod 64) / 32 of word
  // j mod 4 of the generator block with counter (8 (j / 64) + (j mod 32) / 4,
  // row, b * H_q + h, offset).  A tile is one 64-key window, and the lane's
  // keys 32 jb + 8 u + 4 g + e of it (register 4 u + e of block jb) take
  // half jb of word e of block 8 (n0 / 64) + 2 u + g: four blocks per tile.
  static_assert(BN == 64, "the dropout counters assume 64-key tiles");
  auto keep_bits = [&](const int it) __attribute__((always_inline)) -> uint32_t {
    const int n0 = wtile(it) * BN;
    const uint32_t c0 = (uint32_t)(n0 >> 3) + (uint32_t)g;
    uint32_t bits = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 wd = philox4x32_10(c0 + 2u * (uint32_t)u, plane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bits |= ((wd[e] & 0xFFFFu) >= a.drop_thr ? 1u : 0u) << (4 * u + e);
        bits |= ((wd[e] >> 16) >= a.drop_thr ? 1u : 0u) << (16 + 4 * u + e);
      }
    }
    return bits;
  };
  auto prepare = [&](const int it, f32x16 (&s)[2]) {
    if (has_bias) {
      f32x4 bv[8];
      bias_load(it, bv);
      bias_add(s, bv);
    }
    if (tile_masked(it)) mask_tile(it, s);
    raise_max(tile_max(s));
  };

  // Probabilities of a prepared tile, packed to the input type, and their sum.
  // While a row has seen no visible key its reference is 0, so that no
  // exp(-inf - (-inf)) is formed.
  // With dropout (keep bits other than all ones) the row sum takes every
  // probability and the P·V operand only the kept ones.
  auto softmax_exp = [&](const f32x16 (&s)[2], uint32_t (&pk)[2][8], const uint32_t keep) {
    const float nm = m_ref == kNegInf ? 0.f : -m_ref;
    float ps[2] = {0.f, 0.f};  // two partial sums: shorter dependency chains
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[jb][r], sc2, nm));
        const float p1 = fast_exp2(fmaf(s[jb][r + 1], sc2, nm));
        ps[jb] += p0 + p1;
        if constexpr (EXT) {
          pk[jb][r >> 1] = T::pack2((keep >> (16 * jb + r)) & 1u ? p0 : 0.f,
                                    (keep >> (16 * jb + r + 1)) & 1u ? p1 : 0.f);
        } else {
          pk[jb][r >> 1] = T::pack2(p0, p1);
        }
      }
    }
    l_run += ps[0] + ps[1];
  };

  // Oᵀ += Vᵀ Pᵀ over four 16-key steps of tile t.
  auto pv = [&](const int t, const uint32_t (&pk)[2][8]) {
    const uint16_t* vbuf = Vs[t % NS] + gw * BN * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int jb = ks >> 1, mh = ks & 1;
      const u32x4 bp = {pk[jb][4 * mh], pk[jb][4 * mh + 1], pk[jb][4 * mh + 2], pk[jb][4 * mh + 3]};
      const uint16_t* vt = vbuf + 16 * ks * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = lds_read_tr(vt + vofs[0][db]);
        const u32x2 hi = lds_read_tr(vt + vofs[1][db]);
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = T::mma(av, bp, o[db]);
      }
    }
  };

  // Instruction order for the block {Sᵀ of tile t+1, exponentials of tile t,
  // P·V of tile t, maximum of tile t+1}: keep a few K reads ahead of the Sᵀ
  // MFMAs and put the exponential work between them, so that neither the LDS
  // latency nor the vector work leaves the matrix cores idle; then P·V with
  // its transposed V reads three MFMAs ahead and the maximum between them.
  auto interleave_schedule = [&]() {
    constexpr int kMfma = 0x008, kValu = 0x002 | 0x400, kDsRead = 0x100;
    constexpr int NQK = 2 * KK, NPV = 4 * DB;
    __builtin_amdgcn_sched_group_barrier(kDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kValu, 5, 0);
      if (i + 4 < NQK) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kDsRead, 6, 0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      if (i + 3 < NPV) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kValu, 4, 0);
    }
  };

  // The two phases of a pipelined step, each in a fixed instruction order
  // (a scheduling barrier closes every chunk): left free, the scheduler
  // either bunched the vector work behind the matrix work or, with ALiBi,
  // started P·V before Sᵀ and left the exponentials exposed.  The sixteen
  // pairs of exponentials of the current tile are split between the phases:
  // the first EQ under the Sᵀ MFMAs of the next tile, the rest under the
  // first P·V MFMAs (those that use only the first EQ pairs).
  constexpr int NQK = 2 * KK, NPV = 4 * DB, EQ = 8;
  // P·V MFMAs 0 .. NPV/2-1 use only pairs 0 .. 7 (keys 0 .. 31 of the tile).
  static_assert(EQ >= 8 && EQ <= 16, "pair split");
  // One pair of probabilities: exponentials, packed to the input type, summed.
  auto exp_pair = [&](const f32x16 (&s)[2], const int pi, const float nm, uint32_t (&pk)[2][8],
                      float (&ps)[2], const uint32_t keep) {
    const int jb = pi >> 3, r = 2 * (pi & 7);
    const float p0 = fast_exp2(fmaf(s[jb][r], sc2, nm));
    const float p1 = fast_exp2(fmaf(s[jb][r + 1], sc2, nm));
    ps[jb] += p0 + p1;
    if constexpr (EXT) {
      pk[jb][r >> 1] = T::pack2((keep >> (16 * jb + r)) & 1u ? p0 : 0.f,
                                (keep >> (16 * jb + r + 1)) & 1u ? p1 : 0.f);
    } else {
      pk[jb][r >> 1] = T::pack2(p0, p1);
    }
  };
  // Phase 1: Sᵀ of the tile of iteration t1 (K fragments read four MFMAs
  // ahead) with pairs 0 .. EQ-1 of the current tile s.
  auto qk_exp = [&](const int t1, f32x16 (&sn)[2], const f32x16 (&s)[2], const float nm,
                    uint32_t (&pk)[2][8], float (&ps)[2], const uint32_t keep) {
    const uint16_t* kbuf = Ks[t1 % NS] + gw * BN * D;
    u32x4 ak[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ak[i] = k_frag(kbuf, i);
    init_scores(t1, 0, sn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      sn[i & 1] = T::mma(ak[i & 3], qreg[i >> 1], sn[i & 1]);
      if (i + 4 < NQK) ak[i & 3] = k_frag(kbuf, i + 4);
      if (i == 0) init_scores(t1, 1, sn);
#pragma unroll
      for (int pi = i * EQ / NQK; pi < (i + 1) * EQ / NQK; ++pi) exp_pair(s, pi, nm, pk, ps, keep);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Phase 2: Oᵀ += Vᵀ Pᵀ for the tile of iteration t (transposed V reads three
  // MFMAs ahead) with pairs EQ .. 15 under its first MFMAs, and the row
  // maximum of the next tile sn (as if no key were hidden) in two chains.
  auto pv_max = [&](const int t, const f32x16 (&s)[2], const float nm, uint32_t (&pk)[2][8],
                    float (&ps)[2], const f32x16 (&sn)[2], const uint32_t keep) -> float {
    const uint16_t* vbuf = Vs[t % NS] + gw * BN * D;
    auto v_frag = [&](const int i) -> u32x4 {
      const int ks = i / DB, db = i % DB;
      const uint16_t* vt = vbuf + 16 * ks * D;
      const u32x2 lo = lds_read_tr(vt + vofs[0][db]);
      const u32x2 hi = lds_read_tr(vt + vofs[1][db]);
      return (u32x4){lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 av[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) av[i] = v_frag(i);
    float mx[2] = {kNegInf, kNegInf};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int ks = i / DB, db = i % DB, jb = ks >> 1, mh = ks & 1;
      const u32x4 bp = {pk[jb][4 * mh], pk[jb][4 * mh + 1], pk[jb][4 * mh + 2], pk[jb][4 * mh + 3]};
      o[db] = T::mma(av[i % 3], bp, o[db]);
      if (i + 3 < NPV) av[i % 3] = v_frag(i + 3);
      constexpr int H = NPV / 2;
      if (i < H) {
#pragma unroll
        for (int pi = EQ + i * (16 - EQ) / H; pi < EQ + (i + 1) * (16 - EQ) / H; ++pi)
          exp_pair(s, pi, nm, pk, ps, keep);
      }
#pragma unroll
      for (int e = 0; e < 32 / NPV; e += 2) {
        const int vi = i * (32 / NPV) + e;  // score 0..31
        const int sj = vi >> 4, r = vi & 15;
        mx[sj] = fmaxf(fmaxf(mx[sj], sn[sj][r]), sn[sj][r + 1]);
      }
      // Pin this step of the maximum here (it depends on nothing in the loop
      // and would otherwise be sunk past it).
      __asm__ volatile("" : "+v"(mx[0]), "+v"(mx[1]));
      __builtin_amdgcn_sched_barrier(0);
    }
    return max_halves(fmaxf(mx[0], mx[1])) * sc2;
  };

  // Tiles this wave needs: all of them, or under the causal rule those that
  // start at or before the wave's furthest visible key.  They are the
  // iterations [t0w, t1w): in key order the first ntw, in band-first (or
  // descending) order the last ntw (the tiles past the wave's diagonal come
  // first and are the ones it skips).
  int ntw = wave_active ? nt : 0;
  if (CAUSAL) {
    if (wave_last < 0) {
      ntw = 0;
    } else if constexpr (SPARSE) {
      // Entries of the (ascending) list at or before the wave's last tile.
      const int last_tile = wave_last / BN;
      int lo = 0, hi = ntw;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane((int)Tl[mid]) <= last_tile) lo = mid + 1;
        else hi = mid;
      }
      ntw = lo;
    } else {
      ntw = min(ntw, wave_last / BN + 1);
    }
  }
  // In iterations: those whose sweep position NG t + gw lies in that range.
  const int t0w = DESC ? (max(nt - ntw - gw, 0) + NG - 1) / NG : 0;
  const int t1w = DESC ? (max(nt - gw, 0) + NG - 1) / NG : (max(ntw - gw, 0) + NG - 1) / NG;
  const bool wact = t1w > t0w;

  // Iteration t issues K of tile t+NS (into the buffer K(t) left, whose Sᵀ
  // was formed in iteration t-1) and V of tile t+NS-1 (into the buffer of
  // V(t-1)).  Before the barrier that ends iteration t, K(t+2) and V(t+1)
  // must have landed: they were issued NS-2 iterations earlier, so only the
  // copies issued in this iteration may still be in flight.
  auto copies = [&](const int t) -> int {
    int n = 0;
    if (t + NS < nti) {
      issue_k(t + NS);
      n += NI;
    }
    if (t + NS - 1 < nti) {
      issue_v(t + NS - 1);
      n += NI;
    }
    return n;
  };
  auto finish = [&](const int in_flight) {
    if (NS == 2 || in_flight == 0) wait_vmem();
    else if (in_flight == NI) wait_vmem_n<NI>();
    else wait_vmem_n<2 * NI>();
    __syncthreads();
  };
  // A full step: Sᵀ of tile t+1, probabilities and P·V of tile t, then the
  // preparation of tile t+1.
  // The maximum of tile t+1 is first taken as if no key were hidden, during
  // the matrix work (every score is finite); a tile that has hidden keys
  // masks them and takes it again.  With ALiBi the step runs in the fixed
  // order above; otherwise the scheduler places the same work after the
  // pattern of interleave_schedule, which measured faster there.
  // `keep` holds the dropout bits of tile t (all ones without dropout).
  auto full_step = [&](const int t, f32x16 (&s)[2], f32x16 (&sn)[2], const uint32_t keep) {
    const int n = copies(t);
    uint32_t pk[2][8];
    float tmax;
    // Extended mode: the next tile's bias is loaded under this step's matrix
    // work.
    f32x4 bvn[8];
    if (has_bias) bias_load(t + 1, bvn);
    if constexpr (ALIBI) {
      float ps[2] = {0.f, 0.f};
      const float nm = m_ref == kNegInf ? 0.f : -m_ref;
      qk_exp(t + 1, sn, s, nm, pk, ps, keep);
      tmax = pv_max(t, s, nm, pk, ps, sn, keep);
      l_run += ps[0] + ps[1];
    } else {
      qk(t + 1, sn);
      softmax_exp(s, pk, keep);
      pv(t, pk);
      tmax = tile_max(sn);
      interleave_schedule();
      // Keep the row sum in this block, where the matrix work hides it (the
      // compiler would otherwise sink it past the masking branch).
      __asm__ volatile("" : "+v"(l_run));
    }
    bool remax = false;
    if (has_bias) {
      bias_add(sn, bvn);
      remax = true;
    }
    if (tile_masked(t + 1)) {
      mask_tile(t + 1, sn);
      remax = true;
    }
    if (remax) tmax = tile_max(sn);
    raise_max(tmax);
    finish(n);
  };
  // The wave's last tile: probabilities and P·V only.
  auto last_step = [&](const int t, f32x16 (&s)[2], const uint32_t keep) {
    const int n = copies(t);
    uint32_t pk[2][8];
    softmax_exp(s, pk, keep);
    pv(t, pk);
    finish(n);
  };

  wait_vmem();
  // Persistent schedule: no scalar load is left in flight into the sweep
  // (the per-block reloads of kernel arguments), so that the waits for the
  // sweep's LDS reads can count them exactly.
  if constexpr (PERSIST) __builtin_amdgcn_s_waitcnt(0xc07f);
  __syncthreads();

  f32x16 sa[2], sb[2];
  if (wact && t0w == 0) {
    qk(0, sa);
    prepare(0, sa);
  }
  // Iteration 0 overwrites the buffer of K(0): every wave must have read it.
  __syncthreads();
  int t = 0;
  if (DESC) {
    // Iterations before this wave's first tile take part in the copies and
    // barriers only.  In the last of them the wave forms Sᵀ of its first
    // tile: that K landed before the previous barrier, and its buffer is
    // refilled only after the next one.
    for (; t < t0w; ++t) {
      const int n = copies(t);
      if (wact && t + 1 == t0w) {
        qk(t + 1, sa);
        prepare(t + 1, sa);
      }
      finish(n);
    }
  }
  // Dropout bits of the tile of iteration it (formed outside the steps, which
  // stay small enough to be inlined).
  auto keep_of = [&](const int it) __attribute__((always_inline)) -> uint32_t {
    return dropping ? keep_bits(it) : ~0u;
  };
  if (wact) {
    for (; t + 2 < t1w; t += 2) {
      full_step(t, sa, sb, keep_of(t));
      full_step(t + 1, sb, sa, keep_of(t + 1));
    }
    if (t + 1 < t1w) {
      full_step(t, sa, sb, keep_of(t));
      last_step(t + 1, sb, keep_of(t + 1));
    } else {
      last_step(t, sa, keep_of(t));
    }
    t = t1w;
  }
  // Tiles this wave does not need still take part in the copies and barriers.
  for (; t < nti; ++t) finish(copies(t));

  // Two groups, extended mode: each group finalises half of the head
  // dimension (group 0 the d blocks below DB / 2, group 1 the rest), which
  // measured 2 % faster there (and 1 % slower for the plain causal forward,
  // which keeps the hand-over to group 0 below).  Every wave hands the
  // other group's half of its O, its reference maximum and its row-sum share
  // to the wave of the other group that owns the same rows, through the K
  // buffers (O as 16-byte pieces, lane-minor) and the V buffers; both then
  // rescale the two states to the larger maximum and add them, in the same
  // order (group 0's term first), so the two halves share one row sum.  The
  // last barrier of the sweep came after every read of the tiles.
  constexpr bool HALVES = NG == 2 && EXT;
  constexpr int DH = HALVES ? DB / 2 : DB;  // d blocks each group finalises
  auto store_half = [&](const int hf) {
    // out = O / l over half hf (0 for a row that saw no key).
    const float l_tot = sum_halves(l_run);
    if (qvalid) {
      float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if constexpr (EXT) inv *= a.drop_scale;
      uint16_t* op = a.out + ((size_t)(b * (size_t)a.S_q + qi) * a.H_q + h) * D + 4 * g;
#pragma unroll
      for (int dd = 0; dd < DH; ++dd) {
        const int db = hf * DH + dd;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x2 pr = {T::pack2(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv),
                            T::pack2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv)};
          *(u32x2*)(op + 32 * db + 8 * q4) = pr;
        }
      }
    }
  };
  if constexpr (HALVES) {
    static_assert(NW * DH * 4 * 64 * 16 <= (int)sizeof(Ks), "O hand-over fits the K buffers");
    f32x4* xo_w = (f32x4*)&Ks[0][0] + (2 * wi + gw) * (DH * 4 * 64) + lane;
    const f32x4* xo_r = (const f32x4*)&Ks[0][0] + (2 * wi + 1 - gw) * (DH * 4 * 64) + lane;
    float* xm_w = (float*)&Vs[0][0] + (2 * wi + gw) * 128 + lane;
    const float* xm_r = (const float*)&Vs[0][0] + (2 * wi + 1 - gw) * 128 + lane;
    auto hand_over = [&](const int hf) {
      // This wave keeps half hf and hands over half 1 - hf.
#pragma unroll
      for (int dd = 0; dd < DH; ++dd)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int db = (1 - hf) * DH + dd;
          xo_w[(dd * 4 + q4) * 64] = (f32x4){o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]};
        }
      xm_w[0] = m_ref;
      xm_w[64] = l_run;
      __syncthreads();
      const float mo = xm_r[0], lo = xm_r[64];
      const float m0 = hf == 0 ? m_ref : mo, m1 = hf == 0 ? mo : m_ref;
      const float l0 = hf == 0 ? l_run : lo, l1 = hf == 0 ? lo : l_run;
      const float mn = fmaxf(m0, m1);
      if (mn != kNegInf) {
        const float f0 = m0 == kNegInf ? 0.f : fast_exp2(m0 - mn);
        const float f1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - mn);
        l_run = l0 * f0 + l1 * f1;
#pragma unroll
        for (int dd = 0; dd < DH; ++dd)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int db = hf * DH + dd;
            const f32x4 x = xo_r[(dd * 4 + q4) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float own = o[db][4 * q4 + e];
              o[db][4 * q4 + e] = hf == 0 ? own * f0 + x[e] * f1 : x[e] * f0 + own * f1;
            }
          }
        m_ref = mn;
      }
      store_half(hf);
    };
    if (gw == 0) hand_over(0);
    else hand_over(1);
  } else if constexpr (NG == 2) {
    // Group 1 hands its state (reference maximum, row-sum share and O, per
    // lane) to the wave of group 0 that owns the same rows, through the K
    // buffers (O as 16-byte pieces, lane-minor) and the V buffers (maximum
    // and sum); group 0 rescales both to the larger maximum and adds them.
    // The last barrier of the sweep came after every read of the tiles.
    f32x4* xo = (f32x4*)&Ks[0][0] + wi * (DB * 4 * 64) + lane;
    float* xm = (float*)&Vs[0][0] + wi * 128 + lane;
    static_assert(NWG * DB * 16 * 64 * 4 <= (int)sizeof(Ks), "O hand-over fits the K buffers");
    if (gw == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xo[(db * 4 + q4) * 64] = (f32x4){o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]};
      xm[0] = m_ref;
      xm[64] = l_run;
    }
    __syncthreads();
    if (gw == 0) {
      const float m1 = xm[0], l1 = xm[64];
      const float mn = fmaxf(m_ref, m1);
      if (mn != kNegInf) {
        const float f0 = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - mn);
        const float f1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - mn);
        l_run = l_run * f0 + l1 * f1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 x = xo[(db * 4 + q4) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[db][4 * q4 + e] = o[db][4 * q4 + e] * f0 + x[e] * f1;
          }
        m_ref = mn;
      }
    }
  }

  // Epilogue: out = O / l (0 for a row that saw no key; in halves written
  // above), lse = ln of the sum.
  const float l_tot = sum_halves(l_run);
  if (qvalid && gw == 0) {
    if constexpr (!HALVES) {
      float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if constexpr (EXT) inv *= a.drop_scale;
      uint16_t* op = a.out + ((size_t)(b * (size_t)a.S_q + qi) * a.H_q + h) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x2 pr = {T::pack2(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv),
                            T::pack2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv)};
          *(u32x2*)(op + 32 * db + 8 * q4) = pr;
        }
      }
    }
    if (g == 0 && a.lse)
      a.lse[((size_t)b * a.H_q + h) * a.S_q + qi] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
  }
  if constexpr (!PERSIST) {
    break;
  } else {
    // Every wave has read the unit and is done with the buffers (the next
    // block's copies reuse them, after the two-group hand-over too); then the
    // next unit or block.
    __syncthreads();
    if (tid == 0) {
      const int q = s_unit[0], upb = persist_upb<CAUSAL>(a);
      const int x = q % upb;
      if (CAUSAL && s_unit[1] == 0 && x < a.nmb - 1 - x) {
        s_unit[1] = 1;
      } else {
        s_unit[0] = q + persist_stride();
        s_unit[1] = 0;
      }
    }
    __syncthreads();
  }
  }
}

}  // namespace sa
