// Decode kernel (one query token per sequence) over a key/value cache.
//
// A workgroup owns one (batch, KV head, group of up to 16 query heads sharing
// that KV head, key split).  Its four waves stream disjoint 32-key sub-tiles
// of the split, so every key/value row is read from memory once for all query
// heads of the group (the "StreamAttention" page, "Seed-Only Serving Wedge"
// and "Engine Direction", argues against re-reading K/V per query head under
// GQA).  Each wave keeps its own online-softmax state (running maximum,
// running sum, unnormalised output) for the group's heads; the four states are
// merged through LDS and the split writes a normalised partial output and its
// log-sum-exp to the workspace.
//
// A second kernel combines the splits of every (batch, query head) with
// log-sum-exp weights into the output: the "partial online-softmax states
// merged" of the "StreamAttention" page, "Engine Direction", and the
// "log-sum-exp weighted combining" of its "Distributed and Long-Context
// Variants".  It is spread over one workgroup per (batch, query head, 16-wide
// slice of D), so that it costs about one memory round trip.
//
// Matrix-core mapping: 16x16x32 MFMAs with the group's query heads as the 16
// columns: S^T = K Q^T (K straight from global memory into A-operand
// registers, one key row per lane), then O^T += V^T P^T with V copied from
// global memory into a wave-private LDS slot and read transposed with
// ds_read_b64_tr_b16.  Each wave issues every copy and load of a round of
// NSUB sub-tiles before computing any of them.
//
// Single-kernel mode (the "StreamAttention" page, "Seed-Only Serving Wedge",
// finds the merge and its launch dominant at small batch and calls for a
// single-kernel split design): each workgroup hands its partial over with
// device-coherent stores and then counts itself on its head group's arrival
// counter (a device-scope atomic in the workspace).  The workgroup that
// arrives last has every partial of the group available: it resets the
// counter to zero for the next call and merges the group's splits itself.
// No workgroup ever waits for another, so the launch is an ordinary one of
// any size.
#pragma once
#include "common.hpp"
#include "host_logic.hpp"

namespace sa {

// A wave rescales its state only when a sub-tile maximum exceeds the running
// reference by more than this (base 2), bounding every probability by 2^8.
constexpr float kDecodeSlack = 8.0f;

struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* mask;
  const float* slopes;
  uint16_t* out;      // [B, 1, H_q, D]
  float* lse;         // [B, H_q, 1] or null
  float* ws_o;        // [B, H_q, splits, D] normalised partial outputs
  float* ws_lse;      // [B, H_q, splits] base-2 partial lse
  int B, S_k, H_q, H_kv, G, n_hg, splits, chunk;
  float scale2;       // scale * log2(e)
  float alibi2;       // 1 / |scale|: bias to accumulator units
  // Single-kernel mode: one arrival counter per head group (zero between calls).
  unsigned* arrive;
};

// Chunk swizzle of a V row in a wave's LDS slot (16-byte chunks): spreads the
// 16 rows x 32 bytes of one transposed read over the banks.
template <int D>
__device__ inline int dec_swizzle(int r) {
  if constexpr (D == 128) return 2 * (r & 7);
  else return 2 * ((r >> 1) & 3);
}

template <class T, int D>
__device__ void merge_group(const DecArgs& a, int b, int h0, int g_heads);

template <class T, int D, bool MASK, bool ALIBI, bool FUSED = false>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecArgs a) {
  constexpr int KK = D / 32;             // MFMA k-steps (32 wide) over the head dimension
  constexpr int DB = D / 16;             // 16-row blocks of O^T
  constexpr int NSUB = D == 64 ? 4 : 2;  // 32-key sub-tiles per wave per round
  constexpr int NK = 2 * KK;             // K loads per lane per sub-tile
  constexpr int NV = 32 * D * 2 / 1024;  // 1 KiB V copies per wave per sub-tile
  constexpr int SLOT = 32 * D;           // 16-bit words per sub-tile slot
  constexpr int VBYTES = 4 * NSUB * SLOT * 2;
  constexpr int MBYTES = 3 * (2 + D) * 16 * 4;
  constexpr int SBYTES = VBYTES > MBYTES ? VBYTES : MBYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SBYTES];
  __shared__ __attribute__((aligned(1024))) uint16_t Qsh[kDecodeHeadGroup * D];  // the group's query rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g4 = lane >> 4;

  const int s = blockIdx.x % a.splits;
  const int grp = blockIdx.x / a.splits;   // (b, hk, hg)
  const int hg = grp % a.n_hg;
  const int bk = grp / a.n_hg;
  const int hk = bk % a.H_kv;
  const int b = bk / a.H_kv;
  const int g_heads = min(16, a.G - 16 * hg);   // query heads in this group
  const int h0 = hk * a.G + 16 * hg;            // first query head of the group
  const int h = h0 + li;                        // this lane's query head
  const bool hvalid = li < g_heads;

  const int k0 = s * a.chunk;
  const int k1 = min(a.S_k, k0 + a.chunk);
  const int nsub = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;   // 32-key sub-tiles in the split
  const int rounds = (nsub + 4 * NSUB - 1) / (4 * NSUB);
  const int ipos = a.S_k - 1;  // the query's position on the key axis

  // Q^T as the B operand: lane (column li, quarter g4) holds q[li][8 g4 + 32 kk .. +7].
  // The group's query rows (contiguous, g_heads * D values) are copied into
  // LDS by wave 0 ahead of its first loads of K and V, and read after those
  // loads are all issued (see the first round below): loaded into registers
  // here, they would have been awaited (for the sign flip) before any K/V
  // load left, and every split would have started its stream one memory
  // round trip late.
  const uint32_t qflip = a.scale2 < 0.f ? 0x80008000u : 0u;
  const float sc2 = __builtin_fabsf(a.scale2);
  constexpr int NQ = kDecodeHeadGroup * D * 2 / 1024;  // 1 KiB copies of the query rows
  if (w == 0) {
    const i32x4 rq = buffer_rsrc(a.q + ((size_t)b * a.H_q + h0) * D, (uint32_t)(g_heads * D * 2));
#pragma unroll
    for (int c = 0; c < NQ; ++c) load_lds16(rq, Qsh + c * 512, (uint32_t)(c * 1024 + 16 * lane));
  }
  u32x4 qreg[KK];

  // One buffer resource per split: rows past k1 read as zero.
  const size_t rs = (size_t)a.H_kv * D;  // key/value row stride (16-bit words)
  const size_t base = ((size_t)b * a.S_k * a.H_kv + hk) * D + (size_t)k0 * rs;
  const uint32_t bytes = k1 > k0 ? (uint32_t)((size_t)(k1 - k0 - 1) * rs * 2 + 2 * D) : 0u;
  const auto rk = buffer_rsrc_t(a.k + base, bytes);
  const i32x4 rv = buffer_rsrc(a.v + base, bytes);
  const uint8_t* mrow = MASK ? a.mask + (size_t)b * a.S_k : nullptr;

  uint16_t* slots = (uint16_t*)smem + w * NSUB * SLOT;
  // V copy c of a sub-tile: lane l's 16 bytes are LDS row r, position p of the
  // slot, holding global chunk p ^ f(r) of key row r.
  uint32_t vsrc[NV];
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int byte = c * 1024 + 16 * lane;
    const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
    vsrc[c] = (uint32_t)(r * rs * 2 + 16 * (p ^ dec_swizzle<D>(r)));
  }
  // Transposed V read of key step hi (keys 16 hi + 4 g4 + t/4, t = lane % 16)
  // and d block db (d = 16 db + 4 (t % 4)): word offset in a slot.
  int vofs[2][DB];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r = 16 * hi + 4 * g4 + (li >> 2);
      const int d = 16 * db + 4 * (li & 3);
      vofs[hi][db] = r * D + 8 * ((d >> 3) ^ dec_swizzle<D>(r)) + (d & 7);
    }

  float m_ref = kNegInf, l_run = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x4){};
  const float slope_acc = (ALIBI && hvalid) ? a.slopes[h] * a.alibi2 : 0.f;

  for (int rd = 0; rd < rounds; ++rd) {
    // Sub-tile v of this round covers keys k0 + 32 u .. +31, u = w + 4 (NSUB rd + v).
    // Copies of V go first, then the K loads, so that the wait for K(v) also
    // covers V(v).
#pragma unroll
    for (int v = 0; v < NSUB; ++v) {
      const uint32_t row0 = (uint32_t)(32 * (w + 4 * (NSUB * rd + v)));
#pragma unroll
      for (int c = 0; c < NV; ++c)
        load_lds16(rv, slots + v * SLOT + c * 512, vsrc[c] + row0 * (uint32_t)rs * 2);
    }
    u32x4 kr[NSUB][2][KK];
#pragma unroll
    for (int v = 0; v < NSUB; ++v) {
      const uint32_t row0 = (uint32_t)(32 * (w + 4 * (NSUB * rd + v)));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          kr[v][kb][kk] = buffer_load16(rk, (row0 + 16 * kb + li) * (uint32_t)rs * 2 + 2 * (8 * g4 + 32 * kk), 0);
    }
    // Keep every load of the round ahead of the first wait for one of them.
    __builtin_amdgcn_sched_barrier(0);
    if (rd == 0) {
      // Wave 0's query copies were issued before its loads of this round;
      // once only those loads are in flight they have landed.  The barrier
      // does not wait for any wave's loads.
      if (w == 0) wait_vmem_upto(NSUB * NV + NSUB * NK);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qreg[kk] = *(const u32x4*)&Qsh[li * D + 8 * g4 + 32 * kk] ^ qflip;
    }
#pragma unroll
    for (int v = 0; v < NSUB; ++v) {
      // Sub-tiles past the split's end are computed too (their keys read as
      // zero and are masked out), so that the loads above stay where they are
      // issued rather than being sunk behind a branch.
      const int kbase = k0 + 32 * (w + 4 * (NSUB * rd + v));
      // Sᵀ for keys kbase + 16 kb + 4 g4 + r (register r of block kb).  With
      // ALiBi the accumulator starts at -slope (ipos - key) / |scale|.
      f32x4 sc[2];
      if (ALIBI) {
        const float b0 = slope_acc * (float)(kbase + 4 * g4 - ipos);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[kb][r] = fmaf(slope_acc, (float)(16 * kb + r), b0);
      } else {
        sc[0] = (f32x4){};
        sc[1] = (f32x4){};
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[kb] = T::mma16(kr[v][kb][kk], qreg[kk], sc[kb]);
      if (MASK || kbase + 32 > k1) {
        // Padding bits of the sub-tile's 32 keys: lane l (and l + 32) reads
        // the byte of key kbase + l % 32, one ballot gathers them, shifted to
        // this lane's quarter (keys from 4 g4 on).
        uint64_t keep = ~uint64_t(0);
        if (MASK) {
          const int kl = kbase + (lane & 31);
          const bool kept = kl < k1 && mrow[kl < k1 ? kl : 0] != 0;
          keep = __builtin_amdgcn_ballot_w64(kept) >> (4 * g4);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kj = kbase + 16 * kb + 4 * g4 + r;
            bool vis = kj < k1;
            if (MASK) vis = vis && ((keep >> (16 * kb + r)) & 1u);
            sc[kb][r] = vis ? sc[kb][r] : kNegInf;
          }
      }
      float tmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sc[kb][r]);
      tmax = max_quarters(tmax) * sc2;
      if (wave_any(tmax > m_ref + kDecodeSlack)) {
        const float m_new = fmaxf(m_ref, tmax);
        const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      const float nm = m_ref == kNegInf ? 0.f : -m_ref;
      uint32_t pk[4];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const float p0 = fast_exp2(fmaf(sc[kb][r], sc2, nm));
          const float p1 = fast_exp2(fmaf(sc[kb][r + 1], sc2, nm));
          psum += p0 + p1;
          pk[2 * kb + (r >> 1)] = T::pack2(p0, p1);
        }
      l_run += psum;
      // V(v) was copied before every K load of the round: once only the
      // copies and loads issued after it are in flight, its slot is complete.
      wait_vmem_upto((NSUB - 1 - v) * NV + NSUB * NK);
      __asm__ volatile("" ::: "memory");
      const u32x4 bp = {pk[0], pk[1], pk[2], pk[3]};
      const uint16_t* vs = slots + v * SLOT;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = lds_read_tr(vs + vofs[0][db]);
        const u32x2 hi = lds_read_tr(vs + vofs[1][db]);
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = T::mma16(av, bp, o[db]);
      }
    }
    // The next round's copies reuse the slots: every transposed read of this
    // round must have returned (they have: their results fed the MFMAs).
    __asm__ volatile("" ::: "memory");
  }

  // Merge the four waves' states through LDS (reusing the V slots).
  const float l_tot = sum_quarters(l_run);
  wait_vmem();
  __syncthreads();
  float* mg = (float*)smem;
  constexpr int MREG = (2 + D) * 16;
  if (w > 0) {
    float* r = mg + (w - 1) * MREG;
    if (g4 == 0) {
      r[li] = m_ref;
      r[16 + li] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) r[32 + (16 * db + 4 * g4 + e) * 16 + li] = o[db][e];
  }
  __syncthreads();
  if (w == 0) {
    float M = m_ref;
#pragma unroll
    for (int x = 0; x < 3; ++x) M = fmaxf(M, mg[x * MREG + li]);
    const float Mu = M == kNegInf ? 0.f : M;
    const float s0 = fast_exp2(m_ref - Mu);
    float L = s0 * l_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= s0;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const float* r = mg + x * MREG;
      const float sx = fast_exp2(r[li] - Mu);
      L = fmaf(sx, r[16 + li], L);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db][e] = fmaf(sx, r[32 + (16 * db + 4 * g4 + e) * 16 + li], o[db][e]);
    }
    if (hvalid) {
      const size_t idx = ((size_t)b * a.H_q + h) * a.splits + s;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const float lv = L > 0.f ? M + __log2f(L) : kNegInf;
      if constexpr (FUSED) {
        // Handed to another workgroup: device-coherent stores (the partial
        // area is below 4 GiB, checked on the host).
        const auto ro = buffer_rsrc_t(a.ws_o, 0xFFFFFFFFu);
        const uint32_t ob = (uint32_t)((idx * D + 4 * g4) * 4);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          buffer_store16_coherent(ro, ob + 64 * db, __builtin_bit_cast(u32x4, o[db] * inv));
        if (g4 == 0) __hip_atomic_store(a.ws_lse + idx, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        float* op = a.ws_o + idx * D + 4 * g4;
#pragma unroll
        for (int db = 0; db < DB; ++db) *(f32x4*)(op + 16 * db) = o[db] * inv;
        if (g4 == 0) a.ws_lse[idx] = lv;
      }
    }
  }
  if constexpr (FUSED) {
    // Count this split on the head group's arrival counter; the last of the
    // group's splits to arrive resets the counter and merges them all.  The
    // partials were stored by wave 0, the wave of thread 0, so they precede
    // its count in program order: the count releases them at agent scope.
    // The last arriver then acquires (agent scope) every other split's
    // partials, which the barrier hands to the whole workgroup.
    __shared__ int s_last;
    __syncthreads();
    if (tid == 0) {
      unsigned* cnt = a.arrive + grp;
      const bool last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) ==
                        (unsigned)a.splits - 1u;
      if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      s_last = last;
    }
    __syncthreads();
    if (s_last) merge_group<T, D>(a, b, h0, g_heads);
  }
}

// Online log-sum-exp state (m, l, acc) of one (head, 4-wide d chunk) over a
// subset of splits: l = sum 2^(lse_s - m), acc = sum 2^(lse_s - m) o_s.
// Combining two states rescales both to the larger maximum (a state with m =
// -inf holds nothing and is scaled by zero).
__device__ inline float lse_scale(float m, float mn) { return m == kNegInf ? 0.f : fast_exp2(m - mn); }

// The merge of one head group (query heads h0 .. h0 + g_heads - 1 of batch b)
// by the workgroup that completed it: for each head and d, out = sum_s w_s
// o_s / sum_s w_s with w_s = 2^(lse_s - max lse), and lse = (max + log2 sum)
// ln 2 (a split with lse_s = -inf weighs nothing).  The group's partial rows
// (head-major, split-minor) are contiguous in the workspace.  Each thread
// owns one (head, d chunk) pair and the splits part, part + P, ... of it (P
// threads per pair, adjacent lanes), reads XC of those splits at a time with
// every load of the chunk issued before any is used, and keeps an online
// state in registers; the P states of a pair are then combined by lane
// exchanges.  Pairs beyond 256 / P are taken in further sweeps.
template <class T, int D>
__device__ void merge_group(const DecArgs& a, int b, int h0, int g_heads) {
  constexpr int TD = D / 4, XC = 32;
  const int tid = threadIdx.x;
  const int ns = a.splits;
  const int npair = g_heads * TD;
  int P = 1;
  while (2 * P * npair <= 256 && P < ns) P *= 2;
  const int per = 256 / P;  // pairs per sweep
  const size_t row0 = ((size_t)b * a.H_q + h0) * ns;
  const auto ro = buffer_rsrc_t(a.ws_o, 0xFFFFFFFFu);
  for (int pb = 0; pb < npair; pb += per) {
    const int pi = pb + tid / P, part = tid % P;
    const bool act = pi < npair;
    const int hh = pi / TD, d4 = pi - hh * TD;
    const size_t rbase = row0 + (size_t)(act ? hh : 0) * ns;
    float m = kNegInf, l = 0.f;
    f32x4 acc = {};
    for (int x0 = 0; x0 * P < ns; x0 += XC) {
      float lv[XC];
      f32x4 ov[XC];
#pragma unroll
      for (int x = 0; x < XC; ++x) {
        const int sp = part + P * (x0 + x);
        const bool ok = act && sp < ns;
        lv[x] = ok ? __hip_atomic_load(a.ws_lse + rbase + sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kNegInf;
        ov[x] = ok ? __builtin_bit_cast(f32x4, buffer_load16_coherent(
                                                   ro, (uint32_t)(((rbase + sp) * D + 4 * d4) * 4)))
                   : (f32x4){};
      }
      float cm = kNegInf;
#pragma unroll
      for (int x = 0; x < XC; ++x) cm = fmaxf(cm, lv[x]);
      const float mn = fmaxf(m, cm);
      if (mn != kNegInf) {
        const float sc = lse_scale(m, mn);
        l *= sc;
        acc *= sc;
#pragma unroll
        for (int x = 0; x < XC; ++x) {
          const float e = fast_exp2(lv[x] - mn);
          l += e;
          acc += e * ov[x];
        }
        m = mn;
      }
    }
    for (int k = 1; k < P; k <<= 1) {
      const float om = __shfl_xor(m, k), ol = __shfl_xor(l, k);
      f32x4 oa;
#pragma unroll
      for (int e = 0; e < 4; ++e) oa[e] = __shfl_xor(acc[e], k);
      const float mn = fmaxf(m, om);
      const float s1 = lse_scale(m, mn), s2 = lse_scale(om, mn);
      l = l * s1 + ol * s2;
      acc = acc * s1 + oa * s2;
      m = mn;
    }
    if (act && part == 0) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const uint2 pk = {T::pack2(acc[0] * inv, acc[1] * inv), T::pack2(acc[2] * inv, acc[3] * inv)};
      *(uint2*)(a.out + ((size_t)b * a.H_q + h0 + hh) * D + 4 * d4) = pk;
      if (a.lse && d4 == 0) a.lse[(size_t)b * a.H_q + h0 + hh] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
    }
  }
}

struct MergeArgs {
  const float* ws_o;   // [B * H_q, splits, D]
  const float* ws_lse; // [B * H_q, splits], base 2
  uint16_t* out;       // [B * H_q, D]
  float* lse;          // [B * H_q] or null
  int splits;
};

// One (batch * query head, 16-wide slice of D) item: out = sum_s w_s o_s /
// sum_s w_s with w_s = exp2(lse_s - max lse) (splits with lse_s = -inf weigh
// nothing); lse = (max + log2 sum w) ln 2.  Thread t of the 256 loads the
// 4-wide d chunk t % 4 of split t / 4 (+ 64 x): every load of the workgroup is
// issued before any is used.
template <class T, int D>
__device__ void merge_one(const float* ws_o, const float* ws_lse, uint16_t* out, float* lse, int splits,
                          int item, float* s_w, float (*s_red)[4], f32x4 (*s_acc)[4]) {
  constexpr int NX = kDecodeMaxSplits / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = item / (D / 16), slice = item % (D / 16);
  const int ns = splits;
  const float* lp = ws_lse + (size_t)bh * ns;
  const size_t obase = (size_t)bh * ns * D + 16 * slice + 4 * (tid & 3);
  const float lv = tid < ns ? lp[tid] : kNegInf;
  const float* op = ws_o + obase;
  f32x4 ov[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int sp = (tid >> 2) + 64 * x;
    ov[x] = sp < ns ? *(const f32x4*)(op + (size_t)sp * D) : (f32x4){};
  }
  // Largest lse over the splits, then the weights and their sum.
  float m = lv;
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
  if (lane == 0) s_red[0][w] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  const float wgt = fast_exp2(lv - (M == kNegInf ? 0.f : M));
  if (tid < kDecodeMaxSplits) s_w[tid] = wgt;
  float tot = wgt;
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) tot += __shfl_xor(tot, k);
  if (lane == 0) s_red[1][w] = tot;
  __syncthreads();
  tot = s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];
  // Weighted sum over this thread's splits, then over the 16 threads of the
  // wave that hold the same d chunk, then over the four waves.
  f32x4 acc = {};
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int sp = (tid >> 2) + 64 * x;
    acc += (sp < ns ? s_w[sp] : 0.f) * ov[x];
  }
#pragma unroll
  for (int k = 32; k >= 4; k >>= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], k);
  if (lane < 4) s_acc[w][lane] = acc;
  __syncthreads();
  if (tid < 4) {
    const f32x4 sum = s_acc[0][tid] + s_acc[1][tid] + s_acc[2][tid] + s_acc[3][tid];
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    const uint2 pk = {T::pack2(sum[0] * inv, sum[1] * inv), T::pack2(sum[2] * inv, sum[3] * inv)};
    *(uint2*)(out + (size_t)bh * D + 16 * slice + 4 * tid) = pk;
    if (tid == 0 && slice == 0 && lse) lse[bh] = tot > 0.f ? (M + __log2f(tot)) * kLn2 : kNegInf;
  }
}

// The second kernel of the two-kernel decode: one workgroup per item.
template <class T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeArgs a) {
  __shared__ float s_w[kDecodeMaxSplits];
  __shared__ float s_red[4][4];
  __shared__ f32x4 s_acc[4][4];
  merge_one<T, D>(a.ws_o, a.ws_lse, a.out, a.lse, a.splits, blockIdx.x, s_w, s_red, s_acc);
}

}  // namespace sa
