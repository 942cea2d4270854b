// Decode kernels (one query token per sequence) over a key/value cache.
//
// Split phase: a workgroup owns one (batch, KV head, group of up to 32 query
// heads sharing that KV head, key split).  Its four waves stream disjoint
// 32-key sub-tiles of the split, so every key/value row is read from memory
// once for all query heads of the group (the "StreamAttention" page, "Seed-Only
// Serving Wedge" and "Engine Direction", argues against re-reading K/V per
// query head under GQA).  Each wave keeps its own online-softmax state
// (running maximum, running sum, unnormalised output) for the group's heads;
// at the end the four states are merged through LDS and the split writes a
// normalised partial output and its log-sum-exp.
//
// Merge phase: one workgroup per (batch, query head) combines the splits with
// log-sum-exp weights, the "partial online-softmax states merged in a second
// kernel" of "Engine Direction" and the log-sum-exp weighted combining of
// "Distributed and Long-Context Variants".
//
// The matrix-core mapping is the prefill kernel's: S^T = K Q^T with the group's
// query heads as the 32 MFMA columns (unused columns hold zero queries), then
// O^T += V^T P^T with V read transposed from LDS.  K goes straight from global
// memory into the A-operand registers (one key row per lane); V passes through
// a wave-private LDS slot.  Each wave issues the loads of NSUB sub-tiles at
// once before computing any of them, to keep many bytes in flight per CU.
#pragma once
#include "common.hpp"

namespace sa {

struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* mask;
  const float* slopes;
  float* ws_o;    // [B, H_q, splits, D] normalised partial outputs
  float* ws_lse;  // [B, H_q, splits] natural-log partial lse
  int B, S_k, H_q, H_kv, G, n_hg, splits, chunk;
  float scale2;   // scale * log2(e)
};

template <class T, int D, bool MASK, bool ALIBI>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecArgs a) {
  constexpr int VSTR = D + 32;           // V row stride in LDS (16-bit words)
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int VCH = 32 * D / 8 / 64;   // 16-byte V chunks per lane per 32-key sub-tile
  constexpr int RCH = D / 8;
  constexpr int NSUB = D == 64 ? 4 : 2;  // sub-tiles loaded together per wave
  constexpr int VBYTES = 4 * 32 * VSTR * 2;
  constexpr int MBYTES = 3 * (2 + D) * 32 * 4;
  constexpr int SBYTES = VBYTES > MBYTES ? VBYTES : MBYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;

  const int s = blockIdx.x % a.splits;
  int rest = blockIdx.x / a.splits;
  const int hg = rest % a.n_hg;
  rest /= a.n_hg;
  const int hk = rest % a.H_kv;
  const int b = rest / a.H_kv;
  const int g_heads = min(32, a.G - 32 * hg);   // query heads in this group
  const int h = hk * a.G + 32 * hg + li;         // this lane's query head
  const bool hvalid = li < g_heads;

  const int k0 = s * a.chunk;
  const int k1 = min(a.S_k, k0 + a.chunk);
  const int nsub_total = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;   // 32-key sub-tiles in the split
  const int nsteps = (nsub_total + 4 * NSUB - 1) / (4 * NSUB);
  const int ipos = a.S_k - 1;  // the query's position on the key axis

  const uint32_t qflip = a.scale2 < 0.f ? 0x80008000u : 0u;
  const float sc2 = __builtin_fabsf(a.scale2);
  u32x4 qreg[KK];
  {
    const uint16_t* qp = a.q + ((size_t)b * a.H_q + (hvalid ? h : 0)) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qreg[kk] = hvalid ? *(const u32x4*)(qp + 16 * kk) : (u32x4){0, 0, 0, 0};
      qreg[kk] ^= qflip;
    }
  }

  const size_t rs = (size_t)a.H_kv * D;
  const uint16_t* kb = a.k + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint16_t* vb = a.v + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  uint16_t* Vw = (uint16_t*)smem + w * 32 * VSTR;
  const uint8_t* mrow = MASK ? a.mask + (size_t)b * a.S_k : nullptr;

  float m_ref = kNegInf, l_run = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  const float slope2 = (ALIBI && hvalid) ? a.slopes[h] * kLog2e : 0.f;
  const int tr_key = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int st = 0; st < nsteps; ++st) {
    // Sub-tiles are dealt to the waves round-robin: sub-tile u = w + 4 (st NSUB + v).
    u32x4 kr[NSUB][KK], vr[NSUB][VCH];
#pragma unroll
    for (int v = 0; v < NSUB; ++v) {
      const int base = k0 + 32 * (w + 4 * (st * NSUB + v));
      const int j = base + li;
      const bool ok = j < k1;
      const uint16_t* kp = kb + (size_t)(ok ? j : k0) * rs + 8 * g;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        kr[v][kk] = *(const u32x4*)(kp + 16 * kk);
        if (!ok) kr[v][kk] = (u32x4){0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < VCH; ++u) {
        const int c = lane + 64 * u, row = c / RCH, col = (c % RCH) * 8;
        const bool okv = base + row < k1;
        vr[v][u] = *(const u32x4*)(vb + (size_t)(okv ? base + row : k0) * rs + col);
        if (!okv) vr[v][u] = (u32x4){0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int v = 0; v < NSUB; ++v) {
      const int base = k0 + 32 * (w + 4 * (st * NSUB + v));
      if (base >= k1) break;  // wave-uniform
      f32x16 sc = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc = T::mma(kr[v][kk], qreg[kk], sc);
      // Stage this sub-tile's V rows in the wave's LDS slot.  LDS operations
      // of one wave complete in order; the waits and compiler barriers keep
      // the compiler from moving the reads of the previous sub-tile past
      // these writes or these writes past the reads below.
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < VCH; ++u) {
        const int c = lane + 64 * u, row = c / RCH, col = (c % RCH) * 8;
        *(u32x4*)&Vw[row * VSTR + col] = vr[v][u];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __asm__ volatile("" ::: "memory");

      const bool need_mask = MASK || base + 32 > k1;
      const float rel0 = (float)(ipos - base - 4 * g);
      const float bb = -slope2 * rel0;
      float tmax = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kofs = 8 * (r >> 2) + (r & 3);
        float x = ALIBI ? fmaf(sc[r], sc2, fmaf(slope2, (float)kofs, bb)) : sc[r];
        if (need_mask) {
          const int kj = base + 4 * g + kofs;
          bool vis = kj < k1;
          if (MASK) vis = vis && mrow[vis ? kj : 0] != 0;
          x = vis ? x : kNegInf;
        }
        sc[r] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = max_halves(tmax);
      if (!ALIBI) tmax *= sc2;
      const float m_new = fmaxf(m_ref, tmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_ref - m_use);
      m_ref = m_new;
      float psum = 0.f;
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = ALIBI ? fast_exp2(sc[r] - m_use) : fast_exp2(fmaf(sc[r], sc2, -m_use));
        const float p1 = ALIBI ? fast_exp2(sc[r + 1] - m_use) : fast_exp2(fmaf(sc[r + 1], sc2, -m_use));
        psum += p0 + p1;
        pk[r >> 1] = T::pack2(p0, p1);
      }
      l_run = fmaf(l_run, alpha, psum);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 bp = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
        const uint16_t* vrow0 = &Vw[(16 * ks + tr_key) * VSTR + tr_col];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 lo = lds_read_tr(vrow0 + 32 * db);
          const u32x2 hi = lds_read_tr(vrow0 + 8 * VSTR + 32 * db);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = T::mma(av, bp, o[db]);
        }
      }
      __asm__ volatile("" ::: "memory");
    }
  }

  // Merge the four waves' states through LDS (reusing the V slots).
  const float l_tot = sum_halves(l_run);
  __syncthreads();
  float* mg = (float*)smem;
  constexpr int MREG = (2 + D) * 32;
  if (w > 0) {
    float* r = mg + (w - 1) * MREG;
    if (g == 0) {
      r[li] = m_ref;
      r[32 + li] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) r[64 + (32 * db + 8 * (e >> 2) + 4 * g + (e & 3)) * 32 + li] = o[db][e];
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
      L = fmaf(sx, r[32 + li], L);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          o[db][e] = fmaf(sx, r[64 + (32 * db + 8 * (e >> 2) + 4 * g + (e & 3)) * 32 + li], o[db][e]);
    }
    if (hvalid) {
      const size_t idx = ((size_t)b * a.H_q + h) * a.splits + s;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* op = a.ws_o + idx * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = {o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                             o[db][4 * q4 + 3] * inv};
          *(float4*)(op + 32 * db + 8 * q4) = v4;
        }
      if (g == 0) a.ws_lse[idx] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
    }
  }
}

struct MergeArgs {
  const float* ws_o;
  const float* ws_lse;
  uint16_t* out;   // [B, 1, H_q, D]
  float* lse;      // [B, H_q, 1] or null
  int splits;
};

// One workgroup of 256 threads per (batch, query head).  The split weights
// exp(lse_s - M) / sum are formed once in LDS; then thread (column d, lane
// group sg) sums its share of splits and the groups are added through LDS.
template <class T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeArgs a) {
  constexpr int NG = 256 / D;
  __shared__ float wts[256];
  __shared__ float red[256];
  __shared__ float part[NG][D];
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* L = a.ws_lse + (size_t)bh * a.splits;
  const float lv = t < a.splits ? L[t] : kNegInf;
  red[t] = lv;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) red[t] = fmaxf(red[t], red[t + off]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  const float wv = (M == kNegInf || t >= a.splits) ? 0.f : fast_exp2((lv - M) * kLog2e);
  wts[t] = wv;
  red[t] = wv;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) red[t] += red[t + off];
    __syncthreads();
  }
  const float tot = red[0];
  const int d = t % D, sg = t / D;
  const float* O = a.ws_o + (size_t)bh * a.splits * D + d;
  float acc = 0.f;
  int x = sg;
  for (; x + 3 * NG < a.splits; x += 4 * NG) {
    const float o0 = O[(size_t)x * D], o1 = O[(size_t)(x + NG) * D];
    const float o2 = O[(size_t)(x + 2 * NG) * D], o3 = O[(size_t)(x + 3 * NG) * D];
    acc = fmaf(wts[x], o0, acc);
    acc = fmaf(wts[x + NG], o1, acc);
    acc = fmaf(wts[x + 2 * NG], o2, acc);
    acc = fmaf(wts[x + 3 * NG], o3, acc);
  }
  for (; x < a.splits; x += NG) acc = fmaf(wts[x], O[(size_t)x * D], acc);
  part[sg][d] = acc;
  __syncthreads();
  if (sg == 0) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) sum += part[q][d];
    const float val = tot > 0.f ? sum / tot : 0.f;
    a.out[(size_t)bh * D + d] = (uint16_t)(T::pack2(val, 0.f) & 0xffffu);
    if (d == 0 && a.lse) a.lse[bh] = tot > 0.f ? M + __logf(tot) : kNegInf;
  }
}

}  // namespace sa
