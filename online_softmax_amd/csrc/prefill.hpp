// Prefill kernel: exact attention forward in one streaming sweep over key/value
// tiles with float32 running row maximum and row sum (online softmax), as the
// "StreamAttention: Fused Online Softmax Attention" page describes in section
// "Kernel Design (Fused Online Softmax)": per key tile, raise the running
// maximum, rescale the running numerator and denominator by
// exp(old_max - new_max), add exp(score - new_max) and its product with V;
// finish with numerator / denominator and lse = max + log(denominator).
//
// Mapping onto gfx950:
//  * a workgroup of four waves owns 128 query rows of one (batch, head); each
//    wave owns 32 rows and keeps their Q slice in registers for the whole sweep;
//  * key/value tiles of 64 rows are staged through LDS, double-buffered: the
//    global loads for tile t+1 are issued before tile t is computed and land
//    in the other buffer afterwards, so one barrier per tile suffices;
//  * scores are computed transposed, S^T = K Q^T, with 32x32x16 MFMAs: the
//    accumulator then holds one query per lane (keys along the registers and
//    across the two wave halves), so row statistics are per-lane values plus
//    one exchange between the wave halves, and the probabilities already sit
//    in the B-operand layout of the next product O^T += V^T P^T;
//  * V stays row-major in LDS and is read transposed with ds_read_b64_tr_b16;
//  * exponentials are base 2 on the hardware exp unit with log2(e) folded into
//    the score scale; the running maximum lives in that base-2 domain.
#pragma once
#include "common.hpp"

namespace sa {

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
  int nmb;       // query blocks of 128 rows per (batch, head)
  int nitems;    // B * H_q * nmb
};

template <class T, int D, bool CAUSAL, bool MASK, bool ALIBI>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  constexpr int BM = 128;            // query rows per workgroup
  constexpr int BN = 64;             // keys per tile
  constexpr int KSTR = D + 8;        // K row stride in LDS (16-bit words)
  constexpr int VSTR = D + 32;       // V row stride in LDS
  constexpr int KK = D / 16;         // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int CPT = BN * D / 8 / 256;  // 16-byte chunks per thread per tile
  constexpr int RCH = D / 8;         // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * VSTR];
  __shared__ uint32_t Ms[2][BN / 4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, g = lane >> 5;

  const int item = xcd_contiguous(blockIdx.x, a.nitems);
  const int bh = item / a.nmb, mbi = item - bh * a.nmb;
  // Causal blocks are issued heaviest (last rows) first.
  const int mb = CAUSAL ? a.nmb - 1 - mbi : mbi;
  const int b = bh / a.H_q, h = bh - b * a.H_q, hk = h / a.G;
  const int m0 = mb * BM;
  const int off = a.S_k - a.S_q;  // bottom-right alignment of the causal rule
  const int qi = m0 + 32 * w + li;
  const int ipos = qi + off;      // this row's position on the key axis

  int n_end = a.S_k;
  if (CAUSAL) n_end = min(n_end, m0 + BM + off);
  const int nt = n_end > 0 ? (n_end + BN - 1) / BN : 0;

  // Q^T as the B operand: lane (row li, half g) holds q[row][16kk + 8g .. +7].
  u32x4 qreg[KK];
  const bool qvalid = qi < a.S_q;
  {
    const uint16_t* qp = a.q + ((size_t)(b * (size_t)a.S_q + (qvalid ? qi : 0)) * a.H_q + h) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = qvalid ? *(const u32x4*)(qp + 16 * kk) : (u32x4){0, 0, 0, 0};
  }

  const size_t rs = (size_t)a.H_kv * D;  // key/value row stride
  const uint16_t* kb = a.k + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint16_t* vb = a.v + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint8_t* mrow = MASK ? a.mask + (size_t)b * a.S_k : nullptr;

  u32x4 kst[CPT], vst[CPT];
  uint32_t mst = 0;
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u, row = c / RCH, col = (c % RCH) * 8;
      const bool ok = n0 + row < a.S_k;
      const size_t go = (size_t)(ok ? n0 + row : 0) * rs + col;
      kst[u] = ok ? *(const u32x4*)(kb + go) : (u32x4){0, 0, 0, 0};
      vst[u] = ok ? *(const u32x4*)(vb + go) : (u32x4){0, 0, 0, 0};
    }
    if (MASK && tid < BN / 4) {
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = n0 + 4 * tid + e;
        m |= (uint32_t)((j < a.S_k && mrow[j] != 0) ? 1u : 0u) << (8 * e);
      }
      mst = m;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u, row = c / RCH, col = (c % RCH) * 8;
      *(u32x4*)&Ks[buf][row * KSTR + col] = kst[u];
      *(u32x4*)&Vs[buf][row * VSTR + col] = vst[u];
    }
    if (MASK && tid < BN / 4) Ms[buf][tid] = mst;
  };

  float m_run = kNegInf;  // running row maximum, base-2 domain
  float l_run = 0.f;      // this lane's share of the running row sum
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};

  const float slope2 = ALIBI ? a.slopes[h] * kLog2e : 0.f;
  const int wrow0 = m0 + 32 * w;                       // first row of this wave
  const bool wave_active = wrow0 < a.S_q;
  const int wave_last = min(wrow0 + 31, a.S_q - 1) + off;  // furthest key the wave may see

  // Lane constants of the transposed V read (see lds_read_tr).
  const int tr_key = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1, n0 = t * BN;
    if (t + 1 < nt) load_tile(n0 + BN);
    const bool skip = !wave_active || (CAUSAL && n0 > wave_last);
    if (!skip) {
      // S^T = K Q^T for two 32-key blocks.
      f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const u32x4 ak = *(const u32x4*)&Ks[buf][(32 * jb + li) * KSTR + 16 * kk + 8 * g];
          s[jb] = T::mma(ak, qreg[kk], s[jb]);
        }
      }
      // Register r of block jb holds key n0 + 32 jb + 8 (r/4) + 4 g + r%4.
      const bool need_mask = MASK || (n0 + BN > a.S_k) || (CAUSAL && n0 + BN - 1 > wrow0 + off);
      const float rel0 = (float)(ipos - n0 - 4 * g);  // ipos - key for r = 0, jb = 0
      float mx = kNegInf;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        uint32_t mw[4] = {~0u, ~0u, ~0u, ~0u};
        if (MASK) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) mw[q4] = Ms[buf][8 * jb + 2 * q4 + g];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kofs = 32 * jb + 8 * (r >> 2) + (r & 3);  // key - n0 - 4g
          float x = s[jb][r] * a.scale2;
          if (ALIBI) x = fmaf(-slope2, __builtin_fabsf(rel0 - (float)kofs), x);
          if (need_mask) {
            const int kj = n0 + 4 * g + kofs;
            bool vis = kj < a.S_k;
            if (CAUSAL) vis = vis && kj <= ipos;
            if (MASK) vis = vis && ((mw[r >> 2] >> (8 * (r & 3))) & 0xffu) != 0;
            x = vis ? x : kNegInf;
          }
          s[jb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      // While a row has seen no visible key its reference point is 0, so that
      // no exp(-inf - (-inf)) is ever formed.
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
      uint32_t pk[2][8];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(s[jb][r] - m_use);
          const float p1 = fast_exp2(s[jb][r + 1] - m_use);
          psum += p0 + p1;
          pk[jb][r >> 1] = T::pack2(p0, p1);
        }
      }
      l_run = fmaf(l_run, alpha, psum);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;

      // O^T += V^T P^T over four 16-key steps.
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int jb = ks >> 1, mh = ks & 1;
        const u32x4 bp = {pk[jb][4 * mh], pk[jb][4 * mh + 1], pk[jb][4 * mh + 2], pk[jb][4 * mh + 3]};
        const uint16_t* vrow0 = &Vs[buf][(16 * ks + tr_key) * VSTR + tr_col];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 lo = lds_read_tr(vrow0 + 32 * db);
          const u32x2 hi = lds_read_tr(vrow0 + 8 * VSTR + 32 * db);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = T::mma(av, bp, o[db]);
        }
      }
    }
    if (t + 1 < nt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: out = O / l (0 for a row that saw no key), lse = ln of the sum.
  const float l_tot = l_run + swap_halves(l_run);
  if (qvalid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
    if (g == 0 && a.lse)
      a.lse[((size_t)b * a.H_q + h) * a.S_q + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace sa
