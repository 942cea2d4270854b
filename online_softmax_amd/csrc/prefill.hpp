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
//  * key/value tiles of 64 rows are copied from global memory straight into
//    LDS (buffer loads with the LDS destination, 16 bytes per lane), double-
//    buffered: the copies for tile t+1 are issued before tile t is computed
//    and land in the other buffer, so one barrier per tile suffices; the
//    buffer bounds return zeros past the last key;
//  * LDS rows are unpadded; 16-byte chunks are placed at (chunk XOR f(row))
//    so that the K reads (16 rows, one chunk) and the transposed V reads
//    (4 consecutive rows, 4 chunks) each touch distinct banks;
//  * scores are computed transposed, S^T = K Q^T, with 32x32x16 MFMAs: the
//    accumulator then holds one query per lane (keys along the registers and
//    across the two wave halves), so row statistics are per-lane values plus
//    one exchange between the wave halves, and the probabilities already sit
//    in the B-operand layout of the next product O^T += V^T P^T;
//  * V stays row-major in LDS and is read transposed with ds_read_b64_tr_b16;
//  * exponentials are base 2 on the hardware exp unit with log2(e) folded into
//    the score scale; the running maximum lives in that base-2 domain;
//  * tiles that no rule hides any key of (the bulk of the sweep) take a path
//    without masking arithmetic; tiles on the causal diagonal, the ragged end
//    of the keys or with hidden padded keys take the masked path;
//  * the reference maximum is raised only when a tile's maximum exceeds it by
//    more than kRescaleSlack (base 2): the final out = numerator / denominator
//    and lse = reference + log(denominator) are exact for any reference, and
//    the slack bounds every probability by 2^kRescaleSlack, so most tiles skip
//    rescaling the output accumulator.
#pragma once
#include "common.hpp"

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
  int nmb;       // query blocks of 128 rows per (batch, head)
  int nitems;    // B * H_q * nmb
};

// Chunk swizzle of LDS row r (16-byte chunks, D / 8 per row).
template <int D>
__device__ inline int lds_swizzle(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <class T, int D, bool CAUSAL, bool MASK, bool ALIBI>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  constexpr int BM = 128;            // query rows per workgroup
  constexpr int BN = 64;             // keys per tile
  constexpr int KK = D / 16;         // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int NI = BN * D / 2048;  // 1 KiB copies per wave per tensor per tile

  __shared__ __attribute__((aligned(1024))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[2][BN * D];
  __shared__ uint32_t Ms[2][BN / 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // A negative scale is applied as |scale| on negated Q (exact in fp16/bf16),
  // so the row maximum of the raw products is the maximum of the scaled ones.
  u32x4 qreg[KK];
  const bool qvalid = qi < a.S_q;
  const uint32_t qflip = a.scale2 < 0.f ? 0x80008000u : 0u;
  const float sc2 = __builtin_fabsf(a.scale2);
  {
    const uint16_t* qp = a.q + ((size_t)(b * (size_t)a.S_q + (qvalid ? qi : 0)) * a.H_q + h) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qreg[kk] = qvalid ? *(const u32x4*)(qp + 16 * kk) : (u32x4){0, 0, 0, 0};
      qreg[kk] ^= qflip;
    }
  }

  const size_t rs = (size_t)a.H_kv * D;  // key/value row stride
  const uint16_t* kb = a.k + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint16_t* vb = a.v + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint8_t* mrow = MASK ? a.mask + (size_t)b * a.S_k : nullptr;

  // Copy u of this wave fills LDS bytes [cb KiB, cb KiB + 1 KiB), cb = 4u + w;
  // lane l's 16 bytes are LDS row r, position p, holding global chunk p ^ f(r).
  uint32_t voff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int byte = (4 * u + w) * 1024 + 16 * lane;
    const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
    voff[u] = (uint32_t)(r * rs * 2 + 16 * (p ^ lds_swizzle<D>(r)));
  }
  auto issue_tile = [&](int n0, int buf) {
    const int rows = min(BN, a.S_k - n0);
    const uint32_t bytes = (uint32_t)((rows - 1) * rs * 2 + 2 * D);
    const auto rk = buffer_rsrc(kb + (size_t)n0 * rs, bytes);
    const auto rv = buffer_rsrc(vb + (size_t)n0 * rs, bytes);
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      load_lds16(rk, &Ks[buf][(4 * u + w) * 512], voff[u]);
      load_lds16(rv, &Vs[buf][(4 * u + w) * 512], voff[u]);
    }
  };
  uint32_t mst = 0;
  auto load_mask = [&](int n0) {
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
  auto store_mask = [&](int buf) {
    if (MASK && tid < BN / 4) Ms[buf][tid] = mst;
  };

  float m_ref = kNegInf;  // reference maximum, base-2 domain (raised lazily)
  float l_run = 0.f;      // this lane's share of the running row sum
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};

  const float slope2 = ALIBI ? a.slopes[h] * kLog2e : 0.f;
  const int wrow0 = m0 + 32 * w;                       // first row of this wave
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

  // One tile: scores, softmax update and output accumulation.  MASKED selects
  // the path that applies the causal rule, the end of the keys and the
  // padding mask; otherwise every key of the tile is visible to every row.
  auto tile = [&](auto masked_tag, const int buf, const int n0) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const u32x4 ak = *(const u32x4*)&Ks[buf][(32 * jb + li) * D + 8 * ((2 * kk + g) ^ ksw)];
        s[jb] = T::mma(ak, qreg[kk], s[jb]);
      }
    }
    // Register r of block jb holds key n0 + 32 jb + 8 (r/4) + 4 g + r%4.
    uint32_t mw[2][4];
    if (MASKED && MASK) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) mw[jb][q4] = Ms[buf][8 * jb + 2 * q4 + g];
    }
    auto visible = [&](int jb, int r) {
      const int kofs = 32 * jb + 8 * (r >> 2) + (r & 3);
      const int kj = n0 + 4 * g + kofs;
      bool vis = kj < a.S_k;
      if (CAUSAL) vis = vis && kj <= ipos;
      if (MASK) vis = vis && ((mw[jb][r >> 2] >> (8 * (r & 3))) & 0xffu) != 0;
      return vis;
    };
    float tmax = kNegInf;
    if (!ALIBI) {
      // Raw products; the scale enters once, in the exponent's fma.
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (MASKED) s[jb][r] = visible(jb, r) ? s[jb][r] : kNegInf;
          tmax = fmaxf(tmax, s[jb][r]);
        }
      tmax = max_halves(tmax) * sc2;
    } else {
      // Scaled score plus bias -slope * |ipos - key|.  Under the causal rule
      // every visible key satisfies key <= ipos, so the bias is linear there.
      const float rel0 = (float)(ipos - n0 - 4 * g);
      const float bb = -slope2 * rel0;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float kofs = (float)(32 * jb + 8 * (r >> 2) + (r & 3));
          const float bias = CAUSAL ? fmaf(slope2, kofs, bb) : -slope2 * __builtin_fabsf(rel0 - kofs);
          float t = fmaf(s[jb][r], sc2, bias);
          if (MASKED) t = visible(jb, r) ? t : kNegInf;
          s[jb][r] = t;
          tmax = fmaxf(tmax, t);
        }
      tmax = max_halves(tmax);
    }
    // Raise the reference maximum only when some row's tile maximum exceeds
    // it by more than the slack; rows that need no change get alpha = 1.
    if (wave_any(tmax > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    // While a row has seen no visible key its reference is 0, so that no
    // exp(-inf - (-inf)) is formed (only masked tiles can meet such a row).
    const float m_use = (MASKED && m_ref == kNegInf) ? 0.f : m_ref;
    const float nm = -m_use;
    float psum = 0.f;
    uint32_t pk[2][8];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0, p1;
        if (!ALIBI) {
          p0 = fast_exp2(fmaf(s[jb][r], sc2, nm));
          p1 = fast_exp2(fmaf(s[jb][r + 1], sc2, nm));
        } else {
          p0 = fast_exp2(s[jb][r] + nm);
          p1 = fast_exp2(s[jb][r + 1] + nm);
        }
        psum += p0 + p1;
        pk[jb][r >> 1] = T::pack2(p0, p1);
      }
    }
    l_run += psum;

    // O^T += V^T P^T over four 16-key steps.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int jb = ks >> 1, mh = ks & 1;
      const u32x4 bp = {pk[jb][4 * mh], pk[jb][4 * mh + 1], pk[jb][4 * mh + 2], pk[jb][4 * mh + 3]};
      const uint16_t* vt = &Vs[buf][16 * ks * D];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = lds_read_tr(vt + vofs[0][db]);
        const u32x2 hi = lds_read_tr(vt + vofs[1][db]);
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = T::mma(av, bp, o[db]);
      }
    }
  };

  if (nt > 0) {
    issue_tile(0, 0);
    load_mask(0);
    store_mask(0);
  }
  wait_vmem();
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1, n0 = t * BN;
    if (t + 1 < nt) {
      issue_tile(n0 + BN, buf ^ 1);
      load_mask(n0 + BN);
    }
    const bool skip = !wave_active || (CAUSAL && n0 > wave_last);
    if (!skip) {
      bool fast = n0 + BN <= a.S_k && (!CAUSAL || n0 + BN - 1 <= wrow0 + off);
      if (MASK && fast) fast = !wave_any(Ms[buf][lane & 15] != 0x01010101u);
      if (fast)
        tile(std::false_type{}, buf, n0);
      else
        tile(std::true_type{}, buf, n0);
    }
    if (t + 1 < nt) store_mask(buf ^ 1);
    wait_vmem();
    __syncthreads();
  }

  // Epilogue: out = O / l (0 for a row that saw no key), lse = ln of the sum.
  const float l_tot = sum_halves(l_run);
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
      a.lse[((size_t)b * a.H_q + h) * a.S_q + qi] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace sa
