// Backward kernels: gradients dq, dk, dv of the attention output.
//
// The single-sweep backward of the "StreamAttention: Fused Online Softmax
// Attention" page ("Recent Updates": recompute the score tiles from the saved
// lse and stream dQ, dK and dV without materialising the attention matrix),
// whose quantities the "flash-attn-volta" page checks in "Backward
// correctness".  With P = exp(s - lse) over the visible keys of each row:
//
//   Di = <dout_i, out_i>,  dP = dout V^T,  dS = P (dP - Di),
//   dv = P^T dout,  dq = scale dS K,  dk = scale dS^T q.
//
// Two kernels, so that every gradient is summed in registers in a fixed
// order (no atomics, bit-reproducible):
//  * bwd_dq_kernel: the forward's layout (a workgroup of 4 waves owns 128
//    query rows of one (batch, head); K/V tiles of 64 keys stream through LDS
//    with direct buffer-to-LDS copies; S^T = K Q^T puts one query per lane):
//    P^T from the saved lse, dP^T = V dO^T with dO held in registers like Q,
//    dQ^T += K^T dS^T with K read transposed from LDS.  It first forms, for
//    its rows, Di = <dout_i, out_i> and the lse in base 2 (+inf for a row
//    with no visible key, so that its probabilities are 0), and stores them
//    as one float2 per row for the next kernel;
//  * bwd_dkdv_kernel: a workgroup of 4 waves owns 128 keys of one (batch,
//    KV head), each wave 32 keys whose K and V rows stay in registers; tiles
//    of 32 query rows of every query head sharing that KV head stream
//    through LDS (Q, dO, and the rows' lse and Di; from the last tile down
//    to the block's diagonal), S = Q K^T puts one key per lane, and
//    dV^T += dO^T P and dK^T += Q^T dS accumulate over all of them, so the
//    grouped heads' contributions sum in registers.
#pragma once
#include "common.hpp"

namespace sa {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;     // [B, H_q, S_q], natural log
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const uint8_t* mask;
  const float* slopes;
  float2* ld;           // workspace [B, H_q, S_q]: {lse * log2(e) or +inf, Di},
                        // written by the dq kernel, read by the dk/dv kernel
  int B, S_q, S_k, H_q, H_kv, G;
  float scale;          // signed
  float scale2;         // |scale| * log2(e)
  float alibi2;         // 1 / |scale|
  int nqb;              // query blocks of 128 rows per (batch, head)   (dq kernel)
  int nkb;              // key blocks of 128 keys per (batch, KV head)  (dk/dv kernel)
  // dq and dk/dv kernels: the number of CUs when the kernel's causal grid is
  // resident at two workgroups per CU (workgroups j and j + pair_ncu share a
  // CU), else 0.
  int pair_ncu;
  int pair_ncu_kv;
};

template <int D>
__device__ inline int bwd_swizzle(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// ---------------------------------------------------------------------------
// dq: 4 waves x 32 query rows; key/value tiles of 64 keys.
template <class T, int D, bool CAUSAL, bool MASK, bool ALIBI>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = 4, BM = 32 * NW, BN = 64, NS = 2;
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int NI = BN * D * 2 / 1024 / NW;  // 1 KiB copies per wave per tensor per tile
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[NS][BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[NS][BN * D];
  __shared__ int Pw[MASK ? NW : 1];  // per-wave first cleared key

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  int bh, mb;
  if (CAUSAL && a.pair_ncu > 0) {
    // As in the forward: workgroups j and j + pair_ncu share a CU and take
    // blocks nqb - 1 - l and l of one head.
    const int ncu = a.pair_ncu, j = blockIdx.x;
    const int p = j < ncu ? j : j - ncu;
    const int nbh = a.B * a.H_q;
    bh = p % nbh;
    const int lvl = p / nbh;
    mb = j < ncu ? a.nqb - 1 - lvl : lvl;
  } else {
    const int item = xcd_contiguous(blockIdx.x, a.B * a.H_q * a.nqb);
    bh = item / a.nqb;
    const int mbi = item - bh * a.nqb;
    mb = CAUSAL ? a.nqb - 1 - mbi : mbi;  // heaviest blocks first
  }
  const int b = bh / a.H_q, h = bh - b * a.H_q, hk = h / a.G;
  const int m0 = mb * BM;
  const int off = a.S_k - a.S_q;
  const int qi = m0 + 32 * w + li;
  const int ipos = qi + off;
  const bool qvalid = qi < a.S_q;

  int n_end = a.S_k;
  if (CAUSAL) n_end = min(n_end, m0 + BM + off);
  const int nt = n_end > 0 ? (n_end + BN - 1) / BN : 0;

  const size_t rs = (size_t)a.H_kv * D;
  const uint16_t* kb = a.k + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint16_t* vb = a.v + ((size_t)b * a.S_k * a.H_kv + hk) * D;
  const uint8_t* mrow = MASK ? a.mask + (size_t)b * a.S_k : nullptr;

  uint32_t voff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int byte = (NW * u + w) * 1024 + 16 * lane;
    const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
    voff[u] = (uint32_t)(r * rs * 2 + 16 * (p ^ bwd_swizzle<D>(r)));
  }
  auto issue = [&](const uint16_t* base, uint16_t* buf, int t) {
    const int n0 = t * BN, rows = min(BN, a.S_k - n0);
    const auto r = buffer_rsrc(base + (size_t)n0 * rs, (uint32_t)((rows - 1) * rs * 2 + 2 * D));
#pragma unroll
    for (int u = 0; u < NI; ++u) load_lds16(r, buf + (NW * u + w) * 512, voff[u]);
  };
  if (nt > 0) {
    issue(kb, Ks[0], 0);
    issue(vb, Vs[0], 0);
  }

  // Q (sign-flipped for a negative scale) and dO as B operands: lane (row li,
  // half g) holds [row][16 kk + 8 g .. +7].
  const uint32_t qflip = a.scale < 0.f ? 0x80008000u : 0u;
  u32x4 qreg[KK], doreg[KK];
  float l2 = __builtin_huge_valf(), di = 0.f;
  {
    const size_t rowo = ((size_t)(b * (size_t)a.S_q + (qvalid ? qi : 0)) * a.H_q + h) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qreg[kk] = qvalid ? *(const u32x4*)(a.q + rowo + 16 * kk) : (u32x4){0, 0, 0, 0};
      qreg[kk] ^= qflip;
      doreg[kk] = qvalid ? *(const u32x4*)(a.dout + rowo + 16 * kk) : (u32x4){0, 0, 0, 0};
    }
    // Di = <dout_i, out_i> (each half of the row on one lane half, summed in
    // a fixed order) and the lse in base 2, stored for the dk/dv kernel.
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 o4 = qvalid ? *(const u32x4*)(a.out + rowo + 16 * kk) : (u32x4){0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 of = T::unpack2(o4[e]), df = T::unpack2(doreg[kk][e]);
        acc = fmaf(of[0], df[0], acc);
        acc = fmaf(of[1], df[1], acc);
      }
    }
    acc += __shfl_xor(acc, 32);
    if (qvalid) {
      const size_t x = ((size_t)b * a.H_q + h) * a.S_q + qi;
      const float l = a.lse[x];
      l2 = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
      di = acc;
      if (g == 0) a.ld[x] = make_float2(l2, di);
    }
  }
  const float sc2 = a.scale2;
  const float slope_acc = ALIBI ? a.slopes[h] * a.alibi2 : 0.f;
  // The first key the padding mask clears among the keys of the sweep (S_k
  // if none): only tiles reaching it read mask bytes.  Each lane checks 16
  // consecutive keys per round, all loads in flight together; the minimum
  // goes over the wave by shuffles and over the waves through LDS.
  int pad_start = a.S_k;
  if (MASK) {
    const auto mr = buffer_rsrc_t(mrow, (uint32_t)a.S_k);
    int first = a.S_k;
    for (int j0 = 16 * (64 * w + lane); j0 < nt * BN; j0 += 16 * 64 * NW) {
      uint32_t kept[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) kept[e] = __builtin_amdgcn_raw_buffer_load_b8(mr, (uint32_t)(j0 + e), 0, 0);
#pragma unroll
      for (int e = 15; e >= 0; --e) first = kept[e] == 0 ? min(first, j0 + e) : first;
    }
#pragma unroll
    for (int k = 32; k > 0; k >>= 1) first = min(first, __shfl_xor(first, k));
    if (lane == 0) Pw[w] = first;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NW; ++x) pad_start = min(pad_start, Pw[x]);
    pad_start = __builtin_amdgcn_readfirstlane(pad_start);
  }
  // Everything read into registers above has landed before the sweep.  The
  // tile copies are inline assembly the compiler does not count, so a wait
  // it placed inside the loop for these loads would wait for the copies in
  // flight too.
  wait_vmem();
  const int wrow0 = m0 + 32 * w;
  const int wave_last = min(wrow0 + 31, a.S_q - 1) + off;
  int ntw = wrow0 < a.S_q ? nt : 0;
  if (CAUSAL) ntw = wave_last < 0 ? 0 : min(ntw, wave_last / BN + 1);

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = (f32x16){};

  const int ksw = bwd_swizzle<D>(li);
  const int tr_key = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int tofs[2][DB];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r = 8 * q2 + tr_key;
      tofs[q2][db] = r * D + 8 * ((4 * db + (tr_col >> 3)) ^ bwd_swizzle<D>(r)) + (tr_col & 7);
    }

  for (int t = 0; t < nt; ++t) {
    // Tile t is in buffer t % 2, and its copies are the only ones in flight.
    // After the barrier every wave has finished tile t - 1, so tile t + 1
    // goes into that buffer while tile t is worked on: one barrier per tile.
    wait_vmem();
    __syncthreads();
    if (t + 1 < nt) {
      issue(kb, Ks[(t + 1) % NS], t + 1);
      issue(vb, Vs[(t + 1) % NS], t + 1);
    }
    if (t < ntw) {
      const uint16_t* kt = Ks[t % NS];
      const uint16_t* vt = Vs[t % NS];
      const int n0 = t * BN;
      // S^T and dP^T for keys n0 + 32 jb + 8 (r/4) + 4 g + r%4 of this lane's row.
      f32x16 s[2], dp[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        if (ALIBI) {
          const float b0 = slope_acc * (float)(n0 + 4 * g - ipos);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float kofs = (float)(32 * jb + 8 * (r >> 2) + (r & 3));
            s[jb][r] = CAUSAL ? fmaf(slope_acc, kofs, b0) : -slope_acc * __builtin_fabsf(fmaf(1.f, kofs, (float)(n0 + 4 * g - ipos)));
          }
        } else {
          s[jb] = (f32x16){};
        }
        dp[jb] = (f32x16){};
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int off16 = (32 * jb + li) * D + 8 * ((2 * kk + g) ^ ksw);
          s[jb] = T::mma(*(const u32x4*)&kt[off16], qreg[kk], s[jb]);
          dp[jb] = T::mma(*(const u32x4*)&vt[off16], doreg[kk], dp[jb]);
        }
      const bool padded = MASK && n0 + BN > pad_start;
      const bool masked = n0 + BN > a.S_k || (CAUSAL && n0 + BN - 1 > wrow0 + off) || padded;
      // Padding bits of the tile's 64 keys (the same for every row): lane l
      // reads the byte of key n0 + l, one ballot gathers them (bit l kept),
      // shifted to this lane's half (keys from 4 g on).
      uint64_t keep = ~uint64_t(0);
      if (padded) {
        const int kl = n0 + lane;
        const bool kept = kl < a.S_k && mrow[kl < a.S_k ? kl : 0] != 0;
        keep = __builtin_amdgcn_ballot_w64(kept) >> (4 * g);
      }
      // Tiles that no rule hides any key of skip the masking pass.
      if (masked) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 32 * jb + 8 * (r >> 2) + (r & 3);  // from n0 + 4 g
            const int kj = n0 + 4 * g + ko;
            bool vis = kj < a.S_k;
            if (CAUSAL) vis = vis & (kj <= ipos);
            if (MASK) vis = vis & (((keep >> ko) & 1u) != 0);
            s[jb][r] = vis ? s[jb][r] : kNegInf;
          }
      }
      uint32_t pk[2][8];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float ds[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float p = fast_exp2(fmaf(s[jb][r + e], sc2, -l2));
            ds[e] = p * (dp[jb][r + e] - di);
          }
          pk[jb][r >> 1] = T::pack2(ds[0], ds[1]);
        }
      // dQ^T += K^T dS^T over four 16-key steps (K read transposed).
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int jb = ks >> 1, mh = ks & 1;
        const u32x4 bp = {pk[jb][4 * mh], pk[jb][4 * mh + 1], pk[jb][4 * mh + 2], pk[jb][4 * mh + 3]};
        const uint16_t* kt16 = kt + 16 * ks * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 lo = lds_read_tr(kt16 + tofs[0][db]);
          const u32x2 hi = lds_read_tr(kt16 + tofs[1][db]);
          dq[db] = T::mma((u32x4){lo[0], lo[1], hi[0], hi[1]}, bp, dq[db]);
        }
      }
    }
  }

  if (qvalid) {
    uint16_t* op = a.dq + ((size_t)(b * (size_t)a.S_q + qi) * a.H_q + h) * D + 4 * g;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 pr = {T::pack2(dq[db][4 * q4] * sc, dq[db][4 * q4 + 1] * sc),
                          T::pack2(dq[db][4 * q4 + 2] * sc, dq[db][4 * q4 + 3] * sc)};
        *(u32x2*)(op + 32 * db + 8 * q4) = pr;
      }
  }
}

// ---------------------------------------------------------------------------
// dk, dv: 4 waves x 32 keys; tiles of 32 query rows of every query head of
// the KV head.
template <class T, int D, bool CAUSAL, bool MASK, bool ALIBI>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 4, BK = 32 * NW, BQ = 32, NS = 3;
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int NI = BQ * D * 2 / 1024;  // 1 KiB copies per tensor per tile (all by one wave each)
  // Q and dO tiles of one buffer side by side, so that a dO fragment is read
  // at its Q fragment's address plus a constant (the reads' offset field).
  __shared__ __attribute__((aligned(1024))) uint16_t QOs[NS][2][BQ * D];
  __shared__ __attribute__((aligned(256))) float2 Ls[NS][BQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  int bk, kblk;
  if (CAUSAL && a.pair_ncu_kv > 0) {
    // The whole grid is resident, two workgroups per CU: workgroups j and
    // j + pair_ncu_kv share a CU and take key blocks lvl and nkb - 1 - lvl of
    // one KV head, so that every CU carries the same number of query rows.
    const int ncu = a.pair_ncu_kv, j = blockIdx.x;
    const int p = j < ncu ? j : j - ncu;
    const int nbk = a.B * a.H_kv;
    bk = p % nbk;
    const int lvl = p / nbk;
    kblk = j < ncu ? lvl : a.nkb - 1 - lvl;
  } else {
    const int item = xcd_contiguous(blockIdx.x, a.B * a.H_kv * a.nkb);
    bk = item / a.nkb;
    kblk = item - bk * a.nkb;  // under the causal rule the first key blocks carry the most rows
  }
  const int b = bk / a.H_kv, hk = bk - b * a.H_kv;
  const int k0 = kblk * BK;
  const int kj = k0 + 32 * w + li;  // this lane's key
  const int off = a.S_k - a.S_q;
  const bool kvalid = kj < a.S_k;
  const bool key_ok = kvalid && (!MASK || a.mask[(size_t)b * a.S_k + kj] != 0);
  const bool wave_masked = wave_any(!key_ok);

  // Query tiles that can see a key of this block: rows i with i + off >= k0.
  const int nqt = (a.S_q + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? min(nqt, max(0, (k0 - off) / BQ)) : 0;
  const int per_head = nqt - qt0;
  const int niter = per_head * a.G;
  // Iteration it takes query head gi = it / per_head and, within it, the
  // query tiles from the last one down to qt0: every workgroup of a KV head
  // starts on the same (last) tiles, so their reads of Q and dO meet in L2
  // (from the diagonal up, each would start on a tile of its own).
  auto qtile = [&](const int it, const int gi) { return nqt - 1 - (it - gi * per_head); };

  const size_t qrs = (size_t)a.H_q * D;  // q / dout row stride
  // Tile copies: wave 0 copies Q, wave 1 copies dO, wave 2 the rows' {lse2, Di}.
  // Copy u of a lane fills LDS row r, position p, from global chunk
  // p ^ f(r); the offsets are recomputed at each tile (from a lane index the
  // compiler cannot see through) rather than held in registers for the whole
  // sweep.  The swizzle f repeats every 16 rows, which is every P = D / 32
  // copies: copy u is copy u mod P of the lane, u / P times 16 rows further
  // on, so only P offsets are formed and the rest add a scalar.
  auto toff = [&](const int ln, const int u) -> uint32_t {
    const int byte = u * 1024 + 16 * ln;
    const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
    return (uint32_t)(r * qrs * 2 + 16 * (p ^ bwd_swizzle<D>(r)));
  };
  auto issue = [&](int it) {
    const int gi = it / per_head, qt = qtile(it, gi);
    const int h = hk * a.G + gi;
    const int i0 = qt * BQ, rows = min(BQ, a.S_q - i0);
    const int buf = __builtin_amdgcn_readfirstlane(it % NS);
    if (w == 0 || w == 1) {
      const uint16_t* base = (w == 0 ? a.q : a.dout) + (((size_t)b * a.S_q + i0) * a.H_q + h) * D;
      const auto r = buffer_rsrc(base, (uint32_t)((rows - 1) * qrs * 2 + 2 * D));
      uint16_t* dst = QOs[buf][w];
      int ln = lane;
      __asm__ volatile("" : "+v"(ln));
      constexpr int P = D / 32;
      static_assert(NI % P == 0 && 1024 * P == 16 * 2 * D, "P copies span 16 rows");
      uint32_t o0[P];
#pragma unroll
      for (int c = 0; c < P; ++c) o0[c] = toff(ln, c);
#pragma unroll
      for (int u = 0; u < NI; ++u)
        load_lds16(r, dst + u * 512, o0[u % P] + (uint32_t)(u / P) * (uint32_t)(32 * qrs));
    } else if (w == 2) {
      // BQ float2 = 256 bytes: 16 lanes of 16 bytes (the others would write
      // past Ls[buf]); rows past S_q read zero.
      const auto r = buffer_rsrc(a.ld + ((size_t)b * a.H_q + h) * a.S_q + i0, (uint32_t)(rows * 8));
      if (lane < BQ * 8 / 16) load_lds16(r, &Ls[buf][0], 16 * lane);
    }
  };

  // K (sign-flipped for a negative scale) and V rows of this lane's key as B
  // operands: lane (key li, half g) holds [key][16 kk + 8 g .. +7].
  const uint32_t kflip = a.scale < 0.f ? 0x80008000u : 0u;
  u32x4 kreg[KK], vreg[KK];
  {
    const size_t rowk = ((size_t)(b * (size_t)a.S_k + (kvalid ? kj : 0)) * a.H_kv + hk) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kreg[kk] = kvalid ? *(const u32x4*)(a.k + rowk + 16 * kk) : (u32x4){0, 0, 0, 0};
      kreg[kk] ^= kflip;
      vreg[kk] = kvalid ? *(const u32x4*)(a.v + rowk + 16 * kk) : (u32x4){0, 0, 0, 0};
    }
  }
  // These rows (and the mask byte above) have landed before the sweep: the
  // tile copies are inline assembly the compiler does not count, so a wait
  // it placed inside the loop for these loads would wait for the copies in
  // flight too.
  wait_vmem();
  const float sc2 = a.scale2;
  const int kw0 = k0 + 32 * w;  // first key of this wave

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = (f32x16){};
    dv[db] = (f32x16){};
  }

  const int tr_key = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int tofs[2][DB];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r = 8 * q2 + tr_key;
      tofs[q2][db] = r * D + 8 * ((4 * db + (tr_col >> 3)) ^ bwd_swizzle<D>(r)) + (tr_col & 7);
    }
  const int rsw = bwd_swizzle<D>(li);

  // ALiBi slope of the tile's query head, read when the head changes.
  int slope_head = -1;
  float slope_acc = 0.f;
  // Three buffers, one barrier per tile: tile it + 2 is copied right after
  // the barrier of tile it, into the buffer of tile it - 1, which every wave
  // finished reading before that barrier; the copies of two tiles are in
  // flight under each tile's work.
  if (niter > 0) issue(0);
  if (niter > 1) issue(1);
  for (int it = 0; it < niter; ++it) {
    // Tile it has landed once at most the copies of tile it + 1 (issued
    // after it) are in flight.
    if (it + 1 < niter) {
      if (w <= 1) wait_vmem_n<NI>();
      else if (w == 2) wait_vmem_n<1>();
    } else {
      wait_vmem();
    }
    __syncthreads();
    if (it + 2 < niter) issue(it + 2);
    const int gi = it / per_head, qt = qtile(it, gi);
    const int h = hk * a.G + gi;
    const int i0 = qt * BQ;
    // Rows of this tile that see none of the wave's keys contribute nothing;
    // a tile whose rows all end before the wave's first key is skipped.
    const bool active = !CAUSAL || i0 + BQ - 1 + off >= kw0;
    if (active) {
      const int buf = __builtin_amdgcn_readfirstlane(it % NS);
      const uint16_t* qt_ = QOs[buf][0];
      const uint16_t* ot_ = qt_ + BQ * D;
      const float2* lt = Ls[buf];
      if (ALIBI && gi != slope_head) {
        slope_head = gi;
        slope_acc = scalar_load_f32(a.slopes + __builtin_amdgcn_readfirstlane(h)) * a.alibi2;
      }
      // S = Q K^T and dP = dO V^T for rows i0 + 8 (r/4) + 4 g + r%4 and key kj.
      f32x16 s, dp = (f32x16){};
      if (ALIBI) {
        const float b0 = slope_acc * (float)(kj - (i0 + 4 * g + off));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float rofs = (float)(8 * (r >> 2) + (r & 3));
          s[r] = CAUSAL ? fmaf(-slope_acc, rofs, b0) : -slope_acc * __builtin_fabsf(fmaf(-1.f, rofs, (float)(kj - (i0 + 4 * g + off))));
        }
      } else {
        s = (f32x16){};
      }
      // The tile's Q and dO fragments, read RA k-steps ahead of their MFMAs
      // (two waves per SIMD hide the rest of the LDS latency).
      constexpr int RA = 1;
      auto frag = [&](const uint16_t* t, int kk) -> u32x4 {
        return *(const u32x4*)&t[li * D + 8 * ((2 * kk + g) ^ rsw)];
      };
      u32x4 qa[RA], oa[RA];
#pragma unroll
      for (int kk = 0; kk < RA; ++kk) {
        qa[kk] = frag(qt_, kk);
        oa[kk] = frag(ot_, kk);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s = T::mma(qa[kk % RA], kreg[kk], s);
        dp = T::mma(oa[kk % RA], vreg[kk], dp);
        if (kk + RA < KK) {
          qa[kk % RA] = frag(qt_, kk + RA);
          oa[kk % RA] = frag(ot_, kk + RA);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Rows' lse2 and Di: registers r = 4 c .. 4 c + 3 hold rows 8 c + 4 g + 0..3.
      uint32_t pk[8], dk_[8];
      const bool masked = wave_masked || (CAUSAL && i0 + off < kw0 + 31);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int rb = 8 * c + 4 * g;
        const float4 l01 = *(const float4*)&lt[rb];
        const float4 l23 = *(const float4*)&lt[rb + 2];
        const float lsv[4] = {l01.x, l01.z, l23.x, l23.z};
        const float div[4] = {l01.y, l01.w, l23.y, l23.w};
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sv = s[4 * c + e];
          if (masked) {
            bool vis = key_ok;
            if (CAUSAL) vis = vis && kj <= i0 + rb + e + off;
            sv = vis ? sv : kNegInf;
          }
          // Rows past S_q read lse2 = Di = 0 here, and their dO rows are 0.
          p[e] = fast_exp2(fmaf(sv, sc2, -lsv[e]));
          ds[e] = p[e] * (dp[4 * c + e] - div[e]);
        }
        pk[2 * c] = T::pack2(p[0], p[1]);
        pk[2 * c + 1] = T::pack2(p[2], p[3]);
        dk_[2 * c] = T::pack2(ds[0], ds[1]);
        dk_[2 * c + 1] = T::pack2(ds[2], ds[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over two 16-row steps; the
      // transposed fragments of d block i + 1 are read under the MFMAs of
      // block i.
      auto trf = [&](const uint16_t* t, int i) -> u32x4 {
        const int ks = i / DB, db = i % DB;
        const u32x2 lo = lds_read_tr(t + 16 * ks * D + tofs[0][db]);
        const u32x2 hi = lds_read_tr(t + 16 * ks * D + tofs[1][db]);
        return (u32x4){lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4 ov = trf(ot_, 0), qv = trf(qt_, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * DB; ++i) {
        const int ks = i / DB, db = i % DB;
        const u32x4 bp = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
        const u32x4 bd = {dk_[4 * ks], dk_[4 * ks + 1], dk_[4 * ks + 2], dk_[4 * ks + 3]};
        const u32x4 ovc = ov, qvc = qv;
        if (i + 1 < 2 * DB) {
          ov = trf(ot_, i + 1);
          qv = trf(qt_, i + 1);
        }
        dv[db] = T::mma(ovc, bp, dv[db]);
        dk[db] = T::mma(qvc, bd, dk[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if (kvalid) {
    const size_t rowk = ((size_t)(b * (size_t)a.S_k + kj) * a.H_kv + hk) * D + 4 * g;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 pkk = {T::pack2(dk[db][4 * q4] * sc, dk[db][4 * q4 + 1] * sc),
                           T::pack2(dk[db][4 * q4 + 2] * sc, dk[db][4 * q4 + 3] * sc)};
        const u32x2 pvv = {T::pack2(dv[db][4 * q4], dv[db][4 * q4 + 1]),
                           T::pack2(dv[db][4 * q4 + 2], dv[db][4 * q4 + 3])};
        *(u32x2*)(a.dk + rowk + 32 * db + 8 * q4) = pkk;
        *(u32x2*)(a.dv + rowk + 32 * db + 8 * q4) = pvv;
      }
  }
}

}  // namespace sa
