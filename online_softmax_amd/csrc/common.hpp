// Device-side types and helpers shared by the attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;  // log2(e): e^x = 2^(x log2 e)
constexpr float kLn2 = 0.6931471805599453f;    // ln(2)
constexpr float kNegInf = -__builtin_huge_valf();

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Element-type traits.  Storage is raw 16-bit words; these convert and feed
// the 32x32x16 matrix-core instruction of the matching type.
struct F16 {
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Two floats to a packed pair, round to nearest even.
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  // A packed pair to two floats (exact).
  __device__ static inline f32x2 unpack2(uint32_t x) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, x), f32x2);
  }
};

struct BF16 {
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // bf16 is the upper half of a float.
  __device__ static inline f32x2 unpack2(uint32_t x) {
    return (f32x2){__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u)};
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine x with the value the lane 32 positions away holds (the other half
// of the wave), using v_permlane32_swap: with both operands x it returns the
// low-half values in one result and the high-half values in the other.
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Combine x over the four lanes l, l^16, l^32, l^48 (the lanes that hold one
// query column of a 16x16 MFMA accumulator), with v_permlane16_swap and
// v_permlane32_swap.
__device__ inline float max_quarters(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_halves(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ inline float sum_quarters(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return sum_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// True in every lane when the predicate holds in any lane of the wave.
__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
// Number of set bits of a wave mask in the lanes below `lane`.
__device__ inline int lanes_below(uint64_t m, int lane) {
  return __builtin_popcountll(m & ((uint64_t(1) << lane) - 1));
}

// Transposing LDS read: in every group of 16 lanes, lane t supplies the
// address of four consecutive 16-bit words; lane u receives word (u % 4) of
// the chunks supplied by lanes u/4, 4 + u/4, 8 + u/4 and 12 + u/4.
__device__ inline u32x2 lds_read_tr(const uint16_t* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Buffer resource (V#) over [base, base + bytes): loads beyond the end read
// zero.  Word 3 selects raw 32-bit data with no swizzle or stride.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return (i32x4){(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// Direct global-to-LDS copy of 16 bytes per lane: lane l's bytes land at
// lds + 16 l (lds must be the same for the whole wave).  Written as inline
// assembly so that the compiler does not treat later LDS reads of other
// buffers as dependent on the copy (it would wait for every copy before
// them); completion is awaited explicitly with wait_vmem() before the
// barrier that publishes the buffer.  The copy has no register results; M0
// carries the LDS base and needs one wait state before the load.
__device__ inline void load_lds16(i32x4 rsrc, const void* lds, uint32_t voffset) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(lds_addr), "v"(voffset), "s"(rsrc) : "m0");
}

// A 32-bit load through the scalar data cache from a wave-uniform address,
// awaited in the same statement.  Unlike a vector load it is counted apart
// from the vector-memory operations (the LDS-destination copies above are
// among those, and the compiler does not see them), so waiting for it never
// waits for copies in flight.
__device__ inline float scalar_load_f32(const float* p) {
  float v;
  __asm__ volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// The same resource in the form the buffer-load builtins take.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc_t(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16-byte buffer load into registers (zero past the end of the resource).
__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, soffset, 0));
}

// Device-coherent (sc1) 16-byte buffer store and load: they write through and
// read past the per-XCD L2 caches, so workgroups on different XCDs see each
// other's data once the store has completed, without a cache-wide write-back
// or invalidation.
__device__ inline void buffer_store16_coherent(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, voffset, 0, 16);
}
__device__ inline u32x4 buffer_load16_coherent(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, 0, 16));
}

// Wait for this wave's outstanding vector-memory operations, including
// global-to-LDS copies (vmcnt(0); the other counters are left alone).
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Wait until at most N of this wave's vector-memory operations are in flight
// (they complete in issue order, so everything older than the last N is done).
template <int N>
__device__ inline void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// wait_vmem_n for a count known only after loop unrolling (the switch folds
// to one wait when n is a constant); counts past 47 wait for everything.
__device__ inline void wait_vmem_upto(int n) {
  switch (n) {
    case 0: wait_vmem_n<0>(); break;
    case 1: wait_vmem_n<1>(); break;
    case 2: wait_vmem_n<2>(); break;
    case 3: wait_vmem_n<3>(); break;
    case 4: wait_vmem_n<4>(); break;
    case 5: wait_vmem_n<5>(); break;
    case 6: wait_vmem_n<6>(); break;
    case 7: wait_vmem_n<7>(); break;
    case 8: wait_vmem_n<8>(); break;
    case 9: wait_vmem_n<9>(); break;
    case 10: wait_vmem_n<10>(); break;
    case 11: wait_vmem_n<11>(); break;
    case 12: wait_vmem_n<12>(); break;
    case 13: wait_vmem_n<13>(); break;
    case 14: wait_vmem_n<14>(); break;
    case 15: wait_vmem_n<15>(); break;
    case 16: wait_vmem_n<16>(); break;
    case 17: wait_vmem_n<17>(); break;
    case 18: wait_vmem_n<18>(); break;
    case 19: wait_vmem_n<19>(); break;
    case 20: wait_vmem_n<20>(); break;
    case 21: wait_vmem_n<21>(); break;
    case 22: wait_vmem_n<22>(); break;
    case 23: wait_vmem_n<23>(); break;
    case 24: wait_vmem_n<24>(); break;
    case 25: wait_vmem_n<25>(); break;
    case 26: wait_vmem_n<26>(); break;
    case 27: wait_vmem_n<27>(); break;
    case 28: wait_vmem_n<28>(); break;
    case 29: wait_vmem_n<29>(); break;
    case 30: wait_vmem_n<30>(); break;
    case 31: wait_vmem_n<31>(); break;
    case 32: wait_vmem_n<32>(); break;
    case 33: wait_vmem_n<33>(); break;
    case 34: wait_vmem_n<34>(); break;
    case 35: wait_vmem_n<35>(); break;
    case 36: wait_vmem_n<36>(); break;
    case 37: wait_vmem_n<37>(); break;
    case 38: wait_vmem_n<38>(); break;
    case 39: wait_vmem_n<39>(); break;
    case 40: wait_vmem_n<40>(); break;
    case 41: wait_vmem_n<41>(); break;
    case 42: wait_vmem_n<42>(); break;
    case 43: wait_vmem_n<43>(); break;
    case 44: wait_vmem_n<44>(); break;
    case 45: wait_vmem_n<45>(); break;
    case 46: wait_vmem_n<46>(); break;
    case 47: wait_vmem_n<47>(); break;
    default: wait_vmem(); break;
  }
}

// Workgroups are dealt to the eight XCDs round-robin (id % 8).  Renumber them
// so that each XCD receives one contiguous run of work items, keeping the
// items that share key/value rows inside one XCD's L2.
__device__ inline int xcd_contiguous(int id, int n) {
  const int per = n >> 3, rem = n & 7, x = id & 7, slot = id >> 3;
  return x < rem ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}

}  // namespace sa
