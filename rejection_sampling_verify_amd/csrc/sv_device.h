// sv_device.h — device building blocks of the verify kernels (gfx950, wave64).
//
// Counter-based random words (Philox4x32-10, Salmon et al. SC'11), the uniform
// and Gumbel maps, logit loads (bf16 / fp32, 16-byte vectors), and wave /
// workgroup reductions with fixed trees so that results do not depend on which
// workgroup computes what.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;  // threads per workgroup: 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------------------
// Philox4x32-10. c1..c3 and the key are the same for every lane of a row, so
// the compiler keeps part of the first two rounds on the scalar unit.
// --------------------------------------------------------------------------
struct Words4 {
  uint32_t w[4];
};

// a ^ b ^ c in one gfx950 three-input bit operation (truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ Words4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                           uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Words4 o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}

// Two independent Philox4x32-10 blocks (counters differing only in word 0),
// with their rounds interleaved so that one block's multiplies issue while
// the other's are in flight.
__device__ __forceinline__ void philox10x2(uint32_t a0, uint32_t b0, uint32_t c1, uint32_t c2, uint32_t c3,
                                           uint32_t k0, uint32_t k1, Words4& wa, Words4& wb) {
  uint32_t a1 = c1, a2 = c2, a3 = c3, b1 = c1, b2 = c2, b3 = c3;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r < 3) {
      // In the first rounds some operands are still the same on every lane
      // (c1, c2, c3 and the key; word 0 of both blocks after round 0): plain
      // two-input xors let the compiler combine those on the scalar unit.
      const uint64_t pa0 = (uint64_t)0xD2511F53u * a0;
      const uint64_t pb0 = (uint64_t)0xD2511F53u * b0;
      const uint64_t pa1 = (uint64_t)0xCD9E8D57u * a2;
      const uint64_t pb1 = (uint64_t)0xCD9E8D57u * b2;
      const uint32_t na0 = (uint32_t)(pa1 >> 32) ^ (a1 ^ k0);
      const uint32_t nb0 = (uint32_t)(pb1 >> 32) ^ (b1 ^ k0);
      const uint32_t na2 = (uint32_t)(pa0 >> 32) ^ (a3 ^ k1);
      const uint32_t nb2 = (uint32_t)(pb0 >> 32) ^ (b3 ^ k1);
      a1 = (uint32_t)pa1;
      b1 = (uint32_t)pb1;
      a3 = (uint32_t)pa0;
      b3 = (uint32_t)pb0;
      a0 = na0;
      b0 = nb0;
      a2 = na2;
      b2 = nb2;
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
      continue;
    }
    const uint64_t pa0 = (uint64_t)0xD2511F53u * a0;
    const uint64_t pb0 = (uint64_t)0xD2511F53u * b0;
    const uint64_t pa1 = (uint64_t)0xCD9E8D57u * a2;
    const uint64_t pb1 = (uint64_t)0xCD9E8D57u * b2;
    const uint32_t na0 = xor3((uint32_t)(pa1 >> 32), a1, k0);
    const uint32_t nb0 = xor3((uint32_t)(pb1 >> 32), b1, k0);
    const uint32_t na2 = xor3((uint32_t)(pa0 >> 32), a3, k1);
    const uint32_t nb2 = xor3((uint32_t)(pb0 >> 32), b3, k1);
    a1 = (uint32_t)pa1;
    b1 = (uint32_t)pb1;
    a3 = (uint32_t)pa0;
    b3 = (uint32_t)pb0;
    a0 = na0;
    b0 = nb0;
    a2 = na2;
    b2 = nb2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  wa.w[0] = a0;
  wa.w[1] = a1;
  wa.w[2] = a2;
  wa.w[3] = a3;
  wb.w[0] = b0;
  wb.w[1] = b1;
  wb.w[2] = b2;
  wb.w[3] = b3;
}

// Word k (0..3) of a block, by selects rather than an indexed array.
__device__ __forceinline__ uint32_t word_at(const Words4& w, int k) {
  const uint32_t lo = (k & 1) ? w.w[1] : w.w[0];
  const uint32_t hi = (k & 1) ? w.w[3] : w.w[2];
  return (k & 2) ? hi : lo;
}

// u = (w >> 8) * 2^-24, exact in fp32, in [0, 1).
__device__ __forceinline__ float uniform_accept(uint32_t w) {
  return (float)(w >> 8) * 0x1p-24f;
}

// Gumbel noise G = -ln(-ln U), U = ((w >> 8) + 0.5) * 2^-24.
// fp32 cannot hold U near 1, so E = -ln U is formed from whichever of U or
// t = 1 - U is at most 1/2 (both are exact multiples of 2^-25 there):
//   U <= 1/2          : E = -ln U;
//   t < 2^-8          : E = -ln(1 - t) by its series t + t^2/2 + t^3/3 + t^4/4;
//   otherwise         : E = -ln(1 - t) = -(ln u - e/u) where u = fl(1 - t) and
//                       e = (u - 1) + t is the exact rounding error of u
//                       (first-order correction; 1/u by its short series).
__device__ __forceinline__ float gumbel(uint32_t w) {
  const uint32_t j = w >> 8;
  const bool low = j < (1u << 23);
  const uint32_t k = low ? j : ((1u << 24) - 1u - j);
  const float z = ((float)k + 0.5f) * 0x1p-24f;  // exact, in (0, 1/2]
  const float u = 1.0f - z;                      // rounded when !low
  const float arg = low ? z : u;
  const float lnarg = __builtin_amdgcn_logf(arg) * kLn2;
  const float e = (u - 1.0f) + z;                // exact rounding error of u
  const float inv_u = 1.0f + z * (1.0f + z * (1.0f + z));
  const float e_log = -(lnarg - e * inv_u);
  const float e_ser = z * (1.0f + z * (0.5f + z * (0.33333334f + z * 0.25f)));
  const float E = low ? -lnarg : (z < 0x1p-8f ? e_ser : e_log);
  // The outer logarithm by the library's logf (about 1 ulp; the hardware
  // log2 is a few ulp off here): G decides comparisons of totals.
  return -logf(E);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ln(1 - e^x) for x < 0, accurate near x = 0 (Maechler's log1mexp split).
__device__ __forceinline__ float log1mexp(float x) {
  return (x > -kLn2) ? logf(-expm1f(x)) : log1pf(-expf(x));
}

// --------------------------------------------------------------------------
// Logit access. Elements per 16-byte vector: 8 bf16 or 4 fp32.
// --------------------------------------------------------------------------
template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float load(const uint8_t* row, int64_t v) {
    const uint16_t h = *(const uint16_t*)(row + 2 * v);
    return __uint_as_float((uint32_t)h << 16);
  }
  // Unpack one 16-byte vector to 8 floats.
  __device__ static __forceinline__ void unpack(const u32x4& q, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(q[k] << 16);
      f[2 * k + 1] = __uint_as_float(q[k] & 0xFFFF0000u);
    }
  }
};

template <>
struct Elem<false> {
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float load(const uint8_t* row, int64_t v) {
    return *(const float*)(row + 4 * v);
  }
  __device__ static __forceinline__ void unpack(const u32x4& q, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(q[k]);
  }
};

__device__ __forceinline__ u32x4 load_vec_stream(const uint8_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// A buffer resource over [p, p + bytes): loads through it take their whole
// offset from one vector register (no 64-bit address arithmetic per load),
// and a load at or past `bytes` returns zeros instead of reading memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes at byte offset off of a buffer, nontemporal (aux bit 1).
__device__ __forceinline__ u32x4 load_vec_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}

// --------------------------------------------------------------------------
// Reductions. Partial log-sum-exp states (M, s) mean sum exp2((l - M) * c)
// over a set of raw logits l with max M, c = log2(e) / T.
// --------------------------------------------------------------------------
struct LseState {
  float M;
  float s;
};

__device__ __forceinline__ LseState lse_merge(LseState a, LseState b, float c) {
  if (b.M == -INFINITY) return a;
  if (a.M == -INFINITY) return b;
  const float M = fmaxf(a.M, b.M);
  // fp32 addition is commutative, so merge(a, b) and merge(b, a) agree
  // bitwise: both lanes of a butterfly step hold the same result.
  const float ta = a.s * fast_exp2((a.M - M) * c);
  const float tb = b.s * fast_exp2((b.M - M) * c);
  LseState r;
  r.M = M;
  r.s = ta + tb;
  return r;
}

struct ArgMax {
  float v;
  int32_t i;
};

// Larger value wins; equal values go to the lower index. Logits are assumed
// not to be NaN.
__device__ __forceinline__ ArgMax argmax_merge(ArgMax a, ArgMax b) {
  if (b.i < 0) return a;
  if (a.i < 0) return b;
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ LseState wave_lse(LseState a, float c) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    LseState o;
    o.M = shfl_xor_f(a.M, m);
    o.s = shfl_xor_f(a.s, m);
    a = lse_merge(a, o, c);
  }
  return a;
}


// Lane exchanges without LDS: DPP within 16-lane rows, then the gfx950 row
// swaps (16 lanes, then 32). After lane_swaps(v), each lane holds v of the
// lane its row swap pairs it with in one of the two results (the other holds
// its own v), so a reduction over v and both results is a reduction with that
// partner row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Wave-wide maximum, in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  float a, b;
  swap16(x, a, b);
  x = fmaxf(x, fmaxf(a, b));
  swap32(x, a, b);
  return fmaxf(x, fmaxf(a, b));
}

// Wave-wide sum, the same value in every lane (fixed order): DPP steps
// within each 16-lane row (after each step both lanes of a pair hold the same
// sum, fp32 addition being commutative), then the four row sums read into
// scalar registers and added in row order.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int wave_or(int x) { return __builtin_amdgcn_ballot_w64(x != 0) != 0ull ? 1 : 0; }

template <int CTRL>
__device__ __forceinline__ ArgMax dpp_am(ArgMax a) {
  ArgMax o;
  o.v = dpp_f<CTRL>(a.v);
  o.i = __builtin_amdgcn_update_dpp(0, a.i, CTRL, 0xF, 0xF, false);
  return o;
}
__device__ __forceinline__ ArgMax readlane_am(ArgMax a, int lane) {
  ArgMax o;
  o.v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a.v), lane));
  o.i = __builtin_amdgcn_readlane(a.i, lane);
  return o;
}

// Wave-wide argmax (larger value, lower index on ties), the same in every
// lane: the DPP steps of wave_sum within each 16-lane row, then the four row
// results merged in row order.
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
  a = argmax_merge(a, dpp_am<0xB1>(a));
  a = argmax_merge(a, dpp_am<0x4E>(a));
  a = argmax_merge(a, dpp_am<0x141>(a));
  a = argmax_merge(a, dpp_am<0x140>(a));
  return argmax_merge(argmax_merge(readlane_am(a, 0), readlane_am(a, 16)),
                      argmax_merge(readlane_am(a, 32), readlane_am(a, 48)));
}

// --------------------------------------------------------------------------
// Cross-workgroup exchange. Workgroups on different XCDs do not share an L2,
// and agent-scope fences make coherent by writing back and invalidating the
// whole L2 of the XCD, which costs far more than the data exchanged here.
// Instead every word one workgroup hands to another is written and read with
// atomic read-modify-write operations, which the device performs at its
// coherence point for all XCDs; a wave that must publish data before a
// signal waits for its outstanding memory operations to complete first.
// --------------------------------------------------------------------------
__device__ __forceinline__ void xput(uint32_t* p, uint32_t v) { atomicExch(p, v); }
__device__ __forceinline__ void xput(int32_t* p, int32_t v) { atomicExch(p, v); }
__device__ __forceinline__ void xput(float* p, float v) { atomicExch((uint32_t*)p, __float_as_uint(v)); }
__device__ __forceinline__ uint32_t xget(uint32_t* p) { return atomicOr(p, 0u); }
__device__ __forceinline__ int32_t xget(int32_t* p) { return atomicOr(p, 0); }
__device__ __forceinline__ float xget(float* p) { return __uint_as_float(atomicOr((uint32_t*)p, 0u)); }
// Plain device-scope atomic load of a 32-bit word (no read-modify-write: many
// readers of one word do not serialize).
__device__ __forceinline__ uint32_t xload(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 64-bit words: device-scope atomic loads and stores (single-copy atomic).
__device__ __forceinline__ void xput64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t xget64(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All vector memory operations of this wave (loads, stores, atomics) done.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Index of the XCD (accelerator complex die) this workgroup runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11));  // HW_REG_XCC_ID[3:0]
}

}  // namespace sv
