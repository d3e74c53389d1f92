// Device helpers shared by the gfx950 kernels: bf16 packing, wave64 reductions,
// packed argmax keys and cross-workgroup completion counters.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mtp {

constexpr int kWave = 64;

// Native 16-byte vector (the unit of every global load in the weight streams).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// v ~= hi + lo with hi = bf16(v) and lo = bf16(v - hi): a pair of bf16 values that
// keeps about 16 significant bits of v.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(v);
  lo = f32_to_bf16(v - bf16_to_f32(hi));
}

__device__ __forceinline__ void load8_f32(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void store8_lds(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<float4*>(p + 4) = float4{v[4], v[5], v[6], v[7]};
}

// Element type tags: storage of weights / activations in memory.
struct F32 {
  using T = float;
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ static float get(const T* p, long i) { return p[i]; }
  // Unpack one 16-byte vector to kVec floats.
  __device__ static void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static void put(T* p, long i, float f) { p[i] = f; }
  // 8 consecutive elements (16-byte aligned) as floats.
  __device__ static void load8(const T* p, float* o) { load8_f32(p, o); }
  // N consecutive elements (N = 1 or 2) loaded as one naturally aligned access.
  template <int N>
  struct VecT { float v[N]; };
  template <int N>
  using Vec = VecT<N>;
  template <int N>
  __device__ static Vec<N> load_vec(const T* p) {
    Vec<N> r;
    if constexpr (N == 2) {
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
      r.v[0] = t.x; r.v[1] = t.y;
    } else {
      r.v[0] = __builtin_nontemporal_load(p);
    }
    return r;
  }
  template <int N>
  __device__ static void unpack_vec(const Vec<N>& r, float* o) {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = r.v[i];
  }
};
struct BF16 {
  using T = uint16_t;
  static constexpr int kVec = 8;
  __device__ static float get(const T* p, long i) { return bf16_to_f32(p[i]); }
  __device__ static void unpack(const u32x4& v, float* o) {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
  __device__ static void put(T* p, long i, float f) { p[i] = f32_to_bf16(f); }
  __device__ static void load8(const T* p, float* o) {
    unpack(*reinterpret_cast<const u32x4*>(p), o);
  }
  // N consecutive elements (N = 1 or 2) loaded as one naturally aligned access.
  template <int N>
  using Vec = typename std::conditional<N == 2, uint32_t, uint16_t>::type;
  template <int N>
  __device__ static Vec<N> load_vec(const T* p) {
    if constexpr (N == 2) {
      return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else {
      return __builtin_nontemporal_load(p);
    }
  }
  template <int N>
  __device__ static void unpack_vec(const Vec<N>& r, float* o) {
    if constexpr (N == 2) {
      o[0] = bf16_lo(r);
      o[1] = bf16_hi(r);
    } else {
      o[0] = bf16_to_f32(r);
    }
  }
};

// ---------------------------------------------------------------- DPP lane movement
// gfx9 DPP controls: quad_perm(a,b,c,d) = a | b<<2 | c<<4 | d<<6, row_mirror = 0x140,
// row_half_mirror = 0x141. Rows are groups of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of W lanes (W = 2, 4, 8 or 16) with DPP; every lane of the
// group ends with the group's sum.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group of 2..16 lanes");
  v += dpp<0xB1>(v);                      // lane ^ 1
  if constexpr (W >= 4) v += dpp<0x4E>(v);  // lane ^ 2
  if constexpr (W >= 8) v += dpp<0x141>(v); // mirror within 8 lanes
  if constexpr (W >= 16) v += dpp<0x140>(v); // mirror within 16 lanes
  return v;
}
// Sum over the 64-lane wave, result uniform in every lane.
__device__ __forceinline__ float wave_sum_fast(float v) {
  v = dpp_group_sum<16>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}
__device__ __forceinline__ float wave_max_fast(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned long long o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Sum of `v` over the workgroup; `red` holds >= blockDim/64 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum_fast(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Maximum of `v` over the workgroup; `red` as for block_sum.
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max_fast(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

// ---------------------------------------------------------------- RoPE
// cos / sin of position * theta^(-2i/d) for rotate-half pair i (0 <= i < d/2), evaluated
// in double precision from the integer position and rounded to fp32.
__device__ __forceinline__ void rope_cs(int position, int i, int d, float theta, float& c,
                                        float& s) {
  const double inv = pow((double)theta, -2.0 * (double)i / (double)d);
  const double ang = (double)position * inv;
  c = (float)cos(ang);
  s = (float)sin(ang);
}

// ---------------------------------------------------------------- counter-based random numbers
// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1,
// 2, 3", SC'11): ten rounds of two 64x64->128-bit multiplies with the key bumped by Weyl
// constants between rounds. Any (counter, key) is evaluated independently, so every
// vocabulary entry draws its own number wherever and in whatever order it is computed.
struct Philox4 {
  uint64_t w[4];
};
// 64 x 64 -> 128-bit product from four 32 x 32 + 64 -> 64-bit multiply-adds: with a, c split
// into 32-bit halves, p1 = ah*cl + hi(al*cl) and p2 = al*ch + lo(p1) stay below 2^64, and
// a*c = (ah*ch + hi(p1) + hi(p2)) * 2^64 + lo(p2) * 2^32 + lo(al*cl).
__host__ __device__ __forceinline__ void mul64_wide(uint64_t a, uint64_t c, uint64_t& hi,
                                                    uint64_t& lo) {
  const uint64_t al = (uint32_t)a, ah = a >> 32, cl = (uint32_t)c, ch = c >> 32;
  const uint64_t p0 = al * cl;
  const uint64_t p1 = ah * cl + (p0 >> 32);
  const uint64_t p2 = al * ch + (uint32_t)p1;
  hi = ah * ch + (p1 >> 32) + (p2 >> 32);
  lo = (p2 << 32) | (uint32_t)p0;
}
__device__ __forceinline__ Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                 uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mul64_wide(M0, c0, hi0, lo0);
    mul64_wide(M1, c2, hi1, lo1);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  return Philox4{{c0, c1, c2, c3}};
}
// Counter layout of the sampling streams: (c0, row, purpose, offset) under key (seed, 0).
// Vocabulary entry v of a row uses word v & 3 of block c0 = v >> 2.
enum RngPurpose : uint64_t {
  RNG_DRAFT = 0,     // the draft's Gumbel noise at draft step `row`
  RNG_ACCEPT = 1,    // acceptance uniform of draft `row` (c0 = 0, word 0)
  RNG_RESAMPLE = 2,  // Gumbel noise of the resampled / bonus token (row = accepted length)
};
__device__ __forceinline__ Philox4 rng_block(uint64_t seed, uint64_t offset, uint64_t purpose,
                                             uint64_t row, uint64_t c0) {
  return philox4x64_10(c0, row, purpose, offset, seed, 0ull);
}
__device__ __forceinline__ uint64_t philox_word(const Philox4& b, int i) {
  return i == 0 ? b.w[0] : i == 1 ? b.w[1] : i == 2 ? b.w[2] : b.w[3];
}
// A word as a uniform number in (0, 1): its top 24 bits with the lowest forced to one,
// times 2^-24 (an odd multiple of 2^-24, exact in fp32).
__device__ __forceinline__ float rng_uniform(uint64_t w) {
  return (float)((uint32_t)(w >> 40) | 1u) * 0x1p-24f;
}
// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32, about 1 ulp).
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
// Standard Gumbel variate -ln(-ln U), in base 2: -ln2 * log2(-ln2 * log2 U). Adding one to
// each log-weight and taking the argmax samples the categorical distribution of the weights.
__device__ __forceinline__ float gumbel_of(uint64_t w) {
  return -kLn2 * hw_log2(-kLn2 * hw_log2(rng_uniform(w)));
}

// ---------------------------------------------------------------- argmax keys
// A logit and its index packed so that a larger key means a larger value and,
// among equal values, a smaller index. Key 0 is below every finite logit.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ unsigned long long pack_key(float v, uint32_t idx) {
  return ((unsigned long long)orderable(v) << 32) | (unsigned long long)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t key_index(unsigned long long k) {
  return 0xffffffffu - (uint32_t)(k & 0xffffffffull);
}
__device__ __forceinline__ float key_value(unsigned long long k) {
  return from_orderable((uint32_t)(k >> 32));
}

// Publish a key; returns the previous value so that callers can wait for completion.
__device__ __forceinline__ unsigned long long atomic_max_key(unsigned long long* p,
                                                             unsigned long long k) {
  return __hip_atomic_fetch_max(p, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Completion counter for workgroups that publish their results only through
// device-scope atomic read-modify-writes (which are performed at the device's
// coherence point). Each thread waits until its own atomics have returned, the
// workgroup synchronises, and one thread bumps the counter; exactly one workgroup,
// the last to arrive, gets true and resets the counter. No cache-wide release or
// acquire fence is needed: the last workgroup reads the published values back with
// atomic read-modify-writes as well.
__device__ __forceinline__ bool last_to_arrive(unsigned int* counter, unsigned int total,
                                               int* flag_lds) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (prev == total - 1);
    if (last) __hip_atomic_exchange(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag_lds = last;
  }
  __syncthreads();
  return *flag_lds != 0;
}

// Force a returned atomic value to be materialised, so that the atomic is issued in
// its returning form and the wait before the completion counter covers it.
__device__ __forceinline__ void keep_alive(unsigned long long v) { asm volatile("" ::"v"(v)); }

// Read a published key and reset it to zero in one atomic step.
__device__ __forceinline__ unsigned long long take_key(unsigned long long* p) {
  return __hip_atomic_exchange(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The only two ways a workgroup publishes a value that the winner of last_to_arrive reads
// back: a returning device-scope atomic whose result is kept live, so that the wait at the
// top of last_to_arrive covers it. A plain or non-returning store in their place would
// not be covered by that wait, and the winner could read a stale value.
__device__ __forceinline__ void publish_max_key(unsigned long long* p, unsigned long long k) {
  keep_alive(atomic_max_key(p, k));
}
__device__ __forceinline__ void publish_exchange(unsigned long long* p, unsigned long long v) {
  keep_alive(__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Steps of sequence b in a call of K steps: its own length kseq[b] clamped to [0, K], or K
// when the call has no per-sequence lengths.
__device__ __forceinline__ int seq_steps(const int* kseq, int b, int K) {
  if (!kseq) return K;
  const int k = kseq[b];
  return k < 0 ? 0 : k > K ? K : k;
}

__device__ __forceinline__ void set_error(unsigned int* err, unsigned int bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mtp
