// Device helpers shared by the gfx950 kernels: bf16 packing, wave64 reductions,
// packed argmax keys and cross-workgroup completion counters.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

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
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
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

__device__ __forceinline__ void set_error(unsigned int* err, unsigned int bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mtp
