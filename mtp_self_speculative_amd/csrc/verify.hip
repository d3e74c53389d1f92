// Greedy verification and MTP-cache rollback.
//
// Verify: grid (vocabulary chunk, row j = 0..K, sequence b). Each workgroup reduces its
// chunk of target-logit row (b, j) to a packed (value, index) key — larger value wins,
// lowest index on ties — and folds it into a per-row key with an atomic max, which is
// order independent and hence deterministic. The last workgroup of sequence b turns the
// K+1 keys into the target's tokens, scans the longest prefix of drafts that match them
// and writes accepted_len and the bonus token.
// Rows of a length divisible by 4 take a variant with 16-byte loads and larger chunks.
// Rollback: one lane per sequence moves len/pos to the committed prefix.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kVerifyThreads = 256;
constexpr int kVerifyPer = 8;  // logits per lane; a workgroup covers kVerifyThreads * kVerifyPer

__global__ __launch_bounds__(kVerifyThreads) void verify_kernel(VerifyParams p) {
  __shared__ unsigned long long kred[kVerifyThreads / kWave];
  __shared__ int flag;
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* row = p.logits + ((long)b * (p.K + 1) + j) * p.V;
  const int lo = c * p.chunk, hi = min(lo + p.chunk, p.V);
  // All loads are issued before any is used; indexes past the row end are clamped to its
  // last element, whose key then only repeats.
  int idx[kVerifyPer];
  float v[kVerifyPer];
#pragma unroll
  for (int k = 0; k < kVerifyPer; ++k) {
    idx[k] = min(lo + (int)threadIdx.x + k * kVerifyThreads, hi - 1);
    v[k] = __builtin_nontemporal_load(row + idx[k]);
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int k = 0; k < kVerifyPer; ++k) {
    const unsigned long long key = pack_key(v[k], (uint32_t)idx[k]);
    best = key > best ? key : best;
  }
  best = wave_max_u64(best);
  if (lane == 0) kred[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kVerifyThreads / kWave; ++w) best = kred[w] > best ? kred[w] : best;
    if (best) keep_alive(atomic_max_key(p.keys + (long)b * (p.K + 1) + j, best));
  }
  if (last_to_arrive(p.counters + b, gridDim.x * gridDim.y, &flag)) {
    // Take (and reset) the K+1 row keys and scan for the first mismatch.
    if (threadIdx.x == 0) {
      unsigned long long* kb = p.keys + (long)b * (p.K + 1);
      int a = 0, next = -1;
      for (int q = 0; q <= p.K; ++q) {
        const int t = (int)key_index(take_key(kb + q));
        if (next < 0) {
          if (q < p.K && p.draft[(long)b * p.K + q] == t) {
            ++a;
          } else {
            next = t;
          }
        }
      }
      p.accepted[b] = a;
      p.next[b] = next;
    }
  }
}

// Same reduction for rows whose length is a multiple of 4 (16-byte aligned rows): each
// lane keeps kVerifyVecPer float4 loads in flight, a workgroup covers kVerifyVecChunk
// logits, so far fewer workgroups (and same-address atomics) are needed per row.
constexpr int kVerifyVecPer = 8;
constexpr int kVerifyVecChunk = kVerifyThreads * kVerifyVecPer * 4;

__global__ __launch_bounds__(kVerifyThreads) void verify_vec_kernel(VerifyParams p) {
  __shared__ unsigned long long kred[kVerifyThreads / kWave];
  __shared__ int flag;
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const f32x4v* row = reinterpret_cast<const f32x4v*>(p.logits + ((long)b * (p.K + 1) + j) * p.V);
  const int lo = c * (kVerifyVecChunk / 4), hi = min(lo + kVerifyVecChunk / 4, p.V / 4);
  int idx[kVerifyVecPer];
  f32x4v v[kVerifyVecPer];
#pragma unroll
  for (int k = 0; k < kVerifyVecPer; ++k) {
    idx[k] = min(lo + (int)threadIdx.x + k * kVerifyThreads, hi - 1);
    v[k] = __builtin_nontemporal_load(row + idx[k]);
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int k = 0; k < kVerifyVecPer; ++k) {
    const uint32_t i0 = (uint32_t)idx[k] * 4;
    unsigned long long key = pack_key(v[k].x, i0);
    unsigned long long t = pack_key(v[k].y, i0 + 1);
    key = t > key ? t : key;
    t = pack_key(v[k].z, i0 + 2);
    key = t > key ? t : key;
    t = pack_key(v[k].w, i0 + 3);
    key = t > key ? t : key;
    best = key > best ? key : best;
  }
  best = wave_max_u64(best);
  if (lane == 0) kred[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kVerifyThreads / kWave; ++w) best = kred[w] > best ? kred[w] : best;
    if (best) keep_alive(atomic_max_key(p.keys + (long)b * (p.K + 1) + j, best));
  }
  if (last_to_arrive(p.counters + b, gridDim.x * gridDim.y, &flag)) {
    if (threadIdx.x == 0) {
      unsigned long long* kb = p.keys + (long)b * (p.K + 1);
      int a = 0, next = -1;
      for (int q = 0; q <= p.K; ++q) {
        const int t = (int)key_index(take_key(kb + q));
        if (next < 0) {
          if (q < p.K && p.draft[(long)b * p.K + q] == t) {
            ++a;
          } else {
            next = t;
          }
        }
      }
      p.accepted[b] = a;
      p.next[b] = next;
    }
  }
}

__global__ void rollback_kernel(int* len, int* pos, const int* accepted, int B, int K,
                                unsigned* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int a = accepted[b];
  if (a < 0 || a > K) {
    set_error(err, 4u);
    a = a < 0 ? 0 : K;
  }
  const int keep = (a + 1 < K) ? a + 1 : K;
  len[b] += keep - K;
  pos[b] += a + 1 - K;
}

hipError_t launch_verify(const VerifyParams& p, int B, hipStream_t s) {
  if (p.V < 1 || p.K < 0 || B < 1) return hipErrorInvalidValue;
  if (p.V % 4 == 0 && ((uintptr_t)p.logits & 15) == 0) {
    const int nchunk = (p.V + kVerifyVecChunk - 1) / kVerifyVecChunk;
    hipLaunchKernelGGL(verify_vec_kernel, dim3(nchunk, p.K + 1, B), dim3(kVerifyThreads), 0, s, p);
    return hipGetLastError();
  }
  if (p.chunk != kVerifyThreads * kVerifyPer || (long)p.nchunk * p.chunk < p.V ||
      (long)(p.nchunk - 1) * p.chunk >= p.V)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_kernel, dim3(p.nchunk, p.K + 1, B), dim3(kVerifyThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rollback(int* len, int* pos, const int* accepted, int B, int K, unsigned* err,
                           hipStream_t s) {
  hipLaunchKernelGGL(rollback_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, pos, accepted,
                     B, K, err);
  return hipGetLastError();
}

}  // namespace mtp
