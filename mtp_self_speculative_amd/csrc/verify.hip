// Greedy verification and MTP-cache rollback.
//
// Verify: grid (vocabulary chunk, row j = 0..K, sequence b). Each workgroup reduces its
// chunk of target-logit row (b, j) to a packed (value, index) key — larger value wins,
// lowest index on ties — and folds it into a per-row key with an atomic max, which is
// order independent and hence deterministic. The last workgroup of sequence b turns the
// K+1 keys into the target's tokens, scans the longest prefix of drafts that match them
// and writes accepted_len and the bonus token.
// Rows of a length divisible by 4 take a variant with 16-byte loads and larger chunks.
// Sampling verification (temperature > 0) is described above its kernels below.
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

// ---------------------------------------------------------------- sampling verification
// Speculative sampling at temperature T, in two launches.
// (1) grid (chunk, row, sequence) over the K+1 target rows and the K draft rows: each
//     workgroup reduces its chunk to the pair (max m, sum of 2^(y - m)) of y = x log2(e) / T
//     (base 2, so that each entry costs one hardware exp2) and publishes it with a
//     returning atomic exchange. The last workgroup of a sequence
//     merges each row's pairs (one wave per row, lanes over chunks, then a fixed butterfly
//     over the wave) into a log-sum-exp. Wave 0 then evaluates the acceptance tests of up
//     to 64 drafts at once, draft d_{j+1} passing iff
//     log U_j < (t_j[d]/T - lse_t[j]) - (z_j[d]/T - lse_z[j]), i.e. U < p/q; the first
//     failing lane (a ballot) gives the accepted length a. It writes a and the two
//     log-sum-exps of row a.
// (2) grid (chunk, sequence): Gumbel-max draws over row a, one of log(p_a - q_a) where
//     positive (a < K: the residual distribution) and one of t_a / T (the target's own
//     distribution: the bonus token when a = K, the fallback when rounding left no
//     positive residual). Each lane takes groups of four consecutive entries, one random
//     block per group.
// Rows whose length is a multiple of 4 (16-byte aligned) are read with 16-byte loads.
constexpr int kVsThreads = 256;
constexpr int kVsPer = 8;                                  // loads in flight per lane
constexpr int kVsChunkScalar = kVsThreads * kVsPer;        // logits per statistics workgroup
constexpr int kVsChunkVec = kVsThreads * kVsPer * 4;
constexpr int kVsResChunk = kVsThreads * 8;                // logits per resampling workgroup

int vs_chunks(int V) { return (V + kVsChunkScalar - 1) / kVsChunkScalar; }

__device__ __forceinline__ unsigned long long pack_pair(float m, float sum) {
  return ((unsigned long long)__float_as_uint(m) << 32) | (unsigned long long)__float_as_uint(sum);
}

template <bool VEC>
__global__ __launch_bounds__(kVsThreads) void vs_stats_kernel(VSampleParams p) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  __shared__ float red[kVsThreads / kWave];
  __shared__ float lse_s[2 * kVsMaxK + 1];
  __shared__ int flag;
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, V = p.V, R = 2 * K + 1;
  const float* row = r <= K ? p.tlog + ((long)b * (K + 1) + r) * V
                            : p.dlog + ((long)b * K + (r - K - 1)) * V;
  constexpr int N = VEC ? 4 * kVsPer : kVsPer;
  const float sc2 = kLog2e * p.inv_temp;
  float x[N];
  if constexpr (VEC) {
    const f32x4v* row4 = reinterpret_cast<const f32x4v*>(row);
    const int lo = c * (kVsChunkVec / 4);
#pragma unroll
    for (int k = 0; k < kVsPer; ++k) {
      const int i4 = lo + (int)threadIdx.x + k * kVsThreads;
      f32x4v v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (i4 < V / 4) v = __builtin_nontemporal_load(row4 + i4) * sc2;
      x[4 * k] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
    }
  } else {
    const int lo = c * kVsChunkScalar;
#pragma unroll
    for (int k = 0; k < kVsPer; ++k) {
      const int idx = lo + (int)threadIdx.x + k * kVsThreads;
      x[k] = idx < V ? __builtin_nontemporal_load(row + idx) * sc2 : -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k) m = fmaxf(m, x[k]);
  m = block_max(m, red);  // finite: every chunk holds at least one entry
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < N; ++k) sum += hw_exp2(x[k] - m);
  sum = block_sum(sum, red);
  if (threadIdx.x == 0)
    keep_alive(__hip_atomic_exchange(p.part + ((long)b * R + r) * p.nchunk + c, pack_pair(m, sum),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (!last_to_arrive(p.counters + b, gridDim.x * gridDim.y, &flag)) return;
  // Merge each row's pairs: lane-local running (max, rescaled sum), then the wave.
  for (int q = wave; q < R; q += kVsThreads / kWave) {
    unsigned long long* pp = p.part + ((long)b * R + q) * p.nchunk;
    float M = -INFINITY, S = 0.f;
    for (int cc = lane; cc < p.nchunk; cc += kWave) {
      const unsigned long long v = take_key(pp + cc);
      const float mc = __uint_as_float((uint32_t)(v >> 32));
      const float sc = __uint_as_float((uint32_t)v);
      if (mc > M) {
        S = S * hw_exp2(M - mc) + sc;
        M = mc;
      } else {
        S += sc * hw_exp2(mc - M);
      }
    }
    const float Mw = wave_max(M);
    const float Sw = wave_sum(S * hw_exp2(M - Mw));
    // sum_v e^(x_v / T) = 2^Mw * Sw, so its natural log is Mw ln 2 + ln Sw
    if (lane == 0) lse_s[q] = Mw * kLn2 + logf(Sw);
  }
  __syncthreads();
  if (wave != 0) return;
  int a = K;
  for (int base = 0; base < K; base += kWave) {
    const int j = base + lane;
    bool rej = false;
    if (j < K) {
      const int d = p.draft[(long)b * K + j];
      if (d < 0 || d >= V) {  // an invalid draft token is rejected
        set_error(p.err, 1u);
        rej = true;
      } else {
        const float lp = p.tlog[((long)b * (K + 1) + j) * V + d] * p.inv_temp - lse_s[j];
        const float lq = p.dlog[((long)b * K + j) * V + d] * p.inv_temp - lse_s[K + 1 + j];
        const Philox4 rb = rng_block(p.seeds[b], p.offset, RNG_ACCEPT, (uint64_t)j, 0ull);
        rej = !(logf(rng_uniform(rb.w[0])) < lp - lq);
      }
    }
    const unsigned long long m = __ballot(rej);
    if (m) {
      a = base + __ffsll(m) - 1;
      break;
    }
  }
  if (lane == 0) {
    p.accepted[b] = a;
    p.lse[2 * b] = lse_s[a];
    p.lse[2 * b + 1] = a < K ? lse_s[K + 1 + a] : 0.f;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kVsThreads) void vs_resample_kernel(VSampleParams p) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  __shared__ unsigned long long kred[2][kVsThreads / kWave];
  __shared__ int flag;
  const int c = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, V = p.V;
  int a = p.accepted[b];
  a = a < 0 ? 0 : a > K ? K : a;
  const bool resid = a < K;
  const float* trow = p.tlog + ((long)b * (K + 1) + a) * V;
  const float* drow = resid ? p.dlog + ((long)b * K + a) * V : trow;
  const float lt = p.lse[2 * b], lz = p.lse[2 * b + 1];
  const uint64_t seed = p.seeds[b];
  unsigned long long kr = 0ull, kp = 0ull;
#pragma unroll
  for (int g = 0; g < kVsResChunk / (4 * kVsThreads); ++g) {
    const int v0 = c * kVsResChunk + (g * kVsThreads + (int)threadIdx.x) * 4;
    if (v0 >= V) continue;
    float tv[4], zv[4];
    if constexpr (VEC) {  // V % 4 == 0: the whole group is in range
      const f32x4v t4 = *reinterpret_cast<const f32x4v*>(trow + v0);
      tv[0] = t4.x; tv[1] = t4.y; tv[2] = t4.z; tv[3] = t4.w;
      if (resid) {
        const f32x4v z4 = *reinterpret_cast<const f32x4v*>(drow + v0);
        zv[0] = z4.x; zv[1] = z4.y; zv[2] = z4.z; zv[3] = z4.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = v0 + e < V ? v0 + e : V - 1;
        tv[e] = trow[v];
        if (resid) zv[e] = drow[v];
      }
    }
    const Philox4 rb = rng_block(seed, p.offset, RNG_RESAMPLE, (uint64_t)a, (uint64_t)(v0 >> 2));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v0 + e;
      if (v >= V) break;
      const float t = tv[e] * p.inv_temp;
      const float gv = gumbel_of(rb.w[e]);
      const unsigned long long k1 = pack_key(t + gv, (uint32_t)v);
      kp = k1 > kp ? k1 : kp;
      if (resid) {
        const float rv = hw_exp2((t - lt) * kLog2e) - hw_exp2((zv[e] * p.inv_temp - lz) * kLog2e);
        if (rv > 0.f) {
          const unsigned long long k2 = pack_key(hw_log2(rv) * kLn2 + gv, (uint32_t)v);
          kr = k2 > kr ? k2 : kr;
        }
      }
    }
  }
  kr = wave_max_u64(kr);
  kp = wave_max_u64(kp);
  if (lane == 0) {
    kred[0][wave] = kr;
    kred[1][wave] = kp;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    unsigned long long k = 0ull;
    for (int w = 0; w < kVsThreads / kWave; ++w) k = kred[threadIdx.x][w] > k ? kred[threadIdx.x][w] : k;
    if (k) keep_alive(atomic_max_key(p.keys + 2 * b + threadIdx.x, k));
  }
  if (last_to_arrive(p.counters + b, gridDim.x, &flag)) {
    if (threadIdx.x == 0) {
      const unsigned long long r = take_key(p.keys + 2 * b);
      const unsigned long long q = take_key(p.keys + 2 * b + 1);
      p.next[b] = (int)key_index(r ? r : q);
    }
  }
}

hipError_t launch_verify_sample(const VSampleParams& p, int B, hipStream_t s) {
  if (p.V < 1 || p.K < 0 || p.K > kVsMaxK || B < 1 || p.nchunk != vs_chunks(p.V) ||
      !(p.inv_temp > 0.f) || !p.seeds || !p.tlog || (p.K > 0 && (!p.dlog || !p.draft)) || !p.part ||
      !p.lse || !p.keys || !p.counters || !p.accepted || !p.next || !p.err)
    return hipErrorInvalidValue;
  const bool vec = p.V % 4 == 0 && ((uintptr_t)p.tlog & 15) == 0 &&
                   (p.K == 0 || ((uintptr_t)p.dlog & 15) == 0);
  VSampleParams q = p;
  const int nres = (p.V + kVsResChunk - 1) / kVsResChunk;
  if (vec) {
    q.nchunk = (p.V + kVsChunkVec - 1) / kVsChunkVec;
    hipLaunchKernelGGL(vs_stats_kernel<true>, dim3(q.nchunk, 2 * p.K + 1, B), dim3(kVsThreads), 0,
                       s, q);
  } else {
    hipLaunchKernelGGL(vs_stats_kernel<false>, dim3(q.nchunk, 2 * p.K + 1, B), dim3(kVsThreads),
                       0, s, q);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (vec)
    hipLaunchKernelGGL(vs_resample_kernel<true>, dim3(nres, B), dim3(kVsThreads), 0, s, q);
  else
    hipLaunchKernelGGL(vs_resample_kernel<false>, dim3(nres, B), dim3(kVsThreads), 0, s, q);
  return hipGetLastError();
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
