// Greedy verification, sampling verification and MTP-cache rollback.
//
// Greedy verify: grid (segment, row j = 0..K, sequence b). Each workgroup walks its
// segment of target-logit row (b, j) in stages of 8 loads per lane and reduces it to a
// packed (value, index) key — larger value wins, lowest index on ties — which it folds
// into the row's key with an atomic max (order independent, hence deterministic). The
// last workgroup of sequence b turns the K+1 keys into the target's tokens, scans the
// longest prefix of drafts that match them and writes accepted_len and the bonus token.
// The segment count is chosen per launch so that the grid holds about four workgroups per
// CU: enough loads in flight to stream HBM, and few enough completion atomics per
// sequence. Each sequence's counter and keys sit on their own 256-byte line.
// Rows whose length is a multiple of 4 (16-byte aligned) are read with 16-byte loads.
// Sampling verification (temperature > 0) is described above its kernels below.
// Rollback: one lane per sequence moves len/pos to the committed prefix.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kVThreads = 256;
constexpr int kVPer = 8;                      // loads in flight per lane and stage
constexpr int kVStage = kVThreads * kVPer;    // load units (floats or float4s) per stage
constexpr int kTargetGroups = 1024;           // about four workgroups per CU

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Segments of `units` load units for `rows` rows: about kTargetGroups workgroups in all,
// at most one per stage of the row.
static void segments(long rows, int units, int* nseg, int* seg) {
  const int max_seg = (units + kVStage - 1) / kVStage;
  long s = (kTargetGroups + rows - 1) / rows;
  if (s > max_seg) s = max_seg;
  if (s < 1) s = 1;
  *seg = (int)((units + s - 1) / s);
  *nseg = (units + *seg - 1) / *seg;
}

// Loads kVPer units of `row` starting at unit i0 + threadIdx.x with stride kVThreads,
// indexes clamped to hi - 1 (a repeated unit only repeats a key or is masked by the
// caller); VEC units are float4 groups.
template <bool VEC>
__device__ __forceinline__ void load_stage(const float* row, int i0, int hi, int* idx,
                                           f32x4v* v) {
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    idx[k] = min(i0 + (int)threadIdx.x + k * kVThreads, hi - 1);
    if constexpr (VEC) {
      v[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(row) + idx[k]);
    } else {
      const float x = __builtin_nontemporal_load(row + idx[k]);
      v[k] = f32x4v{x, x, x, x};
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kVThreads) void verify_kernel(VerifyParams p) {
  __shared__ unsigned long long kred[kVThreads / kWave];
  __shared__ int flag;
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* row = p.logits + ((long)b * (p.K + 1) + j) * p.V;
  const int units = VEC ? p.V / 4 : p.V;
  const int ks = seq_steps(p.kseq, b, p.K);  // the sequence's own draft count
  const int lo = c * p.seg, hi = j <= ks ? min(lo + p.seg, units) : lo;  // rows past ks: skipped
  unsigned long long best = 0ull;
  auto process = [&](const int (&idx)[kVPer], const f32x4v (&v)[kVPer]) {
#pragma unroll
    for (int k = 0; k < kVPer; ++k) {
      unsigned long long key;
      if constexpr (VEC) {
        const uint32_t e0 = (uint32_t)idx[k] * 4;
        key = pack_key(v[k].x, e0);
        unsigned long long t = pack_key(v[k].y, e0 + 1);
        key = t > key ? t : key;
        t = pack_key(v[k].z, e0 + 2);
        key = t > key ? t : key;
        t = pack_key(v[k].w, e0 + 3);
        key = t > key ? t : key;
      } else {
        key = pack_key(v[k].x, (uint32_t)idx[k]);
      }
      best = key > best ? key : best;
    }
  };
  // Two stages in flight: the next stage's loads go out before this stage's keys are
  // formed (indexes past the segment are clamped, so the extra stage is harmless).
  int ia[kVPer], ib[kVPer];
  f32x4v va[kVPer], vb[kVPer];
  if (lo < hi) {
    load_stage<VEC>(row, lo, hi, ia, va);
    for (int i0 = lo; i0 < hi; i0 += 2 * kVStage) {
      load_stage<VEC>(row, i0 + kVStage, hi, ib, vb);
      process(ia, va);
      if (i0 + kVStage >= hi) break;
      load_stage<VEC>(row, i0 + 2 * kVStage, hi, ia, va);
      process(ib, vb);
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) kred[wave] = best;
  __syncthreads();
  unsigned long long* kb = p.keys + (long)b * p.kstride;
  if (threadIdx.x == 0) {
    for (int w = 1; w < kVThreads / kWave; ++w) best = kred[w] > best ? kred[w] : best;
    if (best) publish_max_key(kb + j, best);
  }
  // the winner reads back only keys published by publish_max_key
  if (last_to_arrive(p.counters + (long)b * kSeqLineU32, gridDim.x * gridDim.y, &flag)) {
    // Take (and reset) the K+1 row keys and scan for the first mismatch.
    if (threadIdx.x == 0) {
      int a = 0, next = -1;
      for (int q = 0; q <= p.K; ++q) {  // every key is reset; rows past kseq decide nothing
        const int t = (int)key_index(take_key(kb + q));
        if (next < 0 && q <= ks) {
          if (q < ks && p.draft[(long)b * p.K + q] == t) {
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

hipError_t launch_verify(const VerifyParams& p, int B, hipStream_t s) {
  if (p.V < 1 || p.K < 0 || B < 1 || !p.logits || !p.keys || !p.counters || !p.accepted ||
      !p.next || (p.K > 0 && !p.draft) || p.kstride < p.K + 1)
    return hipErrorInvalidValue;
  const bool vec = p.V % 4 == 0 && ((uintptr_t)p.logits & 15) == 0;
  VerifyParams q = p;
  int nseg;
  segments((long)B * (p.K + 1), vec ? p.V / 4 : p.V, &nseg, &q.seg);
  if (vec)
    hipLaunchKernelGGL(verify_kernel<true>, dim3(nseg, p.K + 1, B), dim3(kVThreads), 0, s, q);
  else
    hipLaunchKernelGGL(verify_kernel<false>, dim3(nseg, p.K + 1, B), dim3(kVThreads), 0, s, q);
  return hipGetLastError();
}

// ---------------------------------------------------------------- sampling verification
// Speculative sampling at temperature T, in two launches.
// (1) grid (segment, row, sequence) over the K+1 target rows and the K draft rows: each
//     workgroup reduces its segment to the pair (max m, sum of 2^(y - m)) of
//     y = x log2(e) / T (base 2, so that each entry costs one hardware exp2), keeping a
//     running pair per lane across stages, and publishes it with a returning atomic
//     exchange. The last workgroup of a sequence merges each row's pairs (one wave per
//     row, lanes over segments, then a fixed butterfly over the wave) into a log-sum-exp.
//     Wave 0 then evaluates the acceptance tests of up to 64 drafts at once, draft d_{j+1}
//     passing iff log U_j < (t_j[d]/T - lse_t[j]) - (z_j[d]/T - lse_z[j]), i.e. U < p/q; the
//     first failing lane (a ballot) gives the accepted length a. It writes a and the two
//     log-sum-exps of row a.
// (2) grid (segment, sequence): Gumbel-max draws over row a, one of log(p_a - q_a) where
//     positive (a < K: the residual distribution) and one of t_a / T (the target's own
//     distribution: the bonus token when a = K, the fallback when rounding left no
//     positive residual). Each lane takes groups of four consecutive entries, one random
//     block per group.

int vs_chunks(int V) { return (V + kVStage - 1) / kVStage; }

__device__ __forceinline__ unsigned long long pack_pair(float m, float sum) {
  return ((unsigned long long)__float_as_uint(m) << 32) | (unsigned long long)__float_as_uint(sum);
}

template <bool VEC>
__global__ __launch_bounds__(kVThreads) void vs_stats_kernel(VSampleParams p) {
  __shared__ float red[kVThreads / kWave];
  __shared__ float lse_s[2 * kVsMaxK + 1];
  __shared__ int flag;
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, V = p.V, R = 2 * K + 1;
  const float* row = r <= K ? p.tlog + ((long)b * (K + 1) + r) * V
                            : p.dlog + ((long)b * K + (r - K - 1)) * V;
  const int units = VEC ? V / 4 : V;
  const int lo = c * p.seg, hi = min(lo + p.seg, units);
  const float sc2 = kLog2e * p.inv_temp;
  // Running (max, sum of 2^(y - max)) of this lane; units repeated by the index clamp
  // are masked out.
  float m = -INFINITY, sum = 0.f;
  auto process = [&](const f32x4v (&v)[kVPer], int i0) {
    float y[kVPer][4];
    float sm = m;
#pragma unroll
    for (int k = 0; k < kVPer; ++k) {
      const bool live = i0 + (int)threadIdx.x + k * kVThreads < hi;
      y[k][0] = live ? v[k].x * sc2 : -INFINITY;
      y[k][1] = live && VEC ? v[k].y * sc2 : -INFINITY;
      y[k][2] = live && VEC ? v[k].z * sc2 : -INFINITY;
      y[k][3] = live && VEC ? v[k].w * sc2 : -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm = fmaxf(sm, y[k][e]);
    }
    if (sm > -INFINITY) {
      sum = m > -INFINITY ? sum * hw_exp2(m - sm) : 0.f;
      m = sm;
#pragma unroll
      for (int k = 0; k < kVPer; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += hw_exp2(y[k][e] - m);
    }
  };
  // Two stages in flight, as in verify_kernel.
  int ia[kVPer], ib[kVPer];
  f32x4v va[kVPer], vb[kVPer];
  load_stage<VEC>(row, lo, hi, ia, va);
  for (int i0 = lo; i0 < hi; i0 += 2 * kVStage) {
    load_stage<VEC>(row, i0 + kVStage, hi, ib, vb);
    process(va, i0);
    if (i0 + kVStage >= hi) break;
    load_stage<VEC>(row, i0 + 2 * kVStage, hi, ia, va);
    process(vb, i0 + kVStage);
  }
  const float M = block_max(m, red);  // finite: every segment holds at least one entry
  const float S = block_sum(m > -INFINITY ? sum * hw_exp2(m - M) : 0.f, red);
  if (threadIdx.x == 0)
    publish_exchange(p.part + ((long)b * R + r) * p.nchunk + c, pack_pair(M, S));
  // the winner reads back only pairs published by publish_exchange
  if (!last_to_arrive(p.counters + (long)b * kSeqLineU32, gridDim.x * gridDim.y, &flag)) return;
  // Merge each row's pairs: lane-local running (max, rescaled sum), then the wave.
  const int nseg = gridDim.x;
  for (int q = wave; q < R; q += kVThreads / kWave) {
    unsigned long long* pp = p.part + ((long)b * R + q) * p.nchunk;
    float Mq = -INFINITY, Sq = 0.f;
    for (int cc = lane; cc < nseg; cc += kWave) {
      const unsigned long long pv = take_key(pp + cc);
      const float mc = __uint_as_float((uint32_t)(pv >> 32));
      const float sc = __uint_as_float((uint32_t)pv);
      if (mc > Mq) {
        Sq = Sq * hw_exp2(Mq - mc) + sc;
        Mq = mc;
      } else {
        Sq += sc * hw_exp2(mc - Mq);
      }
    }
    const float Mw = wave_max(Mq);
    const float Sw = wave_sum(Mq > -INFINITY ? Sq * hw_exp2(Mq - Mw) : 0.f);
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
    const unsigned long long msk = __ballot(rej);
    if (msk) {
      a = base + __ffsll(msk) - 1;
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
__global__ __launch_bounds__(kVThreads) void vs_resample_kernel(VSampleParams p) {
  __shared__ unsigned long long kred[2][kVThreads / kWave];
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
  const int ngroups = (V + 3) / 4;
  const int lo = c * p.seg, hi = min(lo + p.seg, ngroups);
  unsigned long long kr = 0ull, kp = 0ull;
  for (int g = lo + (int)threadIdx.x; g < hi; g += kVThreads) {
    const int v0 = 4 * g;
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
    const Philox4 rb = rng_block(seed, p.offset, RNG_RESAMPLE, (uint64_t)a, (uint64_t)g);
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
  unsigned long long* kb = p.keys + (long)b * kSeqLineU64;
  if (threadIdx.x < 2) {
    unsigned long long k = 0ull;
    for (int w = 0; w < kVThreads / kWave; ++w) k = kred[threadIdx.x][w] > k ? kred[threadIdx.x][w] : k;
    if (k) publish_max_key(kb + threadIdx.x, k);
  }
  // the winner reads back only keys published by publish_max_key
  if (last_to_arrive(p.counters + (long)b * kSeqLineU32, gridDim.x, &flag)) {
    if (threadIdx.x == 0) {
      const unsigned long long rk = take_key(kb);
      const unsigned long long qk = take_key(kb + 1);
      p.next[b] = (int)key_index(rk ? rk : qk);
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
  int nseg;
  segments((long)B * (2 * p.K + 1), vec ? p.V / 4 : p.V, &nseg, &q.seg);
  if (vec)
    hipLaunchKernelGGL(vs_stats_kernel<true>, dim3(nseg, 2 * p.K + 1, B), dim3(kVThreads), 0, s, q);
  else
    hipLaunchKernelGGL(vs_stats_kernel<false>, dim3(nseg, 2 * p.K + 1, B), dim3(kVThreads), 0, s, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Resampling: groups of four entries; about kTargetGroups workgroups, at least one
  // group per lane.
  const int ngroups = (p.V + 3) / 4;
  long sr = (kTargetGroups + B - 1) / B;
  const long max_sr = (ngroups + kVThreads - 1) / kVThreads;
  if (sr > max_sr) sr = max_sr;
  q.seg = (int)((ngroups + sr - 1) / sr);
  const int nres = (ngroups + q.seg - 1) / q.seg;
  if (vec)
    hipLaunchKernelGGL(vs_resample_kernel<true>, dim3(nres, B), dim3(kVThreads), 0, s, q);
  else
    hipLaunchKernelGGL(vs_resample_kernel<false>, dim3(nres, B), dim3(kVThreads), 0, s, q);
  return hipGetLastError();
}

__global__ void rollback_kernel(int* len, int* pos, const int* accepted, const int* kseq, int B,
                                int K, unsigned* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int k = seq_steps(kseq, b, K);  // the draft's steps for this sequence
  int a = accepted[b];
  if (a < 0 || a > k) {
    set_error(err, 4u);
    a = a < 0 ? 0 : k;
  }
  const int keep = (a + 1 < k) ? a + 1 : k;
  len[b] += keep - k;
  pos[b] += a + 1 - k;
}

hipError_t launch_rollback(int* len, int* pos, const int* accepted, const int* kseq, int B, int K,
                           unsigned* err, hipStream_t s) {
  hipLaunchKernelGGL(rollback_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, pos, accepted,
                     kseq, B, K, err);
  return hipGetLastError();
}

}  // namespace mtp
