// Decode attention of the MTP layer over its own single-layer cache, with RoPE and the
// cache append fused in, split over the context, then merged by a second kernel.
//
// Grid (split, kv head, sequence). A workgroup owns one KV head and all G query heads
// that share it (GQA), and one chunk of cache positions, so every K/V byte is read from
// HBM once per step. Its K and V rows are requested with 16-byte loads before anything
// else (the new slot excepted), so the HBM round trip overlaps the set-up: q and the new
// key are rotated with the step's cos/sin table (evaluated in fp64 once per call), the
// new key/value are rounded to the cache dtype, and the workgroup whose chunk holds the
// new slot writes them; every workgroup takes that slot's values from LDS, so none
// depends on another's cache write.
// Phase 1: scores (lane groups of LPR lanes reduce one row per head) into LDS.
// Phase 2: per-head max / exp / sum over the chunk.
// Phase 3: P.V with the same row layout, reduced across row groups and waves.
// Each split writes (max, sum, unnormalised o); the merge kernel (one workgroup per
// query head and sequence) combines them with log-sum-exp weights.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kMaxGroup = 8;
constexpr int kRowBatch = 8;  // rows per lane in flight in phases 1 and 3

size_t attn_lds_bytes(int d, int chunk) {
  return sizeof(float) * ((size_t)kMaxGroup * d + 2 * d + (size_t)kMaxGroup * chunk +
                          (size_t)kAttnWaves * kMaxGroup * d);
}

template <class CT, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams p) {
  using T = typename CT::T;
  constexpr int VEC = CT::kVec;
  constexpr int LPR = D / VEC;      // lanes per cache row
  constexpr int PPW = kWave / LPR;  // rows per wave instruction
  constexpr int HALF = D / 2;
  constexpr int RSTEP = kAttnWaves * PPW;  // rows per workgroup instruction
  extern __shared__ __align__(16) float sm[];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, dl = (lane % LPR) * VEC;
  const int G = p.n_q / p.n_kv;
  const int chunk = p.chunk;
  float* q_l = sm;                       // [kMaxGroup][D]
  float* kn = q_l + kMaxGroup * D;       // [D]
  float* vn = kn + D;                    // [D]
  float* sc = vn + D;                    // [kMaxGroup][chunk]
  float* ored = sc + kMaxGroup * chunk;  // [kAttnWaves][kMaxGroup][D]

  const int slot = p.len[b] + p.step;
  const bool overflow = slot >= p.capacity;
  if (overflow && s == 0 && g == 0 && threadIdx.x == 0) set_error(p.err, 2u);
  const int T_valid = overflow ? p.capacity : slot + 1;
  const int t0 = s * chunk;
  const int t1 = min(t0 + chunk, T_valid);
  const long kv_base = ((long)b * p.n_kv + g) * p.capacity;
  T* kc = static_cast<T*>(p.kc);
  T* vc = static_cast<T*>(p.vc);
  const int nj = t1 > t0 ? (t1 - t0 + RSTEP - 1) / RSTEP : 0;  // row iterations per lane
  auto row_of = [&](int j) { return t0 + j * RSTEP + wave * PPW + sub; };

  if (t0 < t1) {
    u32x4 kr[kRowBatch], vr[kRowBatch];
    auto load_rows = [&](u32x4 (&buf)[kRowBatch], const T* base, int j0) {
#pragma unroll
      for (int jj = 0; jj < kRowBatch; ++jj) {
        const int t = row_of(j0 + jj);
        buf[jj] = (j0 + jj < nj && t < t1 && t != slot)
                      ? __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4*>(base + (kv_base + t) * D + dl))
                      : u32x4{0u, 0u, 0u, 0u};
      }
    };
    load_rows(kr, kc, 0);
    load_rows(vr, vc, 0);

    // ---- q (G heads) and the new k, v; RoPE from the step's table; round to cache dtype
    const float* qkv = p.qkv + (long)b * p.ldqkv;
    for (int i = threadIdx.x; i < G * D; i += kAttnThreads) q_l[i] = qkv[(long)g * G * D + i];
    for (int i = threadIdx.x; i < D; i += kAttnThreads) {
      kn[i] = qkv[(long)p.n_q * D + g * D + i];
      vn[i] = qkv[(long)(p.n_q + p.n_kv) * D + g * D + i];
    }
    __syncthreads();
    const float* tab = p.rope + (long)b * D;  // [HALF] cos, then [HALF] sin
    for (int i = threadIdx.x; i < HALF; i += kAttnThreads) {
      const float c = tab[i], sn = tab[HALF + i];
      for (int h = 0; h < G; ++h) {
        const float x1 = q_l[h * D + i], x2 = q_l[h * D + i + HALF];
        q_l[h * D + i] = x1 * c - x2 * sn;
        q_l[h * D + i + HALF] = x2 * c + x1 * sn;
      }
      const float x1 = kn[i], x2 = kn[i + HALF];
      T b1, b2, v1, v2;
      CT::put(&b1, 0, x1 * c - x2 * sn);
      CT::put(&b2, 0, x2 * c + x1 * sn);
      CT::put(&v1, 0, vn[i]);
      CT::put(&v2, 0, vn[i + HALF]);
      kn[i] = CT::get(&b1, 0);
      kn[i + HALF] = CT::get(&b2, 0);
      vn[i] = CT::get(&v1, 0);
      vn[i + HALF] = CT::get(&v2, 0);
      if (!overflow && slot >= t0 && slot < t0 + chunk) {
        const long o = (kv_base + slot) * D;
        kc[o + i] = b1;
        kc[o + i + HALF] = b2;
        vc[o + i] = v1;
        vc[o + i + HALF] = v2;
      }
    }
    __syncthreads();

    // ---- phase 1: scores
    {
      float qr[kMaxGroup][VEC];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) qr[h][e] = (h < G) ? q_l[h * D + dl + e] : 0.f;
      for (int j0 = 0; j0 < nj; j0 += kRowBatch) {
        if (j0 > 0) load_rows(kr, kc, j0);
#pragma unroll
        for (int jj = 0; jj < kRowBatch; ++jj) {
          if (j0 + jj >= nj) break;
          const int t = row_of(j0 + jj);
          float kv[VEC];
          CT::unpack(kr[jj], kv);
          if (t == slot) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) kv[e] = kn[dl + e];
          }
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
              float part = 0.f;
#pragma unroll
              for (int e = 0; e < VEC; ++e) part = fmaf(qr[h][e], kv[e], part);
              part = group_sum<LPR>(part);
              if ((lane % LPR) == 0 && t < t1) sc[h * chunk + (t - t0)] = part * p.scale;
            }
          }
        }
      }
    }
    __syncthreads();

    // ---- phase 2: per-head max, exp, sum over the chunk
    const int n = t1 - t0;
    const long hbase = (long)b * p.n_q + g * G;
    for (int h = wave; h < G; h += kAttnWaves) {
      float m = -INFINITY;
      for (int i = lane; i < n; i += kWave) m = fmaxf(m, sc[h * chunk + i]);
      m = wave_max(m);
      float l = 0.f;
      for (int i = lane; i < n; i += kWave) {
        const float e = expf(sc[h * chunk + i] - m);
        sc[h * chunk + i] = e;
        l += e;
      }
      l = wave_sum(l);
      if (lane == 0) {
        p.part_ml[((hbase + h) * p.nsplit + s) * 2 + 0] = m;
        p.part_ml[((hbase + h) * p.nsplit + s) * 2 + 1] = l;
      }
    }
    __syncthreads();

    // ---- phase 3: unnormalised P.V
    {
      float acc[kMaxGroup][VEC];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
      for (int j0 = 0; j0 < nj; j0 += kRowBatch) {
        if (j0 > 0) load_rows(vr, vc, j0);
#pragma unroll
        for (int jj = 0; jj < kRowBatch; ++jj) {
          if (j0 + jj >= nj) break;
          const int t = row_of(j0 + jj);
          if (t >= t1) continue;
          float vv[VEC];
          CT::unpack(vr[jj], vv);
          if (t == slot) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) vv[e] = vn[dl + e];
          }
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
              const float pr = sc[h * chunk + (t - t0)];
#pragma unroll
              for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(pr, vv[e], acc[h][e]);
            }
          }
        }
      }
      // reduce over the PPW row groups of the wave (lanes with the same dl)
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float v = acc[h][e];
#pragma unroll
            for (int m = LPR; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
            acc[h][e] = v;
          }
        }
      }
      if (sub == 0) {
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
          if (h < G)
#pragma unroll
            for (int e = 0; e < VEC; ++e) ored[(wave * kMaxGroup + h) * D + dl + e] = acc[h][e];
      }
      __syncthreads();
      for (int i = threadIdx.x; i < G * D; i += kAttnThreads) {
        const int h = i / D, dd = i % D;
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) o += ored[(w * kMaxGroup + h) * D + dd];
        p.part_o[((hbase + h) * p.nsplit + s) * D + dd] = o;
      }
    }
  }

}

// Merge the splits of one (query head, sequence): o = sum_q w_q o_q with
// w_q = exp(m_q - M) / sum_q' l_q' exp(m_q' - M). One thread per dimension; the
// split partials are read with all loads of a batch in flight.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnParams p) {
  __shared__ float w[256];
  __shared__ float red[D / kWave];
  const int hq = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int slot = p.len[b] + p.step;
  const int T_valid = slot >= p.capacity ? p.capacity : slot + 1;
  const int nvalid = (T_valid + p.chunk - 1) / p.chunk;
  const long hb = (long)b * p.n_q + hq;
  const float* ml = p.part_ml + hb * p.nsplit * 2;
  float m = -INFINITY;
  for (int q = t; q < nvalid; q += D) m = fmaxf(m, ml[2 * q]);
  m = wave_max(m);
  if (lane == 0) red[wv] = m;
  __syncthreads();
  float M = red[0];
  for (int i = 1; i < D / kWave; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float l = 0.f;
  for (int q = t; q < nvalid; q += D) {
    const float e = expf(ml[2 * q] - M);
    w[q] = e;
    l = fmaf(e, ml[2 * q + 1], l);
  }
  l = wave_sum(l);
  if (lane == 0) red[wv] = l;
  __syncthreads();
  float L = 0.f;
  for (int i = 0; i < D / kWave; ++i) L += red[i];
  const float* po = p.part_o + hb * p.nsplit * D + t;
  constexpr int UB = 16;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < nvalid; q0 += UB) {
    float v[UB];
#pragma unroll
    for (int j = 0; j < UB; ++j) v[j] = (q0 + j < nvalid) ? po[(long)(q0 + j) * D] : 0.f;
#pragma unroll
    for (int j = 0; j < UB; ++j)
      if (q0 + j < nvalid) acc[j & 3] = fmaf(v[j], w[q0 + j], acc[j & 3]);
  }
  p.o[hb * D + t] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) / L;
}

__global__ void rope_tables_kernel(float* tab, const int* pos, int B, int K, int d,
                                   float theta) {
  const int half = d / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= K * B * half) return;
  const int i = e % half, kb = e / half, b = kb % B, k = kb / B;
  const double inv = pow((double)theta, -2.0 * (double)i / (double)d);
  const double ang = (double)(pos[b] + k) * inv;
  tab[(long)kb * d + i] = (float)cos(ang);
  tab[(long)kb * d + half + i] = (float)sin(ang);
}

hipError_t launch_rope_tables(float* tab, const int* pos, int B, int K, int d, float theta,
                              hipStream_t s) {
  const int n = K * B * (d / 2);
  hipLaunchKernelGGL(rope_tables_kernel, dim3((n + 255) / 256), dim3(256), 0, s, tab, pos, B, K,
                     d, theta);
  return hipGetLastError();
}

template <class CT, int D>
static hipError_t launch_attn_t(const AttnParams& p, int B, hipStream_t s) {
  if (p.nsplit > 256 || p.nsplit < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_kernel<CT, D>), dim3(p.nsplit, p.n_kv, B), dim3(kAttnThreads),
                     attn_lds_bytes(D, p.chunk), s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(p.n_q, B), dim3(D), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention(int cdtype, const AttnParams& p, int B, hipStream_t s) {
  if (cdtype == 0) return p.d == 64 ? launch_attn_t<F32, 64>(p, B, s) : launch_attn_t<F32, 128>(p, B, s);
  return p.d == 64 ? launch_attn_t<BF16, 64>(p, B, s) : launch_attn_t<BF16, 128>(p, B, s);
}

}  // namespace mtp
