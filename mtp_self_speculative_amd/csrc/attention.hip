// Decode attention of the MTP layer over its own single-layer cache, with RoPE and the
// cache append fused in, split over the context and combined by the last workgroup.
//
// Grid (split, kv head, sequence). A workgroup owns one KV head and all G query heads
// that share it (GQA), and one chunk of cache positions, so every K/V byte is read from
// HBM once per step. It rotates q and the new key itself (cos/sin evaluated in fp64 from
// the integer position), rounds the new key/value to the cache dtype, and the workgroup
// whose chunk contains the new slot writes it; every workgroup uses the rounded values
// from LDS for that slot, so no workgroup depends on another's cache write.
// Phase 1: scores for the chunk (16-byte K loads, lane groups reduce per row) into LDS.
// Phase 2: per-head max / exp / sum over the chunk. Phase 3: P.V with lanes owning
// dimensions. Each split writes (max, sum, unnormalised o); the last workgroup of a
// (sequence, kv head) merges the splits with the usual log-sum-exp rescaling.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kMaxGroup = 8;

template <class CT, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams p) {
  using T = typename CT::T;
  constexpr int VEC = CT::kVec;
  constexpr int LPR = D / VEC;     // lanes per cache row in phase 1
  constexpr int PPW = kWave / LPR; // rows per wave instruction in phase 1
  constexpr int DPL = D / kWave;   // dimensions per lane in phase 3
  constexpr int HALF = D / 2;
  extern __shared__ float sm[];
  __shared__ int flag;

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = p.n_q / p.n_kv;
  const int chunk = p.chunk;
  float* q_l = sm;                       // [kMaxGroup][D]
  float* kn = q_l + kMaxGroup * D;       // [D]
  float* vn = kn + D;                    // [D]
  float* sc = vn + D;                    // [kMaxGroup][chunk]
  float* ored = sc + kMaxGroup * chunk;  // [kAttnWaves][kMaxGroup][D]

  const int slot = p.len[b] + p.step;
  const int position = p.pos[b] + p.step;
  const bool overflow = slot >= p.capacity;
  if (overflow && s == 0 && g == 0 && threadIdx.x == 0) set_error(p.err, 2u);
  const int T_valid = overflow ? p.capacity : slot + 1;
  const int t0 = s * chunk;
  const int t1 = min(t0 + chunk, T_valid);
  const long kv_base = ((long)b * p.n_kv + g) * p.capacity;
  T* kc = static_cast<T*>(p.kc);
  T* vc = static_cast<T*>(p.vc);

  if (t0 < t1) {
    // ---- q (G heads) and the new k, v of this kv head; RoPE; round k, v to the cache dtype
    const float* qkv = p.qkv + (long)b * p.ldqkv;
    for (int i = threadIdx.x; i < G * D; i += kAttnThreads) q_l[i] = qkv[(long)g * G * D + i];
    for (int i = threadIdx.x; i < D; i += kAttnThreads) {
      kn[i] = qkv[(long)p.n_q * D + g * D + i];
      vn[i] = qkv[(long)(p.n_q + p.n_kv) * D + g * D + i];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < HALF; i += kAttnThreads) {
      const double inv = pow((double)p.theta, -2.0 * (double)i / (double)D);
      const double ang = (double)position * inv;
      const float c = (float)cos(ang), sn = (float)sin(ang);
      for (int h = 0; h < G; ++h) {
        const float x1 = q_l[h * D + i], x2 = q_l[h * D + i + HALF];
        q_l[h * D + i] = x1 * c - x2 * sn;
        q_l[h * D + i + HALF] = x2 * c + x1 * sn;
      }
      const float x1 = kn[i], x2 = kn[i + HALF];
      const float r1 = x1 * c - x2 * sn, r2 = x2 * c + x1 * sn;
      T b1, b2, v1, v2;
      CT::put(&b1, 0, r1); CT::put(&b2, 0, r2);
      CT::put(&v1, 0, vn[i]); CT::put(&v2, 0, vn[i + HALF]);
      kn[i] = CT::get(&b1, 0); kn[i + HALF] = CT::get(&b2, 0);
      vn[i] = CT::get(&v1, 0); vn[i + HALF] = CT::get(&v2, 0);
      if (!overflow && slot >= t0 && slot < t0 + chunk) {
        const long o = (kv_base + slot) * D;
        kc[o + i] = b1; kc[o + i + HALF] = b2;
        vc[o + i] = v1; vc[o + i + HALF] = v2;
      }
    }
    __syncthreads();

    // ---- phase 1: scores
    {
      const int sub = lane / LPR, dl = (lane % LPR) * VEC;
      float qr[kMaxGroup][VEC];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int q = 0; q < VEC; ++q) qr[h][q] = (h < G) ? q_l[h * D + dl + q] : 0.f;
      for (int tb = t0 + wave * PPW; tb < t1; tb += kAttnWaves * PPW) {
        const int t = tb + sub;
        float kv[VEC];
        if (t < t1 && t != slot) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(kc + (kv_base + t) * D + dl);
          CT::unpack(raw, kv);
        } else {
#pragma unroll
          for (int q = 0; q < VEC; ++q) kv[q] = (t == slot) ? kn[dl + q] : 0.f;
        }
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
            float part = 0.f;
#pragma unroll
            for (int q = 0; q < VEC; ++q) part = fmaf(qr[h][q], kv[q], part);
            part = group_sum<LPR>(part);
            if ((lane % LPR) == 0 && t < t1) sc[h * chunk + (t - t0)] = part * p.scale;
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
      float acc[kMaxGroup][DPL];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[h][j] = 0.f;
      const int dim = lane * DPL;
      for (int t = t0 + wave; t < t1; t += kAttnWaves) {
        float vv[DPL];
        if (t == slot) {
#pragma unroll
          for (int j = 0; j < DPL; ++j) vv[j] = vn[dim + j];
        } else {
#pragma unroll
          for (int j = 0; j < DPL; ++j) vv[j] = CT::get(vc, (kv_base + t) * D + dim + j);
        }
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
            const float pr = sc[h * chunk + (t - t0)];
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[h][j] = fmaf(pr, vv[j], acc[h][j]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int j = 0; j < DPL; ++j) ored[(wave * kMaxGroup + h) * D + dim + j] = acc[h][j];
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

  // ---- the last split of this (sequence, kv head) merges all splits
  if (last_to_arrive(p.counters + (long)b * p.n_kv + g, gridDim.x, &flag)) {
    __threadfence();
    const int nvalid = (T_valid + chunk - 1) / chunk;
    const long hbase = (long)b * p.n_q + g * G;
    for (int i = threadIdx.x; i < G * D; i += kAttnThreads) {
      const int h = i / D, dd = i % D;
      const float* ml = p.part_ml + (hbase + h) * p.nsplit * 2;
      float M = -INFINITY;
      for (int q = 0; q < nvalid; ++q) M = fmaxf(M, ml[2 * q]);
      float L = 0.f, acc = 0.f;
      const float* po = p.part_o + (hbase + h) * p.nsplit * D + dd;
      for (int q = 0; q < nvalid; ++q) {
        const float w = expf(ml[2 * q] - M);
        L = fmaf(ml[2 * q + 1], w, L);
        acc = fmaf(po[(long)q * D], w, acc);
      }
      p.o[(hbase + h) * D + dd] = acc / L;
    }
  }
}

size_t attn_lds_bytes(int d, int chunk) {
  return sizeof(float) * ((size_t)kMaxGroup * d + 2 * d + (size_t)kMaxGroup * chunk +
                          (size_t)kAttnWaves * kMaxGroup * d);
}

template <class CT, int D>
static hipError_t launch_attn_t(const AttnParams& p, int B, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<CT, D>), dim3(p.nsplit, p.n_kv, B), dim3(kAttnThreads),
                     attn_lds_bytes(D, p.chunk), s, p);
  return hipGetLastError();
}

hipError_t launch_attention(int cdtype, const AttnParams& p, int B, hipStream_t s) {
  if (cdtype == 0) return p.d == 64 ? launch_attn_t<F32, 64>(p, B, s) : launch_attn_t<F32, 128>(p, B, s);
  return p.d == 64 ? launch_attn_t<BF16, 64>(p, B, s) : launch_attn_t<BF16, 128>(p, B, s);
}

}  // namespace mtp
