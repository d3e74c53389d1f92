// Decode attention of the MTP layer over its own single-layer cache, with RoPE and the
// cache append fused in, split over the context, then merged by a second kernel.
//
// Grid: one workgroup per (split, kv head, sequence). A workgroup owns one KV head and all G query heads
// that share it (GQA), and one chunk of cache positions, so every K/V byte is read from
// HBM once per step. Its K and V rows are requested with 16-byte loads before anything
// else (the new slot excepted), so the HBM round trip overlaps the set-up: q and the new
// key are rotated with the step's cos/sin table (evaluated in fp64 once per call), the
// new key/value are rounded to the cache dtype, and the workgroup whose chunk holds the
// new slot writes them; every workgroup takes that slot's values from LDS, so none
// depends on another's cache write.
// K and V rows stream in double-buffered batches of 16-byte loads (the first V batches
// are in flight while the softmax runs); the new slot is never read back from the cache.
// Phase 1: scores into LDS. With a bf16 cache they come from the matrix cores: 16-row
// tiles of K against the group's query heads (q as bf16 hi/lo planes); with an fp32
// cache, lane groups of LPR lanes reduce one row per head on the VALU.
// Phase 2: per-head max / exp / sum over the chunk.
// Phase 3: P.V with the same row layout, reduced across row groups and waves.
// Each split writes (max, sum, unnormalised o); the merge kernel (one workgroup per
// query head and sequence) combines them with log-sum-exp weights.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kAttnWaves = 8;  // waves per workgroup
constexpr int kAttnThreads = kAttnWaves * kWave;
constexpr int kMaxGroup = 8;
constexpr int kAttnJ = 4;  // cache rows per lane per batch (K and V alike)

// Positions per workgroup must be a multiple of this.
int attn_chunk_quantum() { return 128; }

size_t attn_lds_bytes(int d, int chunk) {
  return sizeof(float) * ((size_t)kMaxGroup * d + 2 * d + (size_t)kMaxGroup * chunk +
                          (size_t)kAttnWaves * kMaxGroup * d);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class CT, int D, int GP>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams p) {
  using T = typename CT::T;
  constexpr bool kMfma = sizeof(T) == 2;   // bf16 cache: scores on the matrix cores
  constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte load
  constexpr int LPR = D / VEC;              // lanes per cache row
  constexpr int PPW = kWave / LPR;          // rows per wave instruction
  constexpr int HALF = D / 2;
  constexpr int R1 = kAttnWaves * PPW;      // rows per workgroup instruction
  constexpr int RB = R1 * kAttnJ;           // rows per batch
  constexpr int KS = D / 32;                // MFMA k-steps per 16-slot score tile
  extern __shared__ __align__(16) float sm[];

  // One-dimensional grid, (kv head, sequence) varying fastest: workgroups are dealt to the
  // XCDs round-robin, so each XCD takes whole heads of every sequence and the ragged split
  // work of different sequences spreads evenly (split-major order would give XCD i all of
  // split i, the late splits of short sequences being empty).
  const int ngb = p.n_kv * p.batch;
  const int s = (int)blockIdx.x / ngb;
  const int g = (int)blockIdx.x % p.n_kv, b = ((int)blockIdx.x % ngb) / p.n_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  if (overflow && s == 0 && g == 0 && tid == 0) set_error(p.err, 2u);
  const int T_valid = overflow ? p.capacity : slot + 1;
  const int t0 = s * chunk;
  const int t1 = min(t0 + chunk, T_valid);
  if (t0 >= t1) return;  // nothing cached in this split (the merge skips it)
  // Cached rows [t0, te) are streamed from memory; the new slot (when it falls in this
  // chunk) is handled from LDS, so every streamed row is real, finite cache data.
  const bool has_new = !overflow && slot >= t0 && slot < t1;
  const int te = has_new ? slot : t1;
  const int ns = te - t0;  // streamed rows (0 when the chunk holds only the new slot)
  const long kv_base = ((long)b * p.n_kv + g) * p.capacity;
  T* kc = static_cast<T*>(p.kc);
  T* vc = static_cast<T*>(p.vc);
  const int n = t1 - t0;
  const int nbat = (ns + RB - 1) / RB;  // V batches
  const int ntile = (ns + 15) / 16;     // score tiles (matrix-core path)
  const int last = ns > 0 ? te - 1 : t0;  // clamp target of rows past the stream (real data
                                          // whenever anything is streamed)

  // ---- set-up operands first (small, cache-resident): q pairs, new k/v, cos/sin. Every
  // thread loads (threads past HALF duplicate), so no load sits behind a branch.
  float qa[GP], qb[GP];
  const float* qkv = p.qkv + (long)b * p.ldqkv;
  const int ti = tid % HALF;
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    const int hh = g * G + (h < G ? h : G - 1);
    qa[h] = qkv[(long)hh * D + ti];
    qb[h] = qkv[(long)hh * D + ti + HALF];
  }
  const float k1 = qkv[(long)p.n_q * D + g * D + ti];
  const float k2 = qkv[(long)p.n_q * D + g * D + ti + HALF];
  const float v1 = qkv[(long)(p.n_q + p.n_kv) * D + g * D + ti];
  const float v2 = qkv[(long)(p.n_q + p.n_kv) * D + g * D + ti + HALF];
  const float cs = p.rope[(long)b * D + ti];
  const float sn = p.rope[(long)b * D + HALF + ti];
  __builtin_amdgcn_sched_barrier(0);  // set-up loads stay ahead of the K/V stream

  // ---- K stream. Matrix-core path: wave w takes 16-row tiles w, w + 8, ...; lane l reads
  // 16 bytes of row (tile * 16 + l % 16) at dims 8 * (l / 16) + 32 * k. VALU path: lane
  // (sub, dl) reads elements dl..dl+VEC-1 of row t0 + batch * RB + jj * R1 + w * PPW + sub.
  auto row_of = [&](int bt, int jj) { return t0 + bt * RB + jj * R1 + wave * PPW + sub; };
  auto clamp_row = [&](int t) { return t < te ? t : last; };
  u32x4 kt0[KS], kt1[KS];
  auto load_tile = [&](u32x4 (&buf)[KS], int j) {
    const int t = clamp_row(t0 + (wave + j * kAttnWaves) * 16 + (lane & 15));
#pragma unroll
    for (int k = 0; k < KS; ++k)
      buf[k] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kc + (kv_base + t) * D + k * 32 + (lane >> 4) * 8));
  };
  u32x4 buf0[kAttnJ], buf1[kAttnJ];
  auto load_batch = [&](const T* base, u32x4 (&buf)[kAttnJ], int bt) {
#pragma unroll
    for (int jj = 0; jj < kAttnJ; ++jj) {
      const int t = clamp_row(row_of(bt, jj));
      buf[jj] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(base + (kv_base + t) * D + dl));
    }
  };
  if constexpr (kMfma) {
    load_tile(kt0, 0);
    load_tile(kt1, 1);
  } else {
    load_batch(kc, buf0, 0);
    load_batch(kc, buf1, 1);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- RoPE (rotate-half) on q and the new key; round k, v to the cache dtype
  if (tid < HALF) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h < G) {
        q_l[h * D + tid] = qa[h] * cs - qb[h] * sn;
        q_l[h * D + tid + HALF] = qb[h] * cs + qa[h] * sn;
      }
    }
    T b1, b2, w1, w2;
    CT::put(&b1, 0, k1 * cs - k2 * sn);
    CT::put(&b2, 0, k2 * cs + k1 * sn);
    CT::put(&w1, 0, v1);
    CT::put(&w2, 0, v2);
    kn[tid] = CT::get(&b1, 0);
    kn[tid + HALF] = CT::get(&b2, 0);
    vn[tid] = CT::get(&w1, 0);
    vn[tid + HALF] = CT::get(&w2, 0);
  }
  __syncthreads();

  // ---- phase 1: scores s[h][t] = q_h . k_t * scale into LDS
  if constexpr (kMfma) {
    // S^T (16 rows x 16 heads) = K (16 x D) . Q^T (D x 16): q enters as bf16 planes
    // hi + lo (two MFMAs per k-step), so it keeps ~16 bits; heads >= G are zero.
    const int hq = lane & 15;
    bf16x8 qh[KS], qlo[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = hq < G ? q_l[hq * D + k * 32 + (lane >> 4) * 8 + e] : 0.f;
        uint16_t hi, lo;
        split_bf16(v, hi, lo);
        qh[k][e] = __builtin_bit_cast(__bf16, hi);
        qlo[k][e] = __builtin_bit_cast(__bf16, lo);
      }
    }
    auto score_tile = [&](u32x4 (&buf)[KS], int j) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const bf16x8 kk = __builtin_bit_cast(bf16x8, buf[k]);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qh[k], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qlo[k], a, 0, 0, 0);
      }
      // lane l holds rows 4 * (l / 16) + i of the tile for head l % 16
      const int r0 = (wave + j * kAttnWaves) * 16 + (lane >> 4) * 4;
      if (hq < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < ns) sc[hq * chunk + r0 + i] = a[i] * p.scale;
      }
    };
    const int my_tiles = wave < ntile ? (ntile - 1 - wave) / kAttnWaves + 1 : 0;
    for (int j = 0; j < my_tiles; j += 2) {
      score_tile(kt0, j);
      load_tile(kt0, j + 2);
      if (j + 1 >= my_tiles) break;
      score_tile(kt1, j + 1);
      load_tile(kt1, j + 3);
    }
    // the first V batches go out before the softmax
    load_batch(vc, buf0, 0);
    load_batch(vc, buf1, 1);
  } else {
    float qr[GP][VEC];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) qr[h][e] = q_l[(h < G ? h : 0) * D + dl + e];
    auto scores = [&](u32x4 (&buf)[kAttnJ], int bt) {
#pragma unroll
      for (int jj = 0; jj < kAttnJ; ++jj) {
        const int t = row_of(bt, jj);
        float kv[VEC];
        CT::unpack(buf[jj], kv);
        float part[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          part[h] = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) part[h] = fmaf(qr[h][e], kv[e], part[h]);
        }
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if constexpr (LPR <= 16) {
            part[h] = dpp_group_sum<LPR>(part[h]);
          } else {
            part[h] = dpp_group_sum<16>(part[h]);
            part[h] += __shfl_xor(part[h], 16, kWave);
          }
        }
        if ((lane % LPR) == 0 && t < te) {
#pragma unroll
          for (int h = 0; h < GP; ++h)
            if (h < G) sc[h * chunk + (t - t0)] = part[h] * p.scale;
        }
      }
    };
    for (int bt = 0; bt < nbat; bt += 2) {
      scores(buf0, bt);
      load_batch(kc, buf0, bt + 2);
      if (bt + 1 >= nbat) break;
      scores(buf1, bt + 1);
      load_batch(kc, buf1, bt + 3);
    }
    load_batch(vc, buf0, 0);
    load_batch(vc, buf1, 1);
  }
  // the new slot's score, from LDS (q and the rounded new key)
  if (has_new && wave == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h < G) {
        float d0 = 0.f;
        for (int e = lane; e < D; e += kWave) d0 = fmaf(q_l[h * D + e], kn[e], d0);
        d0 = wave_sum_fast(d0);
        if (lane == 0) sc[h * chunk + (slot - t0)] = d0 * p.scale;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: per-head max, exp, sum over the chunk (the first V batches are in flight)
  const long hbase = (long)b * p.n_q + g * G;
  for (int h = wave; h < G; h += kAttnWaves) {
    float m = -INFINITY;
    for (int i = lane; i < n; i += kWave) m = fmaxf(m, sc[h * chunk + i]);
    m = wave_max_fast(m);
    float l = 0.f;
    for (int i = lane; i < n; i += kWave) {
      const float e = expf(sc[h * chunk + i] - m);
      sc[h * chunk + i] = e;
      l += e;
    }
    l = wave_sum_fast(l);
    if (lane == 0) {
      p.part_ml[((hbase + h) * p.nsplit + s) * 2 + 0] = m;
      p.part_ml[((hbase + h) * p.nsplit + s) * 2 + 1] = l;
    }
  }
  __syncthreads();

  // ---- phase 3: unnormalised P.V over the streamed rows (rows past the stream get weight
  // 0; their clamped values are real data), then the new slot's row from LDS. Partial sums
  // are reduced over the PPW rows of a wave instruction (lane shuffles) and over the waves
  // (LDS).
  {
    float acc[GP][VEC];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
    auto pv = [&](u32x4 (&buf)[kAttnJ], int bt) {
#pragma unroll
      for (int jj = 0; jj < kAttnJ; ++jj) {
        const int t = row_of(bt, jj);
        const bool live = t < te;
        const int tc = (live ? t : last) - t0;
        float pr[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) pr[h] = live ? sc[(h < G ? h : 0) * chunk + tc] : 0.f;
        float vv[VEC];
        CT::unpack(buf[jj], vv);
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(pr[h], vv[e], acc[h][e]);
      }
    };
    for (int bt = 0; bt < nbat; bt += 2) {
      pv(buf0, bt);
      load_batch(vc, buf0, bt + 2);
      if (bt + 1 >= nbat) break;
      pv(buf1, bt + 1);
      load_batch(vc, buf1, bt + 3);
    }
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float v = acc[h][e];
#pragma unroll
        for (int m = LPR; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
        acc[h][e] = v;
      }
    if (has_new && wave == 0 && lane < LPR) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float pn = sc[(h < G ? h : 0) * chunk + (slot - t0)];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(pn, vn[dl + e], acc[h][e]);
      }
    }
    if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < GP; ++h)
        if (h < G)
#pragma unroll
          for (int e = 0; e < VEC; ++e) ored[(wave * kMaxGroup + h) * D + dl + e] = acc[h][e];
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kAttnThreads) {
      const int h = i / D, dd = i % D;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) o += ored[(w * kMaxGroup + h) * D + dd];
      p.part_o[((hbase + h) * p.nsplit + s) * D + dd] = o;
    }
  }
  // ---- the workgroup whose chunk holds the new slot appends it to the cache
  if (has_new && tid < D) {
    const long o = (kv_base + slot) * D + tid;
    CT::put(kc, o, kn[tid]);
    CT::put(vc, o, vn[tid]);
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
  constexpr int UB = 32;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < nvalid; q0 += UB) {
    float v[UB];
#pragma unroll
    for (int j = 0; j < UB; ++j) v[j] = (q0 + j < nvalid) ? po[(long)(q0 + j) * D] : 0.f;
#pragma unroll
    for (int j = 0; j < UB; ++j)
      if (q0 + j < nvalid) acc[j & 3] = fmaf(v[j], w[q0 + j], acc[j & 3]);
  }
  const float r = ((acc[0] + acc[1]) + (acc[2] + acc[3])) / L;
  if (p.o_bf16) {
    const long i = (long)b * p.ld_o_bf16 + hq * D + t;
    split_bf16(r, p.o_bf16[i], p.o_bf16_lo[i]);
  } else
    p.o[hb * D + t] = r;
}

// Per-call set-up: RoPE tables of the K steps (tab[k][b][0..d/2) = cos, [d/2..d) = sin of
// (pos[b] + k) * theta^(-2i/d), evaluated in fp64 and rounded to fp32) and the verifier
// hidden state widened to fp32 (the first step's input).
template <class CT>
__global__ void draft_setup_kernel(float* tab, const int* pos, int B, int K, int d, float theta,
                                   const void* hidden, float* hf, int H) {
  const int half = d / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < K * B * half) {
    const int i = e % half, kb = e / half, b = kb % B, k = kb / B;
    rope_cs(pos[b] + k, i, d, theta, tab[(long)kb * d + i], tab[(long)kb * d + half + i]);
  }
  if (e < B * H) hf[e] = CT::get(static_cast<const typename CT::T*>(hidden), e);
}

hipError_t launch_draft_setup(int dtype, float* tab, const int* pos, int B, int K, int d,
                              float theta, const void* hidden, float* hf, int H, hipStream_t s) {
  const int n1 = K * B * (d / 2), n2 = B * H;
  const int n = n1 > n2 ? n1 : n2;
  if (dtype == 0)
    hipLaunchKernelGGL(draft_setup_kernel<F32>, dim3((n + 255) / 256), dim3(256), 0, s, tab, pos,
                       B, K, d, theta, hidden, hf, H);
  else
    hipLaunchKernelGGL(draft_setup_kernel<BF16>, dim3((n + 255) / 256), dim3(256), 0, s, tab, pos,
                       B, K, d, theta, hidden, hf, H);
  return hipGetLastError();
}

template <class CT, int D, int GP>
static hipError_t launch_attn_g(const AttnParams& p, int B, hipStream_t s) {
  AttnParams q = p;
  q.batch = B;
  hipLaunchKernelGGL((attn_kernel<CT, D, GP>), dim3(p.nsplit * p.n_kv * B), dim3(kAttnThreads),
                     attn_lds_bytes(D, p.chunk), s, q);
  return hipGetLastError();
}

template <class CT, int D>
static hipError_t launch_attn_t(const AttnParams& p, int B, hipStream_t s) {
  if (p.nsplit > 256 || p.nsplit < 1 || p.chunk % attn_chunk_quantum() != 0)
    return hipErrorInvalidValue;
  const int G = p.n_q / p.n_kv;
  hipError_t e0;
  if (G <= 1) e0 = launch_attn_g<CT, D, 1>(p, B, s);
  else if (G <= 2) e0 = launch_attn_g<CT, D, 2>(p, B, s);
  else if (G <= 4) e0 = launch_attn_g<CT, D, 4>(p, B, s);
  else if (G <= 8) e0 = launch_attn_g<CT, D, 8>(p, B, s);
  else return hipErrorInvalidValue;
  if (e0 != hipSuccess) return e0;
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
