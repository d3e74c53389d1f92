// Decode attention of the MTP layer over its own single-layer cache, with RoPE and the
// cache append fused in, split over the context, then merged by a second kernel.
//
// Grid: one workgroup per (split, kv head, sequence) item, natural index
// (split * B + sequence) * n_kv + kv head. Workgroups are dealt to the XCDs round-robin,
// so with the kv head varying fastest each XCD takes whole heads of every sequence.
// Launched in natural order, the full chunks of long sequences' late splits would start
// last and run alone; with more items than fit at once, a one-workgroup plan kernel
// (once per draft call) orders them longest first instead (attn_plan_kernel).
// A workgroup owns one KV head and all G query heads that share it (GQA), and one chunk
// of cache positions, so every K/V byte is read from HBM once per step. Its first K and V
// rows are requested before anything else, so the HBM round trip overlaps the set-up: q
// and the new key are rotated with the step's cos/sin table (evaluated in fp64 once per
// call), the new key/value are rounded to the cache dtype, and the workgroup whose chunk
// holds the new slot writes them; every workgroup takes that slot's values from LDS, so
// none depends on another's cache write and the new slot is never read back from memory.
//
// bf16 cache (attn_flash_kernel): one pass over the chunk with an online softmax. Each
// wave walks its own 16-row tiles with K and V tiles of several tiles in flight; the
// scores of a tile are one matrix-core product of the K tile with the group's query heads
// (q as bf16 hi/lo planes), the softmax state (running max, sum) lives in registers, and
// P.V is a second matrix-core product with the weights as hi/lo planes and the V tile
// transposed in registers. The waves' (max, sum, o) are combined in LDS at the end.
// fp32 cache (attn_kernel): scores into LDS from lane groups that reduce one row per head
// on the VALU, per-head max / exp / sum over the chunk, then P.V with the same row
// layout, reduced across row groups and waves.
// Each split writes (max, sum, unnormalised o); the merge kernel (one workgroup per
// query head and sequence) combines them with log-sum-exp weights.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kMaxGroup = 8;
constexpr int kAttnWaves = 8;  // waves per workgroup (fp32 cache)
constexpr int kAttnThreads = kAttnWaves * kWave;
constexpr int kAttnJ = 4;  // cache rows per lane per batch (K and V alike)
constexpr int kFlashWaves = 4;  // waves per workgroup (bf16 cache)
constexpr int kFlashThreads = kFlashWaves * kWave;
constexpr int kFlashStages = 3;  // K + V tiles in flight per wave

// Positions per workgroup must be a multiple of this.
int attn_chunk_quantum() { return 128; }
// Longest chunk: the fp32 kernel keeps a chunk's scores in LDS, the bf16 one does not.
int attn_max_chunk(int cdtype) { return cdtype == 0 ? 1024 : 2048; }

size_t attn_lds_bytes(int d, int chunk) {
  return sizeof(float) * ((size_t)kMaxGroup * d + 2 * d + (size_t)kMaxGroup * chunk +
                          (size_t)kAttnWaves * kMaxGroup * d);
}
size_t flash_lds_bytes(int d) {
  return sizeof(float) * ((size_t)kMaxGroup * d + 2 * d + kMaxGroup +
                          (size_t)kFlashWaves * kMaxGroup * (d + 2));
}

// Positions per split of this call.
__device__ __forceinline__ int attn_chunk(const AttnParams& p) {
  return p.chunk_dev ? *p.chunk_dev : p.chunk;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D, int GP>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams p) {
  using CT = F32;
  using T = float;
  constexpr int VEC = 4;                    // elements per 16-byte load
  constexpr int LPR = D / VEC;              // lanes per cache row
  constexpr int PPW = kWave / LPR;          // rows per wave instruction
  constexpr int HALF = D / 2;
  constexpr int R1 = kAttnWaves * PPW;      // rows per workgroup instruction
  constexpr int RB = R1 * kAttnJ;           // rows per batch
  extern __shared__ __align__(16) float sm[];

  const int item = p.perm ? p.perm[blockIdx.x] : (int)blockIdx.x;
  const int ngb = p.n_kv * p.batch;
  const int s = item / ngb;
  const int g = item % p.n_kv, b = (item % ngb) / p.n_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, dl = (lane % LPR) * VEC;
  const int G = p.n_q / p.n_kv;
  const int chunk = attn_chunk(p);  // LDS is sized for p.chunk >= chunk
  float* q_l = sm;                       // [kMaxGroup][D]
  float* kn = q_l + kMaxGroup * D;       // [D]
  float* vn = kn + D;                    // [D]
  float* sc = vn + D;                    // [kMaxGroup][chunk]
  float* ored = sc + kMaxGroup * chunk;  // [kAttnWaves][kMaxGroup][D]

  // A masked sequence (past its own step count) attends to its new key alone: slot 0 of an
  // empty cache, which only split 0 holds and which comes from LDS, never from memory.
  const bool masked = p.kseq && p.step >= seq_steps(p.kseq, b, p.step + 1);
  const int slot = masked ? 0 : p.len[b] + p.step;
  const bool overflow = !masked && slot >= p.capacity;
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
  const int nbat = (ns + RB - 1) / RB;  // K / V batches
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

  // ---- K stream: lane (sub, dl) reads elements dl..dl+VEC-1 of row
  // t0 + batch * RB + jj * R1 + w * PPW + sub.
  auto row_of = [&](int bt, int jj) { return t0 + bt * RB + jj * R1 + wave * PPW + sub; };
  auto clamp_row = [&](int t) { return t < te ? t : last; };
  u32x4 buf0[kAttnJ], buf1[kAttnJ];
  auto load_batch = [&](const T* base, u32x4 (&buf)[kAttnJ], int bt) {
#pragma unroll
    for (int jj = 0; jj < kAttnJ; ++jj) {
      const int t = clamp_row(row_of(bt, jj));
      buf[jj] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(base + (kv_base + t) * D + dl));
    }
  };
  load_batch(kc, buf0, 0);
  load_batch(kc, buf1, 1);
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
  // the first V batches go out before the softmax
  load_batch(vc, buf0, 0);
  load_batch(vc, buf1, 1);
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
  if (has_new && !masked && tid < D) {
    const long o = (kv_base + slot) * D + tid;
    CT::put(kc, o, kn[tid]);
    CT::put(vc, o, vn[tid]);
  }
}

// bf16 cache: one pass over the chunk with an online softmax, both products on the
// matrix cores. Wave w takes the chunk's 16-row tiles w, w + 4, ...; for each it holds
//   K tile (A operand of 16x16x32): lane l has row l % 16 at dims 32 k + 8 (l / 16) + 0..7;
//   V tile: lane (r, c) = (l / 16, l % 16) has rows 4 r .. 4 r + 3 at dims c D/16 ...
//   (c + 1) D/16 - 1.
// The score tile S^T = K Q^T leaves lane l with rows 4 r + i (i = 0..3) of head c, which
// is exactly the B operand layout of the 16x16x16 product O^T += V^T P^T (B[k][n] = P of
// head n at row k, k = 4 r + i), so the weights never leave their lanes. The A operand
// V^T needs, per lane, one dim at four consecutive rows: two byte permutes per pair of
// dims turn the lane's 4 x (D/16) block into D/16 such operands. O^T tile j then holds
// O[head c][dim (D/16)(4 r + i) + j] in lane (r, c), element i.
template <int D, int GP>
__global__ __launch_bounds__(kFlashThreads) void attn_flash_kernel(AttnParams p) {
  constexpr int KS = D / 32;   // 16x16x32 k-steps of a score tile
  constexpr int VD = D / 16;   // dims per lane of a V tile row
  constexpr int VW = VD / 2;   // 32-bit words per lane of a V tile row
  constexpr int NS = kFlashStages;
  constexpr int HALF = D / 2;
  extern __shared__ __align__(16) float sm[];
  const int item = p.perm ? p.perm[blockIdx.x] : (int)blockIdx.x;
  const int ngb = p.n_kv * p.batch;
  const int s = item / ngb;
  const int g = item % p.n_kv, b = (item % ngb) / p.n_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r4 = lane >> 4, c16 = lane & 15;
  const int G = p.n_q / p.n_kv;
  float* q_l = sm;                                // [kMaxGroup][D]
  float* kn = q_l + kMaxGroup * D;                // [D]
  float* vn = kn + D;                             // [D]
  float* snew = vn + D;                           // [kMaxGroup]
  float* wml = snew + kMaxGroup;                  // [kFlashWaves][kMaxGroup][2]
  float* wo = wml + kFlashWaves * kMaxGroup * 2;  // [kFlashWaves][kMaxGroup][D]

  // A masked sequence (past its own step count) attends to its new key alone: slot 0 of an
  // empty cache, which only split 0 holds and which comes from LDS, never from memory.
  const bool masked = p.kseq && p.step >= seq_steps(p.kseq, b, p.step + 1);
  const int slot = masked ? 0 : p.len[b] + p.step;
  const bool overflow = !masked && slot >= p.capacity;
  if (overflow && s == 0 && g == 0 && tid == 0) set_error(p.err, 2u);
  const int T_valid = overflow ? p.capacity : slot + 1;
  const int chunk = attn_chunk(p);
  const int t0 = s * chunk;
  const int t1 = min(t0 + chunk, T_valid);
  if (t0 >= t1) return;  // nothing cached in this split (the merge skips it)
  // Cached rows [t0, te) are streamed; the new slot (when in this chunk) comes from LDS.
  const bool has_new = !overflow && slot >= t0 && slot < t1;
  const int te = has_new ? slot : t1;
  const int ns = te - t0;
  const long kv_base = ((long)b * p.n_kv + g) * p.capacity;
  const uint16_t* kc = static_cast<const uint16_t*>(p.kc);
  const uint16_t* vc = static_cast<const uint16_t*>(p.vc);
  const int ntile = (ns + 15) / 16;
  const int my_tiles = wave < ntile ? (ntile - 1 - wave) / kFlashWaves + 1 : 0;
  const int last = ns > 0 ? te - 1 : t0;  // clamp target of rows past the stream

  // ---- set-up operands (small, cache-resident): q pairs, new k/v, cos/sin
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
  __builtin_amdgcn_sched_barrier(0);

  // ---- the first NS tiles of K and V go out before the set-up is used. Tiles past the
  // wave's last one read clamped rows (real data, never used), so every stage is a load.
  u32x4 kb[NS][KS];
  uint32_t vb[NS][4][VW];
  auto clamp_row = [&](int t) { return t < te ? t : last; };
  auto issue = [&](int st, int j) {
    const int base = t0 + (wave + j * kFlashWaves) * 16;
    const int tk = clamp_row(base + c16);
#pragma unroll
    for (int k = 0; k < KS; ++k)
      kb[st][k] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kc + (kv_base + tk) * D + k * 32 + r4 * 8));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t* src = vc + (kv_base + clamp_row(base + 4 * r4 + e)) * D + c16 * VD;
      if constexpr (VW == 4) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
#pragma unroll
        for (int q = 0; q < 4; ++q) vb[st][e][q] = x[q];
      } else {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
        vb[st][e][0] = x[0];
        vb[st][e][1] = x[1];
      }
    }
  };
#pragma unroll
  for (int st = 0; st < NS; ++st) issue(st, st);
  __builtin_amdgcn_sched_barrier(0);

  // ---- RoPE (rotate-half) on q and the new key; new k, v rounded to bf16
  if (tid < HALF) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h < G) {
        q_l[h * D + tid] = qa[h] * cs - qb[h] * sn;
        q_l[h * D + tid + HALF] = qb[h] * cs + qa[h] * sn;
      }
    }
    kn[tid] = bf16_to_f32(f32_to_bf16(k1 * cs - k2 * sn));
    kn[tid + HALF] = bf16_to_f32(f32_to_bf16(k2 * cs + k1 * sn));
    vn[tid] = bf16_to_f32(f32_to_bf16(v1));
    vn[tid + HALF] = bf16_to_f32(f32_to_bf16(v2));
  }
  __syncthreads();

  // Scores are kept in base 2: s2 = q.k * scale * log2(e), weights 2^(s2 - max).
  const float scale2 = p.scale * kLog2e;
  if (has_new && wave == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h < G) {
        float d0 = 0.f;
        for (int e = lane; e < D; e += kWave) d0 = fmaf(q_l[h * D + e], kn[e], d0);
        d0 = wave_sum_fast(d0);
        if (lane == 0) snew[h] = d0 * scale2;
      }
    }
  }
  // q as bf16 hi / lo planes in the B layout of the score product (heads >= G are zero)
  bf16x8 qh[KS], qlo[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = c16 < G ? q_l[c16 * D + k * 32 + r4 * 8 + e] : 0.f;
      uint16_t hi, lo;
      split_bf16(v, hi, lo);
      qh[k][e] = __builtin_bit_cast(__bf16, hi);
      qlo[k][e] = __builtin_bit_cast(__bf16, lo);
    }
  }

  // Softmax state of head c16 over this wave's rows: running max M, this lane's share of
  // the sum L (rows 4 r4 .. 4 r4 + 3 of each tile) and the O^T tiles.
  float M = -INFINITY, L = 0.f;
  f32x4 acc[VD];
#pragma unroll
  for (int j = 0; j < VD; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](int st, int j) {
    const int base = t0 + (wave + j * kFlashWaves) * 16;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const bf16x8 kk = __builtin_bit_cast(bf16x8, kb[st][k]);
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qh[k], a, 0, 0, 0);
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qlo[k], a, 0, 0, 0);
    }
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (base + 4 * r4 + i < te) ? a[i] * scale2 : -INFINITY;
    float tm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    tm = fmaxf(tm, __shfl_xor(tm, 16, kWave));
    tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
    const float mn = fmaxf(M, tm);  // finite: row base of every processed tile is streamed
    const float alpha = hw_exp2(M - mn);
    M = mn;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = hw_exp2(sv[i] - mn);
    L = fmaf(L, alpha, (pv[0] + pv[1]) + (pv[2] + pv[3]));
#pragma unroll
    for (int jj = 0; jj < VD; ++jj) acc[jj] *= alpha;
    s16x4 ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t hi, lo;
      split_bf16(pv[i], hi, lo);
      ph[i] = (short)hi;
      pl[i] = (short)lo;
    }
#pragma unroll
    for (int q = 0; q < VW; ++q) {
      // rows 0..3 of dims 2q (low halves) and 2q + 1 (high halves)
      const uint32_t x0 = vb[st][0][q], x1 = vb[st][1][q];
      const uint32_t x2 = vb[st][2][q], x3 = vb[st][3][q];
      u32x2 ae, ao;
      ae[0] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
      ae[1] = __builtin_amdgcn_perm(x3, x2, 0x05040100u);
      ao[0] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
      ao[1] = __builtin_amdgcn_perm(x3, x2, 0x07060302u);
      const s16x4 ve = __builtin_bit_cast(s16x4, ae), vo = __builtin_bit_cast(s16x4, ao);
      acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ve, ph, acc[2 * q], 0, 0, 0);
      acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ve, pl, acc[2 * q], 0, 0, 0);
      acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo, ph, acc[2 * q + 1], 0, 0, 0);
      acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo, pl, acc[2 * q + 1], 0, 0, 0);
    }
  };
  for (int j0 = 0; j0 < my_tiles; j0 += NS) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int j = j0 + st;
      if (j >= my_tiles) break;
      process(st, j);
      issue(st, j + NS);
    }
  }

  // ---- combine the waves (and the new slot) per head in LDS; a wave with no rows has
  // M = -inf and contributes nothing. m is stored in natural-log units for the merge.
  L += __shfl_xor(L, 16, kWave);
  L += __shfl_xor(L, 32, kWave);
  if (c16 < G) {
    if (r4 == 0) {
      wml[(wave * kMaxGroup + c16) * 2 + 0] = M;
      wml[(wave * kMaxGroup + c16) * 2 + 1] = L;
    }
    float* o = wo + (wave * kMaxGroup + c16) * D;
#pragma unroll
    for (int jj = 0; jj < VD; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[VD * (4 * r4 + i) + jj] = acc[jj][i];
  }
  __syncthreads();
  const long hbase = (long)b * p.n_q + g * G;
  for (int i = tid; i < G * D; i += kFlashThreads) {
    const int h = i / D, dd = i % D;
    float mx = has_new ? snew[h] : -INFINITY;
#pragma unroll
    for (int w = 0; w < kFlashWaves; ++w) mx = fmaxf(mx, wml[(w * kMaxGroup + h) * 2]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kFlashWaves; ++w) {
      const float mw = wml[(w * kMaxGroup + h) * 2];
      const float f = mw == -INFINITY ? 0.f : hw_exp2(mw - mx);
      o = fmaf(f, wo[(w * kMaxGroup + h) * D + dd], o);
      l = fmaf(f, wml[(w * kMaxGroup + h) * 2 + 1], l);
    }
    if (has_new) {
      const float f = hw_exp2(snew[h] - mx);
      o = fmaf(f, vn[dd], o);
      l += f;
    }
    p.part_o[((hbase + h) * p.nsplit + s) * D + dd] = o;
    if (dd == 0) {
      p.part_ml[((hbase + h) * p.nsplit + s) * 2 + 0] = mx * kLn2;
      p.part_ml[((hbase + h) * p.nsplit + s) * 2 + 1] = l;
    }
  }
  // ---- the workgroup whose chunk holds the new slot appends it to the cache
  if (has_new && !masked && tid < D) {
    const long o = (kv_base + slot) * D + tid;
    static_cast<uint16_t*>(p.kc)[o] = f32_to_bf16(kn[tid]);
    static_cast<uint16_t*>(p.vc)[o] = f32_to_bf16(vn[tid]);
  }
}

// Merge the splits of one (query head, sequence): o = sum_q w_q o_q with
// w_q = exp(m_q - M) / sum_q' l_q' exp(m_q' - M). One thread per dimension. The first
// UB split partials of o are requested together with the (max, sum) pairs, so up to UB
// splits cost one memory round trip; later batches have all their loads in flight.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnParams p) {
  constexpr int UB = 32;
  __shared__ float w[256];
  __shared__ float red[D / kWave];
  const int hq = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const bool masked = p.kseq && p.step >= seq_steps(p.kseq, b, p.step + 1);
  const int slot = masked ? 0 : p.len[b] + p.step;
  const int T_valid = slot >= p.capacity ? p.capacity : slot + 1;
  const int chunk = attn_chunk(p);
  const int nvalid = (T_valid + chunk - 1) / chunk;
  const long hb = (long)b * p.n_q + hq;
  const float* ml = p.part_ml + hb * p.nsplit * 2;
  const float* po = p.part_o + hb * p.nsplit * D + t;
  float v[UB];
#pragma unroll
  for (int j = 0; j < UB; ++j) v[j] = j < nvalid ? po[(long)j * D] : 0.f;
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
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < nvalid; q0 += UB) {
    if (q0 > 0) {
#pragma unroll
      for (int j = 0; j < UB; ++j) v[j] = (q0 + j < nvalid) ? po[(long)(q0 + j) * D] : 0.f;
    }
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

// Longest-first launch order of the attention items of one draft call (the lengths are
// those of its first step): the items whose chunk is full (sequence-major), then each
// sequence's last, partial chunk by decreasing length (ties by sequence), then the items
// that are empty at that step, which a later step of the call may reach. perm[i] is the
// natural index of the i-th workgroup. Every item keeps exactly one position, so the
// attention launches stay correct whatever the later steps' lengths; only the order is
// tuned. One workgroup, B <= kPlanMaxBatch.
constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxBatch = 1024;

// Exclusive prefix sum over the workgroup (kPlanThreads threads); *total gets the sum.
__device__ int plan_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kPlanThreads / kWave; ++w) {
      const int t = wsum[w];
      wsum[w] = acc;
      acc += t;
    }
    *total = acc;
  }
  __syncthreads();
  const int r = wsum[wave] + x - v;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(const int* len, int B, int nkv,
                                                                 int chunk, const int* chunk_dev,
                                                                 int nsplit, int* perm) {
  if (chunk_dev) chunk = *chunk_dev;
  __shared__ int F[kPlanMaxBatch], R[kPlanMaxBatch], FP[kPlanMaxBatch], EP[kPlanMaxBatch];
  __shared__ int RK[kPlanMaxBatch];
  __shared__ int wsum[kPlanThreads / kWave];
  __shared__ int tot[3];
  const int t = threadIdx.x;
  int f = 0, r = 0, e = 0;
  if (t < B) {
    const long T = max((long)len[t] + 1, 0L);  // valid positions at the call's first step
    f = (int)min(T / chunk, (long)nsplit);
    r = f < nsplit ? (int)(T - (long)f * chunk) : 0;
    e = nsplit - f - (r > 0 ? 1 : 0);
    F[t] = f;
    R[t] = r;
  }
  const int fp = plan_scan(f, wsum, &tot[0]);
  const int ep = plan_scan(e, wsum, &tot[2]);
  const int np = plan_scan(r > 0 ? 1 : 0, wsum, &tot[1]);
  (void)np;
  if (t < B) {
    FP[t] = fp;
    EP[t] = ep;
    int rank = 0;
    if (r > 0)
      for (int u = 0; u < B; ++u) {
        const int ru = R[u];
        rank += (ru > r || (ru == r && u < t)) ? 1 : 0;
      }
    RK[t] = rank;
  }
  __syncthreads();
  const int total_full = tot[0], total_part = tot[1];
  const int ngb = B * nkv;
  const long n = (long)nsplit * ngb;
  for (long idx = t; idx < n; idx += kPlanThreads) {
    const int sp = (int)(idx / ngb), b = (int)(idx % ngb) / nkv, g = (int)(idx % nkv);
    long pos;
    if (sp < F[b]) {
      pos = (long)(FP[b] + sp) * nkv + g;
    } else if (sp == F[b] && R[b] > 0) {
      pos = (long)(total_full + RK[b]) * nkv + g;
    } else {
      const int first_empty = F[b] + (R[b] > 0 ? 1 : 0);
      pos = (long)(total_full + total_part + EP[b] + (sp - first_empty)) * nkv + g;
    }
    perm[pos] = (int)idx;
  }
}

bool attn_plan_wanted(int B, int nkv, int nsplit, int num_cu) {
  return B <= kPlanMaxBatch && (long)nsplit * nkv * B > 2L * num_cu;
}

hipError_t launch_attn_plan(const int* len, int B, int nkv, int chunk, const int* chunk_dev,
                            int nsplit, int* perm, hipStream_t s) {
  if (B < 1 || B > kPlanMaxBatch || nsplit < 1 || chunk < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, len, B, nkv, chunk,
                     chunk_dev, nsplit, perm);
  return hipGetLastError();
}

// Per-call set-up: RoPE tables of the K steps (tab[k][b][0..d/2) = cos, [d/2..d) = sin of
// (pos[b] + k) * theta^(-2i/d), evaluated in fp64 and rounded to fp32) and the verifier
// hidden state widened to fp32 (the first step's input).
template <class CT>
__global__ void draft_setup_kernel(float* tab, const int* pos, int B, int K, int d, float theta,
                                   const void* hidden, float* hf, int H, const int* kseq,
                                   unsigned err_bit, unsigned* err, ChunkPlan cp) {
  const int half = d / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (cp.chunk_out && blockIdx.x == 0) {  // the call's attention chunk, from the lengths
    __shared__ int wmax[256 / kWave];
    __shared__ long wsum[256 / kWave];
    int m = 0;
    long sum = 0;  // sum of T_b (balance rule only)
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      m = max(m, cp.len[b]);
      sum += min((long)cp.len[b] + K, (long)cp.capacity);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      m = max(m, __shfl_xor(m, o, kWave));
      sum += __shfl_xor(sum, o, kWave);
    }
    if ((threadIdx.x & 63) == 0) {
      wmax[threadIdx.x >> 6] = m;
      wsum[threadIdx.x >> 6] = sum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < (int)blockDim.x / kWave; ++w) {
        m = max(m, wmax[w]);
        sum += wsum[w];
      }
      long T = (long)m + K;
      if (T > cp.capacity) T = cp.capacity;
      long ch;
      if (cp.balance && T > 0 && sum > 0) {
        const double r = (double)sum / ((double)B * (double)T);  // mean T / max T
        const double S = (double)sum * cp.n_kv / cp.num_cu * r * r;
        long n = (long)((double)T / S + 0.5);
        if (n < 1) n = 1;
        if (n > cp.nsplit) n = cp.nsplit;
        ch = ((T + n - 1) / n + cp.q - 1) / cp.q * cp.q;
      } else {
        const long per = (T + cp.nsplit - 1) / cp.nsplit;
        ch = (per + cp.q - 1) / cp.q * cp.q;
        if (ch > cp.max_chunk) ch = cp.max_chunk;
      }
      if (ch < cp.q) ch = cp.q;
      cp.chunk_out[0] = (int)ch;
    }
  }
  if (e < K * B * half) {
    const int i = e % half, kb = e / half, b = kb % B, k = kb / B;
    rope_cs(pos[b] + k, i, d, theta, tab[(long)kb * d + i], tab[(long)kb * d + half + i]);
  }
  if (e < B * H) hf[e] = CT::get(static_cast<const typename CT::T*>(hidden), e);
  if (kseq && e < B && (kseq[e] < 0 || kseq[e] > K)) set_error(err, err_bit);
}

hipError_t launch_draft_setup(int dtype, float* tab, const int* pos, int B, int K, int d,
                              float theta, const void* hidden, float* hf, int H, const int* kseq,
                              unsigned err_bit, unsigned* err, const ChunkPlan& cp,
                              hipStream_t s) {
  if (kseq && !err) return hipErrorInvalidValue;
  if (cp.chunk_out && (!cp.len || cp.nsplit < 1 || cp.q < 1 || cp.max_chunk < cp.q))
    return hipErrorInvalidValue;
  const int n1 = K * B * (d / 2), n2 = B * H;
  int n = n1 > n2 ? n1 : n2;
  n = n > B ? n : B;
  if (dtype == 0)
    hipLaunchKernelGGL(draft_setup_kernel<F32>, dim3((n + 255) / 256), dim3(256), 0, s, tab, pos,
                       B, K, d, theta, hidden, hf, H, kseq, err_bit, err, cp);
  else
    hipLaunchKernelGGL(draft_setup_kernel<BF16>, dim3((n + 255) / 256), dim3(256), 0, s, tab, pos,
                       B, K, d, theta, hidden, hf, H, kseq, err_bit, err, cp);
  return hipGetLastError();
}

template <int D, int GP>
static hipError_t launch_attn_g(int cdtype, const AttnParams& p, int B, hipStream_t s) {
  AttnParams q = p;
  q.batch = B;
  if (cdtype == 0)
    hipLaunchKernelGGL((attn_kernel<D, GP>), dim3(p.nsplit * p.n_kv * B), dim3(kAttnThreads),
                       attn_lds_bytes(D, p.chunk), s, q);
  else
    hipLaunchKernelGGL((attn_flash_kernel<D, GP>), dim3(p.nsplit * p.n_kv * B),
                       dim3(kFlashThreads), flash_lds_bytes(D), s, q);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_t(int cdtype, const AttnParams& p, int B, hipStream_t s) {
  if (p.nsplit > 256 || p.nsplit < 1 || p.chunk % attn_chunk_quantum() != 0 ||
      p.chunk > attn_max_chunk(cdtype))
    return hipErrorInvalidValue;
  const int G = p.n_q / p.n_kv;
  hipError_t e0;
  if (G <= 1) e0 = launch_attn_g<D, 1>(cdtype, p, B, s);
  else if (G <= 2) e0 = launch_attn_g<D, 2>(cdtype, p, B, s);
  else if (G <= 4) e0 = launch_attn_g<D, 4>(cdtype, p, B, s);
  else if (G <= 8) e0 = launch_attn_g<D, 8>(cdtype, p, B, s);
  else return hipErrorInvalidValue;
  if (e0 != hipSuccess) return e0;
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(p.n_q, B), dim3(D), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention(int cdtype, const AttnParams& p, int B, hipStream_t s) {
  return p.d == 64 ? launch_attn_t<64>(cdtype, p, B, s) : launch_attn_t<128>(cdtype, p, B, s);
}

}  // namespace mtp
