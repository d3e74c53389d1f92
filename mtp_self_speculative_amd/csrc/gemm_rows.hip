// Tiled bf16 contraction on the matrix cores for many input rows (the input side of a prompt
// prefill: every prompt row through eh_proj and the K / V projections).
//
// The weight-streaming contraction (gemm_mfma.hip) keeps W in registers and reads it from HBM
// once per group of up to 64 input rows, which suits decode; with thousands of rows that
// re-reads W dozens of times and pays its launches per group. Here a workgroup computes a
// 256 (W rows) x 128 (input rows) tile: each 64-column stage of W and of both input planes
// (hi, lo) goes from HBM through registers into LDS once, and the eight waves (4 x 2, two per
// SIMD, so that one wave's products overlap the other's LDS reads) each take 64 x 64 of the
// tile from LDS as 4 x 4 v_mfma_f32_16x16x32_bf16 blocks, the A operand (16 W rows x 32
// columns) shared by four input tiles and the B operands (16 input rows x 32 columns, hi and
// lo) by four W slices. Stages are double-buffered in LDS: the next stage's global loads are
// in flight while the current one is multiplied. (Four waves of 128 x 64, one per SIMD, were
// 26-35% slower on the same shapes.)
//
// EPI_STORE gives the same K-split partial sums, in the same layout, as the weight-streaming
// contraction's EPI_STORE (part[split][bp][N]; a row kernel adds the splits): split s covers
// columns [s * Kd / nsplit, (s + 1) * Kd / nsplit) in 256-column chunks, and each output
// accumulates its 32-column steps in column order, the hi product before the lo one, so the
// two contractions give bit-identical partials for the same split. EPI_ARGMAX (one split;
// the greedy lm_head of verification from hidden states) reduces each input row's values over
// its W rows to a packed (value, index) key, publishes one key per input row and workgroup by
// atomic max, and the last workgroup to arrive writes each input row's argmax.
#include "common.h"
#include "kernels.h"

namespace mtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGmTM = 256;            // W rows per tile
constexpr int kGmTN = 128;            // input rows per tile
constexpr int kGmBK = 64;             // columns per stage
constexpr int kGmLd = kGmBK + 8;      // LDS row stride (bf16): 144 B, conflict-free reads
constexpr int kGmThreads = 512;       // eight waves
constexpr int kGmChunk = 256;         // columns per K-split unit (as the streaming kernel)
constexpr int kGmMaxSplit = 16;

constexpr size_t kGmLdsA = (size_t)2 * kGmTM * kGmLd;       // bf16 elements, two buffers
constexpr size_t kGmLdsB = (size_t)2 * 2 * kGmTN * kGmLd;   // two buffers x two planes
size_t gm_lds_bytes() { return (kGmLdsA + kGmLdsB) * sizeof(uint16_t); }

template <int EPI>
__global__ __launch_bounds__(kGmThreads, 1) void gm_kernel(GmParams p) {
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;             // [2][kGmTM][kGmLd]
  uint16_t* Bs = smem + kGmLdsA;   // [2][2 planes][kGmTN][kGmLd]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int N = p.nrows, Kd = p.ncols;
  const int tiles_m = (N + kGmTM - 1) / kGmTM;
  const int tiles_n = (p.B + kGmTN - 1) / kGmTN;
  const int bid = blockIdx.x;
  const int tm = bid % tiles_m;
  const int tn = (bid / tiles_m) % tiles_n;
  const int split = bid / (tiles_m * tiles_n);
  const int nch = (Kd + kGmChunk - 1) / kGmChunk;
  const int cps = nch / p.nsplit;                        // chunks per split
  const int k0 = split * cps * kGmChunk;
  const int k1 = min(k0 + cps * kGmChunk, (nch * kGmChunk));
  const int S = (k1 - k0) / kGmBK;                       // stages (kGmChunk % kGmBK == 0)
  const int m0 = tm * kGmTM, n0 = tn * kGmTN;

  // Global -> register staging: 4 16-byte chunks of W and 4 of the input per thread and
  // stage. Thread t takes column chunk t % 8 of rows t / 8 + 64 i. Rows past the end read
  // the last row (never stored); columns past Kd read the row's last 8 values, and the
  // input chunk is zeroed in LDS there, so they add nothing.
  const int cc = (tid & 7) * 8;
  u32x4 ra[4], rb[4];
  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(m0 + (tid >> 3) + 64 * i, N - 1);
    arow[i] = r < p.seg1 ? static_cast<const uint16_t*>(p.w0) + (long)r * Kd
                         : static_cast<const uint16_t*>(p.w1) + (long)(r - p.seg1) * Kd;
    const int b = min(n0 + (tid >> 3) + 64 * (i & 1), p.B - 1);
    brow[i] = (i < 2 ? p.x : p.x_lo) + (long)b * p.ldx;
  }
  auto gload = [&](int st) {
    const int c = k0 + st * kGmBK + cc;
    const int cl = c < Kd ? c : Kd - 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(arow[i] + cl);
      rb[i] = *reinterpret_cast<const u32x4*>(brow[i] + cl);
    }
  };
  auto lstore = [&](int st, int buf) {
    const bool live = k0 + st * kGmBK + cc < Kd;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(As + ((size_t)buf * kGmTM + (tid >> 3) + 64 * i) * kGmLd + cc) = ra[i];
      const int pl = i >> 1;
      *reinterpret_cast<u32x4*>(Bs + (((size_t)buf * 2 + pl) * kGmTN + (tid >> 3) + 64 * (i & 1)) * kGmLd + cc) =
          live ? rb[i] : z;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Lane l reads row l % 16 of a 16-row slice, columns 8 (l / 16) .. + 7 of a 32-column step.
  const int fr = lane & 15, fc = (lane >> 4) * 8;
  auto compute = [&](int buf) {
    const uint16_t* a = As + ((size_t)buf * kGmTM + wm * 64 + fr) * kGmLd + fc;
    const uint16_t* bh = Bs + (((size_t)buf * 2 + 0) * kGmTN + wn * 64 + fr) * kGmLd + fc;
    const uint16_t* bl = Bs + (((size_t)buf * 2 + 1) * kGmTN + wn * 64 + fr) * kGmLd + fc;
#pragma unroll
    for (int kk = 0; kk < kGmBK / 32; ++kk) {
      bf16x8 fa[4], fh[4], fl[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        fa[m] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a + m * 16 * kGmLd + kk * 32));
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        fh[n] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bh + n * 16 * kGmLd + kk * 32));
        fl[n] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bl + n * 16 * kGmLd + kk * 32));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[m], fh[n], acc[m][n], 0, 0, 0);
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[m], fl[n], acc[m][n], 0, 0, 0);
        }
    }
  };

  if (S > 0) {
    gload(0);
    lstore(0, 0);
    __syncthreads();
    for (int st = 0; st < S; ++st) {
      if (st + 1 < S) gload(st + 1);  // in flight while stage st is multiplied
      compute(st & 1);
      if (st + 1 < S) lstore(st + 1, (st + 1) & 1);
      __syncthreads();
    }
  }

  // Lane l holds W rows 4 (l / 16) + i (i < 4) of each slice for input row l % 16 of each tile.
  if constexpr (EPI == EPI_ARGMAX) {
    __shared__ unsigned long long kred[kGmThreads / kWave][64];  // [wave][its 64 input rows]
    __shared__ int flag;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      unsigned long long k = 0ull;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r0 = m0 + wm * 64 + m * 16 + (lane >> 4) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned long long ki = r0 + i < N ? pack_key(acc[m][n][i], (uint32_t)(r0 + i)) : 0ull;
          k = ki > k ? ki : k;
        }
      }
      unsigned long long o = __shfl_xor(k, 16, kWave);
      k = o > k ? o : k;
      o = __shfl_xor(k, 32, kWave);
      k = o > k ? o : k;
      if (lane < 16) kred[wave][n * 16 + lane] = k;
    }
    __syncthreads();
    if (tid < kGmTN) {  // input row n0 + tid: the four waves that share its columns
      const int g = tid >> 6, j = tid & 63;
      unsigned long long k = 0ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) k = kred[q + 4 * g][j] > k ? kred[q + 4 * g][j] : k;
      if (n0 + tid < p.B && k) publish_max_key(p.keys + n0 + tid, k);
    }
    // the winner reads back only keys published by publish_max_key
    if (last_to_arrive(p.counter, gridDim.x, &flag)) {
      for (int b = tid; b < p.B; b += kGmThreads) p.tok_out[b] = (int)key_index(take_key(p.keys + b));
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r0 = m0 + wm * 64 + m * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int b = n0 + wn * 64 + n * 16 + (lane & 15);
      if (b >= p.B) continue;
      float* dst = p.part + ((long)split * p.bp + b) * N + r0;
      if (r0 + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = float4{acc[m][n][0], acc[m][n][1], acc[m][n][2], acc[m][n][3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < N) dst[i] = acc[m][n][i];
      }
    }
  }
}

// K splits for a grid of at least one workgroup per CU: the smallest divisor s of the
// chunk count with tiles * s >= num_cu, else the largest allowed; allowed are s <=
// kGmMaxSplit with s * B * nrows <= max_part (the partial sums' room), and always s = 1.
int gm_split(int nrows, int ncols, int B, int num_cu, long max_part) {
  const long tiles = (long)((nrows + kGmTM - 1) / kGmTM) * ((B + kGmTN - 1) / kGmTN);
  const int nch = (ncols + kGmChunk - 1) / kGmChunk;
  int best = 1;
  for (int s = 2; s <= kGmMaxSplit && s <= nch && (long)s * B * nrows <= max_part; ++s) {
    if (tiles * best >= num_cu) break;
    if (nch % s == 0) best = s;
  }
  return best;
}

hipError_t gm_prepare() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gm_kernel<EPI_STORE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)gm_lds_bytes());
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gm_kernel<EPI_ARGMAX>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)gm_lds_bytes());
  return e;
}

hipError_t launch_gm(Epi epi, const GmParams& p, hipStream_t s) {
  if (epi != EPI_STORE && epi != EPI_ARGMAX) return hipErrorInvalidValue;
  if (epi == EPI_STORE ? !p.part : (p.nsplit != 1 || !p.keys || !p.counter || !p.tok_out))
    return hipErrorInvalidValue;
  if (!p.w0 || !p.w1 || !p.x || !p.x_lo || p.nrows < 1 || p.ncols < 8 ||
      p.ncols % 8 != 0 || p.ldx < p.ncols || p.ldx % 8 != 0 || p.B < 1 || p.bp < p.B ||
      p.seg1 < 0 || p.seg1 > p.nrows || p.nsplit < 1 || p.nsplit > kGmMaxSplit)
    return hipErrorInvalidValue;
  const int nch = (p.ncols + kGmChunk - 1) / kGmChunk;
  if (nch % p.nsplit != 0) return hipErrorInvalidValue;
  const long grid = (long)((p.nrows + kGmTM - 1) / kGmTM) * ((p.B + kGmTN - 1) / kGmTN) * p.nsplit;
  if (epi == EPI_ARGMAX)
    hipLaunchKernelGGL(gm_kernel<EPI_ARGMAX>, dim3((unsigned)grid), dim3(kGmThreads), gm_lds_bytes(), s, p);
  else
    hipLaunchKernelGGL(gm_kernel<EPI_STORE>, dim3((unsigned)grid), dim3(kGmThreads), gm_lds_bytes(), s, p);
  return hipGetLastError();
}

}  // namespace mtp
