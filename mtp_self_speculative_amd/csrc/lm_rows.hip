// Greedy verification from the target's hidden states for up to 16 rows in one launch:
// final RMSNorm of each row, the shared lm_head read in place (row-major, no re-laid-out
// copy) on the matrix cores, the vocabulary argmax of every row and the accepted-prefix
// scan (OpenVINO GenAI "Speculative Decoding", Overview).
//
// v_mfma_f32_16x16x32_bf16 wants every lane's 16-byte A operand from a different weight
// row (a 16-row x 32-column tile per instruction), so loading A straight from a row-major
// matrix reads 64-byte pieces of 16 rows per wave instruction. Here a wave instead loads a
// 16-row x 256-column tile with 1 KB per instruction (two 512-byte row pieces), writes it
// to its own LDS tile with an XOR swizzle (row r's 16-byte group g at unit g ^ r, so the
// MFMA reads of 16 rows at one column group hit 16 different bank groups) and reads the A
// operands back from there. Two such tiles are in flight per wave in registers while one
// is staged and multiplied.
//
// The eight waves of a workgroup split the hidden dimension, 512 columns each, so that a
// wave's share of the normalised input rows stays in registers for the whole launch as the
// MFMA B operands (bf16 hi and lo planes of the fp32 values, 16 rows: rows past the count
// are zero). Each workgroup owns a contiguous range of 16-row vocabulary slices; the eight
// partial 16 x 16 tiles of a slice are added in LDS in a fixed order (a ring of eight
// slots, one barrier per four slices), and the row values become packed (value, index)
// argmax keys. Keys leave through device-scope atomic max and the last workgroup to
// finish (common.h protocol) writes the tokens and runs the prefix scan.
#include "common.h"
#include "kernels.h"

namespace mtp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLrWaves = 8;
constexpr int kLrThreads = kLrWaves * kWave;
constexpr int kLrCols = 512;           // hidden columns per wave
constexpr int kLrKS = kLrCols / 32;    // MFMA k-steps per wave
constexpr int kLrTile = 16 * 256;      // elements of one staged tile (16 rows x 256 columns)
constexpr int kLrRing = 8;             // partial-sum slots
constexpr size_t kLrLds = (size_t)kLrWaves * kLrTile * 2 + (size_t)kLrRing * kLrWaves * 64 * 16;

// s_waitcnt immediates (gfx9 encoding): vmcnt(8) alone, lgkmcnt(0) alone.
constexpr int kVm8 = 0x0F78;
constexpr int kLgkm0 = 0xC07F;

}  // namespace

__global__ __launch_bounds__(kLrThreads, 1) void lm_rows_kernel(LmRowsParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* tiles = reinterpret_cast<uint16_t*>(smem);                            // [wave][tile]
  float* part = reinterpret_cast<float*>(smem + (size_t)kLrWaves * kLrTile * 2);  // [slot][wave][64][4]
  __shared__ float rsq[16];
  __shared__ unsigned long long kred[kLrWaves][16];
  __shared__ int flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.V, H = p.H, R = p.R;
  const int nsl = (N + 15) / 16;
  const int s0 = (int)((long)nsl * blockIdx.x / gridDim.x);
  const int s1 = (int)((long)nsl * (blockIdx.x + 1) / gridDim.x);
  const int col0 = wave * kLrCols;

  // ---- final RMSNorm of the rows: 32 threads per row, loads in batches of eight groups
  // (addresses clamped into the row, values past its end masked)
  {
    const int n = tid >> 5, sub = tid & 31;
    const uint16_t* hr = p.h + (long)(n < R ? n : 0) * H;
    float ss = 0.f;
    for (int c0 = sub * 8; c0 < H; c0 += 8 * 32 * 8) {
      u32x4 raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        raw[u] = *reinterpret_cast<const u32x4*>(hr + min(c0 + u * 256, H - 8));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float v[8];
        BF16::unpack(raw[u], v);
        const bool in = n < R && c0 + u * 256 < H;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(in ? v[e] : 0.f, in ? v[e] : 0.f, ss);
      }
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
    if (sub == 0) rsq[n] = 1.0f / sqrtf(ss / (float)H + p.eps);
  }
  __syncthreads();

  // ---- B operands: lane (n = lane % 16, q = lane / 16) holds, per k-step t, the 8 values
  // at columns col0 + 32 t + 8 q of normalised row n (zero past the row count or width);
  // loaded eight k-steps at a time
  bf16x8 bh[kLrKS], bl[kLrKS];
  {
    const int n = lane & 15, q = lane >> 4;
    const bool live = n < R;
    const float rs = live ? rsq[n] : 0.f;
    const uint16_t* hr = p.h + (long)(live ? n : 0) * H;
#pragma unroll
    for (int t0 = 0; t0 < kLrKS; t0 += 8) {
      u32x4 hv[8], gv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = min(col0 + 32 * (t0 + u) + 8 * q, H - 8);
        hv[u] = *reinterpret_cast<const u32x4*>(hr + c);
        gv[u] = *reinterpret_cast<const u32x4*>(p.gain + c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = live && col0 + 32 * (t0 + u) + 8 * q < H;
        float hf[8], gf[8];
        BF16::unpack(hv[u], hf);
        BF16::unpack(gv[u], gf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint16_t hi, lo;
          split_bf16(in ? hf[e] * rs * gf[e] : 0.f, hi, lo);
          bh[t0 + u][e] = __builtin_bit_cast(__bf16, hi);
          bl[t0 + u][e] = __builtin_bit_cast(__bf16, lo);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // only weight loads stay outstanding from here on

  // ---- weight tiles. Tile h: slice s0 + h / 2, columns col0 + 256 (h % 2) .. + 256 of its
  // 16 rows (clamped to the last row and column: such loads read real data, never used).
  // Load instruction j covers rows 2j, 2j+1 (lanes 0-31, 32-63), lane l the 8-column group
  // l % 32 of its row.
  uint16_t* mytile = tiles + wave * kLrTile;
  const int nh = 2 * (s1 - s0);
  auto wload = [&](int h, u32x4 (&buf)[8]) {
    const int hh = max(0, min(h, nh - 1));
    const int s = s0 + (hh >> 1);
    const int c = min(col0 + 256 * (hh & 1) + 8 * (lane & 31), H - 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = min(16 * s + 2 * j + (lane >> 5), N - 1);
      buf[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.W + (long)r * H + c));
    }
  };
  unsigned long long best = 0ull;
  u32x4 WA[8], WB[8];
  wload(0, WA);
  __builtin_amdgcn_sched_barrier(0);  // WA strictly before WB, the order the loop keeps
  wload(1, WB);
  __builtin_amdgcn_sched_barrier(0);
  // Stage the tile in buf, refill buf with tile h + 2, then multiply.
  auto tile = [&](int h, u32x4 (&buf)[8], f32x4& acc, int t0) {
    __builtin_amdgcn_s_waitcnt(kVm8);  // buf has landed; the other buffer is in flight
    {
      const int g = lane & 31;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rl = 2 * j + (lane >> 5);
        *reinterpret_cast<u32x4*>(mytile + rl * 256 + 8 * (g ^ rl)) = buf[j];
      }
    }
    wload(h + 2, buf);
    __builtin_amdgcn_s_waitcnt(kLgkm0);  // the tile is staged
    bf16x8 a[8];
    {
      const int r = lane & 15, q = lane >> 4;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int g = 4 * t + q;
        a[t] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(mytile + r * 256 + 8 * (g ^ r)));
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], bh[t0 + t], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], bl[t0 + t], acc, 0, 0, 0);
    }
  };
  // Lane l of the summed tile holds rows 4 (l / 16) + i of the slice for input row l % 16.
  auto reduce = [&](int s) {
    const int slot = (s - s0) & (kLrRing - 1);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kLrWaves; ++w)
      t += *reinterpret_cast<const f32x4*>(part + ((slot * kLrWaves + w) * 64 + lane) * 4);
    if ((lane & 15) < R) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * s + 4 * (lane >> 4) + i;
        if (row < N) {
          const unsigned long long k = pack_key(t[i], (uint32_t)row);
          best = k > best ? k : best;
        }
      }
    }
  };
  int sr = s0;  // first slice not yet reduced
  for (int s = s0; s < s1; ++s) {
    const int h = 2 * (s - s0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    tile(h, WA, acc, 0);
    tile(h + 1, WB, acc, 8);
    *reinterpret_cast<f32x4*>(
        part + ((((s - s0) & (kLrRing - 1)) * kLrWaves + wave) * 64 + lane) * 4) = acc;
    if (((s - s0) & 3) == 3 || s + 1 == s1) {
      // A barrier without a memory fence: the weight loads in flight stay in flight. A
      // slot is written again eight slices later, after the next barrier, by which time
      // its reducer is done with it.
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      for (; sr <= s; ++sr)
        if (wave == sr % kLrWaves) reduce(sr);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the tail refills (clamped re-reads) have landed

  // ---- argmax keys: lanes of one input row, then waves, then workgroups
  unsigned long long o = __shfl_xor(best, 16, kWave);
  best = o > best ? o : best;
  o = __shfl_xor(best, 32, kWave);
  best = o > best ? o : best;
  if (lane < 16) kred[wave][lane] = best;
  __syncthreads();
  if (tid < R) {
    unsigned long long k = 0ull;
    for (int w = 0; w < kLrWaves; ++w) k = kred[w][tid] > k ? kred[w][tid] : k;
    if (k) publish_max_key(p.keys + tid, k);
  }
  // the winner reads back only keys published by publish_max_key
  if (last_to_arrive(p.counter, gridDim.x, &flag)) {
    if (tid < R) p.tok_out[tid] = (int)key_index(take_key(p.keys + tid));
    __syncthreads();
    if (p.accepted) {
      const int K = p.K;
      for (int b = tid; b < p.B; b += kLrThreads) {
        int a = 0;
        while (a < K && p.draft[(long)b * K + a] == p.tok_out[(long)b * (K + 1) + a]) ++a;
        p.accepted[b] = a;
        p.next[b] = p.tok_out[(long)b * (K + 1) + a];
      }
    }
  }
}

bool lm_rows_fits(int H, int R) { return R >= 1 && R <= 16 && H >= 8 && H % 8 == 0 && H <= kLrWaves * kLrCols; }

hipError_t lm_rows_prepare() {
  return hipFuncSetAttribute((const void*)lm_rows_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLrLds);
}

hipError_t launch_lm_rows(const LmRowsParams& p, int grid, hipStream_t s) {
  if (!lm_rows_fits(p.H, p.R) || p.V < 1 || grid < 1 || !p.h || !p.gain || !p.W || !p.keys ||
      !p.counter || !p.tok_out)
    return hipErrorInvalidValue;
  if (p.accepted && (!p.next || p.B < 1 || p.K < 0 || (p.K > 0 && !p.draft) ||
                     p.B * (p.K + 1) != p.R))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(lm_rows_kernel, dim3(grid), dim3(kLrThreads), kLrLds, s, p);
  return hipGetLastError();
}

}  // namespace mtp
