// Row-wise steps of the batched draft path: one workgroup per sequence where a norm needs
// the whole row, column blocks otherwise.
//
// The MFMA contraction writes fp32 partial sums per K split. Each kernel here adds the
// splits in a fixed order (deterministic), applies the step's epilogue (residual add,
// SwiGLU, plain store) and, where the next contraction starts with an RMSNorm, also
// produces that contraction's bf16 operand row: the whole row is in this workgroup, so
// the norm needs no second pass over memory. Operand rows are written as bf16 hi / lo
// planes, so the contraction sees the fp32 values to about 16 bits. PREP_EH builds the eh_proj operand
// [RMSNorm(h) * g_h ; RMSNorm(embed[tok]) * g_e] (speculators user guide, "MTP
// (Multi-Token Prediction)", How It Works > Architecture: both inputs are normalised
// separately, then concatenated).
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kRedThreads = 512;       // column modes: one float4 group per thread
constexpr int kRedNormThreads = 1024;  // norm modes: one workgroup per sequence
constexpr int kRedNormVPT = 2;         // float4 groups per thread in the norm modes
constexpr int kRedMaxSplit = 16;
constexpr int kRedBatch = 8;  // split partials of a group requested together

int red_max_cols() { return 4 * kRedNormVPT * kRedNormThreads; }

// Four values as bf16 hi / lo planes (see split_bf16).
__device__ __forceinline__ void store4_split(uint16_t* hi, uint16_t* lo, float a, float b, float c,
                                             float d) {
  uint16_t h[4], l[4];
  split_bf16(a, h[0], l[0]);
  split_bf16(b, h[1], l[1]);
  split_bf16(c, h[2], l[2]);
  split_bf16(d, h[3], l[3]);
  *reinterpret_cast<uint2*>(hi) = uint2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
  *reinterpret_cast<uint2*>(lo) = uint2{l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16)};
}
__device__ __forceinline__ float4 load4_bf16(const uint16_t* src) {
  const uint2 u = *reinterpret_cast<const uint2*>(src);
  return float4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
}
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return float4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
}
__device__ __forceinline__ float dot4(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }

// Sum over the splits of the partial sums of NG float4 column groups c[0..NG), added in
// split order (deterministic). The loads of all groups for a batch of kRedBatch splits are
// issued together (indexes past nsplit repeat the last split and are not added), so a row
// costs one memory round trip per batch.
template <int NG>
__device__ __forceinline__ void sum_splits(const RedParams& p, int b, const int (&c)[NG],
                                           float4 (&v)[NG]) {
  for (int s0 = 0; s0 < p.nsplit; s0 += kRedBatch) {
    float4 t[NG][kRedBatch];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int s = 0; s < kRedBatch; ++s) {
        const int sc = s0 + s < p.nsplit ? s0 + s : p.nsplit - 1;
        t[g][s] = *reinterpret_cast<const float4*>(p.part + ((long)sc * p.bp + b) * p.n_part + c[g]);
      }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int s = 0; s < kRedBatch; ++s) {
        if (s0 + s == 0) v[g] = t[g][s];
        else if (s0 + s < p.nsplit) v[g] = add4(v[g], t[g][s]);
      }
  }
}

template <int MODE>
__global__ __launch_bounds__(MODE == RED_QKV || MODE == RED_SWIGLU ? kRedThreads : kRedNormThreads)
void red_kernel(RedParams p) {
  // Column modes (QKV, SwiGLU): grid (column block, sequence), one float4 group per thread.
  // Norm modes: one workgroup per sequence, kRedNormVPT groups per thread.
  constexpr bool kCols = MODE == RED_QKV || MODE == RED_SWIGLU;
  constexpr int NT = kCols ? kRedThreads : kRedNormThreads;
  __shared__ float red[NT / kWave];
  const int b = kCols ? (int)blockIdx.y : (int)blockIdx.x, tid = threadIdx.x;
  const int n = p.n;

  if constexpr (MODE == RED_QKV) {
    const int c = 4 * ((int)blockIdx.x * kRedThreads + tid);
    const int cc[1] = {c < n ? c : n - 4};
    float4 v[1];
    sum_splits<1>(p, b, cc, v);
    if (c < n) *reinterpret_cast<float4*>(p.out + (long)b * n + c) = v[0];
  } else if constexpr (MODE == RED_SWIGLU) {
    const int c = 4 * ((int)blockIdx.x * kRedThreads + tid);
    const int cl = c < n ? c : n - 4;
    const int cc[2] = {cl, n + cl};
    float4 v[2];
    sum_splits<2>(p, b, cc, v);
    if (c < n) {
      const float4 g = v[0], u = v[1];
      const long o = (long)b * p.ldq + c;
      store4_split(p.xq + o, p.xq_lo + o, g.x / (1.0f + expf(-g.x)) * u.x,
                  g.y / (1.0f + expf(-g.y)) * u.y, g.z / (1.0f + expf(-g.z)) * u.z,
                  g.w / (1.0f + expf(-g.w)) * u.w);
    }
  } else {
    // Norm modes: the row stays in registers between the sum of squares and the scaling.
    constexpr int NPART = (MODE == PREP_EH) ? 2 : 1;
    int t = 0;
    if constexpr (MODE == PREP_EH) {
      t = p.tok[(long)b * p.tok_stride];
      if (t < 0 || t >= p.vocab) {
        if (tid == 0) set_error(p.err, 1u);
        t = 0;
      }
    }
#pragma unroll
    for (int q = 0; q < NPART; ++q) {
      float4 v[kRedNormVPT];
      float ss = 0.f;
      if constexpr (MODE == RED_EH || MODE == RED_RESID) {
        int cc[kRedNormVPT];
#pragma unroll
        for (int j = 0; j < kRedNormVPT; ++j) {
          const int c = 4 * (tid + j * kRedNormThreads);
          cc[j] = c < n ? c : n - 4;
        }
        sum_splits<kRedNormVPT>(p, b, cc, v);
      }
#pragma unroll
      for (int j = 0; j < kRedNormVPT; ++j) {
        const int c = 4 * (tid + j * kRedNormThreads);
        if (c < n) {
          if constexpr (MODE == PREP_NORM) {
            v[j] = p.h16 ? load4_bf16(p.h16 + (long)b * n + c)
                         : *reinterpret_cast<const float4*>(p.h + (long)b * n + c);
          } else if constexpr (MODE == PREP_EH) {
            v[j] = q == 0 ? *reinterpret_cast<const float4*>(p.h + (long)b * n + c)
                          : load4_bf16(p.embed + (long)t * n + c);
          } else {
            if constexpr (MODE == RED_RESID)
              v[j] = add4(*reinterpret_cast<const float4*>(p.res + (long)b * n + c), v[j]);
            *reinterpret_cast<float4*>(p.out + (long)b * n + c) = v[j];
            if (MODE == RED_RESID && p.dbg)
              *reinterpret_cast<float4*>(p.dbg + (long)b * p.dbg_ld + c) = v[j];
          }
          ss += dot4(v[j]);
        } else {
          v[j] = float4{0.f, 0.f, 0.f, 0.f};
        }
      }
      const float tot = block_sum(ss, red);
      const float r = 1.0f / sqrtf(tot / (float)n + p.eps);
      const uint16_t* g = q == 0 ? p.gain : p.gain2;
#pragma unroll
      for (int j = 0; j < kRedNormVPT; ++j) {
        const int c = 4 * (tid + j * kRedNormThreads);
        if (c < n) {
          const float4 gv = load4_bf16(g + c);
          const long o = (long)b * p.ldq + q * n + c;
          store4_split(p.xq + o, p.xq_lo + o, v[j].x * r * gv.x, v[j].y * r * gv.y,
                       v[j].z * r * gv.z, v[j].w * r * gv.w);
        }
      }
    }
  }
}

hipError_t launch_red(RedMode mode, const RedParams& p, int B, hipStream_t s) {
  if (B < 1 || p.n < 4 || p.n % 4 != 0 || p.ldq % 4 != 0) return hipErrorInvalidValue;
  if ((mode != RED_QKV && (!p.xq || !p.xq_lo)) ||
      (mode != RED_SWIGLU && mode != PREP_EH && mode != PREP_NORM && !p.out))
    return hipErrorInvalidValue;
  const bool norm = mode == RED_EH || mode == RED_RESID || mode == PREP_EH || mode == PREP_NORM;
  if (norm && (p.n > red_max_cols() || !p.gain || p.ldq < (mode == PREP_EH ? 2 : 1) * p.n))
    return hipErrorInvalidValue;
  if (mode == PREP_EH && (!p.gain2 || !p.h || !p.embed || !p.tok || !p.err))
    return hipErrorInvalidValue;
  if (mode == RED_RESID && !p.res) return hipErrorInvalidValue;
  if (mode == PREP_NORM && !p.h && !p.h16) return hipErrorInvalidValue;
  if (mode != PREP_EH && mode != PREP_NORM &&
      (!p.part || p.nsplit < 1 || p.nsplit > kRedMaxSplit || p.bp < B || p.n_part % 4 != 0))
    return hipErrorInvalidValue;
  const dim3 g(B), t(kRedNormThreads);
  const dim3 gc((p.n / 4 + kRedThreads - 1) / kRedThreads, B), tc(kRedThreads);  // column modes
  switch (mode) {
    case RED_EH: hipLaunchKernelGGL(red_kernel<RED_EH>, g, t, 0, s, p); break;
    case RED_QKV: hipLaunchKernelGGL(red_kernel<RED_QKV>, gc, tc, 0, s, p); break;
    case RED_RESID: hipLaunchKernelGGL(red_kernel<RED_RESID>, g, t, 0, s, p); break;
    case RED_SWIGLU: hipLaunchKernelGGL(red_kernel<RED_SWIGLU>, gc, tc, 0, s, p); break;
    case PREP_EH: hipLaunchKernelGGL(red_kernel<PREP_EH>, g, t, 0, s, p); break;
    case PREP_NORM: hipLaunchKernelGGL(red_kernel<PREP_NORM>, g, t, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ void widen_kernel(const uint16_t* src16, const float* src32, float* dst, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = src16 ? bf16_to_f32(src16[i]) : src32[i];
}

hipError_t launch_widen(int dtype, const void* src, float* dst, long n, hipStream_t s) {
  if (!src || !dst || n < 0) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(widen_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     dtype == 1 ? static_cast<const uint16_t*>(src) : nullptr,
                     dtype == 1 ? nullptr : static_cast<const float*>(src), dst, n);
  return hipGetLastError();
}

// One lane per sequence: accept drafts while they equal the target's tokens; the first
// mismatch (or row K) gives the next token (OpenVINO GenAI, Speculative Decoding,
// Overview).
__global__ void accept_kernel(const int* tokens, const int* draft, int B, int K, int* accepted,
                              int* next) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int a = 0;
  while (a < K && draft[(long)b * K + a] == tokens[(long)b * (K + 1) + a]) ++a;
  accepted[b] = a;
  next[b] = tokens[(long)b * (K + 1) + a];
}

hipError_t launch_accept(const int* tokens, const int* draft, int B, int K, int* accepted,
                         int* next, hipStream_t s) {
  if (!tokens || (K > 0 && !draft) || !accepted || !next || B < 1 || K < 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_kernel, dim3((B + 255) / 256), dim3(256), 0, s, tokens, draft, B, K,
                     accepted, next);
  return hipGetLastError();
}

__global__ void gather_rows_kernel(const uint16_t* src16, const float* src32, float* dst, int r0,
                                   int rows, int per, int src_per, int H) {
  const int i = blockIdx.y;
  const int r = r0 + i;
  const long srow = (long)(r / per) * src_per + r % per;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < H; c += gridDim.x * blockDim.x)
    dst[(long)i * H + c] = src16 ? bf16_to_f32(src16[srow * H + c]) : src32[srow * H + c];
}

hipError_t launch_gather_rows(int dtype, const void* src, float* dst, int r0, int rows, int per,
                              int src_per, int H, hipStream_t s) {
  if (!src || !dst || rows < 1 || per < 1 || src_per < per || H < 1 || r0 < 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((H + 255) / 256, rows), dim3(256), 0, s,
                     dtype == 1 ? static_cast<const uint16_t*>(src) : nullptr,
                     dtype == 1 ? nullptr : static_cast<const float*>(src), dst, r0, rows, per,
                     src_per, H);
  return hipGetLastError();
}

// Grid (row, kv head); thread i handles the rotate-half pair (i, i + d/2).
template <class CT>
__global__ void catchup_write_kernel(CatchupParams p) {
  using T = typename CT::T;
  const int i = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int half = p.d / 2;
  const int r = p.r0 + i;
  const int b = r / p.per, j = r % p.per;
  int lim = p.limit ? p.limit[b] : p.per;
  lim = lim < 0 ? 0 : lim > p.per ? p.per : lim;
  if (j >= lim || t >= half) return;
  const int slot = p.len[b] + p.off + j;
  const int position = p.pos[b] + p.off + j;
  if (slot < 0 || slot >= p.capacity) {
    if (t == 0) set_error(p.err, 2u);
    return;
  }
  float c, sn;
  rope_cs(position, t, p.d, p.theta, c, sn);
  const float* kr = p.kvrows + (long)i * p.ld + g * p.d;
  const float* vr = kr + p.n_kv * p.d;
  const float k1 = kr[t], k2 = kr[t + half];
  const long o = (((long)b * p.n_kv + g) * p.capacity + slot) * p.d;
  CT::put(static_cast<T*>(p.kc), o + t, k1 * c - k2 * sn);
  CT::put(static_cast<T*>(p.kc), o + t + half, k2 * c + k1 * sn);
  CT::put(static_cast<T*>(p.vc), o + t, vr[t]);
  CT::put(static_cast<T*>(p.vc), o + t + half, vr[t + half]);
}

hipError_t launch_catchup_write(int cdtype, const CatchupParams& p, hipStream_t s) {
  if (!p.kvrows || !p.kc || !p.vc || !p.len || !p.pos || p.per < 1 || p.rows < 1 ||
      p.d < 2 || p.d > 1024 || p.d % 2 != 0)
    return hipErrorInvalidValue;
  const dim3 grid(p.rows, p.n_kv), block((p.d / 2 + 63) / 64 * 64);
  if (cdtype == 1)
    hipLaunchKernelGGL(catchup_write_kernel<BF16>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(catchup_write_kernel<F32>, grid, block, 0, s, p);
  return hipGetLastError();
}

__global__ void catchup_commit_kernel(int* len, int* pos, const int* limit, int B, int per,
                                      int add, unsigned err_bit, unsigned* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int lim = limit ? limit[b] : per;
  if (lim < 0 || lim > per) {
    set_error(err, err_bit);
    lim = lim < 0 ? 0 : per;
  }
  len[b] += lim + add;
  pos[b] += lim + add;
}

hipError_t launch_catchup_commit(int* len, int* pos, const int* limit, int B, int per, int add,
                                 unsigned err_bit, unsigned* err, hipStream_t s) {
  if (!len || !pos || !err || B < 1 || per < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(catchup_commit_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len, pos,
                     limit, B, per, add, err_bit, err);
  return hipGetLastError();
}

}  // namespace mtp
