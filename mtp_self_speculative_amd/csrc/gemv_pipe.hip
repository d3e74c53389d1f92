// Persistent, software-pipelined weight-streaming GEMV for batch 1-2 (the latency path).
//
// Each wave owns the logical rows gw, gw + nw, ... (nw = waves in the grid) and walks
// them in stages of CH 16-byte chunks per lane (CH KiB of one row per wave instruction
// group). Two register buffers alternate: while one stage is consumed the next is in
// flight, so every wave keeps up to 2*CH KiB requested; the grid is sized to a few
// workgroups per CU so that the whole chip streams without re-staging the input. The
// first two stages are requested before the prologue (token gather, RMS reductions,
// staging of the fp32 input vector into LDS), hiding the prologue behind the first
// HBM round trip. Weight loads are non-temporal: each byte is used once.
//
// A logical row has P parts read with the same input vector: P = 2 streams the gate
// and up rows of one SwiGLU unit together. The epilogues are those of the general
// GEMV (store, residual add, SwiGLU, vocabulary argmax with last-workgroup finish).
#include "common.h"
#include "kernels.h"

namespace mtp {

template <class WT>
__device__ __forceinline__ float ld_h(const void* p, long i, int is_f32) {
  return is_f32 ? static_cast<const float*>(p)[i]
                : WT::get(static_cast<const typename WT::T*>(p), i);
}

template <class WT, int NB, int P, int CH, int WPB, int PRO, int EPI>
__global__ __launch_bounds__(WPB * 64) void gemv_pipe_kernel(GemvParams p) {
  using T = typename WT::T;
  constexpr int VEC = WT::kVec;
  constexpr int SW = CH * kWave * VEC;  // columns per stage
  extern __shared__ __align__(16) float xs[];  // [NB][ncols]
  __shared__ float red[WPB];
  __shared__ unsigned long long kred[WPB][NB];
  __shared__ int tok_s[NB];
  __shared__ int flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nthreads = WPB * kWave;
  const int ncols = p.ncols;
  const int nw = gridDim.x * WPB;
  const int gw = blockIdx.x * WPB + wave;
  const int S = (ncols + SW - 1) / SW;
  const int nrows_w = gw < p.nrows ? (p.nrows - 1 - gw) / nw + 1 : 0;
  const int items = nrows_w * S;
  const int B = p.B;

  // Row base pointers of part q of logical row r.
  auto row_ptr = [&](int r, int q) -> const T* {
    if constexpr (P == 2) {
      return static_cast<const T*>(q ? p.w1 : p.w0) + (long)r * ncols;
    } else {
      if (r < p.seg1) return static_cast<const T*>(p.w0) + (long)r * ncols;
      if (r < p.seg2) return static_cast<const T*>(p.w1) + (long)(r - p.seg1) * ncols;
      return static_cast<const T*>(p.w2) + (long)(r - p.seg2) * ncols;
    }
  };

  u32x4 A[P][CH], Bf[P][CH];
  auto load = [&](u32x4 (&buf)[P][CH], int it) {
    const bool ok = it < items;
    const int r = ok ? gw + (it / S) * nw : 0;
    const int c0 = ok ? (it % S) * SW : 0;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const T* rp = row_ptr(r, q) + c0 + lane * VEC;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int col = c0 + c * kWave * VEC + lane * VEC;
        buf[q][c] = (ok && col < ncols)
                        ? __builtin_nontemporal_load(
                              reinterpret_cast<const u32x4*>(rp + c * kWave * VEC))
                        : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  load(A, 0);
  load(Bf, 1);

  // ---- residual operands of this wave's first rows: lane l holds row gw + l*nw
  float resv[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) resv[i] = 0.f;
  if constexpr (EPI == EPI_RESID) {
    if (lane < nrows_w) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i < B) resv[i] = p.res[(long)i * p.ldo + gw + lane * nw];
    }
  }

  // ---- prologue: fp32 input vectors (normalised where needed) into LDS. Every thread
  // owns 8-element groups c = (slot * nthreads + tid) * 8; all loads of a batch are in
  // flight together and the values stay in registers between the reduction and staging.
  constexpr int SLOTS = 2;
  const int per_batch = nthreads * 8 * SLOTS;
  const T* gain = static_cast<const T*>(p.gain);
  const T* gain2 = static_cast<const T*>(p.gain2);
  if constexpr (PRO == PRO_EH) {
    if (threadIdx.x < NB) {
      const int b = threadIdx.x;
      int t = 0;
      if (b < B) {
        t = p.tok[(long)b * p.tok_stride];
        if (t < 0 || t >= p.vocab) {
          if (blockIdx.x == 0) set_error(p.err, 1u);
          t = 0;
        }
      }
      tok_s[b] = t;
    }
    __syncthreads();
  }
  const int Hh = (PRO == PRO_EH) ? ncols / 2 : ncols;  // length of one normalised part
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float* dst = xs + i * ncols;
    if (i >= B) {
      for (int c = threadIdx.x; c < ncols; c += nthreads) dst[c] = 0.f;
      continue;
    }
    if constexpr (PRO == PRO_PLAIN) {
      const float* xb = p.x + (long)i * p.ldx;
      for (int base = 0; base < ncols; base += per_batch) {
        float v[SLOTS][8];
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
          const int c = base + (sl * nthreads + threadIdx.x) * 8;
          if (c < ncols) load8_f32(xb + c, v[sl]);
        }
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
          const int c = base + (sl * nthreads + threadIdx.x) * 8;
          if (c < ncols) store8_lds(dst + c, v[sl]);
        }
      }
    } else {
      // One or two parts of length Hh, each RMS-normalised with its own gain.
      constexpr int NPART = (PRO == PRO_EH) ? 2 : 1;
      float ssum[NPART];
#pragma unroll
      for (int q = 0; q < NPART; ++q) ssum[q] = 0.f;
      const bool one_batch = Hh <= per_batch;
      float v[NPART][SLOTS][8];
      auto fetch = [&](int q, int base) {
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
          const int c = base + (sl * nthreads + threadIdx.x) * 8;
          if (c < Hh) {
            if constexpr (PRO == PRO_RMS) {
              load8_f32(p.x + (long)i * p.ldx + c, v[q][sl]);
            } else if (q == 0) {
              if (p.h_is_f32)
                load8_f32(static_cast<const float*>(p.h) + (long)i * p.ldh + c, v[q][sl]);
              else
                WT::load8(static_cast<const T*>(p.h) + (long)i * p.ldh + c, v[q][sl]);
            } else {
              WT::load8(static_cast<const T*>(p.embed) + (long)tok_s[i] * Hh + c, v[q][sl]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[q][sl][e] = 0.f;
          }
        }
      };
      for (int base = 0; base < Hh; base += per_batch) {
#pragma unroll
        for (int q = 0; q < NPART; ++q) fetch(q, base);
#pragma unroll
        for (int q = 0; q < NPART; ++q)
#pragma unroll
          for (int sl = 0; sl < SLOTS; ++sl)
#pragma unroll
            for (int e = 0; e < 8; ++e) ssum[q] = fmaf(v[q][sl][e], v[q][sl][e], ssum[q]);
      }
      float tot[NPART];
#pragma unroll
      for (int q = 0; q < NPART; ++q) tot[q] = block_sum(ssum[q], red);
      float rsq[NPART];
#pragma unroll
      for (int q = 0; q < NPART; ++q) rsq[q] = 1.0f / sqrtf(tot[q] / (float)Hh + p.eps);
      for (int base = 0; base < Hh; base += per_batch) {
        if (!one_batch) {
#pragma unroll
          for (int q = 0; q < NPART; ++q) fetch(q, base);
        }
#pragma unroll
        for (int q = 0; q < NPART; ++q) {
          const T* gq = q == 0 ? gain : gain2;
#pragma unroll
          for (int sl = 0; sl < SLOTS; ++sl) {
            const int c = base + (sl * nthreads + threadIdx.x) * 8;
            if (c < Hh) {
              float gv[8];
              WT::load8(gq + c, gv);
              float o[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = v[q][sl][e] * rsq[q] * gv[e];
              store8_lds(dst + q * Hh + c, o);
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- main pipeline
  float acc[P][NB];
#pragma unroll
  for (int q = 0; q < P; ++q)
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[q][i] = 0.f;
  unsigned long long best[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) best[i] = 0ull;

  auto consume = [&](u32x4 (&buf)[P][CH], int it) {
    const int c0 = (it % S) * SW;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = c0 + c * kWave * VEC + lane * VEC;
      if (col < ncols) {
        float wf[P][VEC];
#pragma unroll
        for (int q = 0; q < P; ++q) WT::unpack(buf[q][c], wf[q]);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          float xv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; e += 4) {
            const float4 t4 = *reinterpret_cast<const float4*>(xs + i * ncols + col + e);
            xv[e] = t4.x; xv[e + 1] = t4.y; xv[e + 2] = t4.z; xv[e + 3] = t4.w;
          }
#pragma unroll
          for (int q = 0; q < P; ++q)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[q][i] = fmaf(wf[q][e], xv[e], acc[q][i]);
        }
      }
    }
    if (it % S == S - 1) {
      const int r = gw + (it / S) * nw;
      const int j = it / S;  // this wave's j-th row
#pragma unroll
      for (int q = 0; q < P; ++q)
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[q][i] = wave_sum(acc[q][i]);
      float rvv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) rvv[i] = j < kWave ? __shfl(resv[i], j, kWave) : 0.f;
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (i >= B) continue;
          const long o = (long)i * p.ldo + r;
          if constexpr (EPI == EPI_SWIGLU) {
            const float gt = acc[0][i], up = acc[P - 1][i];
            p.out[o] = gt / (1.0f + expf(-gt)) * up;
          } else if constexpr (EPI == EPI_STORE) {
            p.out[o] = acc[0][i];
          } else if constexpr (EPI == EPI_RESID) {
            const float rv = j < kWave ? rvv[i] : p.res[o];
            const float v = rv + acc[0][i];
            p.out[o] = v;
            if (p.dbg) p.dbg[(long)i * p.dbg_ld + r] = v;
          } else {
            const unsigned long long k = pack_key(acc[0][i], (uint32_t)r);
            best[i] = k > best[i] ? k : best[i];
            if (p.logits) p.logits[(long)i * p.logits_ld + r] = acc[0][i];
          }
        }
      }
#pragma unroll
      for (int q = 0; q < P; ++q)
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[q][i] = 0.f;
    }
  };

  for (int it = 0; it < items; it += 2) {
    consume(A, it);
    load(A, it + 2);
    if (it + 1 >= items) break;
    consume(Bf, it + 1);
    load(Bf, it + 3);
  }

  if constexpr (EPI == EPI_ARGMAX) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) kred[wave][i] = best[i];
    }
    __syncthreads();
    if (threadIdx.x < NB && (int)threadIdx.x < B) {
      unsigned long long k = 0ull;
      for (int w = 0; w < WPB; ++w) k = kred[w][threadIdx.x] > k ? kred[w][threadIdx.x] : k;
      if (k) keep_alive(atomic_max_key(p.keys + threadIdx.x, k));
    }
    if (last_to_arrive(p.counter, gridDim.x, &flag)) {
      for (int b = threadIdx.x; b < B; b += nthreads) {
        const unsigned long long k = take_key(p.keys + b);
        p.tok_out[(long)b * p.tok_out_stride] = (int)key_index(k);
        if (p.maxlogit) p.maxlogit[b] = key_value(k);
        if (p.advance > 0) {
          p.len[b] += p.advance;
          p.pos[b] += p.advance;
        }
      }
    }
  }
}

constexpr int kPipeWPB = 4;
constexpr int kPipeCH = 4;
constexpr size_t kPipeMaxLds = 64 * 1024;

bool gemv_pipe_fits(int ncols, int B) {
  return B >= 1 && B <= 2 && (size_t)B * ncols * sizeof(float) <= kPipeMaxLds;
}

template <class WT, int NB, int P, int PRO, int EPI>
static hipError_t pipe_one(const GemvParams& p, int grid, hipStream_t s) {
  const size_t lds = (size_t)NB * p.ncols * sizeof(float);
  hipLaunchKernelGGL((gemv_pipe_kernel<WT, NB, P, kPipeCH, kPipeWPB, PRO, EPI>), dim3(grid),
                     dim3(kPipeWPB * 64), lds, s, p);
  return hipGetLastError();
}

template <class WT, int PRO, int EPI>
static hipError_t pipe_nb(const GemvParams& p, int grid, hipStream_t s) {
  constexpr int P = (EPI == EPI_SWIGLU) ? 2 : 1;
  if (p.B <= 1) return pipe_one<WT, 1, P, PRO, EPI>(p, grid, s);
  return pipe_one<WT, 2, P, PRO, EPI>(p, grid, s);
}

template <class WT>
static hipError_t pipe_dt(Pro pro, Epi epi, const GemvParams& p, int grid, hipStream_t s) {
  if (pro == PRO_EH && epi == EPI_STORE) return pipe_nb<WT, PRO_EH, EPI_STORE>(p, grid, s);
  if (pro == PRO_RMS && epi == EPI_STORE) return pipe_nb<WT, PRO_RMS, EPI_STORE>(p, grid, s);
  if (pro == PRO_PLAIN && epi == EPI_RESID) return pipe_nb<WT, PRO_PLAIN, EPI_RESID>(p, grid, s);
  if (pro == PRO_RMS && epi == EPI_SWIGLU) return pipe_nb<WT, PRO_RMS, EPI_SWIGLU>(p, grid, s);
  if (pro == PRO_RMS && epi == EPI_ARGMAX) return pipe_nb<WT, PRO_RMS, EPI_ARGMAX>(p, grid, s);
  return hipErrorInvalidValue;
}

int gemv_pipe_grid(int nrows, int num_cu) {
  // Huge matrices: a few persistent workgroups per CU stream best. Smaller ones: about
  // one logical row per wave, capped at eight workgroups per CU.
  if (nrows >= 64 * 1024) return 2 * num_cu;
  int g = (nrows + kPipeWPB - 1) / kPipeWPB;
  const int cap = 8 * num_cu;
  return g < cap ? (g < 1 ? 1 : g) : cap;
}

hipError_t launch_gemv_pipe(int wdtype, Pro pro, Epi epi, const GemvParams& p, int grid,
                            hipStream_t s) {
  if (!gemv_pipe_fits(p.ncols, p.B)) return hipErrorInvalidValue;
  return wdtype == 0 ? pipe_dt<F32>(pro, epi, p, grid, s) : pipe_dt<BF16>(pro, epi, p, grid, s);
}

}  // namespace mtp
