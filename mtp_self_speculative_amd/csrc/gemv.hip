// Weight-streaming GEMV for the MTP head's projections at small batch (VALU, fp32 accumulate).
//
// Every projection of the draft step (eh_proj, QKV, O, gate/up, down, lm_head) reads
// each weight byte once per step at about B flops per byte, so the kernels are bound
// by HBM bandwidth. A workgroup of four wave64s stages its fp32 input vector(s) in LDS
// (applying the RMSNorm / embedding-gather prologue on the fly), then each wave streams
// whole rows with 16-byte loads (64 lanes x 16 B = 1 KiB per instruction, several rows
// and column chunks in flight) and reduces across the wave. Epilogues fuse the residual
// add, SwiGLU and the vocabulary argmax (plain, or over logit / temperature + Gumbel
// noise to sample), so no [B, V] logits tensor has to be written.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

template <class WT>
__device__ __forceinline__ float load_h(const void* p, long i, int is_f32) {
  return is_f32 ? static_cast<const float*>(p)[i]
                : WT::get(static_cast<const typename WT::T*>(p), i);
}

template <class WT, int NB, int RPW, int U, int PRO, int EPI>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p) {
  using T = typename WT::T;
  constexpr int VEC = WT::kVec;
  constexpr int ROWS = (EPI == EPI_SWIGLU) ? RPW / 2 : RPW;  // logical rows per wave
  extern __shared__ __align__(16) float xs[];                 // [NB][col_block]
  __shared__ float rs[2][NB];
  __shared__ float red[kWavesPerBlock];
  __shared__ unsigned long long kred[kWavesPerBlock][NB];
  __shared__ int tok_s[NB];
  __shared__ int flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b0 = blockIdx.y * NB;
  const int ncols = p.ncols, CB = p.col_block;
  const int nblk = (ncols + CB - 1) / CB;
  const T* gain = static_cast<const T*>(p.gain);
  const T* gain2 = static_cast<const T*>(p.gain2);
  const int H = ncols / 2;  // PRO_EH only

  // ---- prologue: per-row RMS scales over the full input vectors
  if constexpr (PRO == PRO_EH) {
    if (threadIdx.x < NB) {
      int b = b0 + threadIdx.x, t = 0;
      if (b < p.B) {
        t = p.tok[(long)b * p.tok_stride];
        if (t < 0 || t >= p.vocab) {
          if (blockIdx.x == 0) set_error(p.err, 1u);
          t = 0;
        }
      }
      tok_s[threadIdx.x] = t;
    }
    __syncthreads();
  }
  if constexpr (PRO == PRO_RMS || PRO == PRO_EH) {
    for (int i = 0; i < NB; ++i) {
      const int b = b0 + i;
      float s1 = 0.f, s2 = 0.f;
      if (b < p.B) {
        if constexpr (PRO == PRO_RMS) {
          const float* xb = p.x + (long)b * p.ldx;
          for (int c = threadIdx.x; c < ncols; c += kThreads) s1 += xb[c] * xb[c];
        } else {
          const T* eb = static_cast<const T*>(p.embed) + (long)tok_s[i] * H;
          for (int c = threadIdx.x; c < H; c += kThreads) {
            float hv = load_h<WT>(p.h, (long)b * p.ldh + c, p.h_is_f32);
            float ev = WT::get(eb, c);
            s1 += hv * hv;
            s2 += ev * ev;
          }
        }
      }
      float t1 = block_sum(s1, red);
      float t2 = 0.f;
      if constexpr (PRO == PRO_EH) t2 = block_sum(s2, red);
      if (threadIdx.x == 0) {
        const float n = (PRO == PRO_EH) ? (float)H : (float)ncols;
        rs[0][i] = 1.0f / sqrtf(t1 / n + p.eps);
        rs[1][i] = 1.0f / sqrtf(t2 / n + p.eps);
      }
    }
    __syncthreads();
  }

  auto stage = [&](int blk) {
    const int c0 = blk * CB, cl = min(CB, ncols - c0);
    for (int i = 0; i < NB; ++i) {
      const int b = b0 + i;
      float* dst = xs + i * CB;
      for (int c = threadIdx.x; c < cl; c += kThreads) {
        const int cc = c0 + c;
        float v = 0.f;
        if (b < p.B) {
          if constexpr (PRO == PRO_PLAIN) {
            v = p.x[(long)b * p.ldx + cc];
          } else if constexpr (PRO == PRO_RMS) {
            v = p.x[(long)b * p.ldx + cc] * rs[0][i] * WT::get(gain, cc);
          } else {
            if (cc < H)
              v = load_h<WT>(p.h, (long)b * p.ldh + cc, p.h_is_f32) * rs[0][i] * WT::get(gain, cc);
            else
              v = WT::get(static_cast<const T*>(p.embed), (long)tok_s[i] * H + (cc - H)) *
                  rs[1][i] * WT::get(gain2, cc - H);
          }
        }
        dst[c] = v;
      }
    }
  };

  const int rows_per_group = kWavesPerBlock * ROWS;
  const int ngroups = (p.nrows + rows_per_group - 1) / rows_per_group;
  unsigned long long best[NB];
  int exr[NB];  // row that never wins (second-best pass), or -1
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    best[i] = 0ull;
    exr[i] = (epi_is_argmax(EPI) && p.excl && b0 + i < p.B)
                 ? p.excl[(long)(b0 + i) * p.excl_stride] : -1;
  }

  if (nblk == 1) {
    stage(0);
    __syncthreads();
  }

  for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const T* rp[RPW];
    bool valid[RPW];
    int lrow[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if constexpr (EPI == EPI_SWIGLU) {
        const int pr = g * rows_per_group + wave * ROWS + r / 2;
        lrow[r] = pr;
        valid[r] = pr < p.nrows;
        const T* base = static_cast<const T*>((r & 1) ? p.w1 : p.w0);
        rp[r] = base + (long)(valid[r] ? pr : 0) * ncols;
      } else {
        const int lr = g * rows_per_group + wave * ROWS + r;
        lrow[r] = lr;
        valid[r] = lr < p.nrows;
        const int rr = valid[r] ? lr : 0;
        const T* base;
        long loc;
        if (rr < p.seg1) {
          base = static_cast<const T*>(p.w0); loc = rr;
        } else if (rr < p.seg2) {
          base = static_cast<const T*>(p.w1); loc = rr - p.seg1;
        } else {
          base = static_cast<const T*>(p.w2); loc = rr - p.seg2;
        }
        rp[r] = base + loc * ncols;
      }
    }
    float acc[RPW][NB];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[r][i] = 0.f;

    for (int blk = 0; blk < nblk; ++blk) {
      if (nblk > 1) {
        __syncthreads();
        stage(blk);
        __syncthreads();
      }
      const int c0 = blk * CB, cl = min(CB, ncols - c0);
      for (int cb = lane * VEC; cb < cl; cb += kWave * VEC * U) {
        u32x4 wv[U][RPW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + u * kWave * VEC;
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            if (valid[r] && c < cl)
              wv[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp[r] + c0 + c));
            else
              wv[u][r] = u32x4{0u, 0u, 0u, 0u};
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + u * kWave * VEC;
          if (c < cl) {
            float wf[RPW][VEC];
#pragma unroll
            for (int r = 0; r < RPW; ++r) WT::unpack(wv[u][r], wf[r]);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
              float xv[VEC];
#pragma unroll
              for (int q = 0; q < VEC; q += 4) {
                const float4 t4 = *reinterpret_cast<const float4*>(xs + i * CB + c + q);
                xv[q] = t4.x; xv[q + 1] = t4.y; xv[q + 2] = t4.z; xv[q + 3] = t4.w;
              }
#pragma unroll
              for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int q = 0; q < VEC; ++q) acc[r][i] = fmaf(wf[r][q], xv[q], acc[r][i]);
            }
          }
        }
      }
    }

#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[r][i] = wave_sum(acc[r][i]);

    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int b = b0 + i;
        if (b >= p.B) continue;
        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int r = 0; r < RPW; r += 2) {
            if (!valid[r]) continue;
            const float gt = acc[r][i], up = acc[r + 1][i];
            p.out[(long)b * p.ldo + lrow[r]] = gt / (1.0f + expf(-gt)) * up;
          }
        } else {
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            if (!valid[r]) continue;
            const float y = acc[r][i];
            const long o = (long)b * p.ldo + lrow[r];
            if constexpr (EPI == EPI_STORE) {
              p.out[o] = y;
            } else if constexpr (EPI == EPI_RESID) {
              const float v = p.res[o] + y;
              p.out[o] = v;
              if (p.dbg) p.dbg[(long)b * p.dbg_ld + lrow[r]] = v;
            } else {  // EPI_ARGMAX / EPI_SAMPLE
              float val = y;
              if constexpr (EPI == EPI_SAMPLE) {
                const Philox4 rb = rng_block(p.smp.seeds[b], p.smp.offset, RNG_DRAFT,
                                             (uint64_t)p.smp.row, (uint64_t)(lrow[r] >> 2));
                val = y * p.smp.inv_temp + gumbel_of(philox_word(rb, lrow[r] & 3));
              }
              const unsigned long long k =
                  lrow[r] == exr[i] ? 0ull : pack_key(val, (uint32_t)lrow[r]);
              best[i] = k > best[i] ? k : best[i];
              if (p.logits) p.logits[(long)b * p.logits_ld + lrow[r]] = y;
            }
          }
        }
      }
    }
  }

  if constexpr (epi_is_argmax(EPI)) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) kred[wave][i] = best[i];
    }
    __syncthreads();
    if (threadIdx.x < NB) {
      const int b = b0 + threadIdx.x;
      unsigned long long k = 0ull;
      for (int w = 0; w < kWavesPerBlock; ++w) k = kred[w][threadIdx.x] > k ? kred[w][threadIdx.x] : k;
      if (b < p.B && k) publish_max_key(p.keys + b, k);
    }
    // the winner reads back only keys published by publish_max_key
    if (last_to_arrive(p.counter, gridDim.x * gridDim.y, &flag)) {
      for (int b = threadIdx.x; b < p.B; b += kThreads) {
        const unsigned long long k = take_key(p.keys + b);
        p.tok_out[(long)b * p.tok_out_stride] = (int)key_index(k);
        if (p.maxlogit) p.maxlogit[(long)b * (p.maxlogit_stride ? p.maxlogit_stride : 1)] = key_value(k);
        if (p.advance > 0) {
          const int adv = seq_steps(p.kseq, b, p.advance);  // the sequence's own steps
          p.len[b] += adv;
          p.pos[b] += adv;
        }
      }
    }
  }
}

template <class WT, int NB, int RPW, int U, int PRO, int EPI>
static hipError_t launch_one(const GemvParams& p, int max_grid, hipStream_t s) {
  constexpr int ROWS = (EPI == EPI_SWIGLU) ? RPW / 2 : RPW;
  const int rows_per_group = kWavesPerBlock * ROWS;
  const int ngroups = (p.nrows + rows_per_group - 1) / rows_per_group;
  int gx = ngroups < max_grid ? ngroups : max_grid;
  if (gx < 1) gx = 1;
  const int gy = (p.B + NB - 1) / NB;
  const size_t lds = (size_t)NB * p.col_block * sizeof(float);
  hipLaunchKernelGGL((gemv_kernel<WT, NB, RPW, U, PRO, EPI>), dim3(gx, gy), dim3(kThreads), lds, s,
                     p);
  return hipGetLastError();
}

template <class WT, int PRO, int EPI>
static hipError_t launch_nb(const GemvParams& p, int max_grid, hipStream_t s) {
  if (p.B <= 1) return launch_one<WT, 1, 4, 4, PRO, EPI>(p, max_grid, s);
  if (p.B <= 2) return launch_one<WT, 2, 4, 2, PRO, EPI>(p, max_grid, s);
  if (p.B <= 4) return launch_one<WT, 4, 2, 2, PRO, EPI>(p, max_grid, s);
  return launch_one<WT, 8, 2, 2, PRO, EPI>(p, max_grid, s);
}

template <class WT>
static hipError_t launch_dt(Pro pro, Epi epi, const GemvParams& p, int max_grid, hipStream_t s) {
  if (pro == PRO_EH && epi == EPI_STORE) return launch_nb<WT, PRO_EH, EPI_STORE>(p, max_grid, s);
  if (pro == PRO_RMS && epi == EPI_STORE) return launch_nb<WT, PRO_RMS, EPI_STORE>(p, max_grid, s);
  if (pro == PRO_PLAIN && epi == EPI_RESID) return launch_nb<WT, PRO_PLAIN, EPI_RESID>(p, max_grid, s);
  if (pro == PRO_RMS && epi == EPI_SWIGLU) return launch_nb<WT, PRO_RMS, EPI_SWIGLU>(p, max_grid, s);
  if (pro == PRO_RMS && epi == EPI_ARGMAX) return launch_nb<WT, PRO_RMS, EPI_ARGMAX>(p, max_grid, s);
  if (pro == PRO_RMS && epi == EPI_SAMPLE) return launch_nb<WT, PRO_RMS, EPI_SAMPLE>(p, max_grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int wdtype, Pro pro, Epi epi, const GemvParams& p, int max_grid,
                       hipStream_t s) {
  const int step = 64 * (wdtype == 0 ? F32::kVec : BF16::kVec);
  if (p.col_block < step || p.col_block % step != 0 || p.ncols < 1 || p.nrows < 1)
    return hipErrorInvalidValue;
  if (epi == EPI_SAMPLE && (!(p.smp.inv_temp > 0.f) || !p.smp.seeds)) return hipErrorInvalidValue;
  return wdtype == 0 ? launch_dt<F32>(pro, epi, p, max_grid, s)
                     : launch_dt<BF16>(pro, epi, p, max_grid, s);
}

}  // namespace mtp
