// Persistent, software-pipelined weight-streaming GEMV for batch 1-2 (the latency path).
//
// Each wave owns the logical rows gw, gw + nw, ... (nw = waves in the grid) and walks
// them in stages of CH 16-byte chunks per lane (CH KiB of one row per wave instruction
// group). Two register buffers alternate: while one stage is consumed the next is in
// flight. Every load is unconditional (addresses past the end are clamped to valid
// data and meet zeros in the LDS copy of the input), so the compiler can count
// outstanding loads exactly and wait only for the buffer being consumed. The grid is
// sized to a few workgroups per CU so that the whole chip streams without re-staging
// the input. The input-vector loads of the prologue go out first, then the first two
// weight stages, so the norm reduction and the staging of the fp32 input vector into
// LDS overlap the first HBM round trip. Weight loads are non-temporal (used once).
//
// A logical row has P parts read with the same input vector: P = 2 streams the gate
// and up rows of one SwiGLU unit together. The epilogues are those of the general
// GEMV (store, residual add, SwiGLU, vocabulary argmax with last-workgroup finish, and
// the sampling argmax over value / temperature + Gumbel noise).
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kPipeWPB = 4;
constexpr int kPipeCH = 4;
constexpr size_t kPipeMaxLds = 64 * 1024;

template <class WT, int NB, int P, int CH, int WPB, int PRO, int EPI>
__global__ __launch_bounds__(WPB * 64) void gemv_pipe_kernel(GemvParams p) {
  using T = typename WT::T;
  constexpr int VEC = WT::kVec;
  constexpr int SW = CH * kWave * VEC;  // columns per stage
  constexpr int NT = WPB * kWave;
  constexpr int SLOTS = 2;              // prologue: 8-element groups per thread per batch
  constexpr int NPART = (PRO == PRO_EH) ? 2 : 1;
  extern __shared__ __align__(16) float xs[];  // [NB][ldl], zero beyond ncols
  __shared__ float red[WPB];
  __shared__ unsigned long long kred[WPB][NB];
  __shared__ int tok_s[NB];
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncols = p.ncols;
  const int nw = gridDim.x * WPB;
  const int gw = blockIdx.x * WPB + wave;
  const int S = (ncols + SW - 1) / SW;
  const int ldl = S * SW;
  const int nrows_w = gw < p.nrows ? (p.nrows - 1 - gw) / nw + 1 : 0;
  const int items = nrows_w * S;
  const int B = p.B;

  // Row base pointer of part q of logical row r.
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
  // Stages past the wave's last one are prefetched from the small dummy region (the
  // loads stay unconditional, but re-read no weights from HBM).
  auto load = [&](u32x4 (&buf)[P][CH], int it) {
    const bool live = it < items;
    const int r = live ? gw + (it / S) * nw : 0;
    const int c0 = live ? (it % S) * SW : 0;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const T* rp = live ? row_ptr(r, q) : static_cast<const T*>(p.dummy);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        int col = c0 + c * kWave * VEC + lane * VEC;
        col = (col < ncols || !live) ? col : ncols - VEC;
        buf[q][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp + col));
      }
    }
  };

  // ---- residual operands of this wave's first rows: lane l holds row gw + l*nw
  float resv[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) resv[i] = 0.f;
  if constexpr (EPI == EPI_RESID) {
    const int rr = lane < nrows_w ? gw + lane * nw : 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) resv[i] = p.res[(long)(i < B ? i : 0) * p.ldo + rr];
  }

  // ---- prologue loads: thread owns 8-element groups c = (slot * NT + tid) * 8
  if constexpr (PRO == PRO_EH) {
    if (tid < NB) {
      int t = 0;
      if (tid < B) {
        t = p.tok[(long)tid * p.tok_stride];
        if (t < 0 || t >= p.vocab) {
          if (blockIdx.x == 0) set_error(p.err, 1u);
          t = 0;
        }
      }
      tok_s[tid] = t;
    }
    __syncthreads();
  }
  const int Hh = (PRO == PRO_EH) ? ncols / 2 : ncols;  // length of one normalised part
  const int per_batch = NT * 8 * SLOTS;
  float v[NB][NPART][SLOTS][8];
  float gv[NPART][SLOTS][8];
  const T* gains[2] = {static_cast<const T*>(p.gain), static_cast<const T*>(p.gain2)};
  auto fetch = [&](int i, int q, int base) {
    const int ib = i < B ? i : 0;
#pragma unroll
    for (int sl = 0; sl < SLOTS; ++sl) {
      int c = base + (sl * NT + tid) * 8;
      c = c < Hh ? c : Hh - 8;
      if constexpr (PRO != PRO_PLAIN) {
        if (i == 0) WT::load8(gains[q] + c, gv[q][sl]);
      }
      if constexpr (PRO == PRO_PLAIN || PRO == PRO_RMS) {
        load8_f32(p.x + (long)ib * p.ldx + c, v[i][q][sl]);
      } else if (q == 0) {
        load8_f32(static_cast<const float*>(p.h) + (long)ib * p.ldh + c, v[i][q][sl]);
      } else {
        WT::load8(static_cast<const T*>(p.embed) + (long)tok_s[ib] * Hh + c, v[i][q][sl]);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int q = 0; q < NPART; ++q) fetch(i, q, 0);
  __builtin_amdgcn_sched_barrier(0);  // keep the input loads ahead of the weight stream

  load(A, 0);
  load(Bf, 1);
  __builtin_amdgcn_sched_barrier(0);

  // ---- prologue: fp32 input vectors (normalised where needed) into LDS
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float* dst = xs + (long)i * ldl;
    const bool live = i < B;
    float rsq[NPART];
    if constexpr (PRO == PRO_PLAIN) {
      rsq[0] = 1.f;
    } else {
      float ssum[NPART];
#pragma unroll
      for (int q = 0; q < NPART; ++q) ssum[q] = 0.f;
      for (int base = 0; base < Hh; base += per_batch) {
        if (base > 0) {
#pragma unroll
          for (int q = 0; q < NPART; ++q) fetch(i, q, base);
        }
#pragma unroll
        for (int q = 0; q < NPART; ++q)
#pragma unroll
          for (int sl = 0; sl < SLOTS; ++sl) {
            const bool in = base + (sl * NT + tid) * 8 < Hh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = in ? v[i][q][sl][e] : 0.f;
              ssum[q] = fmaf(x, x, ssum[q]);
            }
          }
      }
#pragma unroll
      for (int q = 0; q < NPART; ++q) {
        const float tot = block_sum(ssum[q], red);
        rsq[q] = 1.0f / sqrtf(tot / (float)Hh + p.eps);
      }
    }
    for (int base = 0; base < Hh; base += per_batch) {
      if (base > 0 && (PRO == PRO_PLAIN || Hh > per_batch)) {
#pragma unroll
        for (int q = 0; q < NPART; ++q) fetch(i, q, base);
      }
#pragma unroll
      for (int q = 0; q < NPART; ++q) {
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
          const int c = base + (sl * NT + tid) * 8;
          if (c < Hh) {
            float o[8];
            if constexpr (PRO == PRO_PLAIN) {
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = live ? v[i][q][sl][e] : 0.f;
            } else {
              if (base > 0) {
                const int cc = c < Hh ? c : Hh - 8;
                WT::load8(gains[q] + cc, gv[q][sl]);
              }
#pragma unroll
              for (int e = 0; e < 8; ++e)
                o[e] = live ? v[i][q][sl][e] * rsq[q] * gv[q][sl][e] : 0.f;
            }
            store8_lds(dst + q * Hh + c, o);
          }
        }
      }
    }
    for (int c = ncols + tid; c < ldl; c += NT) dst[c] = 0.f;
  }
  __syncthreads();

  // ---- main pipeline
  float acc[P][NB];
#pragma unroll
  for (int q = 0; q < P; ++q)
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[q][i] = 0.f;
  unsigned long long best[NB];
  float gum[NB];
  uint64_t seed[NB];  // EPI_SAMPLE: the sequences' random-stream seeds, read once
  int exr[NB];        // row that never wins (second-best pass), or -1
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    exr[i] = (epi_is_argmax(EPI) && p.excl && i < B) ? p.excl[(long)i * p.excl_stride] : -1;
    best[i] = 0ull;
    gum[i] = 0.f;
    seed[i] = (EPI == EPI_SAMPLE && i < B) ? p.smp.seeds[i] : 0ull;
  }

  auto consume = [&](u32x4 (&buf)[P][CH], int it) {
    const int c0 = (it % S) * SW;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = c0 + c * kWave * VEC + lane * VEC;
      float wf[P][VEC];
#pragma unroll
      for (int q = 0; q < P; ++q) WT::unpack(buf[q][c], wf[q]);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        float xv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 t4 = *reinterpret_cast<const float4*>(xs + (long)i * ldl + col + e);
          xv[e] = t4.x; xv[e + 1] = t4.y; xv[e + 2] = t4.z; xv[e + 3] = t4.w;
        }
#pragma unroll
        for (int q = 0; q < P; ++q)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[q][i] = fmaf(wf[q][e], xv[e], acc[q][i]);
      }
    }
    if (it % S == S - 1) {
      const int r = gw + (it / S) * nw;
      const int j = it / S;  // this wave's j-th row
#pragma unroll
      for (int q = 0; q < P; ++q)
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[q][i] = wave_sum_fast(acc[q][i]);
      float rvv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) rvv[i] = j < kWave ? __shfl(resv[i], j, kWave) : 0.f;
      float nz[NB];
      if constexpr (EPI == EPI_SAMPLE) {
        // Lane l holds the Gumbel noise of this wave's row 64 * (j / 64) + l, drawn for
        // 64 rows at once so that the random blocks are computed by all lanes.
        if ((j & 63) == 0) {
          const int rl = gw + (j + lane) * nw;  // rows past the end are drawn, never used
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            const Philox4 rb = rng_block(seed[i], p.smp.offset, RNG_DRAFT, (uint64_t)p.smp.row,
                                         (uint64_t)(rl >> 2));
            gum[i] = gumbel_of(philox_word(rb, rl & 3));
          }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) nz[i] = __shfl(gum[i], j & 63, kWave);
      }
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
            const float y = rv + acc[0][i];
            p.out[o] = y;
            if (p.dbg) p.dbg[(long)i * p.dbg_ld + r] = y;
          } else {
            float val = acc[0][i];
            if constexpr (EPI == EPI_SAMPLE) val = val * p.smp.inv_temp + nz[i];
            const unsigned long long k = r == exr[i] ? 0ull : pack_key(val, (uint32_t)r);
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

  if constexpr (epi_is_argmax(EPI)) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) kred[wave][i] = best[i];
    }
    __syncthreads();
    if (tid < NB && tid < B) {
      unsigned long long k = 0ull;
      for (int w = 0; w < WPB; ++w) k = kred[w][tid] > k ? kred[w][tid] : k;
      if (k) publish_max_key(p.keys + tid, k);
    }
    // the winner reads back only keys published by publish_max_key
    if (last_to_arrive(p.counter, gridDim.x, &flag)) {
      for (int b = tid; b < B; b += NT) {
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

static int pipe_stage_cols(int wdtype) { return kPipeCH * kWave * (wdtype == 0 ? 4 : 8); }

bool gemv_pipe_fits(int ncols, int B, int wdtype) {
  const int sw = pipe_stage_cols(wdtype);
  const size_t ldl = (size_t)(ncols + sw - 1) / sw * sw;
  return B >= 1 && B <= 2 && ncols >= 8 && ldl * B * sizeof(float) <= kPipeMaxLds;
}

// 16-byte chunks per lane and stage. Measured at batch 1 on MI355X (q8b shapes, caches
// flushed): the lm_head and gate/up streams run best with 2 KB per wave stage (the lm_head
// at 6.97 TB/s against 6.67 with 4 KB), the shorter matrices with 4 KB.
template <int EPI>
constexpr int pipe_ch() {
  return (EPI == EPI_ARGMAX || EPI == EPI_SAMPLE || EPI == EPI_SWIGLU) ? 2 : kPipeCH;
}

template <class WT, int NB, int P, int PRO, int EPI>
static hipError_t pipe_one(const GemvParams& p, int grid, hipStream_t s) {
  constexpr int CH = pipe_ch<EPI>();
  const int sw = CH * kWave * WT::kVec;
  const size_t ldl = (size_t)(p.ncols + sw - 1) / sw * sw;
  const size_t lds = (size_t)NB * ldl * sizeof(float);
  hipLaunchKernelGGL((gemv_pipe_kernel<WT, NB, P, CH, kPipeWPB, PRO, EPI>), dim3(grid),
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
  if (pro == PRO_RMS && epi == EPI_SAMPLE) return pipe_nb<WT, PRO_RMS, EPI_SAMPLE>(p, grid, s);
  return hipErrorInvalidValue;
}

int gemv_pipe_grid(int nrows, int ncols, int wdtype, int num_cu) {
  // Measured on MI355X at batch 1: matrices with many rows or long rows (two or more
  // stages per row) stream best with two workgroups per CU; short-row matrices with a
  // few thousand rows want about one row per wave, four workgroups per CU.
  const int sw = pipe_stage_cols(wdtype);
  const int stages = (ncols + sw - 1) / sw;
  const int per_cu = (nrows >= 64 * 1024 || stages >= 2) ? 2 : 4;
  int g = per_cu * num_cu;
  const int rows_cap = (nrows + kPipeWPB - 1) / kPipeWPB;
  if (g > rows_cap) g = rows_cap;
  return g < 1 ? 1 : g;
}

hipError_t launch_gemv_pipe(int wdtype, Pro pro, Epi epi, const GemvParams& p, int grid,
                            hipStream_t s) {
  if (!gemv_pipe_fits(p.ncols, p.B, wdtype) || p.ncols % 8 != 0 || p.nrows < 1 || grid < 1)
    return hipErrorInvalidValue;
  if (pro == PRO_EH && !p.h_is_f32) return hipErrorInvalidValue;
  if (epi == EPI_SAMPLE && (!(p.smp.inv_temp > 0.f) || !p.smp.seeds)) return hipErrorInvalidValue;
  static_assert(kPipeCH * kWave * 16 <= kDummyBytes, "dummy region too small");
  if (!p.dummy) return hipErrorInvalidValue;
  return wdtype == 0 ? pipe_dt<F32>(pro, epi, p, grid, s) : pipe_dt<BF16>(pro, epi, p, grid, s);
}

}  // namespace mtp
