// Weight-streaming bf16 contraction on the matrix cores, for batches of 3..64 sequences.
//
// At these batch sizes every projection is still HBM-bound (each weight byte feeds B
// multiply-adds), but a VALU dot product per sequence would be compute-bound from about
// B = 20 on, so the multiply-adds go to v_mfma_f32_16x16x32_bf16: a 16-row slice of W
// (A operand, one 16-byte load per lane: row lane%16, columns 8*(lane/16)..+7 of a
// 32-column step) against 16 sequences of the input (B operand, same column mapping).
// The input arrives as two bf16 planes hi + lo of its fp32 values and both are
// multiplied (two MFMAs per step into one fp32 accumulator): rounding the input to one
// bf16 would cost several hundredths in the hidden state at these sizes.
//
// Work is split into items of (128-row tile, K split). A workgroup of four waves takes
// items in turn (a persistent grid); wave w owns two 16-row slices of the tile, which
// share every input fragment it reads from LDS. Each item is walked in chunks of 256
// columns: per chunk a wave streams 32 rows x 512 bytes of W (sixteen 16-byte loads per
// lane, so every row piece is a full 64-byte segment) and runs 32 x NB MFMAs. The input
// rows (both planes) of the chunk are staged once per workgroup in LDS (double-buffered)
// and read from there by all waves. W stages are double-buffered in registers; all loads
// are unconditional (indexes past the end are clamped), so the compiler can wait for
// exactly the buffer being consumed.
//
// With a packed copy of W (launch_pack) the weight loads are contiguous instead: 1 KB per
// wave instruction, each 128 x 256 block one 64 KB region. On packed weights at 33..64
// sequences, items may also be 256 rows (eight waves over two blocks; see mm_plan).
//
// Epilogues: EPI_STORE writes the fp32 partial sums of the item's K split (a row-wise
// reduction kernel adds the splits in a fixed order, so results are deterministic);
// EPI_ARGMAX (one split) folds each row's value into a packed (value, index) key per
// sequence and finishes with the last-workgroup protocol of the GEMV; EPI_SAMPLE does
// the same with value / temperature + Gumbel noise, which samples softmax(value / T).
#include "common.h"
#include "kernels.h"

namespace mtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMmWaves = 4;                       // waves of a 128-row item
constexpr int kMmMT = 2;                          // 16-row slices per wave
constexpr int kMmTileRows = 16 * kMmMT * kMmWaves;  // 128: rows of a packed block
constexpr int kMmChunk = 256;                     // columns per stage
constexpr int kMmKSteps = kMmChunk / 32;          // MFMA k-steps per stage
constexpr int kMmMaxNB = 4;       // 16-sequence tiles of the general kernel
constexpr int kMmMaxNBArgmax = 8;  // of the greedy lm_head on packed weights (half-chunk stages)
constexpr int kMmMaxSplit = 16;  // the row-wise reductions add at most this many splits

__host__ __device__ int mm_chunks(int ncols) { return (ncols + kMmChunk - 1) / kMmChunk; }
constexpr long kMmPackBlock = (long)kMmTileRows * kMmChunk;  // elements per packed block
int mm_batch_pad(int B) { return (B + 15) / 16 * 16; }

// Workgroups a launch is sized for: one per CU of MI355X. Measured over every projection
// shape of the batched workloads (B = 8, 32, 64), one resident workgroup per CU streams
// better than two, and the split that minimises the rounds of items per workgroup times
// the chunks per item is the fastest or within a few percent of it.
constexpr int kMmTargetGroups = 256;

// K splits: the divisor s of the chunk count (s <= 16, and partial sums below an eighth of
// the weight bytes: s * 16NB * 4 B per row <= ncols * 2 B / 8) that minimises
// ceil(items / groups) * (chunks / s), items = tiles * s; ties go to fewer splits (less
// partial traffic).
int mm_split(int nrows, int ncols, int B, int tile_rows) {
  const long ntiles = (nrows + tile_rows - 1) / tile_rows;
  const int nch = mm_chunks(ncols);
  int cap = ncols / (16 * mm_batch_pad(B));
  if (cap > kMmMaxSplit) cap = kMmMaxSplit;
  if (cap > nch) cap = nch;
  int best = 1;
  long best_cost = -1;
  for (int s = 1; s <= cap; ++s) {
    if (nch % s != 0) continue;
    const long items = ntiles * s;
    const long groups = items < kMmTargetGroups ? items : kMmTargetGroups;
    const long cost = (items + groups - 1) / groups * (nch / s);
    if (best_cost < 0 || cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

// Rows per work item. A workgroup stages each chunk of the inputs (16NB rows, hi and lo
// planes: 1 KB per row) in LDS once for all its rows, so at 16NB = 64 the staging equals
// the 64 KB of weights a 128-row item reads per chunk. Items of 256 rows (eight waves, two
// packed blocks) halve that ratio: on packed weights at B = 64 they cut the projections
// and the lm_head by 11-17% when their items still cover most of the grid, while at
// B <= 32 they lose 1-30%, and with a quarter or an eighth of the grid in items (the
// small catch-up contractions) twice the rows per workgroup cost about twice the time.
// So: 256-row items for packed weights at 16NB >= 48 when their split gives at least
// three quarters of num_cu items. The sampling epilogue keeps 128 rows below four tiles (its
// random blocks would spill at eight waves); at four tiles it streams half-chunk stages,
// which leave them room (wide head, 64 sequences: 461-487 -> 347-349 us, the same bits).
MmPlan mm_plan(Epi epi, int nrows, int ncols, int B, bool packed, int num_cu) {
  const bool split = epi == EPI_STORE;
  MmPlan q{kMmTileRows, split ? mm_split(nrows, ncols, B, kMmTileRows) : 1, 0};
  if (packed && mm_batch_pad(B) / 16 >= (epi == EPI_SAMPLE ? 4 : 3)) {
    const int tr = 2 * kMmTileRows;
    const int s8 = split ? mm_split(nrows, ncols, B, tr) : 1;
    if (4L * ((nrows + tr - 1) / tr) * s8 >= 3L * num_cu) {
      q.tile_rows = tr;
      q.nsplit = s8;
    }
  }
  q.grid = mm_grid(nrows, q.tile_rows, q.nsplit, num_cu);
  return q;
}

// LDS: [2 buffers][2 planes][16 NB rows][ck + 8] bf16
static size_t mm_lds_bytes(int nb, int ck) { return (size_t)4 * 16 * nb * (ck + 8) * sizeof(uint16_t); }

// Persistent grid: one workgroup per CU, or one per item when there are fewer items.
int mm_grid(int nrows, int tile_rows, int nsplit, int num_cu) {
  const long items = (long)((nrows + tile_rows - 1) / tile_rows) * nsplit;
  long g = num_cu;
  if (g > items) g = items;
  return (int)(g < 1 ? 1 : g);
}

// OCC: waves per SIMD the register allocation must allow (the sampling epilogue at one or
// two tiles is held to two, which keeps it free of the extra registers its random blocks
// would otherwise take).
// PK: W is read from the packed copy (p.packed). Each instantiation has one straight load
// path: a branch per load (packed or not, live or not) made the compiler serialise loads.
// WV, MT: waves per workgroup and 16-row slices per wave (4 x 2: 128-row items; other
// shapes read packed blocks only, wave w taking slices w*MT .. w*MT+MT-1 of the item, each
// 16-row slice of a packed block being contiguous).
// CK: columns per stage, 256 or (packed only, so that 128 input rows fit the LDS twice)
// 128, each stage then reading one half of every packed block's columns.
template <int NB, int EPI, int OCC, bool PK, int WV, int MT, int CK>
__global__ __launch_bounds__(WV * kWave, OCC) void mm_kernel(MmParams p) {
  static_assert((WV == kMmWaves && MT == kMmMT) || (PK && WV * MT % 8 == 0),
                "other item shapes read whole packed blocks");
  static_assert(CK == kMmChunk || (PK && CK == kMmChunk / 2), "half chunks read packed blocks");
  constexpr int BP = 16 * NB;
  constexpr int NT = WV * kWave;
  constexpr int TR = 16 * MT * WV;   // rows per item
  constexpr int KS = CK / 32;        // MFMA k-steps per stage
  constexpr int LROW = CK + 8;       // bf16 per LDS row: 16-byte pad against bank conflicts
  constexpr int CPR = CK / 8;        // 16-byte column groups per input row and stage
  constexpr int HALVES = kMmChunk / CK;
  constexpr int XQ = BP * CPR;           // 16-byte input groups per plane and stage
  constexpr int XPASS = (XQ + NT - 1) / NT;  // per thread (the last pass may be partial)
  extern __shared__ __align__(16) uint16_t xl[];  // [2 buffers][2 planes][BP][LROW]
  __shared__ unsigned long long kred[WV][BP];
  __shared__ uint64_t seed_s[EPI == EPI_SAMPLE ? BP : 1];  // random-stream seeds, read once
  __shared__ int excl_s[EPI == EPI_ARGMAX ? BP : 1];        // row that never wins, or -1
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.nrows, Kd = p.ncols;
  const int C = mm_chunks(Kd) * HALVES / p.nsplit;  // stages per item
  const int ntiles = (N + TR - 1) / TR;
  const int nblk_rows = (N + kMmTileRows - 1) / kMmTileRows;  // packed block rows
  const int nitems = ntiles * p.nsplit;
  const int G = gridDim.x;
  const int my_items = (int)blockIdx.x < nitems ? (nitems - 1 - (int)blockIdx.x) / G + 1 : 0;
  const int stages = my_items * C;

  auto clampit = [&](int it) { return it < stages ? it : (stages > 0 ? stages - 1 : 0); };
  auto item_of = [&](int it) { return (int)blockIdx.x + (it / C) * G; };
  auto chunk_of = [&](int it) { return (item_of(it) % p.nsplit) * C + it % C; };
  // first row of slice m of this wave in the tile of stage it
  auto slice_row = [&](int it, int m) {
    return (item_of(it) / p.nsplit) * TR + (wave * MT + m) * 16;
  };


  // Streaming (non-temporal) weight loads keep the input operand's lines in L2. Measured on
  // packed weights: the lm_head 4-10% faster at B = 8..64 and the B = 8 projections 2-9%;
  // the K-split projections at B = 32..64 1-7% slower, so they load normally.
  constexpr bool kStream = EPI != EPI_STORE || NB == 1;
  u32x4 A[MT][KS], Bf[MT][KS];
  // The packed path's weight pointer of stage it for this lane: contiguous 1 KB per wave
  // instruction, one base per wave; the second block of a 256-row item past the last block
  // row reads the dummy.
  auto wbase = [&](int it) -> const uint16_t* {
    const bool live = it < stages;
    const int sl0 = wave * MT;  // the wave's first 16-row slice in the item (8 per block)
    const int brow = (item_of(it) / p.nsplit) * (TR / kMmTileRows) + sl0 / 8;
    const bool lw = live && brow < nblk_rows;
    const long blk = (long)brow * mm_chunks(Kd) + chunk_of(it) / HALVES;
    return (lw ? p.packed + blk * kMmPackBlock : static_cast<const uint16_t*>(p.dummy)) +
           (long)(sl0 % 8) * (kMmKSteps * kWave * 8) + (chunk_of(it) % HALVES) * (KS * kWave * 8) +
           lane * 8;
  };
  // Stages past the workgroup's last one are prefetched from the dummy region and never
  // consumed (packed: the same offsets in a 64 KB dummy block; else 16 rows of 256 bf16).
  auto wload = [&](u32x4 (&buf)[MT][KS], int it) {
    const bool live = it < stages;
    if constexpr (PK) {
      const uint16_t* bp = wbase(it);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const u32x4* a = reinterpret_cast<const u32x4*>(bp + (m * kMmKSteps + k) * kWave * 8);
          buf[m][k] = kStream ? __builtin_nontemporal_load(a) : *a;
        }
      return;
    }
    // Row pointers and column clamps as selects (no branch per load): columns past the row
    // end (a ragged last chunk) re-read the row's last 8 elements.
    const int c0 = live ? chunk_of(it) * kMmChunk + (lane >> 4) * 8 : (lane >> 4) * 8;
    const int cmax = live ? Kd - 8 : kMmChunk - 8;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = min(slice_row(it, m) + (lane & 15), N - 1);
      const uint16_t* rp = r < p.seg1 ? static_cast<const uint16_t*>(p.w0) + (long)r * Kd
                         : r < p.seg2 ? static_cast<const uint16_t*>(p.w1) + (long)(r - p.seg1) * Kd
                                      : static_cast<const uint16_t*>(p.w2) + (long)(r - p.seg2) * Kd;
      rp = live ? rp : static_cast<const uint16_t*>(p.dummy) + (lane & 15) * kMmChunk;
#pragma unroll
      for (int k = 0; k < KS; ++k)
        buf[m][k] = *reinterpret_cast<const u32x4*>(rp + min(c0 + k * 32, cmax));
    }
  };

  u32x4 xr[2][XPASS];
  auto xload = [&](int it) {
    const int c0 = chunk_of(clampit(it)) * CK;
#pragma unroll
    for (int j = 0; j < XPASS; ++j) {
      const int q = tid + j * NT;
      const int row = q / CPR, col = c0 + (q % CPR) * 8;
      const int rr = row < p.B ? row : p.B - 1;
      const int cc = col < Kd ? col : Kd - 8;
      const long o = (long)rr * p.ldx + cc;
      xr[0][j] = *reinterpret_cast<const u32x4*>(p.x + o);
      xr[1][j] = *reinterpret_cast<const u32x4*>(p.x_lo + o);
    }
  };
  auto xstore = [&](int it, int bufi) {
    const int c0 = chunk_of(clampit(it)) * CK;
#pragma unroll
    for (int j = 0; j < XPASS; ++j) {
      const int q = tid + j * NT;
      if (XQ % NT != 0 && q >= XQ) continue;  // past the stage's groups (its load was clamped)
      const int row = q / CPR, cp = q % CPR;
      const bool live = row < p.B && c0 + cp * 8 < Kd;
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
        *reinterpret_cast<u32x4*>(xl + ((long)(2 * bufi + pl) * BP + row) * LROW + cp * 8) =
            live ? xr[pl][j] : z;
    }
  };

  f32x4 acc[MT][NB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned long long best[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) best[nb] = 0ull;

  // Each input fragment read from LDS serves both 16-row slices of the wave. With kSteady
  // (the greedy lm_head on packed weights, up to four tiles) each k-step's registers are
  // refilled from nxt, the stage two ahead, as soon as the k-step's last product is issued:
  // a steady stream of weight loads instead of one burst per stage. Timed against the burst
  // (alternating runs, caches flushed): the greedy lm_head 3% faster at 32 sequences and 2%
  // at 64, the same bits; no better for the projections, the sampling epilogue or eight
  // tiles, which keep the burst.
  constexpr bool kSteady = PK && EPI == EPI_ARGMAX && NB <= kMmMaxNB;
  auto consume = [&](u32x4 (&buf)[MT][KS], int it, const uint16_t* nxt) {
    const uint16_t* xb = xl + (long)(it & 1) * 2 * BP * LROW + (lane & 15) * LROW +
                         (lane >> 4) * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 bh = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(xb + nb * 16 * LROW + k * 32));
        const bf16x8 bl = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(xb + (BP + nb * 16) * LROW + k * 32));
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const bf16x8 w = __builtin_bit_cast(bf16x8, buf[m][k]);
          acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, bh, acc[m][nb], 0, 0, 0);
          acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, bl, acc[m][nb], 0, 0, 0);
        }
      }
      if constexpr (kSteady) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4* a = reinterpret_cast<const u32x4*>(nxt + (m * kMmKSteps + k) * kWave * 8);
          buf[m][k] = kStream ? __builtin_nontemporal_load(a) : *a;
        }
      }
    }
  };

  const bool vec_logits =
      p.logits && (p.logits_ld & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0;
  // Lane l holds rows 4*(l/16)+i (i < 4) of slice m for sequence 16*nb + l%16.
  auto finish_item = [&](int it) {
    const int split = item_of(it) % p.nsplit;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r0 = slice_row(it, m) + (lane >> 4) * 4;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int b = nb * 16 + (lane & 15);
        if constexpr (EPI == EPI_STORE) {
          float* dst = p.part + ((long)split * BP + b) * N + r0;
          if (r0 + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<float4*>(dst) =
                float4{acc[m][nb][0], acc[m][nb][1], acc[m][nb][2], acc[m][nb][3]};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (r0 + i < N) dst[i] = acc[m][nb][i];
          }
        } else {
          // EPI_SAMPLE: the lane's four rows r0..r0+3 (r0 % 4 == 0) take the four words
          // of one random block as their Gumbel noise.
          float noise[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (EPI == EPI_SAMPLE) {
            const Philox4 rb = rng_block(seed_s[b], p.smp.offset, RNG_DRAFT, (uint64_t)p.smp.row,
                                         (uint64_t)(r0 >> 2));
#pragma unroll
            for (int i = 0; i < 4; ++i) noise[i] = gumbel_of(rb.w[i]);
            // one random block at a time: interleaving them would exceed the register budget
            __builtin_amdgcn_sched_barrier(0);
          }
          unsigned long long k = 0ull;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (r0 + i < N) {
              float val = acc[m][nb][i];
              if constexpr (EPI == EPI_SAMPLE) val = val * p.smp.inv_temp + noise[i];
              unsigned long long ki = pack_key(val, (uint32_t)(r0 + i));
              if constexpr (EPI == EPI_ARGMAX) ki = r0 + i == excl_s[b] ? 0ull : ki;
              k = ki > k ? ki : k;
            }
          }
          // The lane's four rows in one 16-byte streaming store when aligned: measured at
          // B = 32..64, writing the step's logits this way instead of with 4-byte cached stores
          // takes 5-10% off the sampling lm_head.
          if (p.logits && b < p.B) {
            float* lp = p.logits + (long)b * p.logits_ld + r0;
            if (vec_logits && r0 + 3 < N) {
              __builtin_nontemporal_store(acc[m][nb], reinterpret_cast<f32x4*>(lp));
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (r0 + i < N) lp[i] = acc[m][nb][i];
            }
          }
          unsigned long long o = __shfl_xor(k, 16, kWave);
          k = o > k ? o : k;
          o = __shfl_xor(k, 32, kWave);
          k = o > k ? o : k;
          best[nb] = k > best[nb] ? k : best[nb];
        }
        acc[m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  auto stage = [&](u32x4 (&buf)[MT][KS], int it) {
    xload(it + 1);
    if constexpr (kSteady) {
      consume(buf, it, wbase(it + 2));
    } else {
      consume(buf, it, nullptr);
      wload(buf, it + 2);
    }
    if (it % C == C - 1) finish_item(it);
    xstore(it + 1, (it + 1) & 1);
    __syncthreads();
  };

  if constexpr (EPI == EPI_SAMPLE) {
    if (tid < BP) seed_s[tid] = tid < p.B ? p.smp.seeds[tid] : 0ull;  // visible after the first barrier
  }
  if constexpr (EPI == EPI_ARGMAX) {
    if (tid < BP) excl_s[tid] = (p.excl && tid < p.B) ? p.excl[(long)tid * p.excl_stride] : -1;
  }
  xload(0);
  wload(A, 0);
  wload(Bf, 1);
  xstore(0, 0);
  __syncthreads();
  for (int it = 0; it < stages; it += 2) {
    stage(A, it);
    if (it + 1 >= stages) break;
    stage(Bf, it + 1);
  }

  if constexpr (epi_is_argmax(EPI)) {
    if (lane < 16) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) kred[wave][nb * 16 + lane] = best[nb];
    }
    __syncthreads();
    if (tid < BP && tid < p.B) {
      unsigned long long k = 0ull;
#pragma unroll
      for (int w = 0; w < WV; ++w) k = kred[w][tid] > k ? kred[w][tid] : k;
      if (k) publish_max_key(p.keys + tid, k);
    }
    // the winner reads back only keys published by publish_max_key
    if (last_to_arrive(p.counter, gridDim.x, &flag)) {
      for (int b = tid; b < p.B; b += NT) {
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

size_t mm_packed_elems(int nrows, int ncols) {
  return (size_t)((nrows + kMmTileRows - 1) / kMmTileRows) * mm_chunks(ncols) * kMmPackBlock;
}

// One thread per 16-byte vector of the packed copy: vector v of block (tile, chunk) is the
// load of lane v % 64, k-step (v / 64) % 8, slice v / 512 (wave * 2 + slice).
__global__ void pack_kernel(const uint16_t* w0, const uint16_t* w1, const uint16_t* w2, int seg1,
                            int seg2, int nrows, int ncols, uint16_t* dst, long nvec) {
  const int nch = mm_chunks(ncols);
  for (long v = blockIdx.x * (long)blockDim.x + threadIdx.x; v < nvec;
       v += (long)gridDim.x * blockDim.x) {
    const long blk = v / (kMmPackBlock / 8);
    const int q = (int)(v % (kMmPackBlock / 8));
    const int lane = q % kWave, k = (q / kWave) % kMmKSteps, sm = q / (kWave * kMmKSteps);
    const long row = (blk / nch) * kMmTileRows + sm * 16 + (lane & 15);
    const int col = (int)(blk % nch) * kMmChunk + k * 32 + (lane >> 4) * 8;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row < nrows && col < ncols) {
      const uint16_t* src = row < seg1   ? w0 + row * ncols
                            : row < seg2 ? w1 + (row - seg1) * ncols
                                         : w2 + (row - seg2) * ncols;
      val = *reinterpret_cast<const u32x4*>(src + col);
    }
    *reinterpret_cast<u32x4*>(dst + v * 8) = val;
  }
}

hipError_t launch_pack(const void* w0, const void* w1, const void* w2, int seg1, int seg2,
                       int nrows, int ncols, uint16_t* dst, hipStream_t s) {
  if (!w0 || !w1 || !w2 || !dst || nrows < 1 || ncols < 8 || ncols % 8 != 0 || seg1 > seg2)
    return hipErrorInvalidValue;
  const long nvec = (long)(mm_packed_elems(nrows, ncols) / 8);
  long blocks = (nvec + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w0), static_cast<const uint16_t*>(w1),
                     static_cast<const uint16_t*>(w2), seg1, seg2, nrows, ncols, dst, nvec);
  return hipGetLastError();
}

// The lm_head over three or four 16-sequence tiles in 256-row items (greedy, or sampling at
// four) streams half-chunk stages (128 columns): the wave's two weight stages then take 64
// registers instead of 128, which leaves the compiler room to overlap the products with the
// input reads (timed against full-chunk stages on the wide head's 129280 x 7168 lm_head at
// 64 sequences: 10% faster, the same bits) and the sampling epilogue room for its random
// blocks. The projections keep full chunks (within ±8% either way, no clear gain).
template <int NB, bool PK, int WV, int MT>
static hipError_t mm_nbp(Epi epi, const MmParams& p, int grid, hipStream_t s) {
  constexpr int CK = kMmChunk;
  constexpr int CKA = (PK && NB >= 3 && WV == 2 * kMmWaves) ? kMmChunk / 2 : kMmChunk;
  const size_t lds = mm_lds_bytes(NB, CK);
  const dim3 block(WV * kWave);
  if (epi == EPI_ARGMAX)
    hipLaunchKernelGGL((mm_kernel<NB, EPI_ARGMAX, 1, PK, WV, MT, CKA>), dim3(grid), block,
                       mm_lds_bytes(NB, CKA), s, p);
  else if (epi == EPI_STORE)
    hipLaunchKernelGGL((mm_kernel<NB, EPI_STORE, 1, PK, WV, MT, CK>), dim3(grid), block, lds, s, p);
  else if constexpr (WV == kMmWaves && MT == kMmMT)
    hipLaunchKernelGGL((mm_kernel<NB, EPI_SAMPLE, NB <= 2 ? 2 : 1, PK, WV, MT, CK>), dim3(grid),
                       block, lds, s, p);
  else if constexpr (CKA != CK)
    hipLaunchKernelGGL((mm_kernel<NB, EPI_SAMPLE, 1, PK, WV, MT, CKA>), dim3(grid), block,
                       mm_lds_bytes(NB, CKA), s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
template <int NB>
static hipError_t mm_nb(Epi epi, const MmParams& p, int grid, hipStream_t s) {
  if (!p.packed) return mm_nbp<NB, false, kMmWaves, kMmMT>(epi, p, grid, s);
  if constexpr (NB >= 3) {
    if (p.tile_rows == 2 * kMmTileRows) return mm_nbp<NB, true, 2 * kMmWaves, kMmMT>(epi, p, grid, s);
  }
  return mm_nbp<NB, true, kMmWaves, kMmMT>(epi, p, grid, s);
}

// 65..128 sequences (the greedy lm_head of verification from hidden states): eight
// 16-sequence tiles, so that one pass over the lm_head serves them all. Two input planes of
// 128 rows fit the LDS twice only at 128 columns per stage (136 KB), so each packed block
// is read in two stages. With 256-row items (eight waves, two per SIMD, so that one wave's
// MFMAs overlap another's LDS reads) the 128-row lm_head pass at q8b shapes takes 438 µs,
// against 518 µs with four waves and 2 x 266 µs for two 64-row passes.
static hipError_t mm_argmax_nb8(const MmParams& p, int grid, hipStream_t s) {
  constexpr int CK = kMmChunk / 2;
  if (p.tile_rows == 2 * kMmTileRows)
    hipLaunchKernelGGL((mm_kernel<kMmMaxNBArgmax, EPI_ARGMAX, 1, true, 2 * kMmWaves, kMmMT, CK>),
                       dim3(grid), dim3(2 * kMmWaves * kWave), mm_lds_bytes(kMmMaxNBArgmax, CK),
                       s, p);
  else
    hipLaunchKernelGGL((mm_kernel<kMmMaxNBArgmax, EPI_ARGMAX, 1, true, kMmWaves, kMmMT, CK>),
                       dim3(grid), dim3(kMmWaves * kWave), mm_lds_bytes(kMmMaxNBArgmax, CK), s,
                       p);
  return hipGetLastError();
}

hipError_t launch_mm(Epi epi, const MmParams& p, int grid, hipStream_t s) {
  if (epi != EPI_STORE && !epi_is_argmax(epi)) return hipErrorInvalidValue;
  if (epi == EPI_SAMPLE && (!(p.smp.inv_temp > 0.f) || !p.smp.seeds)) return hipErrorInvalidValue;
  const int max_b = (epi == EPI_ARGMAX && p.packed ? kMmMaxNBArgmax : kMmMaxNB) * 16;
  if (p.B < 1 || p.B > max_b || p.nrows < 1 || p.ncols < 8 || p.ncols % 8 != 0 ||
      p.ldx < p.ncols || p.ldx % 8 != 0 || !p.x || !p.x_lo || p.nsplit < 1 ||
      mm_chunks(p.ncols) % p.nsplit != 0 || grid < 1)
    return hipErrorInvalidValue;
  if (epi_is_argmax(epi) && (p.nsplit != 1 || !p.keys || !p.counter || !p.tok_out))
    return hipErrorInvalidValue;
  if (epi == EPI_STORE && !p.part) return hipErrorInvalidValue;
  if (p.tile_rows != 0 && p.tile_rows != kMmTileRows &&
      !(p.tile_rows == 2 * kMmTileRows && p.packed && p.B > (epi == EPI_SAMPLE ? 48 : 32) &&
        (p.B <= 16 * kMmMaxNB || epi == EPI_ARGMAX)))
    return hipErrorInvalidValue;
  static_assert(16 * kMmChunk * 2 <= kDummyBytes && kMmPackBlock * 2 <= kDummyBytes,
                "dummy region too small");
  if (!p.dummy) return hipErrorInvalidValue;
  switch (mm_batch_pad(p.B) / 16) {
    case 1: return mm_nb<1>(epi, p, grid, s);
    case 2: return mm_nb<2>(epi, p, grid, s);
    case 3: return mm_nb<3>(epi, p, grid, s);
    case 4: return mm_nb<4>(epi, p, grid, s);
    default: return mm_argmax_nb8(p, grid, s);
  }
}

}  // namespace mtp
