// Launch interfaces of the gfx950 kernels (internal to libmtp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

// Prologue: how a workgroup builds the fp32 input vector(s) it multiplies.
enum Pro : int {
  PRO_PLAIN = 0,  // x as given
  PRO_RMS = 1,    // RMSNorm(x) * gain
  PRO_EH = 2,     // [RMSNorm(h) * g_h ; RMSNorm(embed[tok]) * g_e]   (length 2H)
};
// Epilogue: what happens to each dot product y of logical row r, batch row b.
enum Epi : int {
  EPI_STORE = 0,   // out[b, r] = y
  EPI_RESID = 1,   // out[b, r] = res[b, r] + y
  EPI_SWIGLU = 2,  // rows come in (gate, up) pairs: out[b, r] = silu(y_gate) * y_up
  EPI_ARGMAX = 3,  // argmax over r per b, finished by the last workgroup
  EPI_SAMPLE = 4,  // as EPI_ARGMAX over y / temp + Gumbel noise: a sample of softmax(y / temp)
};
constexpr bool epi_is_argmax(int e) { return e == EPI_ARGMAX || e == EPI_SAMPLE; }

// EPI_SAMPLE: the key of vocabulary row r is y * inv_temp + G; the Gumbel noise G of
// batch row b comes from the stream
// (seed seeds[b], offset, purpose draft, row `row`).
struct SampleParams {
  float inv_temp;          // 1 / temperature (> 0)
  const uint64_t* seeds;   // [B] device
  uint64_t offset;
  int row;                 // draft step (0-based)
};

struct GemvParams {
  // Logical rows r in [0, nrows). Segments: r < seg1 -> w0, r < seg2 -> w1, else w2
  // (local row index r - segment start). For EPI_SWIGLU, pair r reads w0[r] and w1[r].
  const void* w0;
  const void* w1;
  const void* w2;
  int seg1, seg2;
  int nrows;
  int ncols;
  int B;
  int col_block;  // columns staged in LDS at a time (multiple of 64 * elements per 16 B)
  // Input
  const float* x;  // [B, ldx] fp32 (PRO_PLAIN, PRO_RMS)
  int ldx;
  const void* gain;   // RMS gain (PRO_RMS) or g_h (PRO_EH), weight dtype
  const void* gain2;  // g_e (PRO_EH)
  float eps;
  const void* h;  // PRO_EH hidden state: fp32 [B, H] if h_is_f32 else weight dtype
  int h_is_f32;
  int ldh;
  const void* embed;   // PRO_EH embedding table [vocab, H]
  const int* tok;      // PRO_EH token of batch row b at tok[b * tok_stride]
  int tok_stride;
  int vocab;
  unsigned* err;
  // Output
  float* out;
  int ldo;
  const float* res;
  float* dbg;  // optional second copy of out (EPI_RESID), [B, dbg_ld]
  int dbg_ld;
  // EPI_ARGMAX
  unsigned long long* keys;  // [B], zero on entry, left zero on exit
  unsigned* counter;         // zero on entry, left zero on exit
  int* tok_out;              // token of b written to tok_out[b * tok_out_stride]
  int tok_out_stride;
  float* maxlogit;  // value of b's winning key at maxlogit[b * maxlogit_stride], or null
  int maxlogit_stride;  // 0 means 1
  // Optional: row excl[b * excl_stride] never wins for batch row b (the second-best pass
  // of the debug draft: the best value with the winner left out).
  const int* excl;
  int excl_stride;
  float* logits;    // [B, logits_ld] or null
  int logits_ld;
  int* len;  // when advance > 0 the last workgroup adds it to len[b] and pos[b]
  int* pos;
  int advance;
  const int* kseq;  // per-sequence step counts of the call (advance by kseq[b]), or null
  // >= kDummyBytes of readable device memory: the target of the weight-streaming
  // kernels' prefetches past a wave's last stage, which are issued but never consumed
  const void* dummy;
  SampleParams smp;  // EPI_SAMPLE
};
constexpr int kDummyBytes = 64 * 1024;

// Column-blocked GEMV for any batch (batch rows in blockIdx.y tiles of up to 8).
hipError_t launch_gemv(int wdtype, Pro pro, Epi epi, const GemvParams& p, int max_grid,
                       hipStream_t s);
// Persistent pipelined GEMV for batch 1-2 when the input vectors fit in LDS.
bool gemv_pipe_fits(int ncols, int B, int wdtype);
int gemv_pipe_grid(int nrows, int ncols, int wdtype, int num_cu);
hipError_t launch_gemv_pipe(int wdtype, Pro pro, Epi epi, const GemvParams& p, int grid,
                            hipStream_t s);

// Per-call set-up: RoPE tables of K consecutive steps (tab[k][b][0..d/2) = cos,
// tab[k][b][d/2..d) = sin of (pos[b] + k) * theta^(-2i/d), evaluated in fp64 and rounded
// to fp32) and hidden [B, H] (weight dtype) widened to fp32 into hf.
// With kseq (per-sequence step counts) it also sets `err_bit` for a count outside [0, K].
// With chunk_out it writes the call's attention chunk. T_b = min(len[b] + K, capacity) is
// what sequence b attends at the call's last step. Without `balance` the longest T_b is
// spread over nsplit splits, rounded up to a multiple of q, at most max_chunk. With
// `balance` (bf16 cache, many items) the longest T_b is cut into n equal splits,
// 1 <= n <= nsplit, with n = round(max T / S) and S = (sum_b T_b * n_kv / num_cu) *
// (mean T / max T)^2, rounded up to a multiple of q (max_chunk does not apply): one item
// per CU when the lengths are equal, smaller items for the longest-first order to balance
// when they are not.
struct ChunkPlan {
  const int* len;
  int capacity, nsplit, q, max_chunk;
  int* chunk_out;
  int balance = 0;  // the rule for many items (bf16 cache only)
  int n_kv = 0, num_cu = 0;
};
hipError_t launch_draft_setup(int dtype, float* tab, const int* pos, int B, int K, int d,
                              float theta, const void* hidden, float* hf, int H, const int* kseq,
                              unsigned err_bit, unsigned* err, const ChunkPlan& cp,
                              hipStream_t s);

struct AttnParams {
  const float* qkv;  // [B, ldqkv] fp32: q (n_q*d) | k (n_kv*d) | v (n_kv*d), before RoPE
  int ldqkv;
  void* kc;  // [Bc, n_kv, capacity, d] cache dtype
  void* vc;
  int n_q, n_kv, d;
  int capacity;
  const int* len;  // start-of-call values
  const int* pos;
  int step;   // 0-based step index: slot len+step, position pos+step
  int batch;  // sequences (set by launch_attention)
  int chunk;  // positions per workgroup (multiple of attn_chunk_quantum())
  int nsplit;
  // When set, the call's chunk as the set-up kernel computed it from the lengths on the
  // device (used instead of `chunk`; never larger for the fp32 cache, whose kernel sizes
  // its LDS from `chunk`; at most chunk * nsplit covers what a sequence attends either way).
  const int* chunk_dev;
  const float* rope;  // [B, d]: cos then sin of the step's position
  float scale;
  float* part_o;   // [B, n_q, nsplit, d]
  float* part_ml;  // [B, n_q, nsplit, 2]
  float* o;  // [B, n_q * d]
  uint16_t* o_bf16;  // when set, the merge writes o as bf16 planes hi / lo (o_bf16, o_bf16_lo,
  uint16_t* o_bf16_lo;  // [b * ld_o_bf16 + ...]) instead of fp32
  int ld_o_bf16;
  unsigned* err;
  const int* perm;  // launch order of the items (attn_plan_kernel), or null: natural order
  // Per-sequence step counts, or null. A sequence past its count at this step is masked:
  // it attends only to the step's own key (no cache read, no cache write, no capacity
  // check), so its output is finite and is discarded by the caller.
  const int* kseq;
};
// Attention (partials per split) followed by the split merge into o. p.chunk must be a
// positive multiple of attn_chunk_quantum() and at most attn_max_chunk(cdtype).
int attn_chunk_quantum();
int attn_max_chunk(int cdtype);
// Longest-first item order for one draft call, written to perm[nsplit * n_kv * B]; wanted
// when the items outnumber what the chip runs at once.
bool attn_plan_wanted(int B, int nkv, int nsplit, int num_cu);
hipError_t launch_attn_plan(const int* len, int B, int nkv, int chunk, const int* chunk_dev,
                            int nsplit, int* perm, hipStream_t s);
hipError_t launch_attention(int cdtype, const AttnParams& p, int B, hipStream_t s);

// ---- verification from hidden states, up to 16 rows, row-major bf16 lm_head (lm_rows.hip)

// One launch: final RMSNorm of the R rows, the argmax of every row over the lm_head and,
// when `accepted` is set (R = B (K + 1)), the accepted-prefix scan of each sequence.
struct LmRowsParams {
  const uint16_t* h;     // [R][H] bf16 target hidden rows, before the final norm
  const uint16_t* gain;  // [H] bf16 final-norm gain
  float eps;
  const uint16_t* W;     // [V][H] bf16 lm_head, row-major
  int V, H, R;
  unsigned long long* keys;  // [>= R], zero on entry, left zero
  unsigned* counter;         // zero on entry, left zero
  int* tok_out;              // [R] argmax of each row
  const int* draft;          // [B][K] draft tokens (K > 0)
  int B, K;
  int* accepted;             // [B] accepted prefix lengths, or null (no scan)
  int* next;                 // [B] the target's token after the accepted prefix
};
// Shapes the kernel takes: 1 <= R <= 16, H a multiple of 8 and at most 4096.
bool lm_rows_fits(int H, int R);
// Once per process and device before the first launch (raises the kernel's LDS limit).
hipError_t lm_rows_prepare();
hipError_t launch_lm_rows(const LmRowsParams& p, int grid, hipStream_t s);

// ---- many input rows (prompt prefill): tiled MFMA contraction (gemm_rows.hip)

// part[s][b][r] = sum over the columns of K split s of W[r, c] * (x[b, c] + x_lo[b, c]), for
// W rows r < nrows (bf16, row-major, leading dimension ncols; rows [0, seg1) from w0, the
// rest from w1) and input rows b < B (bf16 hi / lo planes, leading dimension ldx). Same
// splits, layout and bits as the weight-streaming contraction's EPI_STORE.
struct GmParams {
  const void* w0;
  const void* w1;
  int seg1;
  int nrows, ncols;
  const uint16_t* x;
  const uint16_t* x_lo;
  int ldx, B;
  int nsplit;
  float* part;  // [nsplit][bp][nrows] (EPI_STORE)
  int bp;       // >= B
  // EPI_ARGMAX (nsplit == 1): argmax over the W rows of each input row, keys [B] and the
  // counter zero on entry and left zero, tok_out [B]
  unsigned long long* keys;
  unsigned* counter;
  int* tok_out;
};
// Splits that give at least one workgroup per CU (a divisor of the 256-column chunk count),
// with split x B x nrows <= max_part (the room of the partial sums, in floats) unless that
// leaves 1.
int gm_split(int nrows, int ncols, int B, int num_cu, long max_part);
// Once per process and device before the first launch (raises the kernel's LDS limit).
hipError_t gm_prepare();
hipError_t launch_gm(Epi epi, const GmParams& p, hipStream_t s);

// ---- batched path (bf16 weights, 3..64 sequences): MFMA contraction + row reductions

// y[b, r] = sum_c W[r, c] * x[b, c] for r < nrows, with W bf16 rows (segments as in
// GemvParams) and x a bf16 operand [16*NB, ldx]. Work items are (128- or 256-row item,
// K split); EPI_STORE writes fp32 partial sums per split, EPI_ARGMAX (nsplit == 1)
// finishes an argmax over r per batch row as the GEMV does.
struct MmParams {
  const void* w0;
  const void* w1;
  const void* w2;
  int seg1, seg2;
  int nrows, ncols;
  // The fp32 input rows as two bf16 planes, x = hi + lo (lo = the rounding residue of hi),
  // each [>= B rows, ldx]; the contraction runs on both, so the input keeps ~16 bits.
  const uint16_t* x;
  const uint16_t* x_lo;
  int ldx;
  int B;
  int nsplit;   // divides mm_chunks(ncols)
  // Rows per work item: 0 or 128 (four waves); 256 (eight waves) needs packed weights,
  // 33..64 sequences and the store or greedy epilogue.
  int tile_rows;
  float* part;  // EPI_STORE: [nsplit][16*NB][nrows]
  unsigned long long* keys;  // EPI_ARGMAX, as GemvParams
  unsigned* counter;
  int* tok_out;
  int tok_out_stride;
  float* maxlogit;
  int maxlogit_stride;  // as GemvParams
  const int* excl;
  int excl_stride;
  float* logits;
  int logits_ld;
  int* len;
  int* pos;
  int advance;
  const int* kseq;  // as GemvParams::kseq
  const void* dummy;  // as GemvParams::dummy
  SampleParams smp;   // EPI_SAMPLE
  // When set, W is read from this packed copy (see launch_pack) and w0/w1/w2/seg1/seg2
  // are not used.
  const uint16_t* packed;
};
__host__ __device__ int mm_chunks(int ncols);  // K chunks of the contraction
int mm_batch_pad(int B);                           // 16 * NB for batch B
int mm_split(int nrows, int ncols, int B, int tile_rows);  // K splits used for these sizes
// Packed copy of the logical matrix w0 | w1 | w2 (segments as in MmParams, [nrows, ncols]
// bf16) for mm_kernel: blocks of 128 rows x 256 columns, block (tile, chunk) at element
// (tile * chunks + chunk) * 32768, each block in the order the kernel's lanes load it, so
// that every wave load instruction reads 1 KB of contiguous memory; rows and columns past
// the matrix are zero.
size_t mm_packed_elems(int nrows, int ncols);
hipError_t launch_pack(const void* w0, const void* w1, const void* w2, int seg1, int seg2,
                       int nrows, int ncols, uint16_t* dst, hipStream_t s);
int mm_grid(int nrows, int tile_rows, int nsplit, int num_cu);
// Item rows, K splits (1 outside EPI_STORE) and grid of one contraction.
struct MmPlan {
  int tile_rows, nsplit, grid;
};
MmPlan mm_plan(Epi epi, int nrows, int ncols, int B, bool packed, int num_cu);
hipError_t launch_mm(Epi epi, const MmParams& p, int grid, hipStream_t s);

// Row-wise steps between contractions, one workgroup per sequence b:
//   RED_EH:   x = sum(part) -> out (fp32); xq = split(RMSNorm(x) * gain)
//   RED_QKV:  out = sum(part)
//   RED_RESID: y = res + sum(part) -> out (and dbg); xq = split(RMSNorm(y) * gain)
//   RED_SWIGLU: xq = split(silu(sum(part[gate rows])) * sum(part[up rows]))  (n = nrows/2)
//   PREP_EH:  xq = [split(RMSNorm(h) * g_h), split(RMSNorm(embed[tok]) * g_e)]
// where split(v) writes the bf16 planes hi = bf16(v), lo = bf16(v - hi).
//   PREP_NORM: xq = split(RMSNorm(h) * gain), h read from h16 (bf16) or h (fp32)
enum RedMode : int { RED_EH = 0, RED_QKV = 1, RED_RESID = 2, RED_SWIGLU = 3, PREP_EH = 4,
                     PREP_NORM = 5 };
struct RedParams {
  const float* part;  // [nsplit][bp][n_part]
  int nsplit, bp, n_part;
  int n;              // outputs per row
  const float* res;   // [B, n] (RED_RESID)
  float* out;         // [B, n] fp32 (RED_EH, RED_QKV, RED_RESID)
  float* dbg;         // optional copy of out (RED_RESID), [B, dbg_ld]
  int dbg_ld;
  const uint16_t* gain;   // bf16 [n]
  const uint16_t* gain2;  // PREP_EH: g_e
  float eps;
  uint16_t* xq;       // bf16 planes [B, ldq]: hi = bf16(v) in xq, lo = bf16(v - hi) in xq_lo
  uint16_t* xq_lo;
  int ldq;
  const float* h;     // PREP_EH / PREP_NORM hidden [B, n] fp32
  const uint16_t* h16;  // PREP_NORM hidden [B, n] bf16 (used instead of h when set)
  const uint16_t* embed;
  const int* tok;
  int tok_stride;
  int vocab;
  unsigned* err;
};
int red_max_cols();  // largest n the norm modes accept
hipError_t launch_red(RedMode mode, const RedParams& p, int B, hipStream_t s);

// Per-sequence completion counters and keys of the verification kernels start on their
// own 256-byte line, so that the atomics of different sequences do not queue on one line.
constexpr int kSeqLineU32 = 64;  // counter of sequence b at counters[b * kSeqLineU32]
constexpr int kSeqLineU64 = 32;  // key stride unit (u64)

struct VerifyParams {
  const float* logits;  // [B, K+1, V]
  const int* draft;     // [B, K]
  int K, V;
  int seg;                   // set by launch_verify: load units per workgroup
  unsigned long long* keys;  // row j of sequence b at keys[b * kstride + j], zero on entry/exit
  int kstride;               // >= K + 1, a multiple of kSeqLineU64
  unsigned* counters;        // [B * kSeqLineU32] zero on entry/exit
  int* accepted;
  int* next;
  const int* kseq;  // per-sequence draft counts (rows past kseq[b] are not read), or null
};
hipError_t launch_verify(const VerifyParams& p, int B, hipStream_t s);

// Speculative-sampling verification at temperature temp (two launches, see verify.hip).
struct VSampleParams {
  const float* tlog;  // [B, K+1, V] target logits
  const float* dlog;  // [B, K, V] draft logits (row j produced draft j)
  const int* draft;   // [B, K]
  int K, V, nchunk;   // nchunk = vs_chunks(V): partial slots per row (the most any launch uses)
  int seg;            // set by launch_verify_sample
  float inv_temp;     // 1 / temperature
  const uint64_t* seeds;     // [B]
  uint64_t offset;
  unsigned long long* part;  // [B, 2K+1, nchunk] (max, sum) pairs, left zero
  float* lse;                // [B, 2] log-sum-exps of the target / draft row a
  unsigned long long* keys;  // [B * kSeqLineU64], two used per sequence, zero on entry/exit
  unsigned* counters;        // [B * kSeqLineU32] zero on entry/exit
  int* accepted;
  int* next;
  unsigned* err;
};
constexpr int kVsMaxK = 100;
int vs_chunks(int V);
hipError_t launch_verify_sample(const VSampleParams& p, int B, hipStream_t s);

// kseq: per-sequence draft counts of the call being rolled back (K for all when null).
hipError_t launch_rollback(int* len, int* pos, const int* accepted, const int* kseq, int B, int K,
                           unsigned* err, hipStream_t s);

// dst[i] = src[i] widened to fp32 (src in weight dtype), i < n.
hipError_t launch_widen(int dtype, const void* src, float* dst, long n, hipStream_t s);
// dst[i, :] = fp32(src[(r / per) * src_per + r % per, :]) for r = r0 + i, i < rows: row
// r % per of sequence r / per, where src holds src_per rows per sequence ([B, src_per, H],
// weight dtype). Catch-up reads the verified-input rows j - 1 = r % K (per = K,
// src_per = K + 1); prefill reads every prompt row (per = src_per = n).
hipError_t launch_gather_rows(int dtype, const void* src, float* dst, int r0, int rows, int per,
                              int src_per, int H, hipStream_t s);

// Write side of the input-side passes (exact catch-up and prompt prefill). kv rows
// [rows, 2 * n_kv * d] fp32 hold k (before RoPE) then v of candidate rows r = r0 + i,
// sequence b = r / per, index j = r % per. Rows with j < lim(b) are rotated at position
// pos[b] + off + j and written to slot len[b] + off + j in the cache dtype, where
// lim(b) = limit[b] clamped to [0, per] (per when limit is null).
//   catch-up: per = K, off = 1 - K, limit = accepted lengths (len / pos: after the draft)
//   prefill:  per = n, off = 0, limit = per-sequence row counts or null
struct CatchupParams {
  const float* kvrows;
  int ld;  // floats per kv row
  void* kc;
  void* vc;
  int n_kv, d, capacity;
  const int* len;
  const int* pos;
  const int* limit;
  int per, off, r0, rows;
  float theta;
  unsigned* err;
};
hipError_t launch_catchup_write(int cdtype, const CatchupParams& p, hipStream_t s);
// len[b] += lim + add and pos[b] += lim + add, lim = limit[b] clamped to [0, per] (per when
// limit is null); an entry outside [0, per] sets `err_bit` in the error word.
hipError_t launch_catchup_commit(int* len, int* pos, const int* limit, int B, int per, int add,
                                 unsigned err_bit, unsigned* err, hipStream_t s);

// Prefix scan of verification from per-row target tokens: tokens[b * (K+1) + j] is the
// target's token after input j; accepted[b] / next[b] as launch_verify writes them.
hipError_t launch_accept(const int* tokens, const int* draft, int B, int K, int* accepted,
                         int* next, hipStream_t s);

}  // namespace mtp
