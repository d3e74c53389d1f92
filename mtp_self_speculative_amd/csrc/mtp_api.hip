// Host side of the C ABI declared in include/mtp.h: argument validation, workspace
// layout, kernel selection and the launch sequence of one speculative iteration.
#include <math.h>
#include <cmath>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "kernels.h"
#include "mtp.h"

namespace {

using namespace mtp;

constexpr int kMaxSplits = 256;
// Cache capacity limit: kMaxSplits chunks of the fp32 kernel's longest chunk (1024).
constexpr int kMaxCapacity = kMaxSplits * 1024;
constexpr int kMaxK = 100;
static_assert(kMaxK <= kVsMaxK, "sampling verification holds 2K+1 log-sum-exps in LDS");
constexpr int kMaxGroupHeads = 8;
constexpr size_t kGemvLdsBudget = 32 * 1024;
constexpr uint32_t kCreateFlags = MTP_CREATE_NO_PACKED_COPY;  // flags mtp_create_ex knows
constexpr int kGemvMaxGrid = 2048;

struct Layout {
  size_t x, x1, h, qkv, o, act, rope, part_o, part_ml, attn_perm, lm_keys, lm_cnt, v_keys,
      v_cnt, err;
  size_t dummy;        // zeroed target of never-consumed tail prefetches
  size_t attn_chunk;   // the draft call's attention chunk (int), computed on the device
  size_t t2_tok;       // debug draft's second-best pass: its (discarded) winners [B]
  size_t xq, xq_lo, mm_part;  // batched path: bf16 operand planes, K-split partial sums
  int ldq;
  // verification from hidden states: one group of up to kVhGroupPk rows at a time (with
  // the packed lm_head copy; else kVhGroup)
  size_t vh_x, vh_q, vh_q_lo, vh_keys, vh_cnt, vh_tok;
  int vh_rows, vh_ld;
  // exact cache catch-up: one group of up to kVhGroup candidate rows at a time
  size_t cu_h, cu_x, cu_kv, cu_q, cu_q_lo, cu_part;
  size_t cu_part_elems;  // floats of room at cu_part
  int cu_rows, cu_ld;
  // sampling verification: (max, sum) pairs per (sequence, row, chunk), row a's lse, keys
  size_t vs_part, vs_lse, vs_keys;
  int v_kstride;  // keys per sequence in v_keys
  // batched path: packed copies of the draft step's matrices (launch_pack), 0 when absent
  size_t pk_eh, pk_qkv, pk_o, pk_gu, pk_down, pk_lm;
  size_t total;
};

// Batched (MFMA) path: bf16 weights, 3..64 sequences, rows short enough for the
// row-wise norm kernels.
constexpr int kMmMinBatch = 3;
constexpr int kVhGroup = 64;      // rows per pass of the general lm_head / contraction
constexpr int kVhGroupPk = 128;   // rows per greedy lm_head pass on the packed copy
constexpr int kMmMaxBatch = 64;
// Input-side row groups (catch-up, prompt prefill) of more than kMmMaxBatch rows go to the
// tiled contraction, up to kGmGroup rows per group; the partial sums get room for
// kGmPartRows rows of the wider contraction, which bounds the tiled one's K splits.
// (Prefill of a 4096-token q8b prompt: 1128 us in 1024-row groups, 1045 in 2048, 1026 in
// one group of 4096; the workspace of a batch-1 q8b handle 114, 189 and 374 MB.)
constexpr int kGmGroup = 2048;
constexpr int kGmPartRows = 2048;
bool mm_eligible(const mtp_config& c) {
  return c.dtype == MTP_BF16 && c.hidden <= red_max_cols();
}
bool use_mm(const mtp_config& c, int B) {
  return mm_eligible(c) && B >= kMmMinBatch && B <= kMmMaxBatch;
}

// The contractions of one draft step that end in K-split partial sums: (rows, columns).
void mm_shapes(const mtp_config& c, int shapes[5][2]) {
  const int H = c.hidden, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  const int v[5][2] = {{H, 2 * H}, {qd + 2 * kvd, H}, {H, qd}, {2 * c.ffn, H}, {H, c.ffn}};
  for (int i = 0; i < 5; ++i) {
    shapes[i][0] = v[i][0];
    shapes[i][1] = v[i][1];
  }
}

// Most K splits a contraction of these sizes takes with 128- or 256-row items (sizes the
// partials).
int mm_split_max(int nrows, int ncols, int B) {
  const int s1 = mm_split(nrows, ncols, B, 128);
  const int s2 = mm_split(nrows, ncols, B, 256);
  return s1 > s2 ? s1 : s2;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The re-laid-out weight copy exists for bf16 handles that can take the matrix-core path,
// unless the caller asked for none.
bool wants_packed(const mtp_config& c, int max_batch, uint32_t flags) {
  return mm_eligible(c) && max_batch >= kMmMinBatch && !(flags & MTP_CREATE_NO_PACKED_COPY);
}

Layout make_layout(const mtp_config& c, int max_batch, int max_k, int max_cap, uint32_t flags) {
  Layout L{};
  const bool packed = wants_packed(c, max_batch, flags);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t B = (size_t)max_batch, H = (size_t)c.hidden, d = (size_t)c.head_dim;
  const size_t nq = (size_t)c.n_q_heads, nkv = (size_t)c.n_kv_heads;
  L.x = take(B * H * 4);
  L.x1 = take(B * H * 4);
  L.h = take(B * H * 4);
  L.qkv = take(B * (nq + 2 * nkv) * d * 4);
  L.o = take(B * nq * d * 4);
  L.act = take(B * (size_t)c.ffn * 4);
  L.rope = take((size_t)(max_k > 0 ? max_k : 1) * B * d * 4);
  L.part_o = take(B * nq * kMaxSplits * d * 4);
  L.part_ml = take(B * nq * kMaxSplits * 2 * 4);
  L.attn_perm = take(B * nkv * kMaxSplits * 4);
  L.lm_keys = take(B * 8);
  L.lm_cnt = take(4);
  L.v_kstride = (max_k + 1 + kSeqLineU64 - 1) / kSeqLineU64 * kSeqLineU64;
  L.v_keys = take(B * (size_t)L.v_kstride * 8);
  L.v_cnt = take(B * kSeqLineU32 * 4);
  L.err = take(4);
  L.dummy = take(kDummyBytes);
  L.attn_chunk = take(4);
  L.t2_tok = take(B * 4);
  L.ldq = 0;
  L.xq = L.xq_lo = L.mm_part = off;
  if (mm_eligible(c) && max_batch >= kMmMinBatch) {
    const int bmax = max_batch < kMmMaxBatch ? max_batch : kMmMaxBatch;
    int w = 2 * c.hidden;
    if (c.ffn > w) w = c.ffn;
    if (c.n_q_heads * c.head_dim > w) w = c.n_q_heads * c.head_dim;
    L.ldq = (w + 7) / 8 * 8;
    L.xq = take((size_t)mm_batch_pad(bmax) * L.ldq * 2);
    L.xq_lo = take((size_t)mm_batch_pad(bmax) * L.ldq * 2);
    int shapes[5][2];
    mm_shapes(c, shapes);
    size_t part = 0;
    for (int b = kMmMinBatch; b <= bmax; ++b)
      for (auto& sh : shapes) {
        const size_t e = (size_t)mm_split_max(sh[0], sh[1], b) * mm_batch_pad(b) * sh[0];
        if (e > part) part = e;
      }
    L.mm_part = take(part * 4);
  }
  // verification from the target's hidden states
  {
    const long rows_all = (long)max_batch * (max_k + 1);
    // 128 rows per pass on matrix-core handles (the eight-tile streaming kernel on the packed
    // lm_head copy, else the tiled contraction on the row-major lm_head)
    const int grp = mm_eligible(c) ? kVhGroupPk : kVhGroup;
    L.vh_rows = (int)(rows_all < grp ? rows_all : grp);
    L.vh_ld = (c.hidden + 7) / 8 * 8;
    L.vh_x = take((size_t)L.vh_rows * c.hidden * 4);
    L.vh_q = L.vh_q_lo = off;
    if (mm_eligible(c)) {
      L.vh_q = take((size_t)mm_batch_pad(L.vh_rows) * L.vh_ld * 2);
      L.vh_q_lo = take((size_t)mm_batch_pad(L.vh_rows) * L.vh_ld * 2);
    }
    L.vh_keys = take((size_t)L.vh_rows * 8);
    L.vh_cnt = take(4);
    L.vh_tok = take((size_t)rows_all * 4);
  }
  // exact cache catch-up
  {
    // Catch-up has max_batch * max_k candidate rows, prefill up to max_batch * capacity.
    // Rows per pass: kVhGroup, or on matrix-core handles up to kGmGroup (the tiled
    // contraction above 64 rows), never more than a call can bring.
    L.cu_rows = kVhGroup;
    if (mm_eligible(c)) {
      const long most = (long)max_batch * (max_cap > max_k ? max_cap : max_k);
      L.cu_rows = most < kVhGroup ? kVhGroup : most > kGmGroup ? kGmGroup : (int)most;
    }
    L.cu_ld = (2 * c.hidden + 7) / 8 * 8;
    const int kvd2 = 2 * c.n_kv_heads * c.head_dim;
    const int rr = L.cu_rows > 0 ? L.cu_rows : 1;
    L.cu_h = take((size_t)rr * c.hidden * 4);
    L.cu_x = take((size_t)rr * c.hidden * 4);
    L.cu_kv = take((size_t)rr * kvd2 * 4);
    L.cu_q = L.cu_q_lo = L.cu_part = off;
    if (mm_eligible(c) && L.cu_rows >= kMmMinBatch) {
      L.cu_q = take((size_t)mm_batch_pad(L.cu_rows) * L.cu_ld * 2);
      L.cu_q_lo = take((size_t)mm_batch_pad(L.cu_rows) * L.cu_ld * 2);
      size_t part = 0;
      for (int b = kMmMinBatch; b <= L.cu_rows && b <= kMmMaxBatch; ++b) {
        const size_t e1 =
            (size_t)mm_split_max(c.hidden, 2 * c.hidden, b) * mm_batch_pad(b) * c.hidden;
        const size_t e2 = (size_t)mm_split_max(kvd2, c.hidden, b) * mm_batch_pad(b) * kvd2;
        part = e1 > part ? e1 : part;
        part = e2 > part ? e2 : part;
      }
      if (L.cu_rows > kMmMaxBatch) {  // tiled groups: splits x rows <= kGmPartRows
        const size_t wide = (size_t)(c.hidden > kvd2 ? c.hidden : kvd2);
        const size_t pr = (size_t)(L.cu_rows > kGmPartRows ? L.cu_rows : kGmPartRows);
        part = pr * wide > part ? pr * wide : part;
      }
      L.cu_part = take(part * 4);
      L.cu_part_elems = part;
    }
  }
  // packed weights for the matrix-core draft path (made once by mtp_create)
  L.pk_eh = L.pk_qkv = L.pk_o = L.pk_gu = L.pk_down = L.pk_lm = 0;
  if (packed) {
    const int H = c.hidden, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    L.pk_eh = take(mm_packed_elems(H, 2 * H) * 2);
    L.pk_qkv = take(mm_packed_elems(qd + 2 * kvd, H) * 2);
    L.pk_o = take(mm_packed_elems(H, qd) * 2);
    L.pk_gu = take(mm_packed_elems(2 * c.ffn, H) * 2);
    L.pk_down = take(mm_packed_elems(H, c.ffn) * 2);
    L.pk_lm = take(mm_packed_elems(c.vocab, H) * 2);
  }
  L.vs_part = take((size_t)max_batch * (2 * max_k + 1) * vs_chunks(c.vocab) * 8);
  L.vs_lse = take((size_t)max_batch * 2 * 4);
  L.vs_keys = take((size_t)max_batch * kSeqLineU64 * 8);
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

mtp_status check_config(const mtp_config* c) {
  if (!c) return MTP_ERR_INVALID_ARG;
  if (c->dtype != MTP_F32 && c->dtype != MTP_BF16) return MTP_ERR_DTYPE;
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->ffn <= 0 || c->vocab <= 0)
    return MTP_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads != 0) return MTP_ERR_SHAPE;
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return MTP_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return MTP_ERR_UNSUPPORTED;
  if (c->n_q_heads / c->n_kv_heads > kMaxGroupHeads) return MTP_ERR_UNSUPPORTED;
  if (c->hidden % 8 != 0 || c->ffn % 8 != 0) return MTP_ERR_UNSUPPORTED;
  return MTP_OK;
}

mtp_status check_limits(int max_batch, int max_k, int max_capacity) {
  if (max_batch < 1 || max_k < 0 || max_capacity < 1) return MTP_ERR_SHAPE;
  if (max_k > kMaxK || max_capacity > kMaxCapacity) return MTP_ERR_CAPACITY;
  return MTP_OK;
}

int nb_for(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }

// Writes the packed copies of the batched path's matrices (contiguous matrix-core loads)
// from the weights into the workspace, on stream s.
hipError_t pack_weights(const Layout& L, const mtp_config& c, const mtp_weights& w, char* ws,
                        hipStream_t s) {
  if (!L.pk_lm) return hipSuccess;
  auto pk = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  const int H = c.hidden, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  const int F = c.ffn;
  hipError_t e = launch_pack(w.w_eh, w.w_eh, w.w_eh, H, H, H, 2 * H, pk(L.pk_eh), s);
  if (e == hipSuccess)
    e = launch_pack(w.w_q, w.w_k, w.w_v, qd, qd + kvd, qd + 2 * kvd, H, pk(L.pk_qkv), s);
  if (e == hipSuccess) e = launch_pack(w.w_o, w.w_o, w.w_o, H, H, H, qd, pk(L.pk_o), s);
  if (e == hipSuccess) e = launch_pack(w.w_gate, w.w_up, w.w_up, F, 2 * F, 2 * F, H, pk(L.pk_gu), s);
  if (e == hipSuccess) e = launch_pack(w.w_down, w.w_down, w.w_down, H, H, H, F, pk(L.pk_down), s);
  if (e == hipSuccess)
    e = launch_pack(w.lm_head, w.lm_head, w.lm_head, c.vocab, c.vocab, c.vocab, H, pk(L.pk_lm), s);
  return e;
}

int col_block_for(int ncols, int B, int dtype) {
  const int step = 64 * (dtype == MTP_F32 ? 4 : 8);
  const int nb = nb_for(B);
  int cb = (int)(kGemvLdsBudget / (4 * (size_t)nb)) / step * step;
  if (cb < step) cb = step;
  const int full = (ncols + step - 1) / step * step;
  return cb < full ? cb : full;
}

}  // namespace

struct ProfRec {
  int id;
  hipEvent_t a, b;
};

struct mtp_handle {
  mtp_config cfg;
  mtp_weights w;
  int max_batch, max_k, max_cap;
  uint32_t flags;  // mtp_create_ex flags
  char* ws;
  size_t ws_bytes;
  Layout L;
  int num_cu = 256;
  bool lm_rows_ok = false;  // the single-launch small-row verification kernel is usable
  bool gm_ok = false;       // the tiled contraction is usable (its LDS limit was raised)
  uint32_t prof_mask = 0;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  template <class T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(ws + off);
  }
};

namespace {

enum KernelClass { KC_EH = 0, KC_QKV, KC_ATTN, KC_OPROJ, KC_GATEUP, KC_DOWN, KC_LMHEAD, KC_VERIFY,
                   KC_ROLLBACK, KC_COUNT };

hipEvent_t take_event(mtp_handle* h) {
  if (!h->pool.empty()) {
    hipEvent_t e = h->pool.back();
    h->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch `f` and, when kernel class `id` is being profiled, bracket it with events.
template <class Fn>
hipError_t timed(mtp_handle* h, int id, hipStream_t s, Fn&& f) {
  if (!((h->prof_mask >> id) & 1u)) return f();
  hipEvent_t a = take_event(h), b = take_event(h);
  if (!a || !b) return hipErrorOutOfMemory;
  (void)hipEventRecord(a, s);
  hipError_t e = f();
  (void)hipEventRecord(b, s);
  h->recs.push_back({id, a, b});
  return e;
}

// Pick the pipelined kernel when the batch's input vectors fit in LDS, else the
// column-blocked one.
hipError_t run_gemv(const mtp_handle* h, Pro pro, Epi epi, GemvParams& g, hipStream_t s) {
  g.dummy = h->ws + h->L.dummy;
  if (gemv_pipe_fits(g.ncols, g.B, h->cfg.dtype))
    return launch_gemv_pipe(h->cfg.dtype, pro, epi, g, gemv_pipe_grid(g.nrows, g.ncols, h->cfg.dtype, h->num_cu), s);
  g.col_block = col_block_for(g.ncols, g.B, h->cfg.dtype);
  return launch_gemv(h->cfg.dtype, pro, epi, g, kGemvMaxGrid, s);
}

}  // namespace

extern "C" {

const char* mtp_status_string(mtp_status s) {
  switch (s) {
    case MTP_OK: return "ok";
    case MTP_ERR_INVALID_ARG: return "invalid argument";
    case MTP_ERR_SHAPE: return "inconsistent or non-positive shape";
    case MTP_ERR_DTYPE: return "unknown dtype";
    case MTP_ERR_CAPACITY: return "capacity exceeded (batch, K, workspace or cache)";
    case MTP_ERR_UNSUPPORTED: return "shape not supported by the kernels";
    case MTP_ERR_HIP: return "HIP runtime error";
    case MTP_ERR_DEVICE: return "device-side error (see mtp_get_error bits)";
  }
  return "unknown status";
}

mtp_status mtp_step_weights(float beta, int32_t K, float* out) {
  if (!out || !(beta > 0.f) || !(beta < INFINITY)) return MTP_ERR_INVALID_ARG;
  if (K < 1 || K > kMaxK) return MTP_ERR_SHAPE;
  double total = 0.0, w = 1.0;
  for (int k = 0; k < K; ++k, w *= beta) total += w;
  w = 1.0;
  for (int k = 0; k < K; ++k, w *= beta) out[k] = (float)(w / total);
  return MTP_OK;
}

mtp_status mtp_adapt_k(const int32_t* accepted_len, int32_t B, int32_t K, int32_t k_min,
                       int32_t k_max, int32_t* k_next) {
  if (!accepted_len || !k_next) return MTP_ERR_INVALID_ARG;
  if (B < 1 || K < 0 || k_min < 0 || k_max < k_min || k_max > kMaxK) return MTP_ERR_SHAPE;
  int want = 0;
  for (int b = 0; b < B; ++b) {
    const int a = accepted_len[b];
    if (a < 0 || a > K) return MTP_ERR_INVALID_ARG;
    const int w = a == K ? K + 1 : a + 1;
    want = w > want ? w : want;
  }
  *k_next = want < k_min ? k_min : want > k_max ? k_max : want;
  return MTP_OK;
}

mtp_status mtp_workspace_size_ex(const mtp_config* cfg, int32_t max_batch, int32_t max_k,
                                 int32_t max_capacity, uint32_t flags, size_t* bytes) {
  if (!bytes || (flags & ~kCreateFlags)) return MTP_ERR_INVALID_ARG;
  mtp_status st = check_config(cfg);
  if (st != MTP_OK) return st;
  st = check_limits(max_batch, max_k, max_capacity);
  if (st != MTP_OK) return st;
  *bytes = make_layout(*cfg, max_batch, max_k, max_capacity, flags).total;
  return MTP_OK;
}

mtp_status mtp_workspace_size(const mtp_config* cfg, int32_t max_batch, int32_t max_k,
                              int32_t max_capacity, size_t* bytes) {
  return mtp_workspace_size_ex(cfg, max_batch, max_k, max_capacity, 0u, bytes);
}

mtp_status mtp_create(const mtp_config* cfg, const mtp_weights* w, int32_t max_batch,
                      int32_t max_k, int32_t max_capacity, void* workspace, size_t workspace_bytes,
                      mtp_handle** out) {
  return mtp_create_ex(cfg, w, max_batch, max_k, max_capacity, 0u, workspace, workspace_bytes,
                       out);
}

mtp_status mtp_create_ex(const mtp_config* cfg, const mtp_weights* w, int32_t max_batch,
                         int32_t max_k, int32_t max_capacity, uint32_t flags, void* workspace,
                         size_t workspace_bytes, mtp_handle** out) {
  if (!out) return MTP_ERR_INVALID_ARG;
  *out = nullptr;
  if (flags & ~kCreateFlags) return MTP_ERR_INVALID_ARG;
  mtp_status st = check_config(cfg);
  if (st != MTP_OK) return st;
  st = check_limits(max_batch, max_k, max_capacity);
  if (st != MTP_OK) return st;
  if (!w || !workspace) return MTP_ERR_INVALID_ARG;
  const void* ptrs[] = {w->g_h, w->g_e, w->w_eh, w->g_attn, w->w_q, w->w_k, w->w_v, w->w_o,
                        w->g_mlp, w->w_gate, w->w_up, w->w_down, w->g_final, w->embed, w->lm_head};
  for (const void* p : ptrs)
    if (!p || !aligned(p, 16)) return MTP_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return MTP_ERR_INVALID_ARG;
  const Layout L = make_layout(*cfg, max_batch, max_k, max_capacity, flags);
  if (workspace_bytes < L.total) return MTP_ERR_CAPACITY;
  if (hipMemset(workspace, 0, L.total) != hipSuccess) return MTP_ERR_HIP;
  if (pack_weights(L, *cfg, *w, static_cast<char*>(workspace), 0) != hipSuccess)
    return MTP_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return MTP_ERR_HIP;
  mtp_handle* h = new (std::nothrow) mtp_handle();
  if (!h) return MTP_ERR_CAPACITY;
  h->cfg = *cfg;
  h->w = *w;
  h->max_batch = max_batch;
  h->max_k = max_k;
  h->max_cap = max_capacity;
  h->flags = flags;
  h->ws = static_cast<char*>(workspace);
  h->ws_bytes = workspace_bytes;
  h->L = L;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      ncu > 0)
    h->num_cu = ncu;
  h->lm_rows_ok = cfg->dtype == MTP_BF16 && lm_rows_prepare() == hipSuccess;
  h->gm_ok = mm_eligible(*cfg) && gm_prepare() == hipSuccess;
  *out = h;
  return MTP_OK;
}

mtp_status mtp_refresh_weights(mtp_handle* h, void* stream) {
  if (!h) return MTP_ERR_INVALID_ARG;
  return pack_weights(h->L, h->cfg, h->w, h->ws, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MTP_OK
             : MTP_ERR_HIP;
}

void mtp_destroy(mtp_handle* h) {
  if (!h) return;
  for (auto& r : h->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
  delete h;
}

mtp_status mtp_set_profiling(mtp_handle* h, uint32_t mask) {
  if (!h) return MTP_ERR_INVALID_ARG;
  h->prof_mask = mask;
  return MTP_OK;
}

mtp_status mtp_get_profile(mtp_handle* h, float* total_ms, int32_t* launches, int32_t n) {
  if (!h || !total_ms || !launches || n < 0 || n > 16) return MTP_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.f;
    launches[i] = 0;
  }
  mtp_status st = MTP_OK;
  if (!h->recs.empty() && hipEventSynchronize(h->recs.back().b) != hipSuccess) st = MTP_ERR_HIP;
  for (auto& r : h->recs) {
    float ms = 0.f;
    if (st == MTP_OK && hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) st = MTP_ERR_HIP;
    if (r.id < n) {
      total_ms[r.id] += ms;
      launches[r.id] += 1;
    }
    h->pool.push_back(r.a);
    h->pool.push_back(r.b);
  }
  h->recs.clear();
  return st;
}

static mtp_status check_kv(const mtp_handle* h, const mtp_kv* kv, int B) {
  if (!kv || !kv->k || !kv->v || !kv->len || !kv->pos) return MTP_ERR_INVALID_ARG;
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return MTP_ERR_INVALID_ARG;
  if (kv->batch < 1 || kv->capacity < 1) return MTP_ERR_SHAPE;
  if (B > kv->batch) return MTP_ERR_SHAPE;
  if (kv->capacity > h->max_cap) return MTP_ERR_CAPACITY;
  return MTP_OK;
}

// Attention parameters of step k (shared by both paths).
static AttnParams attn_params(const mtp_handle* h, mtp_kv* kv, int k, int B, int chunk,
                              int nsplit, const int* perm, const int* kseq) {
  const mtp_config& c = h->cfg;
  const Layout& L = h->L;
  AttnParams a{};
  a.qkv = h->at<float>(L.qkv);
  a.ldqkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  a.kc = kv->k; a.vc = kv->v;
  a.n_q = c.n_q_heads; a.n_kv = c.n_kv_heads; a.d = c.head_dim; a.capacity = kv->capacity;
  a.len = kv->len; a.pos = kv->pos; a.step = k;
  a.chunk = chunk; a.nsplit = nsplit;
  a.rope = h->at<float>(L.rope) + (size_t)k * B * c.head_dim;
  a.scale = 1.0f / sqrtf((float)c.head_dim);
  a.part_o = h->at<float>(L.part_o);
  a.part_ml = h->at<float>(L.part_ml);
  a.o = h->at<float>(L.o);
  a.err = h->at<unsigned>(L.err);
  a.perm = perm;
  a.kseq = kseq;
  a.chunk_dev = h->at<int>(L.attn_chunk);
  return a;
}

// The K draft steps for 3..64 sequences with bf16 weights: each projection is an MFMA
// contraction into K-split partials followed by a row-wise kernel that adds the splits,
// applies the epilogue and writes the next contraction's normalised bf16 operand.
// Where the lm_head writes logits (optional) and whether it samples instead of argmax.
struct LmOut {
  float* logits;       // step k, sequence b at logits + k * step_stride + b * ld
  size_t step_stride;
  int ld;
  const SampleParams* smp;  // null: argmax
};

static mtp_status draft_steps_mm(mtp_handle* h, const int32_t* last_tokens, mtp_kv* kv,
                                 int32_t B, int32_t K, int32_t* draft_tokens, float* hidden_out,
                                 float* top2_out, const LmOut& lo, int chunk, int nsplit,
                                 const int* perm, const int* kseq, hipStream_t s) {
  const mtp_config& c = h->cfg;
  const mtp_weights& w = h->w;
  const Layout& L = h->L;
  const int H = c.hidden, d = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads, F = c.ffn;
  const int V = c.vocab, qkvd = (nq + 2 * nkv) * d;
  const int bp = mm_batch_pad(B);
  float* x = h->at<float>(L.x);
  float* x1 = h->at<float>(L.x1);
  float* hb = h->at<float>(L.h);
  float* part = h->at<float>(L.mm_part);
  uint16_t* xq = h->at<uint16_t>(L.xq);
  uint16_t* xq_lo = h->at<uint16_t>(L.xq_lo);
  unsigned* err = h->at<unsigned>(L.err);
  auto g16 = [&](const void* p) { return static_cast<const uint16_t*>(p); };

  // One contraction (rows r of w0|w1|w2 against xq) into partials; returns the splits.
  auto pkp = [&](size_t off) -> const uint16_t* {
    return off ? reinterpret_cast<const uint16_t*>(h->ws + off) : nullptr;
  };
  auto mm = [&](const void* w0, const void* w1, const void* w2, int seg1, int seg2, int N,
                int Kd, size_t pk_off, int* ns) -> hipError_t {
    MmParams m{};
    m.w0 = w0; m.w1 = w1; m.w2 = w2; m.seg1 = seg1; m.seg2 = seg2;
    m.packed = pkp(pk_off);
    m.nrows = N; m.ncols = Kd; m.x = xq; m.x_lo = xq_lo; m.ldx = L.ldq; m.B = B;
    const MmPlan q = mm_plan(EPI_STORE, N, Kd, B, m.packed != nullptr, h->num_cu);
    m.tile_rows = q.tile_rows;
    m.nsplit = q.nsplit;
    m.part = part;
    m.dummy = h->ws + L.dummy;
    *ns = m.nsplit;
    return launch_mm(EPI_STORE, m, q.grid, s);
  };
  auto red = [&](RedMode mode, int ns, int n_part, int n, const float* res, float* out,
                 float* dbg, const void* gain) -> hipError_t {
    RedParams r{};
    r.part = part; r.nsplit = ns; r.bp = bp; r.n_part = n_part; r.n = n;
    r.res = res; r.out = out; r.dbg = dbg; r.dbg_ld = H;
    r.gain = g16(gain); r.eps = c.rms_eps;
    r.xq = mode == RED_QKV ? nullptr : xq;
    r.xq_lo = mode == RED_QKV ? nullptr : xq_lo;
    r.ldq = L.ldq;
    return launch_red(mode, r, B, s);
  };

  for (int k = 0; k < K; ++k) {
    hipError_t e;
    int ns = 1;
    // 1. gather + separate RMSNorms + concat, then eh_proj
    e = timed(h, KC_EH, s, [&] {
      RedParams r{};
      r.n = H; r.gain = g16(w.g_h); r.gain2 = g16(w.g_e); r.eps = c.rms_eps;
      r.xq = xq; r.xq_lo = xq_lo; r.ldq = L.ldq; r.h = hb; r.embed = g16(w.embed);
      r.tok = k == 0 ? last_tokens : draft_tokens + (k - 1);
      r.tok_stride = k == 0 ? 1 : K;
      r.vocab = V; r.err = err;
      hipError_t e2 = launch_red(PREP_EH, r, B, s);
      if (e2 == hipSuccess) e2 = mm(w.w_eh, w.w_eh, w.w_eh, H, H, H, 2 * H, L.pk_eh, &ns);
      if (e2 == hipSuccess) e2 = red(RED_EH, ns, H, H, nullptr, x, nullptr, w.g_attn);
      return e2;
    });
    if (e != hipSuccess) return MTP_ERR_HIP;
    // 2. QKV (the attention norm was applied by the previous row kernel)
    e = timed(h, KC_QKV, s, [&] {
      hipError_t e2 = mm(w.w_q, w.w_k, w.w_v, nq * d, (nq + nkv) * d, qkvd, H, L.pk_qkv, &ns);
      if (e2 == hipSuccess) e2 = red(RED_QKV, ns, qkvd, qkvd, nullptr, h->at<float>(L.qkv), nullptr, nullptr);
      return e2;
    });
    if (e != hipSuccess) return MTP_ERR_HIP;
    // 3. RoPE + cache append + attention; the merge writes o as the next bf16 operand
    AttnParams a = attn_params(h, kv, k, B, chunk, nsplit, perm, kseq);
    a.o_bf16 = xq;
    a.o_bf16_lo = xq_lo;
    a.ld_o_bf16 = L.ldq;
    if (timed(h, KC_ATTN, s, [&] { return launch_attention(c.dtype, a, B, s); }) != hipSuccess)
      return MTP_ERR_HIP;
    // 4. O projection + residual; writes RMSNorm(x1) * g_mlp
    e = timed(h, KC_OPROJ, s, [&] {
      hipError_t e2 = mm(w.w_o, w.w_o, w.w_o, H, H, H, nq * d, L.pk_o, &ns);
      if (e2 == hipSuccess) e2 = red(RED_RESID, ns, H, H, x, x1, nullptr, w.g_mlp);
      return e2;
    });
    if (e != hipSuccess) return MTP_ERR_HIP;
    // 5. gate / up + SwiGLU
    e = timed(h, KC_GATEUP, s, [&] {
      hipError_t e2 = mm(w.w_gate, w.w_up, w.w_up, F, 2 * F, 2 * F, H, L.pk_gu, &ns);
      if (e2 == hipSuccess) e2 = red(RED_SWIGLU, ns, 2 * F, F, nullptr, nullptr, nullptr, nullptr);
      return e2;
    });
    if (e != hipSuccess) return MTP_ERR_HIP;
    // 6. down + residual -> h^(k); writes RMSNorm(h^(k)) * g_final
    e = timed(h, KC_DOWN, s, [&] {
      hipError_t e2 = mm(w.w_down, w.w_down, w.w_down, H, H, H, F, L.pk_down, &ns);
      if (e2 == hipSuccess)
        e2 = red(RED_RESID, ns, H, H, x1, hb, hidden_out ? hidden_out + (size_t)k * B * H : nullptr,
                 w.g_final);
      return e2;
    });
    if (e != hipSuccess) return MTP_ERR_HIP;
    // 7. shared lm_head + argmax -> draft token
    e = timed(h, KC_LMHEAD, s, [&] {
      MmParams m{};
      m.w0 = m.w1 = m.w2 = w.lm_head;
      m.seg1 = m.seg2 = V;
      m.packed = pkp(L.pk_lm);
      m.nrows = V; m.ncols = H; m.x = xq; m.x_lo = xq_lo; m.ldx = L.ldq; m.B = B; m.nsplit = 1;
      m.keys = h->at<unsigned long long>(L.lm_keys);
      m.counter = h->at<unsigned>(L.lm_cnt);
      m.tok_out = draft_tokens + k;
      m.tok_out_stride = K;
      m.maxlogit = top2_out ? top2_out + (size_t)k * B * 2 : nullptr;
      m.maxlogit_stride = 2;
      m.logits = lo.logits ? lo.logits + (size_t)k * lo.step_stride : nullptr;
      m.logits_ld = lo.ld;
      m.len = kv->len; m.pos = kv->pos;
      m.advance = (k == K - 1) ? K : 0;
      m.kseq = kseq;
      m.dummy = h->ws + L.dummy;
      if (lo.smp) {
        m.smp = *lo.smp;
        m.smp.row = k;
      }
      const Epi epi = lo.smp ? EPI_SAMPLE : EPI_ARGMAX;
      const MmPlan q = mm_plan(epi, V, H, B, m.packed != nullptr, h->num_cu);
      m.tile_rows = q.tile_rows;
      hipError_t e2 = launch_mm(epi, m, q.grid, s);
      if (e2 == hipSuccess && top2_out) {
        // second best: the same pass with each sequence's winner left out
        m.tok_out = h->at<int>(L.t2_tok);
        m.tok_out_stride = 1;
        m.maxlogit = top2_out + (size_t)k * B * 2 + 1;
        m.logits = nullptr;
        m.advance = 0;
        m.excl = draft_tokens + k;
        m.excl_stride = K;
        e2 = launch_mm(EPI_ARGMAX, m, q.grid, s);
      }
      return e2;
    });
    if (e != hipSuccess) return MTP_ERR_HIP;
  }
  return MTP_OK;
}

static mtp_status draft_impl(mtp_handle* h, const void* hidden, const int32_t* last_tokens,
                             mtp_kv* kv, int32_t B, int32_t K, int32_t* draft_tokens,
                             float* hidden_out, float* top2_out, const LmOut& lo,
                             void* stream, const int32_t* kseq = nullptr) {
  if (!h || !hidden || !last_tokens) return MTP_ERR_INVALID_ARG;
  if (!aligned(hidden, 16)) return MTP_ERR_INVALID_ARG;
  if (K < 0 || B < 1) return MTP_ERR_SHAPE;
  if (K > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  mtp_status st = check_kv(h, kv, B);
  if (st != MTP_OK) return st;
  if (K == 0) return MTP_OK;
  if (!draft_tokens) return MTP_ERR_INVALID_ARG;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const mtp_config& c = h->cfg;
  const mtp_weights& w = h->w;
  const Layout& L = h->L;
  const int H = c.hidden, d = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads, F = c.ffn;
  const int V = c.vocab, qkvd = (nq + 2 * nkv) * d;
  float* x = h->at<float>(L.x);
  float* x1 = h->at<float>(L.x1);
  float* hb = h->at<float>(L.h);
  float* qkv = h->at<float>(L.qkv);
  float* o = h->at<float>(L.o);
  float* act = h->at<float>(L.act);
  unsigned* err = h->at<unsigned>(L.err);

  // Attention splits: aim for about one workgroup per CU over (split, kv head, sequence),
  // with chunks of q .. attn_max_chunk cache positions (q = the kernels' quantum) and
  // <= kMaxSplits. (Fewer, longer splits also make the merge cheaper; measured on MI355X
  // at batch 1, 256-position chunks beat 128, and for the bf16 cache at 32K contexts 2048
  // beat 1024.)
  const int q = attn_chunk_quantum();
  long want = ((long)kv->capacity * B * nkv + h->num_cu - 1) / h->num_cu;
  int chunk = (int)((want + q - 1) / q * q);
  if (chunk < q) chunk = q;
  if (chunk > attn_max_chunk(c.dtype)) chunk = attn_max_chunk(c.dtype);
  const int min_chunk = (kv->capacity + kMaxSplits - 1) / kMaxSplits;
  if (chunk < min_chunk) chunk = (min_chunk + q - 1) / q * q;
  int nsplit = (kv->capacity + chunk - 1) / chunk;
  // With more items than the chip runs at once (bf16 cache), the grid gets eight times as
  // many splits as one item per CU would need, and the set-up kernel picks how many of
  // them each sequence uses from the lengths (the balance rule of ChunkPlan). Measured on
  // MI355X (attention + merge): 64 sequences of 4096 slots 182 -> 173 us (512 items of
  // 4097 positions instead of 1536 of 1408), 32 ragged sequences of 1109-7733 slots
  // 101 -> 95-97 us (splits of 1152-1536 instead of 2048); 8 sequences of 32768 slots
  // 173 -> 168 us (4 splits of 8320). Item counts between one and two per CU are avoided:
  // 320 items took 227 us there, the CUs holding two being the bottleneck.
  const bool balance = c.dtype != 0 && (long)nsplit * nkv * B > 2L * h->num_cu;
  if (balance) {
    const long want8 = ((long)kv->capacity * B * nkv + 8L * h->num_cu - 1) / (8L * h->num_cu);
    int ch = (int)((want8 + q - 1) / q * q);
    if (ch < q) ch = q;
    if (ch > attn_max_chunk(c.dtype)) ch = attn_max_chunk(c.dtype);
    if (ch < min_chunk) ch = (min_chunk + q - 1) / q * q;
    chunk = ch;
    nsplit = (kv->capacity + chunk - 1) / chunk;
  }

  // The grid has nsplit splits per (kv head, sequence), sized for the capacity; the chunk
  // itself is chosen on the device from the lengths, so a cache much larger than its
  // contents still spreads the attended positions over every split.
  ChunkPlan cp{kv->len, kv->capacity, nsplit, q, chunk, h->at<int>(L.attn_chunk)};
  cp.balance = balance ? 1 : 0;
  cp.n_kv = nkv;
  cp.num_cu = h->num_cu;
  if (launch_draft_setup(c.dtype, h->at<float>(L.rope), kv->pos, B, K, d, c.rope_theta, hidden,
                         hb, H, kseq, MTP_DEVERR_COUNT, err, cp, s) != hipSuccess)
    return MTP_ERR_HIP;
  // With more attention items than run at once, order them longest first (per call).
  const int* perm = nullptr;
  if (attn_plan_wanted(B, nkv, nsplit, h->num_cu)) {
    if (launch_attn_plan(kv->len, B, nkv, chunk, h->at<int>(L.attn_chunk), nsplit,
                         h->at<int>(L.attn_perm), s) != hipSuccess)
      return MTP_ERR_HIP;
    perm = h->at<int>(L.attn_perm);
  }
  if (use_mm(c, B))
    return draft_steps_mm(h, last_tokens, kv, B, K, draft_tokens, hidden_out, top2_out, lo,
                          chunk, nsplit, perm, kseq, s);
  for (int k = 0; k < K; ++k) {
    hipError_t e;
    // 1. embedding gather + separate RMSNorms + concat + eh_proj
    GemvParams g{};
    g.w0 = g.w1 = g.w2 = w.w_eh;
    g.nrows = g.seg1 = g.seg2 = H;
    g.ncols = 2 * H;
    g.B = B;
    g.gain = w.g_h;
    g.gain2 = w.g_e;
    g.eps = c.rms_eps;
    g.h = hb;  // the set-up kernel widened the step-1 hidden state into hb
    g.h_is_f32 = 1;
    g.ldh = H;
    g.embed = w.embed;
    g.tok = k == 0 ? last_tokens : draft_tokens + (k - 1);
    g.tok_stride = k == 0 ? 1 : K;
    g.vocab = V;
    g.err = err;
    g.out = x;
    g.ldo = H;
    if ((e = timed(h, KC_EH, s, [&] { return run_gemv(h, PRO_EH, EPI_STORE, g, s); })) != hipSuccess)
      return MTP_ERR_HIP;

    // 2. attention RMSNorm + fused QKV projection
    g = GemvParams{};
    g.w0 = w.w_q; g.w1 = w.w_k; g.w2 = w.w_v;
    g.seg1 = nq * d; g.seg2 = (nq + nkv) * d; g.nrows = qkvd;
    g.ncols = H; g.B = B;
    g.x = x; g.ldx = H; g.gain = w.g_attn; g.eps = c.rms_eps;
    g.out = qkv; g.ldo = qkvd;
    if ((e = timed(h, KC_QKV, s, [&] { return run_gemv(h, PRO_RMS, EPI_STORE, g, s); })) != hipSuccess)
      return MTP_ERR_HIP;

    // 3. RoPE + cache append + split decode attention + merge
    AttnParams a = attn_params(h, kv, k, B, chunk, nsplit, perm, kseq);
    if ((e = timed(h, KC_ATTN, s, [&] { return launch_attention(c.dtype, a, B, s); })) != hipSuccess)
      return MTP_ERR_HIP;

    // 4. O projection + residual
    g = GemvParams{};
    g.w0 = g.w1 = g.w2 = w.w_o;
    g.nrows = g.seg1 = g.seg2 = H;
    g.ncols = nq * d; g.B = B;
    g.x = o; g.ldx = nq * d;
    g.out = x1; g.ldo = H; g.res = x;
    if ((e = timed(h, KC_OPROJ, s, [&] { return run_gemv(h, PRO_PLAIN, EPI_RESID, g, s); })) != hipSuccess)
      return MTP_ERR_HIP;

    // 5. MLP RMSNorm + gate/up + SiLU * up
    g = GemvParams{};
    g.w0 = w.w_gate; g.w1 = w.w_up; g.w2 = w.w_up;
    g.nrows = g.seg1 = g.seg2 = F;
    g.ncols = H; g.B = B;
    g.x = x1; g.ldx = H; g.gain = w.g_mlp; g.eps = c.rms_eps;
    g.out = act; g.ldo = F;
    if ((e = timed(h, KC_GATEUP, s, [&] { return run_gemv(h, PRO_RMS, EPI_SWIGLU, g, s); })) != hipSuccess)
      return MTP_ERR_HIP;

    // 6. down projection + residual -> h^(k)
    g = GemvParams{};
    g.w0 = g.w1 = g.w2 = w.w_down;
    g.nrows = g.seg1 = g.seg2 = H;
    g.ncols = F; g.B = B;
    g.x = act; g.ldx = F;
    g.out = hb; g.ldo = H; g.res = x1;
    g.dbg = hidden_out ? hidden_out + (size_t)k * B * H : nullptr;
    g.dbg_ld = H;
    if ((e = timed(h, KC_DOWN, s, [&] { return run_gemv(h, PRO_PLAIN, EPI_RESID, g, s); })) != hipSuccess)
      return MTP_ERR_HIP;

    // 7. final RMSNorm + shared lm_head + argmax -> draft token
    g = GemvParams{};
    g.w0 = g.w1 = g.w2 = w.lm_head;
    g.nrows = g.seg1 = g.seg2 = V;
    g.ncols = H; g.B = B;
    g.x = hb; g.ldx = H; g.gain = w.g_final; g.eps = c.rms_eps;
    g.keys = h->at<unsigned long long>(L.lm_keys);
    g.counter = h->at<unsigned>(L.lm_cnt);
    g.tok_out = draft_tokens + k;
    g.tok_out_stride = K;
    g.maxlogit = top2_out ? top2_out + (size_t)k * B * 2 : nullptr;
    g.maxlogit_stride = 2;
    g.logits = lo.logits ? lo.logits + (size_t)k * lo.step_stride : nullptr;
    g.logits_ld = lo.ld;
    g.len = kv->len; g.pos = kv->pos;
    g.advance = (k == K - 1) ? K : 0;
    g.kseq = kseq;
    if (lo.smp) {
      g.smp = *lo.smp;
      g.smp.row = k;
    }
    const Epi lm_epi = lo.smp ? EPI_SAMPLE : EPI_ARGMAX;
    if ((e = timed(h, KC_LMHEAD, s, [&] { return run_gemv(h, PRO_RMS, lm_epi, g, s); })) != hipSuccess)
      return MTP_ERR_HIP;
    if (top2_out) {
      // second best: the same pass with each sequence's winner left out
      g.tok_out = h->at<int>(L.t2_tok);
      g.tok_out_stride = 1;
      g.maxlogit = top2_out + (size_t)k * B * 2 + 1;
      g.logits = nullptr;
      g.advance = 0;
      g.excl = draft_tokens + k;
      g.excl_stride = K;
      if (run_gemv(h, PRO_RMS, EPI_ARGMAX, g, s) != hipSuccess) return MTP_ERR_HIP;
    }
  }
  return MTP_OK;
}

mtp_status mtp_draft(mtp_handle* h, const void* hidden, const int32_t* last_tokens, mtp_kv* kv,
                     int32_t B, int32_t K, int32_t* draft_tokens, void* stream) {
  return draft_impl(h, hidden, last_tokens, kv, B, K, draft_tokens, nullptr, nullptr,
                    LmOut{nullptr, 0, 0, nullptr}, stream);
}

mtp_status mtp_draft_sample(mtp_handle* h, const void* hidden, const int32_t* last_tokens,
                            mtp_kv* kv, int32_t B, int32_t K, float temperature,
                            const uint64_t* seeds, uint64_t offset, int32_t* draft_tokens,
                            float* draft_logits, void* stream) {
  if (!h) return MTP_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !std::isfinite(1.0f / temperature)) return MTP_ERR_INVALID_ARG;
  if (!std::isfinite(temperature)) return MTP_ERR_INVALID_ARG;
  if (K > 0 && (!seeds || !draft_logits || !aligned(draft_logits, 4))) return MTP_ERR_INVALID_ARG;
  SampleParams smp{1.0f / temperature, seeds, offset, 0};
  const int V = h->cfg.vocab;
  return draft_impl(h, hidden, last_tokens, kv, B, K, draft_tokens, nullptr, nullptr,
                    LmOut{draft_logits, (size_t)V, K * V, &smp}, stream);
}

mtp_status mtp_draft_debug(mtp_handle* h, const void* hidden, const int32_t* last_tokens,
                           mtp_kv* kv, int32_t B, int32_t K, int32_t* draft_tokens,
                           float* hidden_out, float* top2_out, float* logits_out,
                           void* stream) {
  if (!h) return MTP_ERR_INVALID_ARG;
  return draft_impl(h, hidden, last_tokens, kv, B, K, draft_tokens, hidden_out, top2_out,
                    LmOut{logits_out, (size_t)B * h->cfg.vocab, h->cfg.vocab, nullptr}, stream);
}

mtp_status mtp_verify(mtp_handle* h, const float* target_logits, const int32_t* draft_tokens,
                      int32_t B, int32_t K, int32_t* accepted_len, int32_t* next_token,
                      void* stream) {
  if (!h || !target_logits || !accepted_len || !next_token) return MTP_ERR_INVALID_ARG;
  if (K < 0 || B < 1) return MTP_ERR_SHAPE;
  if (K > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  if (K > 0 && !draft_tokens) return MTP_ERR_INVALID_ARG;
  VerifyParams p{};
  p.logits = target_logits;
  p.draft = draft_tokens;
  p.K = K;
  p.V = h->cfg.vocab;
  p.keys = h->at<unsigned long long>(h->L.v_keys);
  p.kstride = h->L.v_kstride;
  p.counters = h->at<unsigned>(h->L.v_cnt);
  p.accepted = accepted_len;
  p.next = next_token;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(h, KC_VERIFY, s, [&] { return launch_verify(p, B, s); }) == hipSuccess ? MTP_OK
                                                                                      : MTP_ERR_HIP;
}

mtp_status mtp_verify_sample(mtp_handle* h, const float* target_logits, const float* draft_logits,
                             const int32_t* draft_tokens, int32_t B, int32_t K, float temperature,
                             const uint64_t* seeds, uint64_t offset, int32_t* accepted_len,
                             int32_t* next_token, void* stream) {
  if (!h || !target_logits || !seeds || !accepted_len || !next_token) return MTP_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !std::isfinite(temperature) || !std::isfinite(1.0f / temperature))
    return MTP_ERR_INVALID_ARG;
  if (K < 0 || B < 1) return MTP_ERR_SHAPE;
  if (K > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  if (K > 0 && (!draft_tokens || !draft_logits)) return MTP_ERR_INVALID_ARG;
  VSampleParams p{};
  p.tlog = target_logits;
  p.dlog = draft_logits;
  p.draft = draft_tokens;
  p.K = K;
  p.V = h->cfg.vocab;
  p.nchunk = vs_chunks(p.V);
  p.inv_temp = 1.0f / temperature;
  p.seeds = seeds;
  p.offset = offset;
  p.part = h->at<unsigned long long>(h->L.vs_part);
  p.lse = h->at<float>(h->L.vs_lse);
  p.keys = h->at<unsigned long long>(h->L.vs_keys);
  p.counters = h->at<unsigned>(h->L.v_cnt);
  p.accepted = accepted_len;
  p.next = next_token;
  p.err = h->at<unsigned>(h->L.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(h, KC_VERIFY, s, [&] { return launch_verify_sample(p, B, s); }) == hipSuccess
             ? MTP_OK
             : MTP_ERR_HIP;
}

mtp_status mtp_verify_hidden(mtp_handle* h, const void* target_hidden, const void* target_norm,
                             const int32_t* draft_tokens, int32_t B, int32_t K,
                             int32_t* accepted_len, int32_t* next_token, void* stream) {
  if (!h || !target_hidden || !target_norm || !accepted_len || !next_token)
    return MTP_ERR_INVALID_ARG;
  if (!aligned(target_hidden, 16) || !aligned(target_norm, 16)) return MTP_ERR_INVALID_ARG;
  if (K < 0 || B < 1) return MTP_ERR_SHAPE;
  if (K > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  if (K > 0 && !draft_tokens) return MTP_ERR_INVALID_ARG;
  const mtp_config& c = h->cfg;
  const Layout& L = h->L;
  const int H = c.hidden, V = c.vocab;
  const int R = B * (K + 1);
  const size_t esz = c.dtype == MTP_BF16 ? 2 : 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* tok = h->at<int>(L.vh_tok);
  // Up to 16 rows without the packed lm_head copy: one launch (norm, row-major lm_head on
  // the matrix cores, argmax, prefix scan).
  if (h->lm_rows_ok && !L.pk_lm && lm_rows_fits(H, R)) {
    LmRowsParams q{};
    q.h = static_cast<const uint16_t*>(target_hidden);
    q.gain = static_cast<const uint16_t*>(target_norm);
    q.eps = c.rms_eps;
    q.W = static_cast<const uint16_t*>(h->w.lm_head);
    q.V = V; q.H = H; q.R = R;
    q.keys = h->at<unsigned long long>(L.vh_keys);
    q.counter = h->at<unsigned>(L.vh_cnt);
    q.tok_out = tok;
    q.draft = draft_tokens; q.B = B; q.K = K;
    q.accepted = accepted_len; q.next = next_token;
    return timed(h, KC_VERIFY, s, [&] { return launch_lm_rows(q, h->num_cu, s); }) == hipSuccess
               ? MTP_OK
               : MTP_ERR_HIP;
  }
  // more than 64 rows per pass need the tiled contraction or the packed copy
  const int group = h->gm_ok || L.pk_lm || L.vh_rows <= kMmMaxBatch ? L.vh_rows : kMmMaxBatch;
  auto run = [&]() -> hipError_t {
    hipError_t e = hipSuccess;
    for (int r0 = 0; r0 < R && e == hipSuccess; r0 += group) {
      const int rows = R - r0 < group ? R - r0 : group;
      const char* src = static_cast<const char*>(target_hidden) + (size_t)r0 * H * esz;
      if (mm_eligible(c) && rows >= kMmMinBatch) {
        RedParams r{};
        r.n = H; r.gain = static_cast<const uint16_t*>(target_norm); r.eps = c.rms_eps;
        r.xq = h->at<uint16_t>(L.vh_q); r.xq_lo = h->at<uint16_t>(L.vh_q_lo); r.ldq = L.vh_ld;
        r.h16 = reinterpret_cast<const uint16_t*>(src);
        e = launch_red(PREP_NORM, r, rows, s);
        if (e != hipSuccess) break;
        if (rows > kMmMaxBatch && !L.pk_lm && h->gm_ok) {
          // Without the packed copy: the tiled contraction on the row-major lm_head, argmax
          // epilogue. (With the copy, the eight-tile streaming kernel is faster: its
          // persistent items balance over the CUs, while 151936 vocabulary rows make 594
          // tiles, three rounds of 256 at 77% occupancy.)
          GmParams g{};
          g.w0 = g.w1 = h->w.lm_head; g.seg1 = V; g.nrows = V; g.ncols = H;
          g.x = h->at<uint16_t>(L.vh_q); g.x_lo = h->at<uint16_t>(L.vh_q_lo); g.ldx = L.vh_ld;
          g.B = rows; g.nsplit = 1; g.bp = rows;
          g.keys = h->at<unsigned long long>(L.vh_keys);
          g.counter = h->at<unsigned>(L.vh_cnt);
          g.tok_out = tok + r0;
          e = launch_gm(EPI_ARGMAX, g, s);
          continue;
        }
        MmParams m{};
        m.w0 = m.w1 = m.w2 = h->w.lm_head;
        m.packed = L.pk_lm ? reinterpret_cast<const uint16_t*>(h->ws + L.pk_lm) : nullptr;
        m.seg1 = m.seg2 = V;
        m.nrows = V; m.ncols = H;
        m.x = h->at<uint16_t>(L.vh_q); m.x_lo = h->at<uint16_t>(L.vh_q_lo); m.ldx = L.vh_ld;
        m.B = rows; m.nsplit = 1;
        m.keys = h->at<unsigned long long>(L.vh_keys);
        m.counter = h->at<unsigned>(L.vh_cnt);
        m.tok_out = tok + r0; m.tok_out_stride = 1;
        m.dummy = h->ws + L.dummy;
        const MmPlan q = mm_plan(EPI_ARGMAX, V, H, rows, m.packed != nullptr, h->num_cu);
        m.tile_rows = q.tile_rows;
        e = launch_mm(EPI_ARGMAX, m, q.grid, s);
      } else {
        const float* x = reinterpret_cast<const float*>(src);
        if (c.dtype == MTP_BF16) {
          e = launch_widen(c.dtype, src, h->at<float>(L.vh_x), (long)rows * H, s);
          x = h->at<float>(L.vh_x);
          if (e != hipSuccess) break;
        }
        GemvParams g{};
        g.w0 = g.w1 = g.w2 = h->w.lm_head;
        g.nrows = g.seg1 = g.seg2 = V;
        g.ncols = H; g.B = rows;
        g.x = x; g.ldx = H; g.gain = target_norm; g.eps = c.rms_eps;
        g.keys = h->at<unsigned long long>(L.vh_keys);
        g.counter = h->at<unsigned>(L.vh_cnt);
        g.tok_out = tok + r0; g.tok_out_stride = 1;
        e = run_gemv(h, PRO_RMS, EPI_ARGMAX, g, s);
      }
    }
    if (e == hipSuccess) e = launch_accept(tok, draft_tokens, B, K, accepted_len, next_token, s);
    return e;
  };
  return timed(h, KC_VERIFY, s, run) == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

}  // extern "C"

// The layer's input side over R candidate rows (exact catch-up and prompt prefill): row r
// of sequence b = r / per, index j = r % per, reads hidden row (b * src_per + j) of `src`
// and token tokens[r]; eh_proj, attention norm and K/V projections run in groups of
// L.cu_rows rows (matrix cores from 3 rows on for bf16: the weight-streaming contraction up
// to 64 rows, the tiled one above; else the GEMV); rows with
// j < limit[b] are rotated and written (catchup_write_kernel), then len / pos advance by
// limit[b] + add.
static hipError_t input_side_pass(mtp_handle* h, mtp_kv* kv, const void* src, int per,
                                  int src_per, const int32_t* tokens, const int32_t* limit,
                                  int B, int off, int add, unsigned limit_err, hipStream_t s) {
  const mtp_config& c = h->cfg;
  const mtp_weights& w = h->w;
  const Layout& L = h->L;
  const int H = c.hidden, kvd = c.n_kv_heads * c.head_dim;
  const int R = B * per;
  unsigned* err = h->at<unsigned>(L.err);
  float* hrows = h->at<float>(L.cu_h);
  float* xrows = h->at<float>(L.cu_x);
  float* kvrows = h->at<float>(L.cu_kv);
  hipError_t e = hipSuccess;
  // without the tiled contraction, groups stay within the weight-streaming one's 64 rows
  const int group = h->gm_ok || L.cu_rows <= kMmMaxBatch ? L.cu_rows : kMmMaxBatch;
  for (int r0 = 0; r0 < R && e == hipSuccess; r0 += group) {
    const int rows = R - r0 < group ? R - r0 : group;
    e = launch_gather_rows(c.dtype, src, hrows, r0, rows, per, src_per, H, s);
    if (e != hipSuccess) break;
    if (mm_eligible(c) && rows >= kMmMinBatch) {
      uint16_t* q = h->at<uint16_t>(L.cu_q);
      uint16_t* qlo = h->at<uint16_t>(L.cu_q_lo);
      float* part = h->at<float>(L.cu_part);
      const bool tiled = rows > kMmMaxBatch;  // (group > 64 implies gm_ok)
      const int bp = tiled ? rows : mm_batch_pad(rows);
      RedParams r{};
      r.n = H; r.gain = static_cast<const uint16_t*>(w.g_h);
      r.gain2 = static_cast<const uint16_t*>(w.g_e); r.eps = c.rms_eps;
      r.xq = q; r.xq_lo = qlo; r.ldq = L.cu_ld; r.h = hrows;
      r.embed = static_cast<const uint16_t*>(w.embed);
      r.tok = tokens + r0; r.tok_stride = 1; r.vocab = c.vocab; r.err = err;
      if ((e = launch_red(PREP_EH, r, rows, s)) != hipSuccess) break;
      // packed: the matrix's rows in the handle's packed copy (or null: read w0/w1)
      auto mm = [&](const void* w0, const void* w1, int seg1, int N, int Kd,
                    const uint16_t* packed, int* ns) {
        if (tiled) {
          GmParams g{};
          g.w0 = w0; g.w1 = w1; g.seg1 = seg1; g.nrows = N; g.ncols = Kd;
          g.x = q; g.x_lo = qlo; g.ldx = L.cu_ld; g.B = rows;
          g.nsplit = gm_split(N, Kd, rows, h->num_cu, (long)L.cu_part_elems);
          g.part = part; g.bp = rows;
          *ns = g.nsplit;
          return launch_gm(EPI_STORE, g, s);
        }
        MmParams m{};
        m.w0 = w0; m.w1 = w1; m.w2 = w1; m.seg1 = seg1; m.seg2 = N;
        m.nrows = N; m.ncols = Kd; m.x = q; m.x_lo = qlo; m.ldx = L.cu_ld; m.B = rows;
        const MmPlan pl = mm_plan(EPI_STORE, N, Kd, rows, packed != nullptr, h->num_cu);
        m.tile_rows = pl.tile_rows;
        m.nsplit = pl.nsplit;
        m.part = part;
        m.dummy = h->ws + L.dummy;
        m.packed = packed;
        *ns = m.nsplit;
        return launch_mm(EPI_STORE, m, pl.grid, s);
      };
      // The K/V rows of the packed [W_q; W_k; W_v] copy start at a whole 128-row tile
      // when n_q * d is a multiple of 128; the packed copy is tile-major.
      const int qd = c.n_q_heads * c.head_dim;
      const uint16_t* pk_kv =
          L.pk_qkv && qd % 128 == 0
              ? h->at<uint16_t>(L.pk_qkv) + (size_t)(qd / 128) * mm_packed_elems(128, H)
              : nullptr;
      int ns = 1;
      if ((e = mm(w.w_eh, w.w_eh, H, H, 2 * H, L.pk_eh ? h->at<uint16_t>(L.pk_eh) : nullptr,
                  &ns)) != hipSuccess)
        break;
      r = RedParams{};
      r.part = part; r.nsplit = ns; r.bp = bp; r.n_part = H; r.n = H;
      r.out = xrows; r.gain = static_cast<const uint16_t*>(w.g_attn); r.eps = c.rms_eps;
      r.xq = q; r.xq_lo = qlo; r.ldq = L.cu_ld;
      if ((e = launch_red(RED_EH, r, rows, s)) != hipSuccess) break;
      if ((e = mm(w.w_k, w.w_v, kvd, 2 * kvd, H, pk_kv, &ns)) != hipSuccess) break;
      r = RedParams{};
      r.part = part; r.nsplit = ns; r.bp = bp; r.n_part = 2 * kvd; r.n = 2 * kvd;
      r.out = kvrows; r.ldq = L.cu_ld;
      if ((e = launch_red(RED_QKV, r, rows, s)) != hipSuccess) break;
    } else {
      GemvParams g{};
      g.w0 = g.w1 = g.w2 = w.w_eh;
      g.nrows = g.seg1 = g.seg2 = H;
      g.ncols = 2 * H; g.B = rows;
      g.gain = w.g_h; g.gain2 = w.g_e; g.eps = c.rms_eps;
      g.h = hrows; g.h_is_f32 = 1; g.ldh = H;
      g.embed = w.embed; g.tok = tokens + r0; g.tok_stride = 1; g.vocab = c.vocab;
      g.err = err; g.out = xrows; g.ldo = H;
      if ((e = run_gemv(h, PRO_EH, EPI_STORE, g, s)) != hipSuccess) break;
      g = GemvParams{};
      g.w0 = w.w_k; g.w1 = w.w_v; g.w2 = w.w_v;
      g.seg1 = kvd; g.seg2 = 2 * kvd; g.nrows = 2 * kvd;
      g.ncols = H; g.B = rows;
      g.x = xrows; g.ldx = H; g.gain = w.g_attn; g.eps = c.rms_eps;
      g.out = kvrows; g.ldo = 2 * kvd;
      if ((e = run_gemv(h, PRO_RMS, EPI_STORE, g, s)) != hipSuccess) break;
    }
    CatchupParams cp{};
    cp.kvrows = kvrows; cp.ld = 2 * kvd; cp.kc = kv->k; cp.vc = kv->v;
    cp.n_kv = c.n_kv_heads; cp.d = c.head_dim; cp.capacity = kv->capacity;
    cp.len = kv->len; cp.pos = kv->pos; cp.limit = limit;
    cp.per = per; cp.off = off; cp.r0 = r0; cp.rows = rows; cp.theta = c.rope_theta;
    cp.err = err;
    e = launch_catchup_write(c.dtype, cp, s);
  }
  if (e == hipSuccess)
    e = launch_catchup_commit(kv->len, kv->pos, limit, B, per, add, limit_err, err, s);
  return e;
}

extern "C" {

mtp_status mtp_kv_catchup(mtp_handle* h, mtp_kv* kv, const void* target_hidden,
                          const int32_t* draft_tokens, const int32_t* accepted_len, int32_t B,
                          int32_t K, void* stream) {
  if (!h || !target_hidden || !draft_tokens || !accepted_len) return MTP_ERR_INVALID_ARG;
  if (!aligned(target_hidden, 16)) return MTP_ERR_INVALID_ARG;
  if (K < 1 || B < 1) return MTP_ERR_SHAPE;
  if (K > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  mtp_status st = check_kv(h, kv, B);
  if (st != MTP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // committed pair j = r % K + 1 of sequence b: hidden row j - 1 of K + 1, token d_j, slot
  // len - K + j; len / pos then move by a + 1 - K
  return timed(h, KC_ROLLBACK, s, [&] {
           return input_side_pass(h, kv, target_hidden, K, K + 1, draft_tokens, accepted_len, B,
                                  1 - K, 1 - K, MTP_DEVERR_ACCEPT, s);
         }) == hipSuccess
             ? MTP_OK
             : MTP_ERR_HIP;
}

mtp_status mtp_kv_prefill(mtp_handle* h, mtp_kv* kv, const void* target_hidden,
                          const int32_t* tokens, const int32_t* n_valid, int32_t B, int32_t n,
                          void* stream) {
  if (!h) return MTP_ERR_INVALID_ARG;
  if (n < 0 || B < 1) return MTP_ERR_SHAPE;
  if (B > h->max_batch) return MTP_ERR_CAPACITY;
  mtp_status st = check_kv(h, kv, B);
  if (st != MTP_OK) return st;
  if (n > kv->capacity) return MTP_ERR_CAPACITY;
  if (n == 0) return MTP_OK;  // nothing to read: the row pointers may be null
  if (!target_hidden || !tokens) return MTP_ERR_INVALID_ARG;
  if (!aligned(target_hidden, 16)) return MTP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(h, KC_ROLLBACK, s, [&] {
           return input_side_pass(h, kv, target_hidden, n, n, tokens, n_valid, B, 0, 0,
                                  MTP_DEVERR_COUNT, s);
         }) == hipSuccess
             ? MTP_OK
             : MTP_ERR_HIP;
}

mtp_status mtp_kv_rollback(mtp_handle* h, mtp_kv* kv, const int32_t* accepted_len, int32_t B,
                           int32_t K, void* stream) {
  if (!h || !accepted_len) return MTP_ERR_INVALID_ARG;
  if (K < 0 || B < 1) return MTP_ERR_SHAPE;
  if (K > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  mtp_status st = check_kv(h, kv, B);
  if (st != MTP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(h, KC_ROLLBACK, s, [&] {
           return launch_rollback(kv->len, kv->pos, accepted_len, nullptr, B, K,
                                  h->at<unsigned>(h->L.err), s);
         }) == hipSuccess
             ? MTP_OK
             : MTP_ERR_HIP;
}

mtp_status mtp_draft_seqk(mtp_handle* h, const void* hidden, const int32_t* last_tokens,
                          mtp_kv* kv, const int32_t* k_seq, int32_t B, int32_t K_max,
                          int32_t* draft_tokens, void* stream) {
  if (!h || (K_max > 0 && !k_seq)) return MTP_ERR_INVALID_ARG;
  return draft_impl(h, hidden, last_tokens, kv, B, K_max, draft_tokens, nullptr, nullptr,
                    LmOut{nullptr, 0, 0, nullptr}, stream, k_seq);
}

mtp_status mtp_verify_seqk(mtp_handle* h, const float* target_logits, const int32_t* draft_tokens,
                           const int32_t* k_seq, int32_t B, int32_t K_max, int32_t* accepted_len,
                           int32_t* next_token, void* stream) {
  if (!h || !target_logits || !k_seq || !accepted_len || !next_token) return MTP_ERR_INVALID_ARG;
  if (K_max < 0 || B < 1) return MTP_ERR_SHAPE;
  if (K_max > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  if (K_max > 0 && !draft_tokens) return MTP_ERR_INVALID_ARG;
  VerifyParams p{};
  p.logits = target_logits;
  p.draft = draft_tokens;
  p.K = K_max;
  p.V = h->cfg.vocab;
  p.keys = h->at<unsigned long long>(h->L.v_keys);
  p.kstride = h->L.v_kstride;
  p.counters = h->at<unsigned>(h->L.v_cnt);
  p.accepted = accepted_len;
  p.next = next_token;
  p.kseq = k_seq;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(h, KC_VERIFY, s, [&] { return launch_verify(p, B, s); }) == hipSuccess ? MTP_OK
                                                                                      : MTP_ERR_HIP;
}

mtp_status mtp_kv_rollback_seqk(mtp_handle* h, mtp_kv* kv, const int32_t* accepted_len,
                                const int32_t* k_seq, int32_t B, int32_t K_max, void* stream) {
  if (!h || !accepted_len || !k_seq) return MTP_ERR_INVALID_ARG;
  if (K_max < 0 || B < 1) return MTP_ERR_SHAPE;
  if (K_max > h->max_k || B > h->max_batch) return MTP_ERR_CAPACITY;
  mtp_status st = check_kv(h, kv, B);
  if (st != MTP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(h, KC_ROLLBACK, s, [&] {
           return launch_rollback(kv->len, kv->pos, accepted_len, k_seq, B, K_max,
                                  h->at<unsigned>(h->L.err), s);
         }) == hipSuccess
             ? MTP_OK
             : MTP_ERR_HIP;
}

mtp_status mtp_adapt_k_seq(const int32_t* accepted_hist, const int32_t* k_hist, int32_t W,
                           int32_t B, int32_t k_min, int32_t k_max, int32_t* k_next) {
  if (!accepted_hist || !k_hist || !k_next) return MTP_ERR_INVALID_ARG;
  if (W < 1 || B < 1 || k_min < 0 || k_max < k_min || k_max > kMaxK) return MTP_ERR_SHAPE;
  for (long i = 0; i < (long)W * B; ++i)
    if (k_hist[i] < 0 || k_hist[i] > kMaxK || accepted_hist[i] < 0 ||
        accepted_hist[i] > k_hist[i])
      return MTP_ERR_INVALID_ARG;
  for (int b = 0; b < B; ++b) {
    long sum = 0;
    for (int i = 0; i < W; ++i) {
      const int a = accepted_hist[(long)i * B + b], k = k_hist[(long)i * B + b];
      sum += a >= k ? k + 1 : a + 1;
    }
    const long want = (sum + W - 1) / W;  // mean of the requests, rounded up
    k_next[b] = (int32_t)(want < k_min ? k_min : want > k_max ? k_max : want);
  }
  return MTP_OK;
}

mtp_status mtp_get_error(mtp_handle* h, void* stream, uint32_t* bits) {
  if (!h) return MTP_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Only the caller's stream is waited for: the error word is written by work on it.
  unsigned v = 0;
  unsigned* dev = h->at<unsigned>(h->L.err);
  if (hipMemcpyAsync(&v, dev, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
    return MTP_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MTP_ERR_HIP;
  if (v) {
    if (hipMemsetAsync(dev, 0, sizeof(v), s) != hipSuccess) return MTP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MTP_ERR_HIP;
  }
  if (bits) *bits = v;
  return v ? MTP_ERR_DEVICE : MTP_OK;
}

mtp_status mtp_get_info(const mtp_handle* h, mtp_info* out) {
  if (!h || !out) return MTP_ERR_INVALID_ARG;
  const Layout& L = h->L;
  mtp_info i{};
  i.workspace_bytes = L.total;
  if (L.pk_lm) {
    const mtp_config& c = h->cfg;
    const int H = c.hidden, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    i.packed_weight_bytes =
        2 * (mm_packed_elems(H, 2 * H) + mm_packed_elems(qd + 2 * kvd, H) +
             mm_packed_elems(H, qd) + mm_packed_elems(2 * c.ffn, H) +
             mm_packed_elems(H, c.ffn) + mm_packed_elems(c.vocab, H));
  }
  i.verify_hidden_group_rows =
      h->gm_ok || L.pk_lm || L.vh_rows <= kMmMaxBatch ? L.vh_rows : kMmMaxBatch;
  i.catchup_group_rows = L.cu_rows;
  i.matrix_core_min_batch = mm_eligible(h->cfg) ? kMmMinBatch : 0;
  i.matrix_core_max_batch = mm_eligible(h->cfg) ? kMmMaxBatch : 0;
  *out = i;
  return MTP_OK;
}

}  // extern "C"
