// C ABI of the MTLA hot path: host-side argument checks, workspace layout and
// the launch sequence of each entry point.  Declarations and their contracts
// are in include/mtla.h.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/mtla.h"
#include "kernels.h"

namespace {

thread_local char g_detail[512] = "";

mtla_status fail(mtla_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return st;
}

mtla_status ok() {
  g_detail[0] = '\0';
  return MTLA_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int esize(const mtla_dims *d) { return d->dtype == MTLA_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

float eff_scale(const mtla_dims *d) {
  return d->scale > 0.0f ? d->scale : 1.0f / sqrtf((float)d->d_h);
}

mtla_status check_dims(const mtla_dims *d) {
  if (!d) return fail(MTLA_ERR_ARG, "dims is null");
  if (d->dtype != MTLA_F32 && d->dtype != MTLA_BF16) return fail(MTLA_ERR_ARG, "dtype %d", d->dtype);
  if (d->d <= 0 || d->H <= 0 || d->d_h <= 0 || d->r <= 0 || d->d_hR <= 0)
    return fail(MTLA_ERR_ARG, "non-positive dimension (d=%d H=%d d_h=%d r=%d d_hR=%d)", d->d, d->H,
                d->d_h, d->r, d->d_hR);
  if (d->s < 1) return fail(MTLA_ERR_ARG, "stride s=%d < 1", d->s);
  if (!(d->scale >= 0.0f) || isinf(d->scale)) return fail(MTLA_ERR_ARG, "scale must be finite and >= 0");
  if (d->d % 32 != 0) return fail(MTLA_ERR_UNSUPPORTED, "d=%d is not a multiple of 32", d->d);
  if (!((d->r == 256 && d->d_hR == 32) || (d->r == 512 && d->d_hR == 64)))
    return fail(MTLA_ERR_UNSUPPORTED, "(r, d_hR) = (%d, %d) not in {(256,32), (512,64)}", d->r,
                d->d_hR);
  if (d->H > 64) return fail(MTLA_ERR_UNSUPPORTED, "H=%d > 64", d->H);
  if (d->r == 512 && d->H > 32) return fail(MTLA_ERR_UNSUPPORTED, "H=%d > 32 with r=512", d->H);
  return MTLA_OK;
}

#define CHECK_PTR(p)                                                     \
  do {                                                                   \
    if (!(p)) return fail(MTLA_ERR_ARG, "%s is null", #p);               \
    if (!aligned16(p)) return fail(MTLA_ERR_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

mtla_status check_weights(const mtla_weights *w, bool need_attn) {
  if (!w) return fail(MTLA_ERR_ARG, "weights is null");
  CHECK_PTR(w->W_dkv);
  CHECK_PTR(w->W_gate);
  CHECK_PTR(w->b_hc);
  CHECK_PTR(w->gate_pos);
  if (w->gate_pos_rows <= 0) return fail(MTLA_ERR_ARG, "gate_pos_rows=%d", w->gate_pos_rows);
  if (need_attn) {
    CHECK_PTR(w->A);
    CHECK_PTR(w->Bvo);
  }
  return MTLA_OK;
}

mtla_status check_cache(const mtla_dims *d, const mtla_cache *c) {
  if (!c) return fail(MTLA_ERR_ARG, "cache is null");
  CHECK_PTR(c->slots);
  if (c->max_slots <= 0) return fail(MTLA_ERR_ARG, "max_slots=%d", c->max_slots);
  const int64_t row = d->r + d->d_hR;
  if (c->batch_stride < (int64_t)c->max_slots * row)
    return fail(MTLA_ERR_ARG, "batch_stride %lld < max_slots*(r+d_hR)", (long long)c->batch_stride);
  if ((c->batch_stride * esize(d)) % 16 != 0)
    return fail(MTLA_ERR_ARG, "batch_stride is not a multiple of 16 bytes");
  return MTLA_OK;
}

mtla_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MTLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MTLA_OK;
}

#define LAUNCH(expr, what)                              \
  do {                                                  \
    mtla_status st_ = launched((expr), what);           \
    if (st_ != MTLA_OK) return st_;                     \
  } while (0)

struct DecodeWs {
  size_t status, cg, qt, part_o, part_ml, o, ypart, counters, total;
  int ncount;   // ints cleared at the start of a call: the status word and the counters
};

// Workspace of one decoding step (plan != nullptr) or of a merge-append.  The
// int32 status word (dropped frames of the last call) sits at byte 0 and the
// split counters right after it, so one clear covers both.
DecodeWs decode_ws(const mtla_dims *d, int B, const mtla::DecodePlan *plan) {
  DecodeWs w;
  const size_t e = esize(d), r = d->r, HR = (size_t)d->H * d->r;
  const int nctr = plan ? B + mtla::out_proj_counters((int)e, B, d->d, (int)HR) : 0;
  size_t off = 0;
  w.status = off;
  w.counters = off + 4;
  w.ncount = 1 + nctr;
  off += align_up((size_t)w.ncount * 4);
  w.cg = off; off += align_up(B * 2 * r * 4);
  w.qt = w.part_o = w.part_ml = w.o = w.ypart = 0;
  if (plan) {
    w.qt = off;       off += align_up(B * HR * e);
    w.part_o = off;   off += align_up((size_t)plan->nparts * HR * 4);
    w.part_ml = off;  off += align_up((size_t)plan->nparts * d->H * 2 * 4);
    w.o = off;        off += align_up(B * HR * e);
    w.ypart = off;    off += align_up(mtla::out_proj_part_bytes((int)e, B, d->d, (int)HR));
  }
  w.total = off;
  return w;
}

struct PrefillWs {
  size_t cg, Cp, keys, qt, O, total;
  int64_t keys_stride;
};

PrefillWs prefill_ws(const mtla_dims *d, int B, int T) {
  PrefillWs w;
  const size_t e = esize(d), r = d->r, HR = (size_t)d->H * d->r, M = (size_t)B * T;
  const int64_t nS = (T + d->s - 1) / d->s;
  w.keys_stride = nS * (d->r + d->d_hR);
  size_t off = 0;
  w.cg = off;    off += align_up(M * 2 * r * 4);
  w.Cp = off;    off += align_up(M * r * e);
  w.keys = off;  off += align_up((size_t)B * w.keys_stride * e);
  w.qt = off;    off += align_up(M * HR * e);
  w.O = off;     off += align_up(M * HR * e);
  w.total = off;
  return w;
}

// Workspace of the per-head (unabsorbed) parallel form.
struct HeadsWs {
  size_t cg, Cp, keys, q, KV, O, total;
  int64_t keys_stride;
};

HeadsWs heads_ws(const mtla_dims *d, int B, int T) {
  HeadsWs w;
  const size_t e = esize(d), r = d->r, HD = (size_t)d->H * d->d_h, M = (size_t)B * T;
  const int64_t nS = (T + d->s - 1) / d->s;
  w.keys_stride = nS * (d->r + d->d_hR);
  size_t off = 0;
  w.cg = off;    off += align_up(M * 2 * r * 4);
  w.Cp = off;    off += align_up(M * r * e);
  w.keys = off;  off += align_up((size_t)B * w.keys_stride * e);
  w.q = off;     off += align_up(M * HD * e);
  w.KV = off;    off += align_up(M * 2 * HD * e);
  w.O = off;     off += align_up(M * HD * e);
  w.total = off;
  return w;
}

// Workspace of the backward of the per-head form: the forward's buffers, the
// transposed weights, and the backward's intermediate gradients.
struct BwdWs {
  HeadsWs f;
  // Wc = [W_Q^T | W_dkv^T] and dQc = [dQ | dc] side by side (row stride
  // H d_h + r), so that dX = dQ W_Q + dc W_dkv is one product.
  size_t O_, lse, WOt, WKVt, Whct, Wc, dO, D, dKVc, dKRc, dKV, dKRh, dQc, dCp, da32, dab, dc32, cb,
      dPpart, red_part, red_ctr, total;
  int nctr;   // ints at red_ctr: counters of the bias column sums (zero between uses)
};

BwdWs bwd_ws(const mtla_dims *d, int B, int T) {
  BwdWs w;
  w.f = heads_ws(d, B, T);
  const size_t e = esize(d), r = d->r, HD = (size_t)d->H * d->d_h, M = (size_t)B * T;
  const size_t nS = (T + d->s - 1) / d->s, dd = d->d, H = d->H, dR = d->d_hR;
  size_t off = w.f.total;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
  w.O_ = w.f.O;
  w.lse = take(M * H * 4);
  w.WOt = take(HD * dd * e);
  w.WKVt = take(r * 2 * HD * e);
  w.Whct = take(r * r * e);
  w.Wc = take(dd * (HD + r) * e);
  w.dO = take(M * HD * e);
  w.D = take(M * H * 4);
  w.dKVc = take((size_t)B * nS * 2 * HD * 4);
  w.dKRc = take((size_t)B * nS * H * dR * 4);
  w.dKV = take(M * 2 * HD * e);
  w.dKRh = take(M * H * dR * 4);
  w.dQc = take(M * (HD + r) * e);
  w.dCp = take(M * r * 4);
  w.da32 = take(M * r * 4);
  w.dab = take(M * r * e);
  w.dc32 = take(M * r * 4);
  w.cb = take(M * r * e);
  w.dPpart = take((size_t)B * nS * r * 4);
  // Partials of the ordered reductions (weight-gradient products and the
  // bias column sums run one after another and share one buffer).
  const int Mi = (int)M, HDi = (int)HD, ri = (int)r, di = (int)dd;
  const size_t tp[6] = {mtla::tn_gemm_part_bytes(Mi, di, HDi), mtla::tn_gemm_part_bytes(Mi, HDi, di),
                        mtla::tn_gemm_part_bytes(Mi, HDi, ri), mtla::tn_gemm_part_bytes(Mi, HDi, ri),
                        mtla::tn_gemm_part_bytes(Mi, ri, ri), mtla::tn_gemm_part_bytes(Mi, ri, di)};
  size_t pmax = mtla::colsum_part_bytes(Mi, ri);
  for (int i = 0; i < 6; ++i)
    if (tp[i] > pmax) pmax = tp[i];
  w.red_part = take(pmax);
  w.nctr = mtla::colsum_counters(ri);
  w.red_ctr = take((size_t)w.nctr * 4);
  w.total = off;
  return w;
}

// Workspace of the rotary inputs of M frames: [M, (H + 1) d_hR] fp32.
size_t rope_ws(const mtla_dims *d, int M) {
  return align_up((size_t)M * (d->H + 1) * d->d_hR * 4);
}

// Workspace of a chunked merge-append of L frames: cg [B*L, 2r] fp32.
size_t chunk_ws(const mtla_dims *d, int B, int L) {
  return align_up((size_t)B * L * 2 * d->r * 4);
}

mtla_status check_positions(const mtla_dims *d, const mtla_weights *w, const mtla_cache *c, int B,
                            int max_pos) {
  if (B < 1 || B > 65535) return fail(MTLA_ERR_ARG, "B=%d outside [1, 65535]", B);
  if (max_pos < 0) return fail(MTLA_ERR_ARG, "max_pos=%d < 0", max_pos);
  const int jmax = max_pos / d->s;
  if (jmax >= c->max_slots)
    return fail(MTLA_ERR_CAPACITY, "slot %d (max_pos %d) >= max_slots %d", jmax, max_pos,
                c->max_slots);
  if (jmax >= w->gate_pos_rows)
    return fail(MTLA_ERR_CAPACITY, "slot %d (max_pos %d) >= gate_pos_rows %d", jmax, max_pos,
                w->gate_pos_rows);
  return MTLA_OK;
}

}  // namespace

// Device scratch of mtla_decode_step_noalloc: a file-scope array, so that the
// entry point allocates nothing.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is only a
// stand-in: its device address (per device) comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev` (the current device), looked up
// once per device.
mtla_status scratch_for(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MTLA_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(MTLA_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MTLA_OK;
}

}  // namespace

extern "C" {

const char *mtla_status_string(mtla_status s) {
  switch (s) {
    case MTLA_OK: return "ok";
    case MTLA_ERR_ARG: return "invalid argument";
    case MTLA_ERR_CAPACITY: return "position exceeds cache or gate-table capacity";
    case MTLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MTLA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char *mtla_last_error_detail(void) { return g_detail; }

size_t mtla_workspace_bytes(const mtla_dims *dims, int32_t op, int32_t B, int32_t T_or_max_pos) {
  if (check_dims(dims) != MTLA_OK || B < 1 || T_or_max_pos < 0) return 0;
  if (op == 0) return decode_ws(dims, B, nullptr).total;
  if (op == 1) {
    mtla::DecodePlan plan;
    if (!mtla::decode_plan(dims->dtype, dims->H, dims->r, dims->d_hR, dims->s, B, T_or_max_pos, &plan))
      return 0;
    return decode_ws(dims, B, &plan).total;
  }
  if (op == 2) {
    if (T_or_max_pos < 1) return 0;
    return prefill_ws(dims, B, T_or_max_pos).total;
  }
  if (op == 3) return chunk_ws(dims, B, T_or_max_pos);
  if (op == 4) {
    if (T_or_max_pos < 1) return 0;
    return heads_ws(dims, B, T_or_max_pos).total;
  }
  if (op == 6) return rope_ws(dims, B * T_or_max_pos);
  if (op == 5) {
    if (T_or_max_pos < 1) return 0;
    return bwd_ws(dims, B, T_or_max_pos).total;
  }
  return 0;
}

mtla_status mtla_gate_pos_table(const mtla_dims *dims, const void *pe, int32_t rows, int32_t d_pe,
                                const void *W_hp, const void *b_hp, float *table, void *stream) {
  if (!dims) return fail(MTLA_ERR_ARG, "dims is null");
  if (dims->dtype != MTLA_F32 && dims->dtype != MTLA_BF16) return fail(MTLA_ERR_ARG, "dtype");
  if (dims->r <= 0 || rows <= 0 || d_pe <= 0) return fail(MTLA_ERR_ARG, "r, rows and d_pe must be > 0");
  if (d_pe % 32 != 0) return fail(MTLA_ERR_UNSUPPORTED, "d_pe=%d is not a multiple of 32", d_pe);
  CHECK_PTR(pe);
  CHECK_PTR(W_hp);
  CHECK_PTR(b_hp);
  CHECK_PTR(table);
  LAUNCH(mtla::launch_pos_table(dims->dtype, pe, rows, d_pe, W_hp, b_hp, dims->r, table,
                                (hipStream_t)stream),
         "gate position table");
  return ok();
}

mtla_status mtla_gate_content_map(const mtla_dims *dims, const void *W_hc, const void *W_dkv,
                                  void *W_gate, void *stream) {
  if (!dims) return fail(MTLA_ERR_ARG, "dims is null");
  if (dims->dtype != MTLA_F32 && dims->dtype != MTLA_BF16) return fail(MTLA_ERR_ARG, "dtype");
  if (dims->r <= 0 || dims->d <= 0) return fail(MTLA_ERR_ARG, "r and d must be > 0");
  CHECK_PTR(W_hc);
  CHECK_PTR(W_dkv);
  CHECK_PTR(W_gate);
  LAUNCH(mtla::launch_gate_map(dims->dtype, W_hc, W_dkv, dims->r, dims->d, W_gate,
                               (hipStream_t)stream),
         "gate content map");
  return ok();
}

mtla_status mtla_rope_inputs(const mtla_dims *dims, const void *W_QR, const void *W_KR,
                             const void *X, const int32_t *pos, int32_t M, float base, void *QR,
                             void *KR, void *workspace, size_t ws_bytes, void *stream) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  CHECK_PTR(W_QR);
  CHECK_PTR(W_KR);
  CHECK_PTR(X);
  CHECK_PTR(pos);
  CHECK_PTR(QR);
  CHECK_PTR(KR);
  CHECK_PTR(workspace);
  if (M < 1) return fail(MTLA_ERR_ARG, "M=%d < 1", M);
  if (!(base > 1.0f) || isinf(base)) return fail(MTLA_ERR_ARG, "base must be finite and > 1");
  if (dims->d_hR % 2 != 0) return fail(MTLA_ERR_ARG, "d_hR=%d is odd", dims->d_hR);
  const int N = dims->H * dims->d_hR + dims->d_hR;
  if ((int64_t)M * N > 0x7fffffffLL) return fail(MTLA_ERR_UNSUPPORTED, "M too large");
  const size_t need = rope_ws(dims, M);
  if (ws_bytes < need) return fail(MTLA_ERR_ARG, "workspace %zu < %zu bytes", ws_bytes, need);
  LAUNCH(mtla::launch_rope_inputs(dims->dtype, X, M, dims->d, W_QR, dims->H * dims->d_hR, W_KR,
                                  dims->d_hR, pos, base, (float *)workspace, QR, KR,
                                  (hipStream_t)stream),
         "rotary inputs");
  return ok();
}

mtla_status mtla_merge_append(const mtla_dims *dims, const mtla_weights *w, const mtla_cache *cache,
                              const void *X_t, const void *KR_t, const int32_t *pos, int32_t B,
                              int32_t max_pos, void *workspace, size_t ws_bytes, void *stream) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  if ((st = check_weights(w, false)) != MTLA_OK) return st;
  if ((st = check_cache(dims, cache)) != MTLA_OK) return st;
  CHECK_PTR(X_t);
  CHECK_PTR(KR_t);
  CHECK_PTR(pos);
  CHECK_PTR(workspace);
  if ((st = check_positions(dims, w, cache, B, max_pos)) != MTLA_OK) return st;
  const DecodeWs ws = decode_ws(dims, B, nullptr);
  if (ws_bytes < ws.total) return fail(MTLA_ERR_ARG, "workspace %zu < %zu bytes", ws_bytes, ws.total);
  hipStream_t s = (hipStream_t)stream;
  float *cg = (float *)((char *)workspace + ws.cg);
  int *status = (int *)((char *)workspace + ws.status);
  LAUNCH(mtla::launch_proj(dims->dtype, X_t, B, dims->d, w->W_dkv, w->W_gate, dims->r, nullptr, 0,
                           cg, nullptr, status, ws.ncount, s),
         "latent and gate projection");
  LAUNCH(mtla::launch_merge(dims->dtype, B, dims->r, dims->d_hR, dims->s, pos, max_pos, cg,
                            w->b_hc, w->gate_pos, KR_t, cache->slots, cache->batch_stride, status,
                            s),
         "merge");
  return ok();
}

mtla_status mtla_append_chunk(const mtla_dims *dims, const mtla_weights *w, const mtla_cache *cache,
                              const void *X, const void *KR, const int32_t *pos0,
                              const int32_t *lens, int32_t B, int32_t L, int32_t max_pos,
                              void *Cprime_out, void *workspace, size_t ws_bytes, void *stream) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  if ((st = check_weights(w, false)) != MTLA_OK) return st;
  if ((st = check_cache(dims, cache)) != MTLA_OK) return st;
  CHECK_PTR(pos0);
  if (lens && !aligned16(lens)) return fail(MTLA_ERR_ARG, "lens is not 16-byte aligned");
  if (Cprime_out && !aligned16(Cprime_out)) return fail(MTLA_ERR_ARG, "Cprime_out is not 16-byte aligned");
  if (L < 0) return fail(MTLA_ERR_ARG, "L=%d < 0", L);
  if (B < 1 || B > 65535) return fail(MTLA_ERR_ARG, "B=%d outside [1, 65535]", B);
  if (L == 0) return ok();   // nothing is read: X, KR and the workspace may be null
  CHECK_PTR(X);
  CHECK_PTR(KR);
  CHECK_PTR(workspace);
  if ((int64_t)B * L > 0x7fffffffLL / 4) return fail(MTLA_ERR_UNSUPPORTED, "B*L too large");
  if ((st = check_positions(dims, w, cache, B, max_pos)) != MTLA_OK) return st;
  const size_t need = chunk_ws(dims, B, L);
  if (ws_bytes < need) return fail(MTLA_ERR_ARG, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  float *cg = (float *)workspace;
  const int jlim = cache->max_slots < w->gate_pos_rows ? cache->max_slots : w->gate_pos_rows;
  LAUNCH(mtla::launch_proj(dims->dtype, X, B * L, dims->d, w->W_dkv, w->W_gate, dims->r, nullptr,
                           0, cg, nullptr, nullptr, 0, s),
         "latent and gate projection");
  LAUNCH(mtla::launch_chunk_merge(dims->dtype, B, L, dims->r, dims->d_hR, dims->s, pos0, lens, cg,
                                  w->b_hc, w->gate_pos, jlim, KR, Cprime_out, cache->slots,
                                  cache->batch_stride, s),
         "chunked merge");
  return ok();
}

}  // extern "C"

namespace {

hipEvent_t ev0(void *const *events) { return events ? (hipEvent_t)events[0] : nullptr; }
hipEvent_t ev1(void *const *events) { return events ? (hipEvent_t)events[1] : nullptr; }


mtla_status decode_step_impl(const mtla_dims *dims, const mtla_weights *w, const mtla_cache *cache,
                             const void *X_t, const void *QR_t, const void *KR_t, const int32_t *pos,
                             int32_t B, int32_t max_pos, void *Y, void *workspace, size_t ws_bytes,
                             void *stream, void *const *events) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  if ((st = check_weights(w, true)) != MTLA_OK) return st;
  if ((st = check_cache(dims, cache)) != MTLA_OK) return st;
  CHECK_PTR(X_t);
  CHECK_PTR(QR_t);
  CHECK_PTR(KR_t);
  CHECK_PTR(pos);
  CHECK_PTR(Y);
  CHECK_PTR(workspace);
  if ((st = check_positions(dims, w, cache, B, max_pos)) != MTLA_OK) return st;
  mtla::DecodePlan plan;
  if (!mtla::decode_plan(dims->dtype, dims->H, dims->r, dims->d_hR, dims->s, B, max_pos, &plan))
    return fail(MTLA_ERR_UNSUPPORTED, "no decode plan for this shape");
  const DecodeWs ws = decode_ws(dims, B, &plan);
  if (ws_bytes < ws.total) return fail(MTLA_ERR_ARG, "workspace %zu < %zu bytes", ws_bytes, ws.total);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)workspace;
  float *cg = (float *)(base + ws.cg);
  void *qt = base + ws.qt, *o = base + ws.o;
  float *part_o = (float *)(base + ws.part_o), *part_ml = (float *)(base + ws.part_ml);
  float *ypart = (float *)(base + ws.ypart);
  int *status = (int *)(base + ws.status), *counters = (int *)(base + ws.counters);
  const int HR = dims->H * dims->r;
  LAUNCH(mtla::launch_proj(dims->dtype, X_t, B, dims->d, w->W_dkv, w->W_gate, dims->r, w->A, HR, cg,
                           qt, status, ws.ncount, s),
         "latent, gate and query projection");
  LAUNCH(mtla::launch_decode_attention(dims->dtype, plan, B, dims->H, dims->r, dims->d_hR, dims->s,
                                       eff_scale(dims), pos, max_pos, cache->slots,
                                       cache->batch_stride, qt, QR_t, KR_t, cg, w->b_hc,
                                       w->gate_pos, part_o, part_ml, counters, status, o, s,
                                       ev0(events), ev1(events)),
         "merge and decode attention");
  LAUNCH(mtla::launch_out_proj(dims->dtype, o, B, HR, w->Bvo, dims->d, Y, ypart, counters + B, s),
         "output projection");
  return ok();
}

mtla_status prefill_impl(const mtla_dims *dims, const mtla_weights *w, const void *X,
                         const void *QR, const void *KR, int32_t B, int32_t T, void *Y,
                         const mtla_cache *cache_out, void *Cprime_out, void *workspace,
                         size_t ws_bytes, void *stream, void *const *events) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  if ((st = check_weights(w, true)) != MTLA_OK) return st;
  CHECK_PTR(X);
  CHECK_PTR(QR);
  CHECK_PTR(KR);
  CHECK_PTR(Y);
  CHECK_PTR(workspace);
  if (Cprime_out && !aligned16(Cprime_out)) return fail(MTLA_ERR_ARG, "Cprime_out is not 16-byte aligned");
  if (B < 1 || B > 65535) return fail(MTLA_ERR_ARG, "B=%d outside [1, 65535]", B);
  if (T < 1) return fail(MTLA_ERR_ARG, "T=%d < 1", T);
  if ((int64_t)B * T * dims->H > 0x7fffffffLL / 4)
    return fail(MTLA_ERR_UNSUPPORTED, "B*T*H too large");
  const int nS = (T + dims->s - 1) / dims->s;
  if ((T - 1) / dims->s >= w->gate_pos_rows)
    return fail(MTLA_ERR_CAPACITY, "slot %d >= gate_pos_rows %d", (T - 1) / dims->s, w->gate_pos_rows);
  if (cache_out) {
    if ((st = check_cache(dims, cache_out)) != MTLA_OK) return st;
    if (nS > cache_out->max_slots)
      return fail(MTLA_ERR_CAPACITY, "ceil(T/s)=%d > max_slots %d", nS, cache_out->max_slots);
  }
  if (!mtla::prefill_attention_supported(dims->dtype, dims->H, dims->r, dims->d_hR))
    return fail(MTLA_ERR_UNSUPPORTED, "no prefill kernel for this shape");
  const PrefillWs ws = prefill_ws(dims, B, T);
  if (ws_bytes < ws.total) return fail(MTLA_ERR_ARG, "workspace %zu < %zu bytes", ws_bytes, ws.total);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)workspace;
  float *cg = (float *)(base + ws.cg);
  void *keys = base + ws.keys, *qt = base + ws.qt, *O = base + ws.O;
  void *Cp = Cprime_out ? Cprime_out : (void *)(base + ws.Cp);
  const int M = B * T, HR = dims->H * dims->r;
  LAUNCH(mtla::launch_proj(dims->dtype, X, M, dims->d, w->W_dkv, w->W_gate, dims->r, w->A, HR, cg,
                           qt, nullptr, 0, s),
         "latent, gate and query projection");
  LAUNCH(mtla::launch_group_scan(dims->dtype, cg, w->b_hc, w->gate_pos, KR, B, T, dims->r,
                                 dims->d_hR, dims->s, Cp, keys, ws.keys_stride,
                                 cache_out ? cache_out->slots : nullptr,
                                 cache_out ? cache_out->batch_stride : 0, s),
         "gate and group scan");
  LAUNCH(mtla::launch_prefill_attention(dims->dtype, B, T, dims->H, dims->r, dims->d_hR, dims->s,
                                        eff_scale(dims), qt, QR, keys, ws.keys_stride, Cp, KR, O, s,
                                        ev0(events), ev1(events)),
         "strided attention");
  LAUNCH(mtla::launch_out_proj(dims->dtype, O, M, HR, w->Bvo, dims->d, Y, nullptr, nullptr, s),
         "output projection");
  return ok();
}

mtla_status prefill_unabsorbed_impl(const mtla_dims *dims, const mtla_unabsorbed_weights *w,
                                   const void *X, const void *QR, const void *KR, int32_t B,
                                   int32_t T, void *Y, const mtla_cache *cache_out,
                                   void *Cprime_out, void *workspace, size_t ws_bytes,
                                   void *stream, void *const *events) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  if (!w) return fail(MTLA_ERR_ARG, "weights is null");
  CHECK_PTR(w->W_dkv);
  CHECK_PTR(w->W_gate);
  CHECK_PTR(w->b_hc);
  CHECK_PTR(w->gate_pos);
  if (w->gate_pos_rows <= 0) return fail(MTLA_ERR_ARG, "gate_pos_rows=%d", w->gate_pos_rows);
  CHECK_PTR(w->W_Q);
  CHECK_PTR(w->W_K);
  CHECK_PTR(w->W_V);
  CHECK_PTR(w->W_O);
  CHECK_PTR(X);
  CHECK_PTR(QR);
  CHECK_PTR(KR);
  CHECK_PTR(Y);
  CHECK_PTR(workspace);
  if (Cprime_out && !aligned16(Cprime_out)) return fail(MTLA_ERR_ARG, "Cprime_out is not 16-byte aligned");
  if (B < 1 || B > 65535) return fail(MTLA_ERR_ARG, "B=%d outside [1, 65535]", B);
  if (T < 1) return fail(MTLA_ERR_ARG, "T=%d < 1", T);
  if ((int64_t)B * T * dims->H * dims->d_h > 0x7fffffffLL / 4)
    return fail(MTLA_ERR_UNSUPPORTED, "B*T*H*d_h too large");
  if (!mtla::heads_attention_supported(dims->dtype, dims->H, dims->d_h, dims->d_hR))
    return fail(MTLA_ERR_UNSUPPORTED, "per-head form needs (d_h, d_hR) = (64, 32) or (128, 64)");
  const int nS = (T + dims->s - 1) / dims->s;
  if ((T - 1) / dims->s >= w->gate_pos_rows)
    return fail(MTLA_ERR_CAPACITY, "slot %d >= gate_pos_rows %d", (T - 1) / dims->s, w->gate_pos_rows);
  if (cache_out) {
    if ((st = check_cache(dims, cache_out)) != MTLA_OK) return st;
    if (nS > cache_out->max_slots)
      return fail(MTLA_ERR_CAPACITY, "ceil(T/s)=%d > max_slots %d", nS, cache_out->max_slots);
  }
  const HeadsWs ws = heads_ws(dims, B, T);
  if (ws_bytes < ws.total) return fail(MTLA_ERR_ARG, "workspace %zu < %zu bytes", ws_bytes, ws.total);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)workspace;
  float *cg = (float *)(base + ws.cg);
  void *keys = base + ws.keys, *q = base + ws.q, *KV = base + ws.KV, *O = base + ws.O;
  void *Cp = Cprime_out ? Cprime_out : (void *)(base + ws.Cp);
  const int M = B * T, HD = dims->H * dims->d_h;
  LAUNCH(mtla::launch_proj(dims->dtype, X, M, dims->d, w->W_dkv, w->W_gate, dims->r, w->W_Q, HD,
                           cg, q, nullptr, 0, s),
         "latent, gate and query projection");
  LAUNCH(mtla::launch_group_scan(dims->dtype, cg, w->b_hc, w->gate_pos, KR, B, T, dims->r,
                                 dims->d_hR, dims->s, Cp, keys, ws.keys_stride,
                                 cache_out ? cache_out->slots : nullptr,
                                 cache_out ? cache_out->batch_stride : 0, s),
         "gate and group scan");
  LAUNCH(mtla::launch_gemm_store2(dims->dtype, Cp, dims->r, w->W_K, w->W_V, HD, dims->r, M, 2 * HD,
                                  dims->r, KV, 2 * HD, s),
         "per-head key and value projection");
  if (dims->dtype == MTLA_BF16)
    LAUNCH(mtla::launch_heads_attention(B, T, dims->H, dims->d_h, dims->s, eff_scale(dims), q, QR,
                                        KV, KR, O, nullptr, s, ev0(events), ev1(events)),
           "per-head strided attention");
  else
    LAUNCH(mtla::launch_heads_attention_f32(B, T, dims->H, dims->d_h, dims->s, eff_scale(dims), q,
                                            QR, KV, KR, O, nullptr, s, ev0(events), ev1(events)),
           "per-head strided attention (fp32)");
  LAUNCH(mtla::launch_out_proj(dims->dtype, O, M, HD, w->W_O, dims->d, Y, nullptr, nullptr, s),
         "output projection");
  return ok();
}

// The fp32 backward after the shared forward projections and group scan
// (csrc/backward_f32.hip): the forward attention with its log2-sum-exp,
// then the chain rule of the bf16 path with strided fp32 products in place
// of the transposes and split products.
mtla_status backward_f32_rest(const mtla_dims *dims, const mtla_unabsorbed_weights *w,
                              const void *W_hc, const void *X, const void *QR, const void *KR,
                              int B, int T, const void *dY, void *dX, void *dQR, void *dKR,
                              const mtla_unabsorbed_grads *gr, const BwdWs &ws, char *base,
                              hipStream_t s) {
  auto F = [&](size_t off) { return (float *)(base + off); };
  const int M = B * T, H = dims->H, dh = dims->d_h, HD = H * dh, r = dims->r, d = dims->d;
  const float scale = eff_scale(dims);
  const float *Xf = (const float *)X, *dYf = (const float *)dY;
  const float *WQ = (const float *)w->W_Q, *WK = (const float *)w->W_K, *WV = (const float *)w->W_V;
  const float *WO = (const float *)w->W_O, *Wdkv = (const float *)w->W_dkv;
  const float *Whc = (const float *)W_hc;
  float *q = F(ws.f.q), *KV = F(ws.f.KV), *O = F(ws.f.O), *Cp = F(ws.f.Cp), *cg = F(ws.f.cg);
  float *lse = F(ws.lse), *dO = F(ws.dO), *D = F(ws.D), *dKV = F(ws.dKV), *dKRh = F(ws.dKRh);
  float *dCp = F(ws.dCp), *da = F(ws.da32), *dc32 = F(ws.dc32);
  // [dQ | dc] side by side at row stride HD + r, as in the bf16 path.
  const int ldc2 = HD + r;
  float *dQ = F(ws.dQc), *dc = dQ + HD;
  float *dXf = (float *)dX;
  LAUNCH(mtla::launch_heads_attention_f32(B, T, H, dh, dims->s, scale, q, QR, KV, KR, O, lse, s),
         "forward attention (fp32)");
  // output map: dO = dY W_O (W_O [d, HD])
  LAUNCH(mtla::launch_gemm_f32s(dYf, d, 1, WO, HD, 1, M, HD, d, nullptr, 0, dO, HD, s), "dO");
  LAUNCH(mtla::launch_rowdot_f32(dO, O, M * H, dh, D, s), "rowsum dO * O");
  LAUNCH(mtla::launch_attn_bwd_f32(B, T, H, dh, dims->s, scale, q, (const float *)QR, KV,
                                   (const float *)KR, dO, lse, D, dKV, dKRh, dQ, ldc2,
                                   (float *)dQR, s),
         "attention backward (fp32)");
  LAUNCH(mtla::launch_head_sum(dims->dtype, dKRh, M, H, dims->d_hR, dKR, s), "dK^R over heads");
  // key and value maps: dC' = dK W_K + dV W_V (W_K, W_V [HD, r])
  LAUNCH(mtla::launch_gemm_f32s(dKV, 2 * HD, 1, WK, r, 1, M, r, HD, nullptr, 0, dCp, r, s), "dC' (K)");
  LAUNCH(mtla::launch_gemm_f32s(dKV + HD, 2 * HD, 1, WV, r, 1, M, r, HD, dCp, r, dCp, r, s),
         "dC' (V)");
  // group sums and gate
  int *rctr = (int *)(base + ws.red_ctr);
  LAUNCH(mtla::launch_zero_i32(rctr, ws.nctr, s), "clear the reduction counters");
  LAUNCH(mtla::launch_scan_gate_bwd(dims->dtype, dCp, cg, w->b_hc, w->gate_pos, B, T, r, dims->s,
                                    da, base + ws.dab, dc32, base + ws.cb, F(ws.dPpart),
                                    w->gate_pos_rows, gr->dgate_pos, s),
         "group scan and gate backward");
  LAUNCH(mtla::launch_colsum(da, M, r, F(ws.red_part), rctr, gr->db_hc, s), "db");
  // dc = dU w + W_hc^T da (W_hc [r, r])
  LAUNCH(mtla::launch_gemm_f32s(da, r, 1, Whc, r, 1, M, r, r, dc32, r, dc, ldc2, s), "dc");
  // inputs: dX = dQ W_Q + dc W_dkv (W_Q [HD, d], W_dkv [r, d])
  LAUNCH(mtla::launch_gemm_f32s(dQ, ldc2, 1, WQ, d, 1, M, d, HD, nullptr, 0, dXf, d, s), "dX (Q)");
  LAUNCH(mtla::launch_gemm_f32s(dc, ldc2, 1, Wdkv, d, 1, M, d, r, dXf, d, dXf, d, s), "dX (latent)");
  // weight gradients: A^T B over the frames (A read along its rows)
  LAUNCH(mtla::launch_gemm_f32s(dYf, 1, d, O, HD, 1, d, HD, M, nullptr, 0, gr->dW_O, HD, s), "dW_O");
  LAUNCH(mtla::launch_gemm_f32s(dQ, 1, ldc2, Xf, d, 1, HD, d, M, nullptr, 0, gr->dW_Q, d, s), "dW_Q");
  LAUNCH(mtla::launch_gemm_f32s(dKV, 1, 2 * HD, Cp, r, 1, HD, r, M, nullptr, 0, gr->dW_K, r, s),
         "dW_K");
  LAUNCH(mtla::launch_gemm_f32s(dKV + HD, 1, 2 * HD, Cp, r, 1, HD, r, M, nullptr, 0, gr->dW_V, r, s),
         "dW_V");
  LAUNCH(mtla::launch_gemm_f32s(da, 1, r, cg, 2 * r, 1, r, r, M, nullptr, 0, gr->dW_hc, r, s), "dW_hc");
  LAUNCH(mtla::launch_gemm_f32s(dc, 1, ldc2, Xf, d, 1, r, d, M, nullptr, 0, gr->dW_dkv, d, s),
         "dW_dkv");
  return ok();
}

mtla_status prefill_unabsorbed_backward_impl(
    const mtla_dims *dims, const mtla_unabsorbed_weights *w, const void *W_hc, const void *X,
    const void *QR, const void *KR, int32_t B, int32_t T, const void *dY, void *dX, void *dQR,
    void *dKR, const mtla_unabsorbed_grads *gr, void *workspace, size_t ws_bytes, void *stream) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  if (!w) return fail(MTLA_ERR_ARG, "weights is null");
  if (!gr) return fail(MTLA_ERR_ARG, "grads is null");
  CHECK_PTR(w->W_dkv);
  CHECK_PTR(w->W_gate);
  CHECK_PTR(w->b_hc);
  CHECK_PTR(w->gate_pos);
  if (w->gate_pos_rows <= 0) return fail(MTLA_ERR_ARG, "gate_pos_rows=%d", w->gate_pos_rows);
  CHECK_PTR(w->W_Q);
  CHECK_PTR(w->W_K);
  CHECK_PTR(w->W_V);
  CHECK_PTR(w->W_O);
  CHECK_PTR(W_hc);
  CHECK_PTR(X);
  CHECK_PTR(QR);
  CHECK_PTR(KR);
  CHECK_PTR(dY);
  CHECK_PTR(dX);
  CHECK_PTR(dQR);
  CHECK_PTR(dKR);
  CHECK_PTR(gr->dW_dkv);
  CHECK_PTR(gr->dW_hc);
  CHECK_PTR(gr->db_hc);
  CHECK_PTR(gr->dgate_pos);
  CHECK_PTR(gr->dW_Q);
  CHECK_PTR(gr->dW_K);
  CHECK_PTR(gr->dW_V);
  CHECK_PTR(gr->dW_O);
  CHECK_PTR(workspace);
  if (B < 1 || B > 65535) return fail(MTLA_ERR_ARG, "B=%d outside [1, 65535]", B);
  if (T < 1) return fail(MTLA_ERR_ARG, "T=%d < 1", T);
  if ((int64_t)B * T * dims->H * dims->d_h > 0x7fffffffLL / 4 ||
      (int64_t)B * T * dims->d > 0x7fffffffLL / 4)
    return fail(MTLA_ERR_UNSUPPORTED, "B*T too large");
  const bool f32 = dims->dtype == MTLA_F32;
  if (!(f32 ? mtla::heads_attention_supported(dims->dtype, dims->H, dims->d_h, dims->d_hR)
            : mtla::attn_bwd_supported(dims->dtype, dims->H, dims->d_h, dims->d_hR)))
    return fail(MTLA_ERR_UNSUPPORTED, "backward needs (d_h, d_hR) = (64, 32) or (128, 64)");
  if ((T - 1) / dims->s >= w->gate_pos_rows)
    return fail(MTLA_ERR_CAPACITY, "slot %d >= gate_pos_rows %d", (T - 1) / dims->s, w->gate_pos_rows);
  const BwdWs ws = bwd_ws(dims, B, T);
  if (ws_bytes < ws.total) return fail(MTLA_ERR_ARG, "workspace %zu < %zu bytes", ws_bytes, ws.total);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)workspace;
  auto P = [&](size_t off) { return (void *)(base + off); };
  auto F = [&](size_t off) { return (float *)(base + off); };
  const int M = B * T, HD = dims->H * dims->d_h, r = dims->r, d = dims->d, H = dims->H;
  const int dt = dims->dtype;
  const float scale = eff_scale(dims);
  void *Cp = P(ws.f.Cp), *q = P(ws.f.q), *KV = P(ws.f.KV), *O = P(ws.f.O);
  float *cg = F(ws.f.cg), *lse = F(ws.lse);
  // forward, keeping what the backward reads
  LAUNCH(mtla::launch_proj(dt, X, M, d, w->W_dkv, w->W_gate, r, w->W_Q, HD, cg, q, nullptr, 0, s),
         "forward projection");
  LAUNCH(mtla::launch_group_scan(dt, cg, w->b_hc, w->gate_pos, KR, B, T, r, dims->d_hR, dims->s, Cp,
                                 P(ws.f.keys), ws.f.keys_stride, nullptr, 0, s),
         "forward group scan");
  LAUNCH(mtla::launch_gemm_store2(dt, Cp, r, w->W_K, w->W_V, HD, r, M, 2 * HD, r, KV, 2 * HD, s),
         "forward key and value projection");
  if (f32)
    return backward_f32_rest(dims, w, W_hc, X, QR, KR, B, T, dY, dX, dQR, dKR, gr, ws, base, s);
  LAUNCH(mtla::launch_heads_attention(B, T, H, dims->d_h, dims->s, scale, q, QR, KV, KR, O, lse, s),
         "forward attention");
  // transposed weights for the products against them
  LAUNCH(mtla::launch_transpose(w->W_O, d, HD, HD, P(ws.WOt), d, s), "transpose W_O");
  LAUNCH(mtla::launch_transpose(w->W_K, HD, r, r, P(ws.WKVt), 2 * HD, s), "transpose W_K");
  LAUNCH(mtla::launch_transpose(w->W_V, HD, r, r, (char *)P(ws.WKVt) + (size_t)HD * 2, 2 * HD, s),
         "transpose W_V");
  LAUNCH(mtla::launch_transpose(W_hc, r, r, r, P(ws.Whct), r, s), "transpose W_hc");
  // [dQ | dc] and [W_Q^T | W_dkv^T]: row stride HD + r, dc and W_dkv^T at column HD.
  const int ldc2 = HD + r;
  void *dQ = P(ws.dQc), *dcb = (char *)P(ws.dQc) + (size_t)HD * esize(dims);
  LAUNCH(mtla::launch_transpose(w->W_Q, HD, d, d, P(ws.Wc), ldc2, s), "transpose W_Q");
  LAUNCH(mtla::launch_transpose(w->W_dkv, r, d, d, (char *)P(ws.Wc) + (size_t)HD * esize(dims), ldc2,
                                s),
         "transpose W_dkv");
  // output map
  LAUNCH(mtla::launch_gemm_store(dt, dY, d, P(ws.WOt), d, M, HD, d, P(ws.dO), HD, s), "dO");
  LAUNCH(mtla::launch_rowdot(P(ws.dO), O, M * H, dims->d_h, F(ws.D), s), "rowsum dO * O");
  // attention
  LAUNCH(mtla::launch_attn_bwd(B, T, H, dims->d_h, dims->s, scale, q, QR, KV, KR, P(ws.dO), lse, F(ws.D),
                               F(ws.dKVc), F(ws.dKRc), P(ws.dKV), F(ws.dKRh), dQ, dQR, ldc2, s),
         "attention backward");
  LAUNCH(mtla::launch_head_sum(dt, F(ws.dKRh), M, H, dims->d_hR, dKR, s), "dK^R over heads");
  // key and value maps
  LAUNCH(mtla::launch_gemm_f32(dt, P(ws.dKV), 2 * HD, P(ws.WKVt), 2 * HD, M, r, 2 * HD, F(ws.dCp), r,
                               false, s),
         "dC'");
  // group sums and gate
  int *rctr = (int *)P(ws.red_ctr);
  float *rpart = F(ws.red_part);
  LAUNCH(mtla::launch_zero_i32(rctr, ws.nctr, s), "clear the reduction counters");
  LAUNCH(mtla::launch_scan_gate_bwd(dt, F(ws.dCp), cg, w->b_hc, w->gate_pos, B, T, r, dims->s,
                                    F(ws.da32), P(ws.dab), F(ws.dc32), P(ws.cb), F(ws.dPpart),
                                    w->gate_pos_rows, gr->dgate_pos, s),
         "group scan and gate backward");
  LAUNCH(mtla::launch_colsum(F(ws.da32), M, r, rpart, rctr, gr->db_hc, s), "db");
  LAUNCH(mtla::launch_gemm_add_bf16(P(ws.dab), r, P(ws.Whct), r, M, r, r, F(ws.dc32), r, dcb, ldc2,
                                    s),
         "dc");
  // inputs
  // dX = [dQ | dc] [W_Q^T | W_dkv^T]^T: one product over K = HD + r.
  LAUNCH(mtla::launch_gemm_store(dt, dQ, ldc2, P(ws.Wc), ldc2, M, d, ldc2, dX, d, s),
         "dX from the query and latent maps");
  // weight gradients (each product's partials added in split order)
  LAUNCH(mtla::launch_tn_gemm(dY, d, O, HD, M, d, HD, gr->dW_O, HD, rpart, s), "dW_O");
  LAUNCH(mtla::launch_tn_gemm(dQ, ldc2, X, d, M, HD, d, gr->dW_Q, d, rpart, s), "dW_Q");
  LAUNCH(mtla::launch_tn_gemm(P(ws.dKV), 2 * HD, Cp, r, M, HD, r, gr->dW_K, r, rpart, s),
         "dW_K");
  LAUNCH(mtla::launch_tn_gemm((char *)P(ws.dKV) + (size_t)HD * 2, 2 * HD, Cp, r, M, HD, r, gr->dW_V,
                              r, rpart, s),
         "dW_V");
  LAUNCH(mtla::launch_tn_gemm(P(ws.dab), r, P(ws.cb), r, M, r, r, gr->dW_hc, r, rpart, s),
         "dW_hc");
  LAUNCH(mtla::launch_tn_gemm(dcb, ldc2, X, d, M, r, d, gr->dW_dkv, d, rpart, s),
         "dW_dkv");
  return ok();
}

}  // namespace

extern "C" {

mtla_status mtla_prefill_unabsorbed_backward(const mtla_dims *dims,
                                             const mtla_unabsorbed_weights *w, const void *W_hc,
                                             const void *X, const void *QR, const void *KR,
                                             int32_t B, int32_t T, const void *dY, void *dX,
                                             void *dQR, void *dKR,
                                             const mtla_unabsorbed_grads *grads, void *workspace,
                                             size_t ws_bytes, void *stream) {
  return prefill_unabsorbed_backward_impl(dims, w, W_hc, X, QR, KR, B, T, dY, dX, dQR, dKR, grads,
                                          workspace, ws_bytes, stream);
}

mtla_status mtla_prefill_unabsorbed(const mtla_dims *dims, const mtla_unabsorbed_weights *w,
                                    const void *X, const void *QR, const void *KR, int32_t B,
                                    int32_t T, void *Y, const mtla_cache *cache_out,
                                    void *Cprime_out, void *workspace, size_t ws_bytes,
                                    void *stream) {
  return prefill_unabsorbed_impl(dims, w, X, QR, KR, B, T, Y, cache_out, Cprime_out, workspace,
                                 ws_bytes, stream, nullptr);
}

mtla_status mtla_prefill_unabsorbed_timed(const mtla_dims *dims, const mtla_unabsorbed_weights *w,
                                          const void *X, const void *QR, const void *KR,
                                          int32_t B, int32_t T, void *Y,
                                          const mtla_cache *cache_out, void *Cprime_out,
                                          void *workspace, size_t ws_bytes, void *stream,
                                          void *const *events) {
  if (!events || !events[0] || !events[1]) return fail(MTLA_ERR_ARG, "events must hold two handles");
  return prefill_unabsorbed_impl(dims, w, X, QR, KR, B, T, Y, cache_out, Cprime_out, workspace,
                                 ws_bytes, stream, events);
}

mtla_status mtla_decode_step(const mtla_dims *dims, const mtla_weights *w, const mtla_cache *cache,
                             const void *X_t, const void *QR_t, const void *KR_t, const int32_t *pos,
                             int32_t B, int32_t max_pos, void *Y, void *workspace, size_t ws_bytes,
                             void *stream) {
  return decode_step_impl(dims, w, cache, X_t, QR_t, KR_t, pos, B, max_pos, Y, workspace, ws_bytes,
                          stream, nullptr);
}

mtla_status mtla_decode_step_noalloc(const mtla_dims *dims, const mtla_weights *w,
                                     const mtla_cache *cache, const void *X_t, const void *QR_t,
                                     const void *KR_t, const int32_t *pos, int32_t B,
                                     int32_t max_pos, void *Y, void *stream) {
  mtla_status st;
  if ((st = check_dims(dims)) != MTLA_OK) return st;
  if (B < 1 || B > 65535) return fail(MTLA_ERR_ARG, "B=%d outside [1, 65535]", B);
  if (max_pos < 0) return fail(MTLA_ERR_ARG, "max_pos=%d < 0", max_pos);
  const size_t need = mtla_workspace_bytes(dims, 1, B, max_pos);
  if (need == 0) return fail(MTLA_ERR_UNSUPPORTED, "no decode plan for this shape");
  if (need > kNoAllocScratchBytes)
    return fail(MTLA_ERR_CAPACITY, "decode step needs %zu bytes of scratch > %zu", need,
                kNoAllocScratchBytes);
  int dev = -1, sdev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MTLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  e = hipStreamGetDevice((hipStream_t)stream, &sdev);
  if (e != hipSuccess) return fail(MTLA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  if (sdev != dev)
    return fail(MTLA_ERR_ARG, "stream belongs to device %d, current device is %d", sdev, dev);
  void *ws = nullptr;
  if ((st = scratch_for(dev, &ws)) != MTLA_OK) return st;
  return decode_step_impl(dims, w, cache, X_t, QR_t, KR_t, pos, B, max_pos, Y, ws,
                          kNoAllocScratchBytes, stream, nullptr);
}

mtla_status mtla_decode_step_timed(const mtla_dims *dims, const mtla_weights *w,
                                   const mtla_cache *cache, const void *X_t, const void *QR_t,
                                   const void *KR_t, const int32_t *pos, int32_t B, int32_t max_pos,
                                   void *Y, void *workspace, size_t ws_bytes, void *stream,
                                   void *const *events) {
  if (!events || !events[0] || !events[1]) return fail(MTLA_ERR_ARG, "events must hold two handles");
  return decode_step_impl(dims, w, cache, X_t, QR_t, KR_t, pos, B, max_pos, Y, workspace, ws_bytes,
                          stream, events);
}

mtla_status mtla_prefill_strided(const mtla_dims *dims, const mtla_weights *w, const void *X,
                                 const void *QR, const void *KR, int32_t B, int32_t T, void *Y,
                                 const mtla_cache *cache_out, void *Cprime_out, void *workspace,
                                 size_t ws_bytes, void *stream) {
  return prefill_impl(dims, w, X, QR, KR, B, T, Y, cache_out, Cprime_out, workspace, ws_bytes,
                      stream, nullptr);
}

mtla_status mtla_prefill_strided_timed(const mtla_dims *dims, const mtla_weights *w, const void *X,
                                       const void *QR, const void *KR, int32_t B, int32_t T,
                                       void *Y, const mtla_cache *cache_out, void *Cprime_out,
                                       void *workspace, size_t ws_bytes, void *stream,
                                       void *const *events) {
  if (!events || !events[0] || !events[1]) return fail(MTLA_ERR_ARG, "events must hold two handles");
  return prefill_impl(dims, w, X, QR, KR, B, T, Y, cache_out, Cprime_out, workspace, ws_bytes,
                      stream, events);
}

}  // extern "C"
