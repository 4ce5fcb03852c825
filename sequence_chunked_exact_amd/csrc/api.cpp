// C-ABI layer: argument checks (all before any device call), workspace sizing,
// the SpaCO chunk selector, the sparse backward driver, the layer-stack driver
// (SeCO's inference pass, SpaCO's relayed backward) and the streamed LM head's
// entry points. Kernels live in attention.hip, projection.hip, stack.hip and
// lm_head.hip; this file validates, orders launches and enqueues them.
#include "chunk_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "launch.h"

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(CA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shared checks of a descriptor. `whole_seq` relaxes chunk_start/q_row_offset
// (the sparse driver sets them per chunk).
int check_desc(const chunk_attn_desc* d, bool whole_seq) {
  if (!d) return fail(CA_ERR_NULL, "descriptor is NULL");
  if (d->dtype != CA_F32 && d->dtype != CA_BF16) return fail(CA_ERR_DTYPE, "dtype %d", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(CA_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", d->head_dim);
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(CA_ERR_SHAPE, "batch/heads must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(CA_ERR_SHAPE, "n_q_heads %d not a multiple of n_kv_heads %d", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads > 65535 || d->batch > 65535 || d->n_kv_heads > 65535)
    return fail(CA_ERR_SHAPE, "heads/batch above 65535");
  if (d->chunk_len < 1) return fail(CA_ERR_SHAPE, "chunk_len %d < 1", d->chunk_len);
  if (d->kv_capacity < 1 || d->q_capacity < 1) return fail(CA_ERR_SHAPE, "capacities must be >= 1");
  if (!(d->softmax_scale == d->softmax_scale) || d->softmax_scale > 3.0e38f || d->softmax_scale < -3.0e38f)
    return fail(CA_ERR_SHAPE, "softmax_scale is not finite");
  if (!whole_seq) {
    if (d->chunk_start < 0 || d->q_row_offset < 0) return fail(CA_ERR_SHAPE, "negative chunk_start/q_row_offset");
    if ((int64_t)d->chunk_start + d->chunk_len > d->kv_capacity)
      return fail(CA_ERR_SHAPE, "chunk_start + chunk_len = %lld exceeds kv_capacity %d",
                  (long long)d->chunk_start + d->chunk_len, d->kv_capacity);
    if ((int64_t)d->q_row_offset + d->chunk_len > d->q_capacity)
      return fail(CA_ERR_SHAPE, "q_row_offset + chunk_len exceeds q_capacity %d", d->q_capacity);
  }
  // element offsets must fit the kernels' index arithmetic
  const int64_t qel = (int64_t)d->batch * d->n_q_heads * d->q_capacity;
  const int64_t kel = (int64_t)d->batch * d->n_kv_heads * d->kv_capacity;
  if (qel > (int64_t)1 << 40 || kel > (int64_t)1 << 40) return fail(CA_ERR_SHAPE, "tensors too large");
  if ((int64_t)d->batch * d->n_q_heads * d->chunk_len > INT32_MAX / 32)
    return fail(CA_ERR_SHAPE, "batch * n_q_heads * chunk_len too large");
  return CA_OK;
}

ca::Shape shape_of(const chunk_attn_desc* d) {
  ca::Shape s;
  s.batch = d->batch;
  s.hq = d->n_q_heads;
  s.hkv = d->n_kv_heads;
  s.head_dim = d->head_dim;
  s.kv_cap = d->kv_capacity;
  s.q_cap = d->q_capacity;
  s.q_off = d->q_row_offset;
  s.start = d->chunk_start;
  s.len = d->chunk_len;
  s.scale = d->softmax_scale;
  s.dtype = d->dtype;
  return s;
}

size_t delta_bytes(const chunk_attn_desc* d) {
  return round_up(ca::bwd_ws_bytes((size_t)d->batch * d->n_q_heads * d->chunk_len));
}

// The whole-sequence drivers keep two slots of row statistics when the
// workspace holds both and is not a dS hand-over workspace (CA_OP_BWD_DS):
// each chunk's launch then also computes the next chunk's statistics, and no
// chunk needs a launch of its own for them.
bool two_stat_slots(const chunk_attn_desc* d, size_t ws_bytes) {
  const size_t slot = delta_bytes(d);
  if (ws_bytes < 2 * slot) return false;
  return !(d->dtype == CA_BF16 &&
           ws_bytes >= slot + round_up(ca::bwd_ds_bytes(d->batch, d->n_q_heads, d->chunk_len, d->kv_capacity)));
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return fail(CA_ERR_NULL, "a tensor pointer is NULL");
    if (!aligned16(p)) return fail(CA_ERR_ALIGN, "a tensor pointer is not 16-byte aligned");
  }
  return CA_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return CA_OK;
  if (!ws) return fail(CA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(CA_ERR_ALIGN, "workspace not 16-byte aligned");
  return CA_OK;
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014).
struct SplitMix64 {
  uint64_t x;
  uint64_t next() {
    x += 0x9E3779B97F4A7C15ull;
    uint64_t z = x;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

}  // namespace


// ---------------------------------------------------------------------------
// Launch timing: while profiling is on, each selected launch gets a pair of
// HIP events from a reusable pool, which the dispatch stamps with the
// kernel's start and end (hipExtLaunchKernelGGL).
// ---------------------------------------------------------------------------
namespace ca {
namespace {
struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};
struct ProfState {
  std::mutex mu;
  bool on = false;
  uint32_t mask = 0xFFFFFFFFu;  // kernel ids that get events (bit per id)
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<ProfRec> recs;
};
ProfState& prof() {
  static ProfState s;
  return s;
}

hipEvent_t take_event(ProfState& s) {
  if (s.used == s.pool.size()) {
    hipEvent_t e = nullptr;
    // timing only: no system-scope fence (a default event's fence, per launch,
    // costs the step several percent)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    s.pool.push_back(e);
  }
  return s.pool[s.used++];
}
}  // namespace

ProfPair prof_launch(int kernel) {
  ProfState& s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on || !((s.mask >> kernel) & 1u)) return {nullptr, nullptr};
  hipEvent_t a = take_event(s), b = take_event(s);
  if (!a || !b) return {nullptr, nullptr};
  s.recs.push_back({kernel, a, b});
  return {a, b};
}
}  // namespace ca

namespace {
int check_proj(const chunk_attn_desc* d, int32_t d_model, int32_t h_capacity, int32_t h_row_offset) {
  int rc = check_desc(d, false);
  if (rc) return rc;
  if (d_model < 64 || d_model > 65536 || d_model % 64 != 0)
    return fail(CA_ERR_SHAPE, "d_model %d (a multiple of 64 in [64, 65536])", d_model);
  if (h_row_offset < 0 || h_capacity < 1 || (int64_t)h_row_offset + d->chunk_len > h_capacity)
    return fail(CA_ERR_SHAPE, "h rows [%d, %lld) exceed h_capacity %d", h_row_offset,
                (long long)h_row_offset + d->chunk_len, h_capacity);
  if ((int64_t)d->batch * h_capacity * d_model > ((int64_t)1 << 40) ||
      (int64_t)d_model * d->n_q_heads * d->head_dim > ((int64_t)1 << 40))
    return fail(CA_ERR_SHAPE, "projection tensors too large");
  return CA_OK;
}
ca::ProjShape proj_shape(const chunk_attn_desc* d, int32_t d_model, int32_t h_capacity, int32_t h_row_offset) {
  ca::ProjShape s;
  s.batch = d->batch;
  s.d_model = d_model;
  s.hq = d->n_q_heads;
  s.hkv = d->n_kv_heads;
  s.head_dim = d->head_dim;
  s.h_cap = h_capacity;
  s.h_off = h_row_offset;
  s.q_cap = d->q_capacity;
  s.q_off = d->q_row_offset;
  s.kv_cap = d->kv_capacity;
  s.start = d->chunk_start;
  s.len = d->chunk_len;
  s.dtype = d->dtype;
  return s;
}
}  // namespace

extern "C" {

const char* chunk_attn_strerror(int code) {
  switch (code) {
    case CA_OK: return "ok";
    case CA_ERR_NULL: return "null pointer";
    case CA_ERR_SHAPE: return "invalid shape";
    case CA_ERR_DTYPE: return "invalid dtype";
    case CA_ERR_ALIGN: return "misaligned pointer";
    case CA_ERR_WORKSPACE: return "workspace too small";
    case CA_ERR_UNSUPPORTED: return "unsupported head_dim";
    case CA_ERR_HIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char* chunk_attn_last_error(void) { return g_err; }

size_t chunk_attn_workspace_size(const chunk_attn_desc* d, int32_t op) {
  if (check_desc(d, op == CA_OP_SPARSE_BWD || op == CA_OP_BWD_DS) != CA_OK) return 0;
  switch (op) {
    case CA_OP_FWD: return 0;
    case CA_OP_BWD:
    case CA_OP_BWD_MIN: return delta_bytes(d);  // the chunk's row statistics only
    case CA_OP_SPARSE_BWD: return 2 * delta_bytes(d);  // this chunk's and the next one's
    case CA_OP_BWD_DS:
      // plus room for the dS^T blocks of any chunk of up to chunk_len rows
      // whose prefix fits kv_capacity (bf16)
      return delta_bytes(d) + (d->dtype == CA_BF16 ? round_up(ca::bwd_ds_bytes(d->batch, d->n_q_heads,
                                                                                d->chunk_len, d->kv_capacity))
                                                   : 0);
    default: return 0;
  }
}

int chunk_attn_fwd(const chunk_attn_desc* d, const void* q, const void* k, const void* v, void* o,
                   float* lse, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_desc(d, false);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k, v, o, lse}))) return rc;
  hipError_t e = ca::launch_fwd(shape_of(d), q, k, v, o, lse, (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "chunk_attn_fwd launch");
}

int chunk_attn_bwd(const chunk_attn_desc* d, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, float grad_scale, float* dq, float* dk_acc,
                   float* dv_acc, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(d, false);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k, v, o, lse, dout, dq, dk_acc, dv_acc}))) return rc;
  if (!(grad_scale == grad_scale) || grad_scale > 3.0e38f || grad_scale < -3.0e38f)
    return fail(CA_ERR_SHAPE, "grad_scale is not finite");
  if ((rc = check_ws(ws, ws_bytes, delta_bytes(d)))) return rc;
  hipError_t e = ca::launch_bwd(shape_of(d), q, k, v, o, lse, dout, grad_scale, dq, dk_acc, dv_acc,
                                (float*)ws, ws_bytes, (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "chunk_attn_bwd launch");
}

int chunk_attn_bwd_noalloc(const chunk_attn_desc* d, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, float grad_scale, float* dq, float* dk_acc,
                           float* dv_acc, void* stream) {
  int rc = check_desc(d, false);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k, v, o, lse, dout, dq, dk_acc, dv_acc}))) return rc;
  if (!(grad_scale == grad_scale) || grad_scale > 3.0e38f || grad_scale < -3.0e38f)
    return fail(CA_ERR_SHAPE, "grad_scale is not finite");
  const size_t need = delta_bytes(d);
  if (need > ca::kScratchBytes)
    return fail(CA_ERR_WORKSPACE,
                "chunk_attn_bwd_noalloc: batch * n_q_heads * chunk_len = %lld rows need %zu bytes of scratch; "
                "the static scratch holds %zu",
                (long long)d->batch * d->n_q_heads * d->chunk_len, need, ca::kScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "chunk_attn_bwd_noalloc: hipGetDevice");
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "chunk_attn_bwd_noalloc: hipStreamGetDevice");
    if (sdev != dev)
      return fail(CA_ERR_SHAPE, "chunk_attn_bwd_noalloc: stream is on device %d, current device is %d", sdev, dev);
  }
  void* ws = nullptr;
  if ((e = ca::scratch_address(&ws)) != hipSuccess) return hip_fail(e, "chunk_attn_bwd_noalloc: scratch address");
  e = ca::launch_bwd(shape_of(d), q, k, v, o, lse, dout, grad_scale, dq, dk_acc, dv_acc, (float*)ws, need,
                     (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "chunk_attn_bwd_noalloc launch");
}

int prefix_grad_accumulate(float* acc, const float* src, int32_t batch, int32_t n_heads, int32_t acc_capacity,
                           int32_t src_capacity, int32_t head_dim, int32_t prefix_len, float scale,
                           void* stream) {
  int rc = check_ptrs({acc, src});
  if (rc) return rc;
  if (batch < 1 || n_heads < 1 || head_dim < 4 || head_dim % 4 != 0 || prefix_len < 0 ||
      prefix_len > acc_capacity || prefix_len > src_capacity)
    return fail(CA_ERR_SHAPE, "accumulate: batch %d heads %d head_dim %d prefix %d caps %d/%d", batch, n_heads,
                head_dim, prefix_len, acc_capacity, src_capacity);
  if ((int64_t)batch * n_heads * std::max(acc_capacity, src_capacity) * head_dim > ((int64_t)1 << 40))
    return fail(CA_ERR_SHAPE, "accumulate: tensors too large");
  hipError_t e = ca::launch_accumulate(acc, src, batch, n_heads, acc_capacity, src_capacity, head_dim,
                                       prefix_len, scale, (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "prefix_grad_accumulate launch");
}


size_t qkv_proj_bwd_workspace_size(const chunk_attn_desc* d, int32_t d_model) {
  if (check_proj(d, d_model, d ? d->chunk_len : 1, 0) != CA_OK) return 0;
  return ca::proj_bwd_ws_bytes(proj_shape(d, d_model, d->chunk_len, 0));
}

int qkv_proj_fwd(const chunk_attn_desc* d, int32_t d_model, int32_t h_capacity, int32_t h_row_offset,
                 const void* h, const void* wq, const void* wk, const void* wv, void* q, void* k, void* v,
                 void* stream) {
  int rc = check_proj(d, d_model, h_capacity, h_row_offset);
  if (rc) return rc;
  if ((rc = check_ptrs({h, wq, wk, wv, q, k, v}))) return rc;
  hipError_t e = ca::launch_proj_fwd(proj_shape(d, d_model, h_capacity, h_row_offset), h, wq, wk, wv, q, k, v,
                                     (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "qkv_proj_fwd launch");
}

size_t qkv_proj_weights_t_bytes(const chunk_attn_desc* d, int32_t d_model) {
  if (check_proj(d, d_model, d ? d->chunk_len : 1, 0) != CA_OK) return 0;
  return ca::proj_wt_bytes(proj_shape(d, d_model, d->chunk_len, 0));
}

int qkv_proj_weights_t(const chunk_attn_desc* d, int32_t d_model, const void* wq, const void* wk, const void* wv,
                       void* w_cat_t, void* stream) {
  int rc = check_proj(d, d_model, d ? d->chunk_len : 1, 0);
  if (rc) return rc;
  if (d->dtype != CA_BF16) return fail(CA_ERR_DTYPE, "qkv_proj_weights_t: bf16 layers only");
  if ((rc = check_ptrs({wq, wk, wv, w_cat_t}))) return rc;
  hipError_t e = ca::launch_proj_wt(proj_shape(d, d_model, d->chunk_len, 0), wq, wk, wv, w_cat_t,
                                    (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "qkv_proj_weights_t launch");
}

int qkv_proj_bwd_wt(const chunk_attn_desc* d, int32_t d_model, int32_t h_capacity, int32_t h_row_offset,
                    const void* h, const void* wq, const void* wk, const void* wv, const void* w_cat_t,
                    const float* dq, const float* dk_acc, const float* dv_acc, float* dwq, float* dwk, float* dwv,
                    float* dh, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_proj(d, d_model, h_capacity, h_row_offset);
  if (rc) return rc;
  if ((rc = check_ptrs({h, wq, wk, wv, dq, dk_acc, dv_acc, dwq, dwk, dwv, dh}))) return rc;
  const bool use_wt = d->dtype == CA_BF16;  // float32 layers read the weights directly
  if (use_wt && (rc = check_ptrs({w_cat_t}))) return rc;
  const ca::ProjShape ps = proj_shape(d, d_model, h_capacity, h_row_offset);
  if ((rc = check_ws(ws, ws_bytes, ca::proj_bwd_ws_bytes(ps, use_wt)))) return rc;
  hipError_t e = ca::launch_proj_bwd(ps, h, wq, wk, wv, dq, dk_acc, dv_acc, dwq, dwk, dwv, dh, ws,
                                     (hipStream_t)stream, use_wt ? w_cat_t : nullptr);
  return e == hipSuccess ? CA_OK : hip_fail(e, "qkv_proj_bwd_wt launch");
}

int qkv_proj_bwd(const chunk_attn_desc* d, int32_t d_model, int32_t h_capacity, int32_t h_row_offset,
                 const void* h, const void* wq, const void* wk, const void* wv, const float* dq,
                 const float* dk_acc, const float* dv_acc, float* dwq, float* dwk, float* dwv, float* dh,
                 void* ws, size_t ws_bytes, void* stream) {
  int rc = check_proj(d, d_model, h_capacity, h_row_offset);
  if (rc) return rc;
  if ((rc = check_ptrs({h, wq, wk, wv, dq, dk_acc, dv_acc, dwq, dwk, dwv, dh}))) return rc;
  const ca::ProjShape ps = proj_shape(d, d_model, h_capacity, h_row_offset);
  if ((rc = check_ws(ws, ws_bytes, ca::proj_bwd_ws_bytes(ps)))) return rc;
  hipError_t e = ca::launch_proj_bwd(ps, h, wq, wk, wv, dq, dk_acc, dv_acc, dwq, dwk, dwv, dh, ws,
                                     (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "qkv_proj_bwd launch");
}

int chunk_select(int32_t k, int32_t t, uint64_t seed, int32_t* out_sorted) {
  if (!out_sorted) return fail(CA_ERR_NULL, "chunk_select: out_sorted is NULL");
  if (k < 1 || t < 1 || t > k) return fail(CA_ERR_SHAPE, "chunk_select: need 1 <= t <= k (k=%d t=%d)", k, t);
  std::vector<int32_t> a(k);
  for (int32_t i = 0; i < k; ++i) a[i] = i;
  SplitMix64 gen{seed};
  for (int32_t i = 0; i < t; ++i) {
    const uint64_t span = (uint64_t)(k - i);
    const int32_t j = i + (int32_t)(gen.next() % span);
    std::swap(a[i], a[j]);
  }
  std::sort(a.begin(), a.begin() + t);
  std::memcpy(out_sorted, a.data(), sizeof(int32_t) * t);
  return CA_OK;
}

int sparse_chunk_bwd(const chunk_attn_desc* d, int32_t seq_len, int32_t t, uint64_t seed, const void* q,
                     const void* k, const void* v, const void* o, const float* lse, const void* dout, float* dq,
                     float* dk, float* dv, int32_t* selected_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(d, true);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv}))) return rc;
  if (!selected_out) return fail(CA_ERR_NULL, "selected_out is NULL");
  if (seq_len < 1 || seq_len > d->q_capacity || seq_len > d->kv_capacity)
    return fail(CA_ERR_SHAPE, "seq_len %d must be in [1, min(q_capacity, kv_capacity)]", seq_len);
  const int32_t C = d->chunk_len;
  const int32_t kch = (int32_t)(((int64_t)seq_len + C - 1) / C);
  if (t < 1 || t > kch) return fail(CA_ERR_SHAPE, "t=%d must be in [1, k=%d]", t, kch);
  if ((rc = check_ws(ws, ws_bytes, delta_bytes(d)))) return rc;

  std::vector<int32_t> sel(t);
  if ((rc = chunk_select(kch, t, seed, sel.data()))) return rc;
  const float gamma = (float)kch / (float)t;

  hipStream_t st = (hipStream_t)stream;
  const size_t nq = (size_t)d->batch * d->n_q_heads * d->q_capacity * d->head_dim;
  const size_t nkv = (size_t)d->batch * d->n_kv_heads * d->kv_capacity * d->head_dim;
  // dq rows of the selected chunks are overwritten: with every chunk selected
  // and no rows past seq_len, nothing is left to zero
  hipError_t e = (t < kch || seq_len < d->q_capacity) ? ca::launch_zero(dq, nq, st) : hipSuccess;
  // The first launch (the last selected chunk) stores dk/dv rows [0, its
  // prefix end) instead of adding to them. Rows past that prefix are written
  // by no launch: when there are any (the prefix ends before kv_capacity),
  // the whole of dk and dv is zeroed first, and the first launch's stores
  // then overwrite its prefix rows.
  const int32_t first_end = std::min((sel[t - 1] + 1) * C, seq_len);
  if (first_end < d->kv_capacity) {
    if (e == hipSuccess) e = ca::launch_zero(dk, nkv, st);
    if (e == hipSuccess) e = ca::launch_zero(dv, nkv, st);
  }
  if (e != hipSuccess) return hip_fail(e, "sparse_chunk_bwd zero");

  ca::Shape s = shape_of(d);
  const bool two = two_stat_slots(d, ws_bytes);
  const size_t slot = delta_bytes(d);
  auto slot_of = [&](int32_t idx) { return (float*)((char*)ws + (two && (t - 1 - idx) % 2 ? slot : 0)); };
  for (int32_t idx = t - 1; idx >= 0; --idx) {
    const int32_t i = sel[idx];
    s.start = i * C;
    s.q_off = i * C;
    s.len = std::min(C, seq_len - i * C);
    ca::NextStats nx;
    if (two && idx > 0) {
      nx.q_off = sel[idx - 1] * C;
      nx.len = std::min(C, seq_len - nx.q_off);
      nx.ws = slot_of(idx - 1);
    }
    s.acc_store = idx == t - 1;
    e = ca::launch_bwd(s, q, k, v, o, lse, dout, gamma, dq, dk, dv, slot_of(idx), two ? slot : ws_bytes, st,
                       two && idx < t - 1, nx);
    if (e != hipSuccess) return hip_fail(e, "sparse_chunk_bwd chunk launch");
  }
  std::memcpy(selected_out, sel.data(), sizeof(int32_t) * t);
  return CA_OK;
}

int chunked_fwd_sweep(const chunk_attn_desc* d, int32_t seq_len, const void* q, const void* k, const void* v,
                      void* o, float* lse, void* stream) {
  int rc = check_desc(d, true);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k, v, o, lse}))) return rc;
  if (seq_len < 1 || seq_len > d->q_capacity || seq_len > d->kv_capacity)
    return fail(CA_ERR_SHAPE, "seq_len %d must be in [1, min(q_capacity, kv_capacity)]", seq_len);
  const int32_t C = d->chunk_len;
  ca::Shape s = shape_of(d);
  for (int64_t start = 0; start < seq_len; start += C) {  // ascending: the inference-mode pass
    s.start = s.q_off = (int)start;
    s.len = (int)std::min<int64_t>(C, seq_len - start);
    hipError_t e = ca::launch_fwd(s, q, k, v, o, lse, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "chunked_fwd_sweep chunk launch");
  }
  return CA_OK;
}

int chunked_bwd_sweep(const chunk_attn_desc* d, int32_t seq_len, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, float grad_scale, float* dq,
                      float* dk_acc, float* dv_acc, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(d, true);
  if (rc) return rc;
  if ((rc = check_ptrs({q, k, v, o, lse, dout, dq, dk_acc, dv_acc}))) return rc;
  if (seq_len < 1 || seq_len > d->q_capacity || seq_len > d->kv_capacity)
    return fail(CA_ERR_SHAPE, "seq_len %d must be in [1, min(q_capacity, kv_capacity)]", seq_len);
  if (!(grad_scale == grad_scale) || grad_scale > 3.0e38f || grad_scale < -3.0e38f)
    return fail(CA_ERR_SHAPE, "grad_scale is not finite");
  if ((rc = check_ws(ws, ws_bytes, delta_bytes(d)))) return rc;
  const int32_t C = d->chunk_len;
  const int32_t n = (int32_t)(((int64_t)seq_len + C - 1) / C);
  ca::Shape s = shape_of(d);
  const bool two = two_stat_slots(d, ws_bytes);
  const size_t slot = delta_bytes(d);
  auto slot_of = [&](int32_t i) { return (float*)((char*)ws + (two && (n - 1 - i) % 2 ? slot : 0)); };
  for (int32_t i = n - 1; i >= 0; --i) {  // descending, as SeCO's backward
    s.start = s.q_off = i * C;
    s.len = std::min(C, seq_len - i * C);
    ca::NextStats nx;
    if (two && i > 0) {
      nx.q_off = (i - 1) * C;
      nx.len = std::min(C, seq_len - nx.q_off);
      nx.ws = slot_of(i - 1);
    }
    hipError_t e = ca::launch_bwd(s, q, k, v, o, lse, dout, grad_scale, dq, dk_acc, dv_acc, slot_of(i),
                                  two ? slot : ws_bytes, (hipStream_t)stream, two && i < n - 1, nx);
    if (e != hipSuccess) return hip_fail(e, "chunked_bwd_sweep chunk launch");
  }
  return CA_OK;
}

int chunk_attn_profile_start(void) {
  ca::ProfState& s = ca::prof();
  std::lock_guard<std::mutex> g(s.mu);
  s.recs.clear();
  s.used = 0;
  s.on = true;
  return CA_OK;
}

int chunk_attn_profile_select(uint32_t kernel_mask) {
  ca::ProfState& s = ca::prof();
  std::lock_guard<std::mutex> g(s.mu);
  s.mask = kernel_mask;
  return CA_OK;
}

int chunk_attn_profile_stop(void) {
  ca::ProfState& s = ca::prof();
  std::lock_guard<std::mutex> g(s.mu);
  s.on = false;
  return CA_OK;
}

int chunk_attn_profile_read(int32_t kernel, int64_t* launches, double* total_ms) {
  if (kernel < 0 || kernel >= CA_KERNEL_COUNT) return fail(CA_ERR_SHAPE, "kernel id %d", kernel);
  if (!launches || !total_ms) return fail(CA_ERR_NULL, "profile_read: NULL output");
  ca::ProfState& s = ca::prof();
  std::lock_guard<std::mutex> g(s.mu);
  int64_t n = 0;
  double ms = 0.0;
  for (const ca::ProfRec& r : s.recs) {
    if (r.kernel != kernel || !r.b) continue;
    hipError_t e = hipEventSynchronize(r.b);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "profile_read");
    ++n;
    ms += t;
  }
  *launches = n;
  *total_ms = ms;
  return CA_OK;
}

}  // extern "C"

// ---- SpaCO over a stack of attention layers --------------------------------
namespace {

// Chunk-local buffers in the stack workspace, each on a 256-byte boundary.
struct StackWs {
  size_t hbuf, q, o, lse, dout, dq, dh_a, dh_b, attn_ws, attn_bytes, proj_ws, total;
  size_t h_stride, q_stride, lse_stride;  // per-layer strides (bytes)
};

StackWs stack_ws(const chunk_attn_desc* d, int32_t L) {
  const size_t B = d->batch, C = d->chunk_len, Hq = d->n_q_heads, hd = d->head_dim;
  const size_t dm = Hq * hd, es = d->dtype == CA_BF16 ? 2 : 4;
  StackWs w{};
  w.h_stride = round_up(B * C * dm * es);
  w.q_stride = round_up(B * Hq * C * hd * es);
  w.lse_stride = round_up(B * Hq * C * 4);
  size_t at = 0;
  w.hbuf = at;
  at += w.h_stride * (size_t)std::max(L - 1, 1);
  w.q = at;
  at += w.q_stride * L;
  w.o = at;
  at += w.q_stride * L;
  w.lse = at;
  at += w.lse_stride * L;
  w.dout = at;
  at += w.q_stride;
  w.dq = at;
  at += round_up(B * Hq * C * hd * 4);
  w.dh_a = at;
  at += round_up(B * C * dm * 4);
  w.dh_b = at;
  at += round_up(B * C * dm * 4);
  w.attn_ws = at;
  // the attention backward's row statistics (its dQ passes recompute dS)
  w.attn_bytes = delta_bytes(d);
  at += w.attn_bytes;
  w.proj_ws = at;
  ca::ProjShape ps = proj_shape(d, (int32_t)dm, d->chunk_len, 0);
  at += round_up(ca::proj_bwd_ws_bytes(ps));
  w.total = at;
  return w;
}

int check_stack(const chunk_attn_desc* d, int32_t seq_len, int32_t L, const spaco_layer* layers, const void* h0,
                int32_t h_capacity, bool backward) {
  int rc = check_desc(d, true);
  if (rc) return rc;
  if (L < 1 || L > 4096) return fail(CA_ERR_SHAPE, "n_layers %d", L);
  if (!layers) return fail(CA_ERR_NULL, "layers is NULL");
  const int64_t dm = (int64_t)d->n_q_heads * d->head_dim;
  if (dm % 64 != 0 || dm > 65536) return fail(CA_ERR_SHAPE, "d_model = n_q_heads * head_dim = %lld", (long long)dm);
  if (d->q_capacity < d->chunk_len) return fail(CA_ERR_SHAPE, "q_capacity %d < chunk_len", d->q_capacity);
  if (seq_len < 1 || seq_len > d->kv_capacity || seq_len > h_capacity)
    return fail(CA_ERR_SHAPE, "seq_len %d must be in [1, min(kv_capacity, h_capacity)]", seq_len);
  if ((int64_t)d->batch * h_capacity * dm > ((int64_t)1 << 40)) return fail(CA_ERR_SHAPE, "h too large");
  if ((rc = check_ptrs({h0}))) return rc;
  for (int32_t l = 0; l < L; ++l) {
    const spaco_layer& y = layers[l];
    if ((rc = check_ptrs({y.wq, y.wk, y.wv, y.k_cache, y.v_cache}))) return rc;
    if (backward && (rc = check_ptrs({y.dk_acc, y.dv_acc, y.dwq, y.dwk, y.dwv}))) return rc;
  }
  return CA_OK;
}

// Shapes for layer-local launches on chunk j (rows [s, s + len)).
ca::Shape stack_attn_shape(const chunk_attn_desc* d, int32_t s, int32_t len) {
  ca::Shape a = shape_of(d);
  a.q_cap = d->chunk_len;
  a.q_off = 0;
  a.start = s;
  a.len = len;
  return a;
}
ca::ProjShape stack_proj_shape(const chunk_attn_desc* d, int32_t l, int32_t h_capacity, int32_t s, int32_t len) {
  ca::ProjShape p = proj_shape(d, d->n_q_heads * d->head_dim, l == 0 ? h_capacity : d->chunk_len, l == 0 ? s : 0);
  p.q_cap = d->chunk_len;
  p.q_off = 0;
  p.kv_cap = d->kv_capacity;
  p.start = s;
  p.len = len;
  return p;
}

// Chunk j through every layer: Q/K/V (K, V into the caches), attention, and
// the residual sum feeding the next layer. Leaves each layer's Q, O, LSE and
// input rows in the workspace for a following backward.
hipError_t stack_chunk_forward(const chunk_attn_desc* d, int32_t L, const spaco_layer* layers, const void* h0,
                               int32_t h_capacity, int32_t s, int32_t len, char* ws, const StackWs& w,
                               hipStream_t st) {
  for (int32_t l = 0; l < L; ++l) {
    const spaco_layer& y = layers[l];
    const void* hin = l == 0 ? h0 : (const void*)(ws + w.hbuf + (size_t)(l - 1) * w.h_stride);
    void* q = ws + w.q + (size_t)l * w.q_stride;
    void* o = ws + w.o + (size_t)l * w.q_stride;
    float* lse = (float*)(ws + w.lse + (size_t)l * w.lse_stride);
    hipError_t e = ca::launch_proj_fwd(stack_proj_shape(d, l, h_capacity, s, len), hin, y.wq, y.wk, y.wv, q,
                                       y.k_cache, y.v_cache, st);
    if (e == hipSuccess) e = ca::launch_fwd(stack_attn_shape(d, s, len), q, y.k_cache, y.v_cache, o, lse, st);
    if (e == hipSuccess && l + 1 < L) {
      ca::ResidualShape r{d->batch, d->n_q_heads, d->head_dim, len, d->dtype,
                          l == 0 ? h_capacity : d->chunk_len, l == 0 ? s : 0, d->chunk_len, 0, d->chunk_len, 0};
      e = ca::launch_residual_fwd(r, hin, o, ws + w.hbuf + (size_t)l * w.h_stride, st);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t spaco_stack_workspace_size(const chunk_attn_desc* d, int32_t n_layers) {
  if (check_desc(d, true) != CA_OK || n_layers < 1 || n_layers > 4096) return 0;
  if (((int64_t)d->n_q_heads * d->head_dim) % 64 != 0) return 0;
  return stack_ws(d, n_layers).total;
}

int spaco_stack_forward(const chunk_attn_desc* d, int32_t seq_len, int32_t n_layers, const spaco_layer* layers,
                        const void* h0, int32_t h_capacity, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_stack(d, seq_len, n_layers, layers, h0, h_capacity, false);
  if (rc) return rc;
  const StackWs w = stack_ws(d, n_layers);
  if ((rc = check_ws(ws, ws_bytes, w.total))) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int32_t C = d->chunk_len;
  for (int32_t s = 0; s < seq_len; s += C) {
    hipError_t e = stack_chunk_forward(d, n_layers, layers, h0, h_capacity, s, std::min(C, seq_len - s),
                                       (char*)ws, w, st);
    if (e != hipSuccess) return hip_fail(e, "spaco_stack_forward");
  }
  return CA_OK;
}

int spaco_stack_backward(const chunk_attn_desc* d, int32_t seq_len, int32_t n_layers, const spaco_layer* layers,
                         const void* h0, const float* dy, float* dh0, int32_t h_capacity, const int32_t* chunks,
                         int32_t n_chunks, float relay_factor, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_stack(d, seq_len, n_layers, layers, h0, h_capacity, true);
  if (rc) return rc;
  if ((rc = check_ptrs({dy, dh0}))) return rc;
  if (!chunks) return fail(CA_ERR_NULL, "chunks is NULL");
  if (!(relay_factor == relay_factor) || relay_factor > 3.0e38f || relay_factor < -3.0e38f)
    return fail(CA_ERR_SHAPE, "relay_factor is not finite");
  const int32_t C = d->chunk_len;
  const int32_t kch = (int32_t)(((int64_t)seq_len + C - 1) / C);
  if (n_chunks < 1 || n_chunks > kch) return fail(CA_ERR_SHAPE, "n_chunks %d not in [1, %d]", n_chunks, kch);
  std::vector<int32_t> order(chunks, chunks + n_chunks);
  std::sort(order.begin(), order.end());
  for (int32_t i = 0; i < n_chunks; ++i) {
    if (order[i] < 0 || order[i] >= kch) return fail(CA_ERR_SHAPE, "chunk index %d out of [0, %d)", order[i], kch);
    if (i > 0 && order[i] == order[i - 1]) return fail(CA_ERR_SHAPE, "chunk index %d repeated", order[i]);
  }
  const StackWs w = stack_ws(d, n_layers);
  if ((rc = check_ws(ws, ws_bytes, w.total))) return rc;

  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const int32_t L = n_layers, B = d->batch, Hq = d->n_q_heads, Hkv = d->n_kv_heads, hd = d->head_dim;
  const int32_t dm = Hq * hd;
  const size_t nkv = (size_t)B * Hkv * d->kv_capacity * hd;
  hipError_t e = hipSuccess;
  for (int32_t l = 0; l < L && e == hipSuccess; ++l) {
    e = ca::launch_zero(layers[l].dk_acc, nkv, st);
    if (e == hipSuccess) e = ca::launch_zero(layers[l].dv_acc, nkv, st);
  }
  if (e != hipSuccess) return hip_fail(e, "spaco_stack_backward zero");

  void* dout = wsb + w.dout;
  float* dq = (float*)(wsb + w.dq);
  float* dh_cur = (float*)(wsb + w.dh_a);
  float* dh_nxt = (float*)(wsb + w.dh_b);
  for (int32_t idx = n_chunks - 1; idx >= 0; --idx) {
    const int32_t s = order[idx] * C, len = std::min(C, seq_len - s);
    // rebuild the chunk's graph from the caches
    e = stack_chunk_forward(d, L, layers, h0, h_capacity, s, len, wsb, w, st);
    if (e != hipSuccess) return hip_fail(e, "spaco_stack_backward rebuild");
    for (int32_t l = L - 1; l >= 0; --l) {
      const spaco_layer& y = layers[l];
      const void* hin = l == 0 ? h0 : (const void*)(wsb + w.hbuf + (size_t)(l - 1) * w.h_stride);
      const void* q = wsb + w.q + (size_t)l * w.q_stride;
      const void* o = wsb + w.o + (size_t)l * w.q_stride;
      const float* lse = (const float*)(wsb + w.lse + (size_t)l * w.lse_stride);
      // relay: what later drawn chunks accumulated in this chunk's cache rows
      if (relay_factor != 1.f) {
        const size_t off = (size_t)s * hd;
        e = ca::launch_accumulate(y.dk_acc + off, y.dk_acc + off, B, Hkv, d->kv_capacity, d->kv_capacity, hd, len,
                                  relay_factor - 1.f, st);
        if (e == hipSuccess)
          e = ca::launch_accumulate(y.dv_acc + off, y.dv_acc + off, B, Hkv, d->kv_capacity, d->kv_capacity, hd, len,
                                    relay_factor - 1.f, st);
      }
      // dO_l = dH_{l+1} of the chunk's rows (dy at the top)
      const bool top = l == L - 1;
      const float* src = top ? dy : dh_cur;
      const int32_t src_cap = top ? h_capacity : C, src_off = top ? s : 0;
      if (e == hipSuccess) {
        ca::ResidualShape r{B, Hq, hd, len, d->dtype, src_cap, src_off, 0, 0, C, 0};
        e = ca::launch_residual_bwd(r, src, dout, st);
      }
      if (e == hipSuccess)
        e = ca::launch_bwd(stack_attn_shape(d, s, len), q, y.k_cache, y.v_cache, o, lse, dout, 1.f, dq, y.dk_acc,
                           y.dv_acc, (float*)(wsb + w.attn_ws), w.attn_bytes, st);
      // dH_l = dH_{l+1} + (dQ W_q^T + dK W_k^T + dV W_v^T) over the chunk's rows
      float* dst = l == 0 ? dh0 : dh_nxt;
      const int32_t dst_cap = l == 0 ? h_capacity : C, dst_off = l == 0 ? s : 0;
      if (e == hipSuccess)
        e = ca::launch_proj_bwd(stack_proj_shape(d, l, h_capacity, s, len), hin, y.wq, y.wk, y.wv, dq, y.dk_acc,
                                y.dv_acc, y.dwq, y.dwk, y.dwv, dst, wsb + w.proj_ws, st);
      if (e == hipSuccess)
        e = ca::launch_accumulate(dst + (size_t)dst_off * dm, src + (size_t)src_off * dm, B, 1, dst_cap, src_cap, dm,
                                  len, 1.f, st);
      if (e != hipSuccess) return hip_fail(e, "spaco_stack_backward layer");
      if (l > 0) std::swap(dh_cur, dh_nxt);
    }
  }
  return CA_OK;
}

}  // extern "C"

// ---- Streamed language-model head ------------------------------------------
namespace {

int check_head(const lm_head_desc* d) {
  if (!d) return fail(CA_ERR_NULL, "lm_head descriptor is NULL");
  if (d->dtype != CA_BF16) {
    if (d->dtype != CA_F32) return fail(CA_ERR_DTYPE, "dtype %d", d->dtype);
    return fail(CA_ERR_UNSUPPORTED, "lm_head: only bf16 storage is supported");
  }
  if (d->batch < 1 || d->batch > 65535 || d->seq_capacity < 1) return fail(CA_ERR_SHAPE, "batch/seq_capacity");
  if (d->d_model < 64 || d->d_model > 65536 || d->d_model % 64 != 0)
    return fail(CA_ERR_SHAPE, "d_model %d (a multiple of 64 in [64, 65536])", d->d_model);
  if (d->vocab < 64 || d->vocab % 64 != 0 || d->vocab > (1 << 24))
    return fail(CA_ERR_SHAPE, "vocab %d (a multiple of 64 up to 2^24)", d->vocab);
  if ((int64_t)d->batch * d->seq_capacity * d->d_model > ((int64_t)1 << 40) ||
      (int64_t)d->vocab * d->d_model > ((int64_t)1 << 40))
    return fail(CA_ERR_SHAPE, "lm_head tensors too large");
  return CA_OK;
}

ca::HeadShape head_shape(const lm_head_desc* d, int32_t row_start, int32_t rows, int32_t ps, int32_t group) {
  ca::HeadShape s;
  s.ps = ps;
  s.group = group;
  s.batch = d->batch;
  s.capacity = d->seq_capacity;
  s.d_model = d->d_model;
  s.vocab = d->vocab;
  s.row_start = row_start;
  s.rows = rows;
  return s;
}

}  // namespace

extern "C" {

int lm_head_transpose(const lm_head_desc* d, const void* w, void* wt, void* stream) {
  int rc = check_head(d);
  if (rc) return rc;
  if ((rc = check_ptrs({w, wt}))) return rc;
  hipError_t e = ca::launch_head_transpose(head_shape(d, 0, 1, 1, 1), w, wt, (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "lm_head_transpose launch");
}

size_t lm_head_sft_workspace_size(const lm_head_desc* d, int32_t rows) {
  if (check_head(d) != CA_OK || rows < 1 || (int64_t)d->batch * rows > 65535 * 64) return 0;
  return ca::head_ws_bytes(head_shape(d, 0, rows, rows, 1));
}

int lm_head_sft_partition(const lm_head_desc* d, int32_t row_start, int32_t rows, const void* h, const void* w,
                          const void* wt, const int32_t* labels, const float* row_weight, float loss_scale,
                          float* row_loss, float* dh, float* dw, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_head(d);
  if (rc) return rc;
  if ((rc = check_ptrs({h, w, wt, labels, row_loss, dh, dw}))) return rc;
  if (rows < 1 || row_start < 0 || (int64_t)row_start + rows > d->seq_capacity ||
      (int64_t)d->batch * rows > 65535 * 64)
    return fail(CA_ERR_SHAPE, "partition rows [%d, %lld) outside seq_capacity %d", row_start,
                (long long)row_start + rows, d->seq_capacity);
  if (!(loss_scale == loss_scale) || loss_scale > 3.0e38f || loss_scale < -3.0e38f)
    return fail(CA_ERR_SHAPE, "loss_scale is not finite");
  const ca::HeadShape s = head_shape(d, row_start, rows, rows, 1);
  if ((rc = check_ws(ws, ws_bytes, ca::head_ws_bytes(s)))) return rc;
  if (row_weight && (rc = check_ptrs({row_weight}))) return rc;
  hipError_t e = ca::launch_head_sft(s, h, w, wt, labels, row_weight, loss_scale, row_loss, dh, dw, ws,
                                     (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "lm_head_sft_partition launch");
}

size_t lm_head_sft_sweep_workspace_size(const lm_head_desc* d, int32_t ps, int32_t dw_group) {
  if (check_head(d) != CA_OK || ps < 1 || dw_group < 1 || (int64_t)ps * dw_group > (1 << 20) ||
      (int64_t)d->batch * ps * dw_group > (int64_t)1 << 26)
    return 0;
  return ca::head_ws_bytes(head_shape(d, 0, ps, ps, dw_group));
}

int lm_head_sft_sweep(const lm_head_desc* d, int32_t seq_len, int32_t ps, int32_t dw_group, const void* h,
                      const void* w, const void* wt, const int32_t* labels, const float* row_weight,
                      float loss_scale, float* row_loss, float* dh, float* dw, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_head(d);
  if (rc) return rc;
  if ((rc = check_ptrs({h, w, wt, labels, row_loss, dh, dw}))) return rc;
  if (seq_len < 1 || seq_len > d->seq_capacity) return fail(CA_ERR_SHAPE, "seq_len %d outside [1, %d]", seq_len,
                                                          d->seq_capacity);
  if (ps < 1 || dw_group < 1 || (int64_t)ps * dw_group > (1 << 20) ||
      (int64_t)d->batch * ps * dw_group > (int64_t)1 << 26)
    return fail(CA_ERR_SHAPE, "ps %d, dw_group %d", ps, dw_group);
  if (!(loss_scale == loss_scale) || loss_scale > 3.0e38f || loss_scale < -3.0e38f)
    return fail(CA_ERR_SHAPE, "loss_scale is not finite");
  const ca::HeadShape s = head_shape(d, 0, seq_len, ps, dw_group);
  if ((rc = check_ws(ws, ws_bytes, ca::head_ws_bytes(s)))) return rc;
  if (row_weight && (rc = check_ptrs({row_weight}))) return rc;
  hipError_t e = ca::launch_head_sft(s, h, w, wt, labels, row_weight, loss_scale, row_loss, dh, dw, ws,
                                     (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "lm_head_sft_sweep launch");
}

int lm_head_dpo_finish(const lm_head_desc* d, int32_t seq_len, const float* row_loss, float ref_logp_chosen,
                       float ref_logp_rejected, float beta, float* dh, float* dw, float* loss_out, float* c_out,
                       void* stream) {
  int rc = check_head(d);
  if (rc) return rc;
  if ((rc = check_ptrs({row_loss, dh, dw}))) return rc;
  if (!loss_out || !c_out) return fail(CA_ERR_NULL, "lm_head_dpo_finish: NULL output");
  if (d->batch != 2) return fail(CA_ERR_SHAPE, "DPO needs batch 2 (chosen, rejected), got %d", d->batch);
  if (seq_len < 1 || seq_len > d->seq_capacity) return fail(CA_ERR_SHAPE, "seq_len %d", seq_len);
  if (!(beta == beta) || !(ref_logp_chosen == ref_logp_chosen) || !(ref_logp_rejected == ref_logp_rejected))
    return fail(CA_ERR_SHAPE, "beta / reference log-probabilities must be numbers");
  hipStream_t st = (hipStream_t)stream;
  std::vector<float> rl((size_t)2 * d->seq_capacity);
  hipError_t e = hipMemcpyAsync(rl.data(), row_loss, rl.size() * sizeof(float), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "lm_head_dpo_finish copy");
  double lp[2] = {0.0, 0.0};
  for (int b = 0; b < 2; ++b)
    for (int32_t t = 0; t < seq_len; ++t) lp[b] -= rl[(size_t)b * d->seq_capacity + t];
  const double margin = (lp[0] - ref_logp_chosen) - (lp[1] - ref_logp_rejected);
  const double x = -beta * margin;  // loss = log(1 + e^x), c = beta * sigmoid(x)
  *loss_out = (float)(x > 0 ? x + std::log1p(std::exp(-x)) : std::log1p(std::exp(x)));
  const double c = beta / (1.0 + std::exp(-x));
  *c_out = (float)c;
  // scale in place: acc += (c - 1) * acc
  e = ca::launch_accumulate(dh, dh, 2, 1, d->seq_capacity, d->seq_capacity, d->d_model, seq_len, (float)(c - 1.0), st);
  if (e == hipSuccess)
    e = ca::launch_accumulate(dw, dw, 1, 1, d->vocab, d->vocab, d->d_model, d->vocab, (float)(c - 1.0), st);
  return e == hipSuccess ? CA_OK : hip_fail(e, "lm_head_dpo_finish scale");
}

}  // extern "C"
