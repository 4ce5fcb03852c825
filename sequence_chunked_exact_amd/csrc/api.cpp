// C-ABI layer: argument checks (all before any device call), workspace sizing,
// the SpaCO chunk selector and the sparse backward driver. Kernels live in
// attention.hip and projection.hip; this file only validates and enqueues.
#include "chunk_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
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
// Launch timing: HIP events recorded on the launching stream around each
// kernel while profiling is on. Events come from a reusable pool.
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
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<ProfRec> recs;
};
ProfState& prof() {
  static ProfState s;
  return s;
}
thread_local long t_pending = -1;

hipEvent_t take_event(ProfState& s) {
  if (s.used == s.pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    s.pool.push_back(e);
  }
  return s.pool[s.used++];
}
}  // namespace

void prof_begin(int kernel, hipStream_t st) {
  ProfState& s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  t_pending = -1;
  if (!s.on) return;
  hipEvent_t a = take_event(s);
  if (!a || hipEventRecord(a, st) != hipSuccess) return;
  s.recs.push_back({kernel, a, nullptr});
  t_pending = (long)s.recs.size() - 1;
}

void prof_end(int kernel, hipStream_t st) {
  ProfState& s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on || t_pending < 0 || t_pending >= (long)s.recs.size() || s.recs[t_pending].kernel != kernel) return;
  hipEvent_t b = take_event(s);
  if (b && hipEventRecord(b, st) == hipSuccess) s.recs[t_pending].b = b;
  t_pending = -1;
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
  if (check_desc(d, op == CA_OP_SPARSE_BWD) != CA_OK) return 0;
  switch (op) {
    case CA_OP_FWD: return 0;
    case CA_OP_BWD:
    case CA_OP_SPARSE_BWD: return delta_bytes(d);
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
                                (float*)ws, (hipStream_t)stream);
  return e == hipSuccess ? CA_OK : hip_fail(e, "chunk_attn_bwd launch");
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
  hipError_t e = ca::launch_zero(dq, nq, st);
  if (e == hipSuccess) e = ca::launch_zero(dk, nkv, st);
  if (e == hipSuccess) e = ca::launch_zero(dv, nkv, st);
  if (e != hipSuccess) return hip_fail(e, "sparse_chunk_bwd zero");

  ca::Shape s = shape_of(d);
  for (int32_t idx = t - 1; idx >= 0; --idx) {
    const int32_t i = sel[idx];
    s.start = i * C;
    s.q_off = i * C;
    s.len = std::min(C, seq_len - i * C);
    e = ca::launch_bwd(s, q, k, v, o, lse, dout, gamma, dq, dk, dv, (float*)ws, st);
    if (e != hipSuccess) return hip_fail(e, "sparse_chunk_bwd chunk launch");
  }
  std::memcpy(selected_out, sel.data(), sizeof(int32_t) * t);
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
