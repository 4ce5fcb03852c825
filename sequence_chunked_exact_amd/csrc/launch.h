// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels
// (attention.hip, projection.hip, stack.hip, lm_head.hip). Arguments are
// already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ca {

struct Shape {
  int batch, hq, hkv, head_dim;
  int kv_cap, q_cap, q_off;
  int start, len;       // chunk: first global position and number of rows
  float scale;          // softmax scale
  int dtype;            // CA_F32 / CA_BF16
  // Backward: the dk/dv rows of the prefix are stored, not added to (the
  // caller's accumulators hold nothing yet, e.g. a sweep's first launch).
  bool acc_store = false;
};

// Forward: o, lse for the chunk's rows.
hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v, void* o,
                      float* lse, hipStream_t st);

// Backward workspace: two float arrays of batch*hq*len rows (row delta and
// LSE*log2(e)), each starting on a 256-byte boundary; this much is required.
inline size_t bwd_ws_stride(size_t rows) { return (rows + 63) / 64 * 64; }
inline size_t bwd_ws_bytes(size_t rows) { return 2 * bwd_ws_stride(rows) * sizeof(float); }
// Optional, after the required part rounded up to 256 bytes (bf16 only): the
// chunk's dS^T in blocks of 128 query rows, [batch*hq][len/128][keys][128],
// keys padded to 128, for a dQ pass that reads dS instead of recomputing it.
constexpr int kDsCols = 128, kDsKeyPad = 128;
inline size_t bwd_ws_base(size_t rows) { return (bwd_ws_bytes(rows) + 255) / 256 * 256; }
inline size_t bwd_ds_bytes(size_t batch, size_t hq, size_t len, size_t keys) {
  return batch * hq * ((len + kDsCols - 1) / kDsCols) * ((keys + kDsKeyPad - 1) / kDsKeyPad * kDsKeyPad) *
         kDsCols * 2;
}

// Row statistics of another chunk of the same tensors (rows [q_off, q_off +
// len) of o, dout and lse), written to `ws` laid out as the required part of
// a backward workspace for that chunk; len == 0: none.
struct NextStats {
  int q_off = 0, len = 0;
  float* ws = nullptr;
};

// Backward: row statistics into the workspace (unless stats_ready: a previous
// launch on the stream put them there), then dq (overwritten, times
// grad_scale) and the dk/dv accumulators (incremented). ws_bytes decides the
// dQ pass: with room for the dS^T blocks after the required part (bf16), the
// dK/dV pass stores dS and dQ = dS K streams it; otherwise dQ recomputes dS,
// in the same launch as dK/dV. `next`, if given, is computed by the same
// launch (by a launch of its own on the dS path).
hipError_t launch_bwd(const Shape& s, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, float grad_scale,
                      float* dq, float* dk, float* dv, float* ws, size_t ws_bytes, hipStream_t st,
                      bool stats_ready = false, const NextStats& next = NextStats{});

// Allocation-free backward: the row statistics live in a static device array
// of kScratchBytes per device (attention.hip). scratch_address() returns the
// current device's copy (looked up once per device with hipGetSymbolAddress).
constexpr size_t kScratchBytes = size_t(8) << 20;
hipError_t scratch_address(void** ptr);

// acc[b][h][r][:] += scale * src[b][h][r][:], r < rows.
hipError_t launch_accumulate(float* acc, const float* src, int batch, int heads, int acc_cap,
                             int src_cap, int head_dim, int rows, float scale, hipStream_t st);

// Launch timing: while profiling is on and selects `kernel`, a start/stop
// event pair (from a reusable pool) recorded for one launch, which the
// launch hands to the dispatch (CA_LAUNCH in timed_launch.h); both null
// otherwise.
struct ProfPair {
  hipEvent_t a, b;
};
ProfPair prof_launch(int kernel);

// Projections around one chunk's attention. h is [batch][h_cap][d_model]
// (rows h_off.. are the chunk's positions); wq is [d_model][hq*head_dim], wk and
// wv [d_model][hkv*head_dim]; q, k, v, dq, dk, dv use the attention layout
// (chunk rows at q_off in the q-side tensors, at start in k, v, dk, dv).
struct ProjShape {
  int batch, d_model, hq, hkv, head_dim;
  int h_cap, h_off, q_cap, q_off, kv_cap, start, len;
  int dtype;
};
// q, k, v rows of the chunk = H^(i) W (written in dtype).
hipError_t launch_proj_fwd(const ProjShape& s, const void* h, const void* wq, const void* wk, const void* wv,
                           void* q, void* k, void* v, hipStream_t st);
// dW += H^(i)^T G for G = dq, dk, dv rows of the chunk; dh rows of the chunk
// = dq wq^T + dk wk^T + dv wv^T (float32). ws: proj_bwd_ws_bytes(s, wt != 0)
// bytes, 256-byte aligned (bf16 layers hold the chunk's gradients there as
// bf16, and the weights' transpose unless wt gives it).
size_t proj_bwd_ws_bytes(const ProjShape& s, bool have_wt = false);
hipError_t launch_proj_bwd(const ProjShape& s, const void* h, const void* wq, const void* wk, const void* wv,
                           const float* dq, const float* dk, const float* dv, float* dwq, float* dwk, float* dwv,
                           float* dh, void* ws, hipStream_t st, const void* wt = nullptr);
// W_cat^T = [wq | wk | wv]^T of a bf16 layer into out (proj_wt_bytes(s) bytes;
// 0 for float32 layers, which need none).
size_t proj_wt_bytes(const ProjShape& s);
hipError_t launch_proj_wt(const ProjShape& s, const void* wq, const void* wk, const void* wv, void* out,
                          hipStream_t st);

// Residual connections of a layer stack over one chunk's rows (d_model =
// hq * head_dim). Row-major operands are [batch][cap][d_model] with the chunk
// at row `off`; the per-head operand is [batch][hq][o_cap][head_dim] at row
// o_off.
struct ResidualShape {
  int batch, hq, head_dim, len, dtype;
  int a_cap, a_off;  // h_in (forward) or dh (backward, float32)
  int c_cap, c_off;  // h_out (forward)
  int o_cap, o_off;  // o (forward) or dout (backward)
};
// h_out = h_in + o (heads side by side), in dtype.
hipError_t launch_residual_fwd(const ResidualShape& s, const void* h_in, const void* o, void* h_out, hipStream_t st);
// dout = dh (float32, row-major) in the per-head layout, in dtype.
hipError_t launch_residual_bwd(const ResidualShape& s, const float* dh, void* dout, hipStream_t st);

// Language-model head over one partition of positions [row_start, +rows) of
// h [batch][capacity][d_model] (bf16); w [vocab][d_model], wt = w^T.
struct HeadShape {
  int batch, capacity, d_model, vocab;
  int row_start, rows;  // positions covered: [row_start, row_start + rows)
  int ps, group;        // partition size; partitions per weight-gradient update
};
size_t head_ws_bytes(const HeadShape& s);
hipError_t launch_head_transpose(const HeadShape& s, const void* w, void* wt, hipStream_t st);
hipError_t launch_head_sft(const HeadShape& s, const void* h, const void* w, const void* wt, const int* labels,
                           const float* weight, float scale, float* row_loss, float* dh, float* dw, void* ws,
                           hipStream_t st);

// Fill n floats with zero (a kernel, so it is safe inside captured graphs).
hipError_t launch_zero(float* p, size_t n, hipStream_t st);

}  // namespace ca
