// Residual connections of an attention-layer stack, per chunk (gfx950).
//
// In the layer stack the heads' outputs, side by side, are added to the
// layer's input: H_{l+1} = H_l + O_l with O_l of [batch][Hq][rows][d] read as
// [rows][Hq*d]. A gradient relayed into a chunk's cache reaches the layer
// below through this sum and through the projections (SeCO/SpaCO review,
// "Assumptions": cache gradients move between chunks only from one layer to
// the next). The backward gives the attention's output gradient
// the same per-head layout: dO_l = dH_{l+1} (float32 in, the layer's storage
// type out). Both are memory-bound layout passes over one chunk's rows, four
// elements per thread.
#include "device_common.h"
#include "timed_launch.h"

namespace ca {
namespace {

template <typename T>
struct Vec4;
template <>
struct Vec4<bf16> {
  using type = bf16x4;
};
template <>
struct Vec4<float> {
  using type = f32x4;
};

struct ResidualParams {
  const void* a;  // forward: H_l rows; backward: dH_{l+1} rows (float32)
  long long a_bs;
  const void* o;  // forward: O_l rows
  void* c;        // forward: H_{l+1} rows; backward: dO_l rows
  long long c_bs;
  long long o_hs, o_bs;  // per-head operand strides (forward: o; backward: c)
  int batch, hq, d, len;
};

template <typename T>
__global__ __launch_bounds__(256) void residual_fwd_kernel(ResidualParams p) {
  using V = typename Vec4<T>::type;
  const int dm = p.hq * p.d, per_row = dm / 4;
  const long long total = (long long)p.batch * p.len * per_row;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int col = (int)(i % per_row) * 4;
    const long long br = i / per_row;
    const int r = (int)(br % p.len), b = (int)(br / p.len);
    const V x = *(const V*)((const T*)p.a + b * p.a_bs + (long long)r * dm + col);
    const V y = *(const V*)((const T*)p.o + b * p.o_bs + (col / p.d) * p.o_hs + (long long)r * p.d + col % p.d);
    V z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = (T)((float)x[e] + (float)y[e]);
    *(V*)((T*)p.c + b * p.c_bs + (long long)r * dm + col) = z;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void residual_bwd_kernel(ResidualParams p) {
  using V = typename Vec4<T>::type;
  const int dm = p.hq * p.d, per_row = dm / 4;
  const long long total = (long long)p.batch * p.len * per_row;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int col = (int)(i % per_row) * 4;
    const long long br = i / per_row;
    const int r = (int)(br % p.len), b = (int)(br / p.len);
    const f32x4 x = *(const f32x4*)((const float*)p.a + b * p.a_bs + (long long)r * dm + col);
    V z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = (T)x[e];
    *(V*)((T*)p.c + b * p.o_bs + (col / p.d) * p.o_hs + (long long)r * p.d + col % p.d) = z;
  }
}

int residual_blocks(const ResidualShape& s) {
  const long long vecs = (long long)s.batch * s.len * s.hq * s.head_dim / 4;
  const long long want = (vecs + 255) / 256;
  return (int)(want < 8192 ? (want > 0 ? want : 1) : 8192);
}

ResidualParams residual_params(const ResidualShape& s) {
  ResidualParams p{};
  const long long dm = (long long)s.hq * s.head_dim;
  p.a_bs = (long long)s.a_cap * dm;
  p.c_bs = (long long)s.c_cap * dm;
  p.o_hs = (long long)s.o_cap * s.head_dim;
  p.o_bs = (long long)s.hq * s.o_cap * s.head_dim;
  p.batch = s.batch;
  p.hq = s.hq;
  p.d = s.head_dim;
  p.len = s.len;
  return p;
}

}  // namespace

hipError_t launch_residual_fwd(const ResidualShape& s, const void* h_in, const void* o, void* h_out, hipStream_t st) {
  const long long dm = (long long)s.hq * s.head_dim;
  const size_t es = s.dtype == CA_BF16 ? sizeof(bf16) : sizeof(float);
  ResidualParams p = residual_params(s);
  p.a = (const char*)h_in + (size_t)s.a_off * dm * es;
  p.o = (const char*)o + (size_t)s.o_off * s.head_dim * es;
  p.c = (char*)h_out + (size_t)s.c_off * dm * es;
  if (s.dtype == CA_BF16) {
    CA_LAUNCH(CA_KERNEL_RESIDUAL, residual_fwd_kernel<bf16>, dim3(residual_blocks(s)), dim3(256), 0, st, p);
  } else {
    CA_LAUNCH(CA_KERNEL_RESIDUAL, residual_fwd_kernel<float>, dim3(residual_blocks(s)), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_residual_bwd(const ResidualShape& s, const float* dh, void* dout, hipStream_t st) {
  const long long dm = (long long)s.hq * s.head_dim;
  const size_t es = s.dtype == CA_BF16 ? sizeof(bf16) : sizeof(float);
  ResidualParams p = residual_params(s);
  p.a = dh + (size_t)s.a_off * dm;
  p.c = (char*)dout + (size_t)s.o_off * s.head_dim * es;
  if (s.dtype == CA_BF16) {
    CA_LAUNCH(CA_KERNEL_RESIDUAL, residual_bwd_kernel<bf16>, dim3(residual_blocks(s)), dim3(256), 0, st, p);
  } else {
    CA_LAUNCH(CA_KERNEL_RESIDUAL, residual_bwd_kernel<float>, dim3(residual_blocks(s)), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace ca
