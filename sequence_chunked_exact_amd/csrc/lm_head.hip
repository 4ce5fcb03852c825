// Language-model head streamed over sequence partitions, supervised
// fine-tuning loss (gfx950). StreamBP streams the head by partitioning the
// logits along the sequence, ps_head positions at a time, the SFT loss being
// separable over positions (StreamBP review, "Core claim"; "Assumptions":
// Eq. (3), ps_head = 100). Per partition of `rows` positions:
//
//   Z  = H W^T                       [rows][vocab] float32     (PG_DH GEMM over W^T)
//   per row: lse = logsumexp(Z), loss = lse - Z[y]; dZ = scale (softmax(Z) - onehot(y))
//                                    [rows_pad][vocab] bf16     (ce_stats_kernel, ce_dz_kernel)
//   dH = dZ W                        float32, overwritten      (PG_DH GEMM over W)
//   dW += dZ^T H                     float32, incremented      (PG_DW GEMM)
//
// Only one partition's logits exist at a time. The weight gradient is added
// once per group of consecutive partitions from their dZ rows (bf16, kept in
// the workspace): added per partition, its float32 read-modify-write (8 bytes
// per weight) dominates the step. W^T [d_model][vocab] is written once per
// step by wt_head_kernel: the logits product reads it along k.
#include <algorithm>

#include "gemm_bf16.h"

namespace ca {
namespace {

struct CeParams {
  const float* z;        // [batch][rows][vocab]
  const int* labels;     // partition's first label of batch entry b at labels + b * lab_bs
  const float* weight;   // per-position gradient weights, same layout (NULL: 1)
  long long lab_bs;
  bf16* dz;              // partition's first dZ row of batch entry b at dz + b * dz_bs
  long long dz_bs;
  float* row_loss;       // partition's first row of batch entry b at row_loss + b * lab_bs
  float* part;           // [batch][rows_pad][nseg] (max, exponential sum) of each row segment
  float scale;
  int rows, rows_pad, vocab, batch;  // rows [rows, rows_pad) of dZ are zeroed
  int nseg;                          // segments per row
};

// Each row's vocabulary runs as nseg segments, one workgroup each, so that a
// partition of ~100 rows still spreads over the whole GPU: a first launch
// finds every segment's maximum and exponential sum, a second combines a
// row's segments (in segment order) into its log-sum-exp and writes the
// segment's dZ.
constexpr int kCeSegMax = 16;
int ce_segments(int vocab) { return std::max(1, std::min(kCeSegMax, vocab / 4 / 1024)); }

struct CeRow {
  int b, r, seg, y;  // y < 0: padding row or not a target
  int v0, v1;        // the segment's 4-element vectors [v0, v1)
};
__device__ __forceinline__ CeRow ce_row(const CeParams& p) {
  CeRow c;
  c.seg = blockIdx.x % p.nseg;
  const int rr = blockIdx.x / p.nseg;
  c.r = rr % p.rows_pad;
  c.b = rr / p.rows_pad;
  c.y = c.r < p.rows ? p.labels[c.b * p.lab_bs + c.r] : -1;
  if (c.y >= p.vocab) c.y = -1;  // not a target
  const int nv = p.vocab / 4;
  c.v0 = (int)((long long)nv * c.seg / p.nseg);
  c.v1 = (int)((long long)nv * (c.seg + 1) / p.nseg);
  return c;
}
// (m, s) and (m2, s2) merged: the exponential sum taken against the larger maximum.
__device__ __forceinline__ void ce_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  s = (m == -kInf ? 0.f : s * fexp2((m - mm) * kLog2e)) + (m2 == -kInf ? 0.f : s2 * fexp2((m2 - mm) * kLog2e));
  m = mm;
}

__global__ __launch_bounds__(256) void ce_stats_kernel(CeParams p) {
  __shared__ float red_m[4], red_s[4];
  const CeRow c = ce_row(p);
  if (c.y < 0) return;  // the dZ launch zeroes such rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* z = p.z + ((long long)c.b * p.rows + c.r) * p.vocab;
  float m = -kInf, s = 0.f;
  for (int i = c.v0 + tid; i < c.v1; i += 256) {
    const f32x4 v = *(const f32x4*)(z + 4 * i);
    const float mv = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    if (mv > m) {
      s *= fexp2((m - mv) * kLog2e);
      m = mv;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s += fexp2((v[e] - m) * kLog2e);
  }
  // reduce (m, s) over the wave, then over the 4 waves
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ce_merge(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
  if (lane == 0) {
    red_m[wave] = m;
    red_s[wave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float M = red_m[0], S = red_s[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) ce_merge(M, S, red_m[w], red_s[w]);
    float* out = p.part + ((long long)(c.b * p.rows_pad + c.r) * p.nseg + c.seg) * 2;
    out[0] = M;
    out[1] = S;
  }
}

__global__ __launch_bounds__(256) void ce_dz_kernel(CeParams p) {
  const CeRow c = ce_row(p);
  const int tid = threadIdx.x;
  bf16* dz = p.dz + c.b * p.dz_bs + (long long)c.r * p.vocab;
  if (c.y < 0) {
    for (int i = c.v0 + tid; i < c.v1; i += 256) *(bf16x4*)(dz + 4 * i) = bf16x4{};
    if (c.r < p.rows && c.seg == 0 && tid == 0) p.row_loss[c.b * p.lab_bs + c.r] = 0.f;
    return;
  }
  const float* part = p.part + (long long)(c.b * p.rows_pad + c.r) * p.nseg * 2;
  float M = part[0], S = part[1];
  for (int k = 1; k < p.nseg; ++k) ce_merge(M, S, part[2 * k], part[2 * k + 1]);
  const float lse = M + __logf(S);
  const float* z = p.z + ((long long)c.b * p.rows + c.r) * p.vocab;
  if (c.seg == 0 && tid == 0) p.row_loss[c.b * p.lab_bs + c.r] = lse - z[c.y];
  const float scale = p.weight ? p.scale * p.weight[c.b * p.lab_bs + c.r] : p.scale;
  for (int i = c.v0 + tid; i < c.v1; i += 256) {
    const f32x4 v = *(const f32x4*)(z + 4 * i);
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float g = fexp2((v[e] - lse) * kLog2e);
      if (4 * i + e == c.y) g -= 1.f;
      o[e] = (bf16)(scale * g);
    }
    *(bf16x4*)(dz + 4 * i) = o;
  }
}

// W^T: out[c][v] = w[v][c], 64 x 64 tiles through LDS, 16-byte accesses.
__global__ __launch_bounds__(256) void wt_head_kernel(const bf16* w, bf16* out, int vocab, int d_model) {
  __shared__ bf16 t[64][64 + 8];
  const int vt = blockIdx.x % (vocab / 64), ct = blockIdx.x / (vocab / 64);
  const int v0 = vt * 64, c0 = ct * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + i * 256, r = idx / 8, c = idx % 8;
    *(bf16x8*)&t[r][c * 8] = *(const bf16x8*)(w + (long long)(v0 + r) * d_model + c0 + c * 8);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + i * 256, r = idx / 8, c = idx % 8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[c * 8 + e][r];
    *(bf16x8*)(out + (long long)(c0 + r) * vocab + v0 + c * 8) = v;
  }
}

// dh rows = sum over the split-k partials [splits][rows][d_model].
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* part, float* dh, int splits, int rows, int dm) {
  const long long n4 = (long long)rows * dm / 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long long)gridDim.x * blockDim.x) {
    f32x4 acc = ((const f32x4*)part)[i];
    for (int s = 1; s < splits; ++s) acc += ((const f32x4*)part)[(long long)s * n4 + i];
    ((f32x4*)dh)[i] = acc;
  }
}

constexpr int kWide = 1 << 30;

// Split of the dH product's k range (the vocabulary, in 64-wide slices) into
// S parts of head_kpart elements, the last one shorter where S does not divide
// the slices: the product has few output tiles (rows x d_model; 32 for a
// 4096-wide model), and 16 splits make them 512 workgroups, two on every
// compute unit. (An exact divisor of the LLaMA3 vocabulary's 2004 slices gave
// at most 12, i.e. 384 workgroups: half the units streamed twice the weight
// rows of the other half.) S is the largest count up to 16 whose parts are
// all non-empty.
int head_splits(int vocab) {
  const int slices = vocab / 64;
  for (int s = 16; s > 1; --s)
    if ((s - 1) * ((slices + s - 1) / s) < slices) return s;
  return 1;
}
int head_kpart(int vocab, int splits) { return (vocab / 64 + splits - 1) / splits * 64; }

}  // namespace

// Workspace: logits [batch][ps][vocab] float32; dZ of a group of partitions
// [batch][pad64(group * ps)][vocab] bf16; split-k partials of dH
// [splits][ps][d_model] float32; the row segments' (max, exponential sum)
// [batch][ps + 64][kCeSegMax] float32 pairs; each on a 256-byte boundary.
size_t head_z_bytes(const HeadShape& s) { return ((size_t)s.batch * s.ps * s.vocab * sizeof(float) + 255) / 256 * 256; }
int head_group_rows(const HeadShape& s) { return pg_rows_pad(s.ps * s.group); }
size_t head_dz_bytes(const HeadShape& s) {
  return ((size_t)s.batch * head_group_rows(s) * s.vocab * sizeof(bf16) + 255) / 256 * 256;
}

size_t head_part_bytes(const HeadShape& s) {
  return ((size_t)head_splits(s.vocab) * s.ps * s.d_model * sizeof(float) + 255) / 256 * 256;
}
size_t head_ws_bytes(const HeadShape& s) {
  return head_z_bytes(s) + head_dz_bytes(s) + head_part_bytes(s) +
         (size_t)s.batch * (s.ps + 64) * kCeSegMax * 2 * sizeof(float);
}

hipError_t launch_head_transpose(const HeadShape& s, const void* w, void* wt, hipStream_t st) {
  CA_LAUNCH(CA_KERNEL_HEAD_AUX, wt_head_kernel, dim3((s.vocab / 64) * (s.d_model / 64)), dim3(256), 0, st,
            (const bf16*)w, (bf16*)wt, s.vocab, s.d_model);
  return hipGetLastError();
}

namespace {

// One partition [s0, s0 + rows): logits, loss rows and dZ (at row `off` of the
// group's dZ buffer, with `zero_to` - rows padding rows zeroed after it), dH.
hipError_t head_partition(const HeadShape& s, int s0, int rows, int off, int zero_to, const void* h,
                          const void* w, const void* wt, const int* labels, const float* weight, float scale,
                          float* row_loss, float* dh, char* ws, hipStream_t st) {
  const int dm = s.d_model, V = s.vocab, grows = head_group_rows(s);
  float* z = (float*)ws;
  bf16* dzg = (bf16*)(ws + head_z_bytes(s));
  float* part = (float*)(ws + head_z_bytes(s) + head_dz_bytes(s));
  const int S = head_splits(V), kpart = head_kpart(V, S), klast = V - (S - 1) * kpart;
  const bf16* hp = (const bf16*)h + (size_t)s0 * dm;

  // Z = H W^T
  ProjGemmParams zp{};
  zp.a = hp;
  zp.a_ld = dm;
  zp.a_bs = (long long)s.capacity * dm;
  zp.b[0] = zp.b[1] = zp.b[2] = (const bf16*)wt;
  zp.b_w[0] = V;
  zp.b_w[1] = zp.b_w[2] = kWide;
  zp.c[0] = z;
  zp.c_rs[0] = V;
  zp.c_bs[0] = (long long)rows * V;
  zp.c_hd[0] = kWide;
  zp.c_w[0] = V;
  zp.c_w[1] = zp.c_w[2] = kWide;
  zp.M = rows;
  zp.N = V;
  zp.K = dm;
  zp.a_rows = rows;
  zp.batch = s.batch;
  hipError_t e = pg_launch<PG_DH>(zp, s.batch, CA_KERNEL_HEAD, st);
  if (e != hipSuccess) return e;

  // per-row loss and dZ
  CeParams cp{};
  cp.z = z;
  cp.labels = labels + s0;
  cp.weight = weight ? weight + s0 : nullptr;
  cp.lab_bs = s.capacity;
  cp.dz = dzg + (size_t)off * V;
  cp.dz_bs = (long long)grows * V;
  cp.row_loss = row_loss + s0;
  cp.scale = scale;
  cp.rows = rows;
  cp.rows_pad = zero_to;
  cp.vocab = V;
  cp.batch = s.batch;
  cp.nseg = ce_segments(V);
  cp.part = (float*)(ws + head_z_bytes(s) + head_dz_bytes(s) + head_part_bytes(s));
  const dim3 ce_grid(s.batch * zero_to * cp.nseg);
  CA_LAUNCH(CA_KERNEL_HEAD_AUX, ce_stats_kernel, ce_grid, dim3(256), 0, st, cp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  CA_LAUNCH(CA_KERNEL_HEAD_AUX, ce_dz_kernel, ce_grid, dim3(256), 0, st, cp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // dH = dZ W, the vocabulary split S ways into partials, then summed
  for (int b = 0; b < s.batch; ++b) {
    ProjGemmParams hq{};
    hq.a = dzg + ((size_t)b * grows + off) * V;
    hq.a_ld = V;
    hq.a_bs = kpart;  // split j reads dZ columns [j kpart, (j + 1) kpart)
    hq.b[0] = hq.b[1] = hq.b[2] = (const bf16*)w;
    hq.b_w[0] = dm;
    hq.b_w[1] = hq.b_w[2] = kWide;
    hq.b_bs = (long long)kpart * dm;  // and W rows of the same range
    hq.c[0] = part;
    hq.c_rs[0] = dm;
    hq.c_bs[0] = (long long)rows * dm;
    hq.c_hd[0] = kWide;
    hq.c_w[0] = dm;
    hq.c_w[1] = hq.c_w[2] = kWide;
    hq.M = rows;
    hq.N = dm;
    hq.K = kpart;
    hq.k_last = klast;
    hq.a_rows = rows;
    hq.batch = S;
    e = pg_launch<PG_DH>(hq, S, CA_KERNEL_HEAD, st);
    if (e != hipSuccess) return e;
    const long long n4 = (long long)rows * dm / 4;
    const int blocks = (int)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
    CA_LAUNCH(CA_KERNEL_HEAD_AUX, splitk_sum_kernel, dim3(blocks), dim3(256), 0, st, part,
              dh + ((size_t)b * s.capacity + s0) * dm, S, rows, dm);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_head_sft(const HeadShape& s, const void* h, const void* w, const void* wt, const int* labels,
                           const float* weight, float scale, float* row_loss, float* dh, float* dw, void* ws,
                           hipStream_t st) {
  const int dm = s.d_model, V = s.vocab, grows = head_group_rows(s);
  const bf16* dzg = (const bf16*)((const char*)ws + head_z_bytes(s));
  const int end = s.row_start + s.rows, span = s.ps * s.group;
  for (int gs = s.row_start; gs < end; gs += span) {
    const int ge = gs + span < end ? gs + span : end;
    for (int s0 = gs; s0 < ge; s0 += s.ps) {
      const int rows = s0 + s.ps < ge ? s.ps : ge - s0;
      const bool last = s0 + rows == ge;
      hipError_t e = head_partition(s, s0, rows, s0 - gs, last ? grows - (s0 - gs) : rows, h, w, wt, labels,
                                    weight, scale, row_loss, dh, (char*)ws, st);
      if (e != hipSuccess) return e;
    }
    // dW += dZ^T H over the group's rows, the batch summed along k
    ProjGemmParams wp{};
    wp.a = dzg;
    wp.a_ld = V;
    wp.a_bs = (long long)grows * V;
    wp.b[0] = wp.b[1] = wp.b[2] = (const bf16*)h + (size_t)gs * dm;
    wp.b_w[0] = dm;
    wp.b_w[1] = wp.b_w[2] = kWide;
    wp.b_bs = (long long)s.capacity * dm;
    wp.c[0] = dw;
    wp.c_rs[0] = dm;
    wp.c_hd[0] = kWide;
    wp.c_w[0] = dm;
    wp.c_w[1] = wp.c_w[2] = kWide;
    wp.M = V;
    wp.N = dm;
    wp.K = grows;
    wp.a_rows = grows;    // dZ rows past the group are zero
    wp.b_rows = ge - gs;  // H rows past the group are not read
    wp.batch = s.batch;
    hipError_t e = pg_launch<PG_DW>(wp, 1, CA_KERNEL_HEAD, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ca
