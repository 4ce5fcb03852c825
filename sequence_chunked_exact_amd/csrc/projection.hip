// Projection GEMMs around the attention of one chunk for gfx950 (CDNA4): the
// QKV projections and their weight and input gradients, float32 accumulation
// on the matrix cores.
//
// bf16 layers use proj_gemm_kernel (gemm_bf16.h): one launch per phase and chunk covers the
// three projections at once, the weights taken side by side as one matrix
// W_cat = [W_q | W_k | W_v] of (Hq + 2 Hkv) d columns:
//   forward  Q|K|V (chunk rows) = H_in^(i) W_cat
//   weights  dW_cat += H_in^(i)^T G_cat
//   input    dH_in^(i) = G_cat W_cat^T
// with G_cat the chunk rows of dQ | dK | dV, first rounded to bf16 in a
// workspace by gcat_kernel (rows up to a multiple of 64, the tail zero), and
// W_cat^T written there by wt_kernel, or handed in by the caller, who wrote it
// once for a whole backward sweep (launch_proj_wt): read along its rows in
// 128-byte pieces, W_cat streamed several times slower than its transpose read
// along k. A
// workgroup of 8 waves owns a 128x128 output tile: two groups of 4 waves (2x2
// waves of 64x64) take the even and odd 64-deep k slices of slice pairs, which
// stream by direct global->LDS loads one pair ahead into two statically named
// buffers, and add their partial tiles through LDS at the end.
//
// float32 layers (the exactness path) use gemm_kernel, which reads every
// operand through a strided view (so per-head [heads][rows][d] tensors take
// part as [rows][heads*d] matrices without copies), one launch per projection.
// A 4-wave workgroup owns a 128x128 output tile (2x2 waves of 64x64); 64-deep
// k slices are staged through registers into double-buffered padded LDS.
//
// Both read an operand whose storage has k along its rows through the
// transposing LDS path and the other with two 8-byte reads per lane, both in
// the tile slot order; outputs are computed as C^T tiles so that a lane holds
// four consecutive columns of one row.

#include "gemm_bf16.h"

namespace ca {
namespace {

struct MatView {
  const void* p;  // element (r, c) of batch b at p + b*bs + r*rs + (c / hd)*hs + c % hd
  long long rs, hs, bs;
  int hd;
};
__device__ __forceinline__ long long mv_index(const MatView& v, int b, int r, int c) {
  return (long long)b * v.bs + (long long)r * v.rs + (long long)(c / v.hd) * v.hs + (c % v.hd);
}

struct GemmParams {
  MatView a, b, c;
  int M, N, K;
  float beta;  // float32 output: c = acc + beta * c (beta 0 overwrites)
};

// 8 source elements at (r, c..c+7) converted to T (zero if `zero`).
template <typename T, typename S>
__device__ __forceinline__ typename Elt<T>::vec8 load8_as(const S* p, bool zero);
template <>
__device__ __forceinline__ bf16x8 load8_as<bf16, bf16>(const bf16* p, bool zero) {
  return zero ? bf16x8{} : *(const bf16x8*)p;
}
template <>
__device__ __forceinline__ bf16x8 load8_as<bf16, float>(const float* p, bool zero) {
  bf16x8 r{};
  if (!zero) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = (bf16)a[i];
      r[4 + i] = (bf16)b[i];
    }
  }
  return r;
}
template <>
__device__ __forceinline__ f32x8 load8_as<float, float>(const float* p, bool zero) {
  f32x8 r{};
  if (!zero) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    r = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void store8(T* lds, const typename Elt<T>::vec8& v);
template <>
__device__ __forceinline__ void store8<bf16>(bf16* lds, const bf16x8& v) {
  *(bf16x8*)lds = v;
}
template <>
__device__ __forceinline__ void store8<float>(float* lds, const f32x8& v) {
  *(f32x4*)lds = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(lds + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// One 64-deep k slice of an operand, staged through registers. MN: the stored
// matrix has k along its rows ([64][128] tile), otherwise along its columns
// ([128][64] tile). Rows or columns past the matrix re-read its last one
// (those outputs are never stored); k past K reads zero.
template <typename T, typename S, bool MN>
struct GemmStage {
  static constexpr int ROWS = MN ? 64 : 128, COLS = MN ? 128 : 64;
  static constexpr int VPR = COLS / 8, NV = ROWS * VPR / 256;  // 8-element vectors
  using Lt = PadLay<T, COLS>;
  typename Elt<T>::vec8 r[NV];
  __device__ __forceinline__ void load(const MatView& v, int b, int mn0, int k0, int MNext, int K, int tid) {
    const S* base = (const S*)v.p;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = tid + i * 256, row = vi / VPR, col = (vi % VPR) * 8;
      int rr, cc;
      bool zero;
      if (MN) {  // rows: k, columns: m or n
        rr = k0 + row;
        cc = min(mn0 + col, MNext - 8);
        zero = rr >= K;
        rr = min(rr, K - 1);
      } else {  // rows: m or n, columns: k
        rr = min(mn0 + row, MNext - 1);
        cc = k0 + col;
        zero = cc >= K;
        cc = min(cc, K - 8);
      }
      r[i] = load8_as<T, S>(base + mv_index(v, b, rr, cc), zero);
    }
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = tid + i * 256;
      store8<T>(lds + Lt::off(vi / VPR, (vi % VPR) * 8), r[i]);
    }
  }
};

template <typename T, typename SA, typename SB, bool A_MN, bool B_MN, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  using E = Elt<T>;
  using frag = typename E::frag;
  using StA = GemmStage<T, SA, A_MN>;
  using StB = GemmStage<T, SB, B_MN>;
  constexpr int TA = StA::ROWS * StA::Lt::RS, TB = StB::ROWS * StB::Lt::RS;
  __shared__ __attribute__((aligned(16))) T As[2][TA];
  __shared__ __attribute__((aligned(16))) T Bs[2][TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 128, m0 = blockIdx.y * 128, b = blockIdx.z;
  const int nk = (p.K + 63) / 64;

  StA sa;
  StB sb;
  sa.load(p.a, b, m0, 0, p.M, p.K, tid);
  sb.load(p.b, b, n0, 0, p.N, p.K, tid);
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  sa.store(As[0], tid);
  sb.store(Bs[0], tid);
  wait_loads();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load(p.a, b, m0, (kt + 1) * 64, p.M, p.K, tid);
      sb.load(p.b, b, n0, (kt + 1) * 64, p.N, p.K, tid);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      frag af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mr = wm * 64 + i * 16;
        af[i] = A_MN ? ldT8<typename StA::Lt>(As[cur], ks * 32, mr, lane)
                     : ld8t<typename StA::Lt>(As[cur], mr + n, ks * 32, g);
        const int nr = wn * 64 + i * 16;
        bfr[i] = B_MN ? ldT8<typename StB::Lt>(Bs[cur], ks * 32, nr, lane)
                      : ld8t<typename StB::Lt>(Bs[cur], nr + n, ks * 32, g);
      }
      // C^T tiles: the n-side fragment is the A operand, so a lane ends up
      // holding 4 consecutive n of one m row (rows 4g..4g+3 of C^T).
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) E::mma(acc[i][j], bfr[j], af[i]);
    }
    if (more) {
      sa.store(As[cur ^ 1], tid);
      sb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // acc[i][j] holds C[m][n .. n+3] for m = m0 + wm*64 + i*16 + (lane % 16),
  // n = n0 + wn*64 + j*16 + 4g (C^T tile rows 4g..4g+3); N is a multiple of 4
  // and a head split never cuts such a group.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 64 + i * 16 + n;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nb = n0 + wn * 64 + j * 16 + 4 * g;
      if (nb >= p.N) continue;
      const long long idx = mv_index(p.c, b, m, nb);
      if (OUT_F32) {
        f32x4* c = (f32x4*)((float*)p.c.p + idx);
        *c = p.beta == 0.f ? acc[i][j] : acc[i][j] + p.beta * *c;
      } else {
        store4<T>((T*)p.c.p + idx, acc[i][j], 1.f);
      }
    }
  }
}

// G_cat[b][r][:] = dQ | dK | dV of chunk row r, rounded to bf16, for r < len;
// zero for len <= r < rows_pad. Eight columns per thread.
struct GcatParams {
  const float* g[3];
  long long g_off[3];  // element offset of the chunk's first row in each head
  long long g_hs[3];   // head stride (capacity * d)
  int heads[3];
  int d, len, rows_pad, ncols, batch;
  bf16* out;
};
__global__ __launch_bounds__(256) void gcat_kernel(GcatParams p) {
  const int c8 = p.ncols / 8;
  const long long total = (long long)p.batch * p.rows_pad * c8;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int col = (int)(i % c8) * 8;
    const long long br = i / c8;
    const int r = (int)(br % p.rows_pad), b = (int)(br / p.rows_pad);
    bf16x8 v{};
    if (r < p.len) {
      const int w0 = p.heads[0] * p.d, w1 = p.heads[1] * p.d;
      const int sg = (col >= w0) + (col >= w0 + w1);
      const int lc = col - (sg > 0 ? w0 : 0) - (sg > 1 ? w1 : 0);
      const float* src = (sg == 0 ? p.g[0] : sg == 1 ? p.g[1] : p.g[2]) +
                         ((long long)b * (sg == 0 ? p.heads[0] : sg == 1 ? p.heads[1] : p.heads[2]) + lc / p.d) *
                             (sg == 0 ? p.g_hs[0] : sg == 1 ? p.g_hs[1] : p.g_hs[2]) +
                         (sg == 0 ? p.g_off[0] : sg == 1 ? p.g_off[1] : p.g_off[2]) + (long long)r * p.d + lc % p.d;
      const f32x4 x = *(const f32x4*)src, y = *(const f32x4*)(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = (bf16)x[e];
        v[4 + e] = (bf16)y[e];
      }
    }
    *(bf16x8*)(p.out + br * p.ncols + col) = v;
  }
}

// W_cat^T[k][n] = W_s[n][k - begin_s] for the three weights side by side
// (k < N = (Hq + 2 Hkv) d, n < d_model): 64 x 64 tiles through LDS, 16-byte
// reads and writes.
struct WtParams {
  const bf16* w[3];
  int w_w[3];
  int d_model, ncols;
  bf16* out;
};
__global__ __launch_bounds__(256) void wt_kernel(WtParams p) {
  __shared__ bf16 t[64][64 + 8];
  const int kt = blockIdx.x % (p.ncols / 64), nt = blockIdx.x / (p.ncols / 64);
  const int k0 = kt * 64, n0 = nt * 64;
  int kl;
  const int sg = seg3(k0, p.w_w, kl);
  const bf16* w = sg == 0 ? p.w[0] : sg == 1 ? p.w[1] : p.w[2];
  const int wd = sg == 0 ? p.w_w[0] : sg == 1 ? p.w_w[1] : p.w_w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + i * 256, r = idx / 8, c = idx % 8;
    *(bf16x8*)&t[r][c * 8] = *(const bf16x8*)(w + (long long)(n0 + r) * wd + kl + c * 8);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + i * 256, r = idx / 8, c = idx % 8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[c * 8 + e][r];
    *(bf16x8*)(p.out + (long long)(k0 + r) * p.d_model + n0 + c * 8) = v;
  }
}

template <typename T, typename SA, typename SB, bool A_MN, bool B_MN, bool OUT_F32>
hipError_t gemm_launch(const GemmParams& p, int batch, hipStream_t st) {
  CA_LAUNCH(CA_KERNEL_PROJ, (gemm_kernel<T, SA, SB, A_MN, B_MN, OUT_F32>),
            dim3((p.N + 127) / 128, (p.M + 127) / 128, batch), dim3(256), 0, st, p);
  return hipGetLastError();
}
constexpr int kNoSplit = 1 << 30;

template <typename T>
hipError_t proj_fwd_impl(const ProjShape& s, const void* h, const void* const w[3], void* const out[3],
                         hipStream_t st) {
  const int d = s.head_dim;
  for (int t = 0; t < 3; ++t) {
    const bool isq = t == 0;
    const int H = isq ? s.hq : s.hkv, cap = isq ? s.q_cap : s.kv_cap, off = isq ? s.q_off : s.start;
    GemmParams p{};
    p.M = s.len;
    p.N = H * d;
    p.K = s.d_model;
    p.a = {(const T*)h + (size_t)s.h_off * s.d_model, s.d_model, 0, (long long)s.h_cap * s.d_model, kNoSplit};
    p.b = {w[t], (long long)H * d, 0, 0, kNoSplit};
    p.c = {(T*)out[t] + (size_t)off * d, d, (long long)cap * d, (long long)H * cap * d, d};
    hipError_t e = gemm_launch<T, T, T, false, true, false>(p, s.batch, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
hipError_t proj_bwd_impl(const ProjShape& s, const void* h, const void* const w[3], const float* const g[3],
                         float* const dw[3], float* dh, hipStream_t st) {
  const int d = s.head_dim;
  for (int t = 0; t < 3; ++t) {
    const bool isq = t == 0;
    const int H = isq ? s.hq : s.hkv, cap = isq ? s.q_cap : s.kv_cap, off = isq ? s.q_off : s.start;
    // dW += H_in^T G over the chunk's rows (one launch per batch entry: the
    // batch is summed into the same weight gradient).
    for (int b = 0; b < s.batch; ++b) {
      GemmParams p{};
      p.M = s.d_model;
      p.N = H * d;
      p.K = s.len;
      p.a = {(const T*)h + ((size_t)b * s.h_cap + s.h_off) * s.d_model, s.d_model, 0, 0, kNoSplit};
      p.b = {g[t] + ((size_t)b * H * cap + off) * d, d, (long long)cap * d, 0, d};
      p.c = {dw[t], (long long)H * d, 0, 0, kNoSplit};
      p.beta = 1.f;
      hipError_t e = gemm_launch<T, T, float, true, true, true>(p, 1, st);
      if (e != hipSuccess) return e;
    }
    // dH (+)= G W^T
    GemmParams p{};
    p.M = s.len;
    p.N = s.d_model;
    p.K = H * d;
    p.a = {g[t] + (size_t)off * d, d, (long long)cap * d, (long long)H * cap * d, d};
    p.b = {w[t], (long long)H * d, 0, 0, kNoSplit};
    p.c = {dh + (size_t)s.h_off * s.d_model, s.d_model, 0, (long long)s.h_cap * s.d_model, kNoSplit};
    p.beta = t == 0 ? 0.f : 1.f;
    hipError_t e = gemm_launch<T, float, T, false, false, true>(p, s.batch, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
// bf16: one launch per phase.
// Workspace: G_cat [batch][rows_pad][N] then W_cat^T [N][d_model], bf16, each
// starting on a 256-byte boundary.
size_t pg_gcat_bytes(const ProjShape& s) {
  const size_t b = (size_t)s.batch * pg_rows_pad(s.len) * (s.hq + 2 * s.hkv) * s.head_dim * sizeof(bf16);
  return (b + 255) / 256 * 256;
}

hipError_t pg_fwd(const ProjShape& s, const void* h, const void* const w[3], void* const out[3], hipStream_t st) {
  const int d = s.head_dim;
  const int H[3] = {s.hq, s.hkv, s.hkv};
  ProjGemmParams p{};
  p.a = (const bf16*)h + (size_t)s.h_off * s.d_model;
  p.a_ld = s.d_model;
  p.a_bs = (long long)s.h_cap * s.d_model;
  for (int t = 0; t < 3; ++t) {
    const int cap = t == 0 ? s.q_cap : s.kv_cap, off = t == 0 ? s.q_off : s.start;
    p.b[t] = (const bf16*)w[t];
    p.b_w[t] = H[t] * d;
    p.c[t] = (bf16*)out[t] + (size_t)off * d;
    p.c_rs[t] = d;
    p.c_hs[t] = (long long)cap * d;
    p.c_bs[t] = (long long)H[t] * cap * d;
    p.c_hd[t] = d;
    p.c_w[t] = H[t] * d;
  }
  p.M = s.len;
  p.N = (s.hq + 2 * s.hkv) * d;
  p.K = s.d_model;
  p.a_rows = s.len;
  p.batch = s.batch;
  return pg_launch<PG_FWD>(p, s.batch, CA_KERNEL_PROJ, st);
}

// W_cat^T of the three weights into out ((Hq + 2 Hkv) d rows of d_model).
hipError_t pg_wt(const ProjShape& s, const void* const w[3], bf16* out, hipStream_t st) {
  const int d = s.head_dim;
  const int H[3] = {s.hq, s.hkv, s.hkv};
  const int N = (s.hq + 2 * s.hkv) * d;
  WtParams tp{};
  for (int t = 0; t < 3; ++t) {
    tp.w[t] = (const bf16*)w[t];
    tp.w_w[t] = H[t] * d;
  }
  tp.d_model = s.d_model;
  tp.ncols = N;
  tp.out = out;
  CA_LAUNCH(CA_KERNEL_PROJ_PREP, wt_kernel, dim3((N / 64) * (s.d_model / 64)), dim3(256), 0, st, tp);
  return hipGetLastError();
}

hipError_t pg_bwd(const ProjShape& s, const void* h, const void* const w[3], const float* const g[3],
                  float* const dw[3], float* dh, void* ws, const void* wt_given, hipStream_t st) {
  const int d = s.head_dim;
  const int H[3] = {s.hq, s.hkv, s.hkv};
  const int N = (s.hq + 2 * s.hkv) * d, rows_pad = pg_rows_pad(s.len);
  bf16* gcat = (bf16*)ws;
  // W_cat^T: the caller's (written by launch_proj_wt for these weights), or
  // transposed here into the workspace behind the gradients.
  const bf16* wt = wt_given ? (const bf16*)wt_given : (const bf16*)((char*)ws + pg_gcat_bytes(s));
  GcatParams gp{};
  for (int t = 0; t < 3; ++t) {
    const int cap = t == 0 ? s.q_cap : s.kv_cap, off = t == 0 ? s.q_off : s.start;
    gp.g[t] = g[t];
    gp.g_off[t] = (long long)off * d;
    gp.g_hs[t] = (long long)cap * d;
    gp.heads[t] = H[t];
  }
  gp.d = d;
  gp.len = s.len;
  gp.rows_pad = rows_pad;
  gp.ncols = N;
  gp.batch = s.batch;
  gp.out = gcat;
  const long long vecs = (long long)s.batch * rows_pad * (N / 8);
  const int blocks = (int)((vecs + 255) / 256 < 8192 ? (vecs + 255) / 256 : 8192);
  CA_LAUNCH(CA_KERNEL_PROJ_PREP, gcat_kernel, dim3(blocks), dim3(256), 0, st, gp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (!wt_given && (e = pg_wt(s, w, (bf16*)wt, st)) != hipSuccess) return e;

  // dW_cat += H_in^(i)^T G_cat, the batch summed along k.
  ProjGemmParams p{};
  p.a = (const bf16*)h + (size_t)s.h_off * s.d_model;
  p.a_ld = s.d_model;
  p.a_bs = (long long)s.h_cap * s.d_model;
  p.b[0] = gcat;
  p.b_w[0] = N;
  p.b_bs = (long long)rows_pad * N;
  for (int t = 0; t < 3; ++t) {
    p.c[t] = dw[t];
    p.c_rs[t] = (long long)H[t] * d;
    p.c_hs[t] = 0;
    p.c_bs[t] = 0;
    p.c_hd[t] = 1 << 30;
    p.c_w[t] = H[t] * d;
  }
  p.M = s.d_model;
  p.N = N;
  p.K = rows_pad;
  p.a_rows = s.len;
  p.b_rows = rows_pad;
  p.batch = s.batch;
  e = pg_launch<PG_DW>(p, 1, CA_KERNEL_PROJ, st);
  if (e != hipSuccess) return e;

  // dH_in^(i) = G_cat W_cat^T.
  ProjGemmParams q{};
  q.a = gcat;
  q.a_ld = N;
  q.a_bs = (long long)rows_pad * N;
  q.b[0] = q.b[1] = q.b[2] = wt;
  q.b_w[0] = s.d_model;
  q.b_w[1] = q.b_w[2] = 1 << 30;
  q.c[0] = dh + (size_t)s.h_off * s.d_model;
  q.c_rs[0] = s.d_model;
  q.c_hs[0] = 0;
  q.c_bs[0] = (long long)s.h_cap * s.d_model;
  q.c_hd[0] = 1 << 30;
  q.c_w[0] = s.d_model;
  q.c_w[1] = q.c_w[2] = 1 << 30;
  q.M = s.len;
  q.N = s.d_model;
  q.K = N;
  q.a_rows = s.len;
  q.batch = s.batch;
  return pg_launch<PG_DH>(q, s.batch, CA_KERNEL_PROJ, st);
}
}  // namespace

size_t proj_wt_bytes(const ProjShape& s) {
  if (s.dtype != CA_BF16) return 0;
  return (size_t)(s.hq + 2 * s.hkv) * s.head_dim * s.d_model * sizeof(bf16);
}

size_t proj_bwd_ws_bytes(const ProjShape& s, bool have_wt) {
  if (s.dtype != CA_BF16) return 0;
  return pg_gcat_bytes(s) + (have_wt ? 0 : proj_wt_bytes(s));
}

hipError_t launch_proj_wt(const ProjShape& s, const void* wq, const void* wk, const void* wv, void* out,
                          hipStream_t st) {
  const void* const w[3] = {wq, wk, wv};
  return pg_wt(s, w, (bf16*)out, st);
}

hipError_t launch_proj_fwd(const ProjShape& s, const void* h, const void* wq, const void* wk, const void* wv,
                           void* q, void* k, void* v, hipStream_t st) {
  const void* const w[3] = {wq, wk, wv};
  void* const out[3] = {q, k, v};
  return s.dtype == CA_BF16 ? pg_fwd(s, h, w, out, st) : proj_fwd_impl<float>(s, h, w, out, st);
}

hipError_t launch_proj_bwd(const ProjShape& s, const void* h, const void* wq, const void* wk, const void* wv,
                           const float* dq, const float* dk, const float* dv, float* dwq, float* dwk, float* dwv,
                           float* dh, void* ws, hipStream_t st, const void* wt) {
  const void* const w[3] = {wq, wk, wv};
  const float* const g[3] = {dq, dk, dv};
  float* const dw[3] = {dwq, dwk, dwv};
  return s.dtype == CA_BF16 ? pg_bwd(s, h, w, g, dw, dh, ws, wt, st)
                            : proj_bwd_impl<float>(s, h, w, g, dw, dh, st);
}

}  // namespace ca
