// bf16 GEMM on the matrix cores for gfx950, shared by the projections around
// the attention and the language-model head: C = A B with float32
// accumulation over a 128x128 output tile per workgroup, in three operand
// arrangements (modes):
//   PG_FWD  A [M][K] k-contiguous, B [K][N] n-contiguous, bf16 output
//   PG_DH   same operands, float32 output (overwritten)
//   PG_DW   A stored [K][M] (m-contiguous), B [K][N], float32 output
//           incremented, k running over `batch` stacked blocks of K rows
// A and B may each be up to three matrices side by side (segments along n for
// B, with their own row strides), and the output up to three strided views.
// Operand tiles stream into LDS by direct global->LDS loads (one slice pair or
// one slice ahead); NG groups of 4 waves (1 or 2) share a workgroup, two
// groups taking alternate k slices.
#pragma once

#include "device_common.h"
#include "timed_launch.h"

namespace ca {
namespace {

enum { PG_FWD = 0, PG_DW = 1, PG_DH = 2 };

// [128 rows][64 k] bf16 tile with k along the row (k-contiguous operand): the
// 16-byte chunk c of row r sits at chunk position c ^ ((r >> 1) & 7). Sixteen
// consecutive rows then put one chunk column on 16 distinct 4-bank groups
// (even and odd rows alternate between the two halves of the banks), so the
// two 8-byte fragment reads of a 32-lane half never share a bank.
struct KLay {
  static constexpr int COLS = 64;
  static __device__ __forceinline__ int off(int r, int c) {
    return r * COLS + ((((c >> 3) ^ (r >> 1)) & 7) << 3) + (c & 7);
  }
};
// [64 k rows][128 m or n] bf16 tile (operand with k along the stored rows).
using TLay = SwzLay<bf16, 128>;
constexpr int PG_TILE = 128 * 64;  // elements of one operand tile

struct ProjGemmParams {
  const bf16* a;             // forward, dW: H_in at the chunk's first row; dH: G_cat
  long long a_ld, a_bs;      // row stride and batch stride (elements)
  const bf16* b[3];          // forward: W_q, W_k, W_v; dW: b[0] = G_cat; dH: b[0] = W_cat^T
  int b_w[3];                // widths (= row strides) of the B matrices side by side
  long long b_bs;            // batch stride of B (dW: G_cat; forward/dH: 0 for shared weights)
  void* c[3];                // output segments (three weight/q/k/v blocks, or dH)
  long long c_rs[3], c_hs[3], c_bs[3];
  int c_hd[3];               // element (r, col) of segment s at c + b*bs + r*rs + (col/hd)*hs + col%hd
  int c_w[3];                // segment widths in columns (single segment: c_w[0] = N)
  int M, N, K;               // K per batch entry, a multiple of 64
  int a_rows;                // rows of A (forward, dH; dW: k rows of A) that exist: reads clamp to them
  int b_rows;                // dW: k rows of B per batch entry that exist (reads clamp to them)
  int batch;                 // forward, dH: batch entries in the grid; dW: summed along k
  int k_last;                // forward, dH: K of the last batch entry when > 0 (a shorter split-k tail)
};

// Segment of a column given three widths.
__device__ __forceinline__ int seg3(int x, const int w[3], int& local) {
  const int s = (x >= w[0]) + (x >= w[0] + w[1]);
  local = x - (s > 0 ? w[0] : 0) - (s > 1 ? w[1] : 0);
  return s;
}

// Geometry of the direct global->LDS loads of one operand tile by 8 waves,
// two 1 KB instructions each: a tile row holds CH 16-byte chunks (8: the
// [128][64] k-contiguous tile, 16: the [64][128] tile), instruction i of a
// wave fills rows rb(i) .. rb(i) + 64/CH - 1, and lane l fetches the logical
// chunk c(i) of row r(i) that belongs in its LDS slot (the swizzle is applied
// on the global side).
template <int CH, int NW>
struct PgGeom {
  static constexpr int ROWS = CH == 8 ? 128 : 64, RPI = 64 / CH, PER_WAVE = ROWS / NW;
  static constexpr int NI = PER_WAVE / RPI;  // load instructions per wave and tile
  static_assert(PER_WAVE % RPI == 0, "whole instructions per wave");
  __device__ __forceinline__ static int rb(int wave, int i) { return wave * PER_WAVE + i * RPI; }
  __device__ __forceinline__ static int row(int wave, int i, int lane) { return rb(wave, i) + lane / CH; }
  __device__ __forceinline__ static int chunk(int wave, int i, int lane) {
    const int r = row(wave, i, lane), slot = lane % CH;
    if constexpr (CH == 8) {
      return (slot ^ (r >> 1)) & 7;
    } else {
      return slot ^ TLay::swz(r);
    }
  }
};

template <class G>
__device__ __forceinline__ void pg_load(bf16* lds, int wave, int i, const bf16* src) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + G::rb(wave, i) * (G::ROWS == 128 ? 64 : 128)), 16, 0,
                                   0);
#endif
}

// NG groups of 4 waves per workgroup (1 or 2): with NG = 2 the groups take
// alternate k slices of each step and add their partial tiles at the end;
// with NG = 1 two workgroups share a CU (64 KB of LDS each).
template <int MODE, int NG>
__global__ __launch_bounds__(NG * 256) __attribute__((amdgpu_waves_per_eu(2))) void proj_gemm_kernel(
    ProjGemmParams p) {
  using E = Elt<bf16>;
  using frag = E::frag;
  constexpr int NW = 4 * NG;
  __shared__ __attribute__((aligned(16))) bf16 As0[NG * PG_TILE];
  __shared__ __attribute__((aligned(16))) bf16 Bs0[NG * PG_TILE];
  __shared__ __attribute__((aligned(16))) bf16 As1[NG * PG_TILE];
  __shared__ __attribute__((aligned(16))) bf16 Bs1[NG * PG_TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = NG == 1 ? 0 : wave >> 2, wq = wave & 3;
  const int wm = wq >> 1, wn = wq & 1;
  const int n = lane & 15, g = lane >> 4;
  const int mt = (p.M + 127) / 128, ntl = (p.N + 127) / 128;
  const int id = xcd_order(blockIdx.x, gridDim.x);
  const int bz = id / (mt * ntl), rem = id % (mt * ntl);
  // Weight gradient: the grid walks runs of GM row blocks, each run taking
  // every column block before the next starts. An A block (a slice of dZ^T or
  // H^T), which every column block reads, is then reused from L2 within its
  // run; with row blocks fastest over the whole range, each column pass
  // streamed all of A again (for the LM head's dW, 13 GB of 15.5 GB fetched).
  constexpr int GM = 8;
  const int run = rem / (GM * ntl), in_run = rem % (GM * ntl);
  const int gm = MODE == PG_DW ? min(GM, mt - run * GM) : mt;
  const int m0 = (MODE == PG_DW ? run * GM + in_run % gm : rem % mt) * 128;
  const int n0 = (MODE == PG_DW ? in_run / gm : rem / mt) * 128;
  const int nks = (MODE != PG_DW && p.k_last > 0 && bz == p.batch - 1 ? p.k_last : p.K) / 64;
  const int nk = MODE == PG_DW ? nks * p.batch : nks;
  const int n_pairs = (nk + NG - 1) / NG;  // steps of NG slices

  // Per-lane global sources of the two load instructions of each operand
  // tile, fixed for the whole k loop; a slice adds its k offset.
  constexpr int ACH = MODE == PG_DW ? 16 : 8, BCH = 16;
  using GA = PgGeom<ACH, NW>;
  using GB = PgGeom<BCH, NW>;
  constexpr int NI = GA::NI;
  static_assert(GB::NI == NI, "both tiles take the same number of loads");
  const bf16* const w0 = p.b[0];
  const bf16* const w1 = p.b[1];
  const bf16* const w2 = p.b[2];
  const int bw[3] = {p.b_w[0], p.b_w[1], p.b_w[2]};
  const bf16* asrc[NI];
  const bf16* bsrc[NI];
  long long bld[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ra = GA::row(wave, i, lane), ca = GA::chunk(wave, i, lane);
    const int rbb = GB::row(wave, i, lane), cb = GB::chunk(wave, i, lane);
    if constexpr (MODE != PG_DW) {
      asrc[i] = p.a + (long long)bz * p.a_bs + (long long)min(m0 + ra, p.a_rows - 1) * p.a_ld + 8 * ca;
      int col;
      const int sg = seg3(min(n0 + 8 * cb, p.N - 8), bw, col);
      const bf16* w = sg == 0 ? w0 : sg == 1 ? w1 : w2;
      bld[i] = sg == 0 ? bw[0] : sg == 1 ? bw[1] : bw[2];
      bsrc[i] = w + (long long)bz * p.b_bs + (long long)rbb * bld[i] + col;
    } else {
      asrc[i] = p.a + min(m0 + 8 * ca, p.M - 8);
      bsrc[i] = w0 + min(n0 + 8 * cb, p.N - 8);
      bld[i] = 0;
    }
  }

  // Stage slice t (A and B tiles) into LDS.
  auto stage_slice = [&](bf16* at, bf16* bt, int t) {
    if constexpr (MODE != PG_DW) {
      const int k0 = t * 64;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pg_load<GA>(at, wave, i, asrc[i] + k0);
        pg_load<GB>(bt, wave, i, bsrc[i] + (long long)k0 * bld[i]);
      }
    } else {
      const int bb = t / nks, k0 = (t % nks) * 64;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ra = GA::row(wave, i, lane), rbb = GB::row(wave, i, lane);
        pg_load<GA>(at, wave, i, asrc[i] + (long long)bb * p.a_bs + (long long)min(k0 + ra, p.a_rows - 1) * p.a_ld);
        pg_load<GB>(bt, wave, i, bsrc[i] + (long long)bb * p.b_bs + (long long)min(k0 + rbb, p.b_rows - 1) * p.N);
      }
    }
  };
  auto stage_pair = [&](bf16* at, bf16* bt, int pair) {
    stage_slice(at, bt, NG * pair);
    if (NG == 2 && 2 * pair + 1 < nk) stage_slice(at + PG_TILE, bt + PG_TILE, 2 * pair + 1);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const bf16* at, const bf16* bt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      frag af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mr = wm * 64 + i * 16, nr = wn * 64 + i * 16;
        if constexpr (MODE == PG_DW) {
          af[i] = ldT8<TLay>(at, ks * 32, mr, lane);
        } else {
          af[i] = ld8t<KLay>(at, mr + n, ks * 32, g);
        }
        bfr[i] = ldT8<TLay>(bt, ks * 32, nr, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) E::mma(acc[i][j], bfr[j], af[i]);
    }
  };

  stage_pair(As0, Bs0, 0);
  wait_loads();
  __syncthreads();
  auto pair_step = [&](int i, const bf16* Ac, const bf16* Bc, bf16* An, bf16* Bn) {
    if (i + 1 < n_pairs) stage_pair(An, Bn, i + 1);
    if (NG * i + grp < nk) compute(Ac + grp * PG_TILE, Bc + grp * PG_TILE);
    wait_loads();  // the next pair has landed in LDS
    __syncthreads();
  };
  for (int i = 0; i < n_pairs; i += 2) {
    pair_step(i, As0, Bs0, As1, Bs1);
    if (i + 1 < n_pairs) pair_step(i + 1, As1, Bs1, As0, Bs0);
  }

  // With two groups, group 0 finishes rows i = 0, 1 of every wave tile and
  // group 1 rows i = 2, 3; each hands the other half of its partial sums over
  // through LDS.
  f32x4* give = (f32x4*)(grp == 0 ? As0 : Bs0);
  const f32x4* take = (const f32x4*)(grp == 0 ? Bs0 : As0);
  if constexpr (NG == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((i >> 1) == grp) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) give[((wq * 8 + (i & 1) * 4 + j) * 64) + lane] = acc[i][j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (NG == 2 && (i >> 1) != grp) continue;
    const int m = m0 + wm * 64 + i * 16 + n;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nb = n0 + wn * 64 + j * 16 + 4 * g;
      if (nb >= p.N) continue;
      const f32x4 v = NG == 2 ? acc[i][j] + take[((wq * 8 + (i & 1) * 4 + j) * 64) + lane] : acc[i][j];
      int col;
      const int sg = seg3(nb, p.c_w, col);
      const long long rs = sg == 0 ? p.c_rs[0] : sg == 1 ? p.c_rs[1] : p.c_rs[2];
      const long long hs = sg == 0 ? p.c_hs[0] : sg == 1 ? p.c_hs[1] : p.c_hs[2];
      const long long bs = sg == 0 ? p.c_bs[0] : sg == 1 ? p.c_bs[1] : p.c_bs[2];
      const int hd = sg == 0 ? p.c_hd[0] : sg == 1 ? p.c_hd[1] : p.c_hd[2];
      void* base = sg == 0 ? p.c[0] : sg == 1 ? p.c[1] : p.c[2];
      const long long idx = (long long)bz * bs + (long long)m * rs + (long long)(col / hd) * hs + col % hd;
      if constexpr (MODE == PG_FWD) {
        store4<bf16>((bf16*)base + idx, v, 1.f);
      } else if constexpr (MODE == PG_DW) {
        f32x4* c = (f32x4*)((float*)base + idx);
        *c = *c + v;
      } else {
        *(f32x4*)((float*)base + idx) = v;
      }
    }
  }
}

int pg_rows_pad(int len) { return (len + 63) / 64 * 64; }

// Wave groups per workgroup: with few output tiles (under ~1.5 per CU) one
// 8-wave workgroup per CU splits k over two groups; otherwise 4-wave
// workgroups run two to a CU.
template <int MODE>
hipError_t pg_launch(const ProjGemmParams& p, int grid_batch, int prof_id, hipStream_t st) {
  const int tiles = ((p.M + 127) / 128) * ((p.N + 127) / 128) * grid_batch;
  if (tiles < 384) {
    CA_LAUNCH(prof_id, (proj_gemm_kernel<MODE, 2>), dim3(tiles), dim3(512), 0, st, p);
  } else {
    CA_LAUNCH(prof_id, (proj_gemm_kernel<MODE, 1>), dim3(tiles), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace ca
