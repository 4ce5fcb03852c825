// Chunked exact causal attention for gfx950 (CDNA4): forward, and the
// backward split into a row-delta pass, a dK/dV pass and a dQ pass. Given
// workspace room (bf16), the dK/dV pass also stores the chunk's dS^T in bf16
// and the dQ pass streams it (dQ = dS K, one product per visible pair);
// otherwise the dQ pass recomputes S, P and dP (three products per pair).
// Tile sizes follow the grid: chunks too short to give every compute unit a
// 128-row query tile run 64-row tiles, and the dK/dV pass mixes 128- and
// 64-key tiles so that its last round is a short one (see bwd_impl).
//
// What is computed (StreamBP review, "What carries the argument": Property 3.1
// and the partitioned attention of Eqs. (12)-(14)): chunk i's queries, at
// global positions start + r, attend to keys [0, start + len) with key j
// visible iff j <= start + r. Per q head h and kv head h / (Hq/Hkv):
//   S = scale Q K^T, P = softmax over visible keys, O = P V, LSE = ln sum exp S
//   dS = P * (dO V^T - delta), delta_r = dO_r . O_r
//   dQ = scale dS K,  dK += scale dS^T Q,  dV += P^T dO   (summed over the group)
//
// Matrix products and their fragment slot orders follow the conventions in
// device_common.h; products accumulate in float32.
//
// LDS holds every streamed tile once, row-major. Tiles filled by direct
// global->LDS loads (K/V in the forward and dQ) have their 16-byte chunks
// XOR-swizzled by row (the loads write each wave's kilobyte contiguously);
// tiles written from registers (Q/dO in dK/dV) have each row padded by 32
// bytes. Either way both access patterns are free of bank conflicts: 16 lanes
// reading one chunk column of 16 rows (operands contracted over head_dim), and
// ds_read_b64_tr_b16 transposing reads (operands contracted over rows: V in
// P V, K in dS K, Q and dO in dS^T Q and P^T dO). Tiles are double-buffered:
// the next tile's loads are in flight while the current one is consumed, with
// one barrier per tile (per pair of tiles in the forward and dQ).
//
// Layout choices:
//  * forward / dQ: S^T = K Q^T per key tile, so each lane owns one query column
//    and softmax statistics need only a 4-lane reduction.
//  * dK/dV: S = Q K^T per query tile, so P and dS are already key-major for
//    dV = P^T dO and dK = dS^T Q.
//  * every dK/dV element is owned by one lane of one workgroup, which adds its
//    total into the float32 accumulator once: no atomics.
//  * softmax runs in the exp2 domain with the scale folded into one FMA, and the
//    running maximum is only moved (rescaling O and the row sum) when a new
//    score exceeds it by more than 2^8, which keeps every exponent <= 2^8.
#include "device_common.h"
#include "timed_launch.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

// Scratch of the allocation-free backward (chunk_attn_bwd_noalloc): the
// chunk's row statistics go here instead of into a caller workspace. Every
// device holds its own copy for the life of the process; host code reaches it
// only through the address scratch_address() looks up, never by this name.
static __device__ __align__(256) char scratch[ca::kScratchBytes];

namespace ca {

hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

// ----------------------------------------------------------------------------
// Forward. 1-D grid over (batch, q head, query tile). A workgroup has NG
// groups of NW waves; wave w of each group owns the same NQT*16 query rows
// (held as B fragments of S^T = K Q^T), and group g takes key tiles NG i + g,
// so each SIMD runs two waves (one's LDS reads and softmax overlap the
// other's MFMAs) without more LDS traffic per product. Long chunks run two
// groups of four waves on 64-key tiles; a chunk too short to give every
// compute unit a 128-row tile runs 64-row tiles as four groups of two waves
// on 32-key tiles, which keeps 32 rows per wave (16-row waves would read
// every tile from LDS twice as often per product). The NG tiles of a step
// stream into double-buffered LDS by direct global->LDS loads issued one step
// ahead; the two buffers are separate arrays named statically (the loop is
// unrolled by two), which lets the compiler see that reads of one buffer do
// not depend on the loads into the other. At the end groups 1..NG-1 in turn
// hand their running maximum, row sums and O^T to group 0 through LDS, which
// merges and stores. Tiles past a wave's rows are skipped; only diagonal
// tiles are masked.
// ----------------------------------------------------------------------------
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int hq, hkv, q_cap, kv_cap, q_off, start, len;
  float c2;  // |softmax scale| * log2(e), > 0
  int neg;   // softmax scale < 0: queries enter S negated
};

template <typename T, int D, int NQT, int BK, int NW, int NG = 2>
__global__ __launch_bounds__(NG * NW * 64) void fwd_kernel(FwdParams p) {
  using E = Elt<T>;
  using frag = typename E::frag;
  using Lt = SwzLay<T, D>;
  constexpr int BQ = NW * NQT * 16;
  constexpr int DK = D / 32, MD = D / 16, MK = BK / 16, KB2 = BK / 32;
  // Step i uses buffer i & 1: K tiles NG i .. NG i + NG - 1 in Kb<i&1> (tile
  // NG i + g at rows [g BK, (g + 1) BK)), V tiles likewise in Vb<i&1>.
  __shared__ __attribute__((aligned(16))) T Kb0[NG * BK * D];
  __shared__ __attribute__((aligned(16))) T Vb0[NG * BK * D];
  __shared__ __attribute__((aligned(16))) T Kb1[NG * BK * D];
  __shared__ __attribute__((aligned(16))) T Vb1[NG * BK * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / NW, wq = wave % NW;
  const int n = lane & 15, g = lane >> 4;
  const int nqt = (p.len + BQ - 1) / BQ;
  const int work_id = xcd_order(blockIdx.x, gridDim.x);
  const int qt = nqt - 1 - work_id % nqt;  // longest rows first
  const int h = (work_id / nqt) % p.hq, b = work_id / (nqt * p.hq);
  const int hk = h / (p.hq / p.hkv);
  const T* Q = (const T*)p.q + ((size_t)(b * p.hq + h) * p.q_cap + p.q_off) * D;
  const T* K = (const T*)p.k + (size_t)(b * p.hkv + hk) * p.kv_cap * D;
  const T* V = (const T*)p.v + (size_t)(b * p.hkv + hk) * p.kv_cap * D;
  const int L = p.start + p.len;
  const int r0 = qt * BQ;
  const int n_tiles = (p.start + min(r0 + BQ, p.len) - 1) / BK + 1;
  const int n_pairs = (n_tiles + NG - 1) / NG;
  const int wr0 = r0 + wq * NQT * 16;
  const bool active = wr0 < p.len;
  const int wq_lo = p.start + wr0;
  const int wq_hi = p.start + min(wr0 + NQT * 16, p.len) - 1;
  const float c2 = p.c2;

  auto stage = [&](T* kd, T* vd, int pair) {
    stage_tile<T, NG * BK, D, NG * NW>(kd, K, NG * pair * BK, L, wave, lane);
    stage_tile<T, NG * BK, D, NG * NW>(vd, V, NG * pair * BK, L, wave, lane);
  };
  stage(Kb0, Vb0, 0);

  frag qf[NQT][DK];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int row = min(wr0 + nt * 16 + n, p.len - 1);
#pragma unroll
    for (int kb = 0; kb < DK; ++kb) {
      qf[nt][kb] = ldg8(Q + (size_t)row * D + kb * 32 + 8 * g);
      if (p.neg) qf[nt][kb] = negate<T>(qf[nt][kb]);
    }
  }
  f32x4 oacc[MD][NQT];
  // Row sums of P come out of the matrix cores (ones times P^T): every lane
  // of a query column holds the column's full sum, in all four slots.
  f32x4 lacc[NQT];
  float m2[NQT];
  const frag ones = ones_frag<T>();
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    m2[nt] = -kInf;
    lacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int md = 0; md < MD; ++md) oacc[md][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  wait_loads();
  __syncthreads();

  // Pair i from the buffer (Kc, Vc); the next pair streams into (Kn, Vn).
  auto pair_step = [&](int i, const T* Kc, const T* Vc, T* Kn, T* Vn) {
    if (i + 1 < n_pairs) stage(Kn, Vn, i + 1);
    const int j = NG * i + grp;  // this group's key tile
    const int kb0 = j * BK;
    if (active && j < n_tiles && kb0 <= wq_hi) {
      const T* Kt = Kc + grp * BK * D;
      const T* Vt = Vc + grp * BK * D;
      f32x4 s[MK][NQT];
#pragma unroll
      for (int mk = 0; mk < MK; ++mk)
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) s[mk][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK; ++kb)
#pragma unroll
        for (int mk = 0; mk < MK; ++mk) {
          const frag a = ld8s<Lt>(Kt, mk * 16 + n, kb * 32 + 8 * g);
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) E::mma(s[mk][nt], a, qf[nt][kb]);
        }

      if (kb0 + BK - 1 > wq_lo) {  // tile crosses this wave's diagonal
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
          const int qp = wq_lo + nt * 16 + n;
#pragma unroll
          for (int mk = 0; mk < MK; ++mk)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
              if (kb0 + mk * 16 + 4 * g + ii > qp) s[mk][nt][ii] = -kInf;
        }
      }
      // Each lane tests its own scores against the running maximum; the exact
      // 4-lane maximum (a cross-lane move) is only taken when some lane's score
      // exceeds it by more than 2^8, so the common path has no cross-lane op.
      bool grow = false;
      float mx2[NQT];
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        float mx = -kInf;
#pragma unroll
        for (int mk = 0; mk < MK; ++mk)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) mx = fmaxf(mx, s[mk][nt][ii]);
        mx2[nt] = mx * c2;
        grow |= mx2[nt] > m2[nt] + kRescale;
      }
      if (__any(grow)) {
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
          const float mnew = fmaxf(m2[nt], max4(mx2[nt]));
          const float alpha = mnew == -kInf ? 1.f : fexp2(m2[nt] - mnew);
          m2[nt] = mnew;
          lacc[nt] *= alpha;
#pragma unroll
          for (int md = 0; md < MD; ++md) oacc[md][nt] *= alpha;
        }
      }
      // A row with no visible key yet (possible for group 1) keeps m2 = -inf;
      // its scores are all -inf, and a finite stand-in keeps exp2 at 0.
      float mref[NQT];
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) mref[nt] = fmaxf(m2[nt], -1e30f);
#pragma unroll
      for (int kb2 = 0; kb2 < KB2; ++kb2) {
        frag pf[NQT];
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
              s[2 * kb2 + hh][nt][ii] = fexp2(__builtin_fmaf(s[2 * kb2 + hh][nt][ii], c2, -mref[nt]));
          pf[nt] = pack44<T>(s[2 * kb2][nt], s[2 * kb2 + 1][nt]);
        }
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const frag a = ldT8<Lt>(Vt, kb2 * 32, md * 16, lane);
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) E::mma(oacc[md][nt], a, pf[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) E::mma(lacc[nt], ones, pf[nt]);
      }
    }
    wait_loads();  // the next pair has landed in LDS
    __syncthreads();
  };
  for (int i = 0; i < n_pairs; i += 2) {
    pair_step(i, Kb0, Vb0, Kb1, Vb1);
    if (i + 1 < n_pairs) pair_step(i + 1, Kb1, Vb1, Kb0, Vb0);
  }

  // Merge: group 1 publishes (m2, row sum, O^T) per lane; the matching lane
  // of group 0 rescales both to the larger maximum and adds. The exchange
  // spans three of the (now idle) tile buffers: O^T columns [0, D/2) in Kb0,
  // [D/2, D) in Vb0, the two statistics in Kb1.
  constexpr int HALF = MD / 2 * 4;  // floats per lane and query tile in each O half
  static_assert(sizeof(Kb0) >= (size_t)NQT * NW * 64 * HALF * sizeof(float) &&
                    sizeof(Kb1) >= (size_t)NQT * NW * 64 * 2 * sizeof(float),
                "merge area");
  float* xo0 = (float*)Kb0;
  float* xo1 = (float*)Vb0;
  float* xs = (float*)Kb1;
  for (int src = 1; src < NG; ++src) {  // groups 1 .. NG-1 in turn
    if (grp == src) {
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        const size_t slot = (size_t)(nt * NW + wq);
        xs[(slot * 2 + 0) * 64 + lane] = m2[nt];
        xs[(slot * 2 + 1) * 64 + lane] = lacc[nt][0];
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float* x = md < MD / 2 ? xo0 : xo1;
            x[(slot * HALF + (md % (MD / 2)) * 4 + e) * 64 + lane] = oacc[md][nt][e];
          }
      }
    }
    __syncthreads();
    if (grp == 0 && active) {
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        const size_t slot = (size_t)(nt * NW + wq);
        const float mb = xs[(slot * 2 + 0) * 64 + lane];
        const float mnew = fmaxf(m2[nt], mb);
        // group 0's maximum is finite for every visible row (its tile 0 holds
        // key 0); another group's is -inf where it saw no key of the row
        const float fa = fexp2(m2[nt] - mnew), fb = mb == -kInf ? 0.f : fexp2(mb - mnew);
        lacc[nt][0] = lacc[nt][0] * fa + xs[(slot * 2 + 1) * 64 + lane] * fb;
        m2[nt] = mnew;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float* x = md < MD / 2 ? xo0 : xo1;
            oacc[md][nt][e] = oacc[md][nt][e] * fa + x[(slot * HALF + (md % (MD / 2)) * 4 + e) * 64 + lane] * fb;
          }
      }
    }
    if (src + 1 < NG) __syncthreads();  // the next group overwrites the exchange area
  }
  if (grp != 0 || !active) return;
  float lrow[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) lrow[nt] = lacc[nt][0];
  T* O = (T*)p.o + ((size_t)(b * p.hq + h) * p.q_cap + p.q_off) * D;
  float* LSE = p.lse + (size_t)(b * p.hq + h) * p.q_cap + p.q_off;
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const float l = lrow[nt];
    const int row = wr0 + nt * 16 + n;
    if (row < p.len) {
      const float inv = 1.f / l;
#pragma unroll
      for (int md = 0; md < MD; ++md) store4<T>(O + (size_t)row * D + md * 16 + 4 * g, oacc[md][nt], inv);
      if (g == 0) LSE[row] = (m2[nt] + __builtin_amdgcn_logf(l)) * kLn2;
    }
  }
}

// ----------------------------------------------------------------------------
// delta_r = sum_c dO_rc O_rc (float32) and lse2_r = LSE_r * log2(e) for a
// chunk's rows, both [batch*hq][len]; LPR lanes share one row. Workgroup
// `block` of `nblocks` (THREADS threads each) takes every nblocks-th group of
// THREADS / LPR rows.
// ----------------------------------------------------------------------------
struct StatsArgs {
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;
  float* lse2;
  int q_cap, q_off, len, rows;
  int blocks;  // workgroups of a fused launch that compute these (0: none)
};

template <typename T, int D, int THREADS>
__device__ __forceinline__ void row_stats(const StatsArgs& a, int block, int nblocks) {
  using V = typename Elt<T>::vec;
  constexpr int VEC = Elt<T>::VEC, LPR = D / VEC, RPB = THREADS / LPR;
  const int sub = threadIdx.x % LPR;
  for (int row0 = block * RPB; row0 < a.rows; row0 += nblocks * RPB) {
    const int row = row0 + threadIdx.x / LPR;
    float acc = 0.f;
    size_t qrow = 0;
    if (row < a.rows) {
      const int bh = row / a.len, r = row % a.len;
      qrow = (size_t)bh * a.q_cap + a.q_off + r;
      const V x = *(const V*)((const T*)a.o + qrow * D + sub * VEC);
      const V y = *(const V*)((const T*)a.dout + qrow * D + sub * VEC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc += (float)x[e] * (float)y[e];
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (row < a.rows && sub == 0) {
      a.delta[row] = acc;
      a.lse2[row] = a.lse[qrow] * kLog2e;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(StatsArgs a) {
  row_stats<T, D, 256>(a, blockIdx.x, gridDim.x);
}

// ----------------------------------------------------------------------------
// Backward parameters shared by the dQ and dK/dV passes.
// ----------------------------------------------------------------------------
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;    // natural-log LSE, q-side layout
  const float* delta;  // [batch*hq][len]
  const float* lse2;   // [batch*hq][len], LSE * log2(e)
  float* dq;
  float* dk;
  float* dv;
  int hq, hkv, q_cap, kv_cap, q_off, start, len;
  float c2;        // |softmax scale| * log2(e), > 0
  int neg;         // softmax scale < 0
  float dq_scale;  // grad_scale * softmax scale
  float dk_scale;  // grad_scale * softmax scale
  float dv_scale;  // grad_scale
  // Optional dS^T store (bf16): [batch*hq][ds_nqb blocks of kDsCols query
  // rows][ds_keys][kDsCols]; null when dQ recomputes dS.
  void* ds;
  int ds_nqb, ds_keys;
  int kv_first, kv_end;  // dK/dV pass: the launch's key tiles cover keys [kv_first, kv_end)
  int acc_store;         // dK/dV pass: store the prefix rows instead of adding to them
};

// dQ pass. Same walk, split and staging as the forward: two groups of NW
// waves own the same query rows and take the even / odd key tiles of pairs
// streamed into two statically named LDS buffers. Per tile S^T = K Q^T and
// dP^T = V dO^T with K, V read row-major, P from the stored LSE, and
// dQ^T += K^T dS^T with K read through the transposing path. Group 1 hands
// its partial dQ to group 0 through LDS at the end.
template <typename T, int D, int BK>
struct DqLds {
  __attribute__((aligned(16))) T Kb0[2 * BK * D];
  __attribute__((aligned(16))) T Vb0[2 * BK * D];
  __attribute__((aligned(16))) T Kb1[2 * BK * D];
  __attribute__((aligned(16))) T Vb1[2 * BK * D];
};
// Workgroup `block` of `nblocks` (the pass's own grid) with its LDS in `sm`.
template <typename T, int D, int NQT, int BK, int NW>
__device__ __forceinline__ void dq_body(const BwdParams& p, int block, int nblocks, DqLds<T, D, BK>& sm) {
  using E = Elt<T>;
  using frag = typename E::frag;
  using Lt = SwzLay<T, D>;
  constexpr int BQ = NW * NQT * 16;
  constexpr int DK = D / 32, MD = D / 16, KB2 = BK / 32;
  T* const Kb0 = sm.Kb0;
  T* const Vb0 = sm.Vb0;
  T* const Kb1 = sm.Kb1;
  T* const Vb1 = sm.Vb1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / NW, wq = wave % NW;
  const int n = lane & 15, g = lane >> 4;
  const int nqt = (p.len + BQ - 1) / BQ;
  const int work_id = xcd_order(block, nblocks);
  const int qt = nqt - 1 - work_id % nqt;  // longest rows first
  const int h = (work_id / nqt) % p.hq, b = work_id / (nqt * p.hq);
  const int hk = h / (p.hq / p.hkv);
  const size_t qhead = ((size_t)(b * p.hq + h) * p.q_cap + p.q_off);
  const T* Q = (const T*)p.q + qhead * D;
  const T* dO = (const T*)p.dout + qhead * D;
  const float* LSE2 = p.lse2 + (size_t)(b * p.hq + h) * p.len;
  const float* DL = p.delta + (size_t)(b * p.hq + h) * p.len;
  const T* K = (const T*)p.k + (size_t)(b * p.hkv + hk) * p.kv_cap * D;
  const T* V = (const T*)p.v + (size_t)(b * p.hkv + hk) * p.kv_cap * D;
  const int L = p.start + p.len;
  const int r0 = qt * BQ;
  const int n_tiles = (p.start + min(r0 + BQ, p.len) - 1) / BK + 1;
  const int n_pairs = (n_tiles + 1) / 2;
  const int wr0 = r0 + wq * NQT * 16;
  const bool active = wr0 < p.len;
  const int wq_lo = p.start + wr0;
  const int wq_hi = p.start + min(wr0 + NQT * 16, p.len) - 1;
  const float c2 = p.c2;

  auto stage = [&](T* kd, T* vd, int pair) {
    stage_tile<T, 2 * BK, D, 2 * NW>(kd, K, 2 * pair * BK, L, wave, lane);
    stage_tile<T, 2 * BK, D, 2 * NW>(vd, V, 2 * pair * BK, L, wave, lane);
  };
  stage(Kb0, Vb0, 0);

  frag qf[NQT][DK], df[NQT][DK];
  float lse2[NQT], dl[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int row = wr0 + nt * 16 + n;
    const int rc = min(row, p.len - 1);
#pragma unroll
    for (int kb = 0; kb < DK; ++kb) {
      qf[nt][kb] = ldg8(Q + (size_t)rc * D + kb * 32 + 8 * g);
      if (p.neg) qf[nt][kb] = negate<T>(qf[nt][kb]);
      df[nt][kb] = ldg8(dO + (size_t)rc * D + kb * 32 + 8 * g);
    }
    lse2[nt] = row < p.len ? LSE2[rc] : kInf;
    dl[nt] = DL[rc];
  }
  f32x4 acc[MD][NQT];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) acc[md][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_loads();
  __syncthreads();

  auto pair_step = [&](int i, const T* Kc, const T* Vc, T* Kn, T* Vn) {
    if (i + 1 < n_pairs) stage(Kn, Vn, i + 1);
    const int j = 2 * i + grp;  // this group's key tile
    const int kb0 = j * BK;
    if (active && j < n_tiles && kb0 <= wq_hi) {
      const T* Kt = Kc + grp * BK * D;
      const T* Vt = Vc + grp * BK * D;
      const bool diag = kb0 + BK - 1 > wq_lo;  // tile crosses this wave's diagonal
      // One 32-key half at a time keeps only half the tile's S and dP live.
#pragma unroll
      for (int kb2 = 0; kb2 < KB2; ++kb2) {
        f32x4 s[2][NQT], dp[2][NQT];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) {
            s[hh][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[hh][nt] = f32x4{-dl[nt], -dl[nt], -dl[nt], -dl[nt]};  // the products give dP - delta
          }
#pragma unroll
        for (int kb = 0; kb < DK; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int mk = 2 * kb2 + hh;
            const frag ak = ld8s<Lt>(Kt, mk * 16 + n, kb * 32 + 8 * g);
            const frag av = ld8s<Lt>(Vt, mk * 16 + n, kb * 32 + 8 * g);
#pragma unroll
            for (int nt = 0; nt < NQT; ++nt) {
              E::mma(s[hh][nt], ak, qf[nt][kb]);
              E::mma(dp[hh][nt], av, df[nt][kb]);
            }
          }
        // dS = P (dP - delta), with the causal mask only on tiles that cross
        // the diagonal: two copies of this step, chosen per tile.
        frag dsf[NQT];
        auto make_ds = [&](auto masked) {
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) {
            const int qp = wq_lo + nt * 16 + n;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) {
                float pv = fexp2(__builtin_fmaf(s[hh][nt][ii], c2, -lse2[nt]));
                if constexpr (decltype(masked)::value) {
                  if (kb0 + (2 * kb2 + hh) * 16 + 4 * g + ii > qp) pv = 0.f;
                }
                dp[hh][nt][ii] = pv * dp[hh][nt][ii];
              }
            dsf[nt] = pack44<T>(dp[0][nt], dp[1][nt]);
          }
        };
        if (diag) {
          make_ds(std::true_type{});
        } else {
          make_ds(std::false_type{});
        }
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const frag a = ldT8<Lt>(Kt, kb2 * 32, md * 16, lane);
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) E::mma(acc[md][nt], a, dsf[nt]);
        }
      }
    }
    wait_loads();  // the next pair has landed in LDS
    __syncthreads();
  };
  for (int i = 0; i < n_pairs; i += 2) {
    pair_step(i, Kb0, Vb0, Kb1, Vb1);
    if (i + 1 < n_pairs) pair_step(i + 1, Kb1, Vb1, Kb0, Vb0);
  }

  // Merge: group 1 publishes its partial dQ^T per lane (columns [0, D/2) in
  // Kb0, [D/2, D) in Vb0), group 0 adds it.
  constexpr int HALF = MD / 2 * 4;
  static_assert(sizeof(sm.Kb0) >= (size_t)NQT * NW * 64 * HALF * sizeof(float), "merge area");
  float* xo0 = (float*)Kb0;
  float* xo1 = (float*)Vb0;
  if (grp == 1) {
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      const size_t slot = (size_t)(nt * NW + wq);
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float* x = md < MD / 2 ? xo0 : xo1;
          x[(slot * HALF + (md % (MD / 2)) * 4 + e) * 64 + lane] = acc[md][nt][e];
        }
    }
  }
  __syncthreads();
  if (grp == 1 || !active) return;
  float* DQ = p.dq + qhead * D;
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const size_t slot = (size_t)(nt * NW + wq);
    const int row = wr0 + nt * 16 + n;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const float* x = md < MD / 2 ? xo0 : xo1;
      f32x4 v = acc[md][nt];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += x[(slot * HALF + (md % (MD / 2)) * 4 + e) * 64 + lane];
      if (row < p.len) *(f32x4*)(DQ + (size_t)row * D + md * 16 + 4 * g) = v * p.dq_scale;
    }
  }
}

// dK/dV pass. Grid (key tiles of NP*NKT*16 rows, Hkv, batch); NP pairs of
// waves, each pair owning NKT*16 keys, walk every (q head of the group,
// query tile) block that can see them. Wave w < NP of a pair holds the keys'
// K fragments and dV sums: S = Q K^T, P = exp(S - LSE) (causally masked),
// dV += P^T dO, and P goes to LDS as the packed fragments of that product.
// Its partner, wave NP + w, holds the V fragments and dK sums and runs one
// block behind: dP = dO V^T, dS = P (dP - delta) with that (rounded) P, and
// dK += dS^T Q one iteration later still, at the start of the next
// iteration. Each wave then does two of the four products per block and fits
// in half the register file, so the two waves of a pair share a SIMD, and
// their phase orders differ (products, exponentials, products against
// products, products, dS) so that one's vector work runs under the other's
// products. Q blocks go through four LDS buffers (block it for S, it - 2 for
// dK, it + 1 being filled), dO blocks and row statistics through three; they
// are read row-major as the A operand of S and dP and through the transposing
// path as the B operand of dV and dK.
template <typename T, int D, int NKT, int BQ, int NP>
struct DkdvLds {
  static constexpr int NB = 3, NBQ = 4, KQ = BQ / 32;
  __attribute__((aligned(16))) T Qs[NBQ][BQ * PadLay<T, D>::RS];
  __attribute__((aligned(16))) T Ds[NB][BQ * PadLay<T, D>::RS];
  // per buffer: LSE*log2(e) of the block's rows in [0, BQ), delta in [BQ, 2BQ)
  __attribute__((aligned(16))) float stat_s[NB][2 * BQ];
  // P of a pair's block as the A fragments of dV: [block parity][pair][kq][nk][lane]
  typename Elt<T>::frag Ps[2][NP][KQ][NKT][64];
};
// Workgroup `block` of `nblocks` (the pass's own grid) with its LDS in `sm`.
template <typename T, int D, int NKT, int BQ, int NP>
__device__ __forceinline__ void dkdv_body(const BwdParams& p, int block, int nblocks,
                                          DkdvLds<T, D, NKT, BQ, NP>& sm) {
  using E = Elt<T>;
  using frag = typename E::frag;
  using Lds = DkdvLds<T, D, NKT, BQ, NP>;
  constexpr int BKV = NP * NKT * 16, NB = Lds::NB, NBQ = Lds::NBQ;
  constexpr int DK = D / 32, MD = D / 16, MQ = BQ / 16, KQ = BQ / 32;
  // Only the P/dV waves load Q/dO blocks (and only the dS/dK waves store dS):
  // vector loads and stores complete out of order with respect to each other
  // on this chip, so a wave with both in flight has to wait for its stores
  // whenever it waits for a load.
  constexpr int NL = NP * 64;  // loading threads
  static_assert(2 * BQ <= NL, "row statistics: one value per loading thread");
  auto& Qs = sm.Qs;
  auto& Ds = sm.Ds;
  auto& stat_s = sm.stat_s;
  auto& Ps = sm.Ps;
  // Ring-buffer slot of block i, made wave-uniform and opaque to the
  // compiler: otherwise it strength-reduces i % NB across the loop into one
  // induction variable per LDS address (two instructions per read).
  auto slot = [](int i, int nb) { return __builtin_amdgcn_readfirstlane(i % nb); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pv_wave = wave < NP;  // P/dV role; otherwise dS/dK
  const int pair = pv_wave ? wave : wave - NP;
  const int n = lane & 15, g = lane >> 4;
  const int G = p.hq / p.hkv;
  const int L = p.start + p.len;
  const int nkt = (p.kv_end - p.kv_first + BKV - 1) / BKV;
  const int work_id = xcd_order(block, nblocks);
  const int kt = work_id % nkt;  // ascending: the first key tiles see the most queries
  const int hk = (work_id / nkt) % p.hkv, b = work_id / (nkt * p.hkv);
  const int kb0 = p.kv_first + kt * BKV;
  const int wk0 = kb0 + pair * NKT * 16;
  const float c2 = p.c2;

  // Query rows that can see key kb0: chunk rows r with start + r >= kb0.
  const int qt0 = max(0, kb0 - p.start) / BQ;
  const int qt_end = (p.len + BQ - 1) / BQ;
  const int iters = G * (qt_end - qt0);
  auto next_qt = [&](int q) { return q + 1 == qt_end ? qt0 : q + 1; };

  // Next block to fetch, walked q tile fastest then q head.
  int f_qt = qt0, f_h = hk * G;
  RegTile<T, BQ, D, NL> qreg, dreg;
  float stat;
  bool past;  // this thread's LSE row lies past the chunk: zero weight
  auto fetch = [&]() {
    const int q0 = f_qt * BQ;
    const size_t qhead = (size_t)(b * p.hq + f_h) * p.q_cap + p.q_off;
    const size_t rhead = (size_t)(b * p.hq + f_h) * p.len;
    qreg.load((const T*)p.q + qhead * D, q0, p.len, tid);
    dreg.load((const T*)p.dout + qhead * D, q0, p.len, tid);
    const int r = q0 + tid % BQ;
    stat = (tid < BQ ? p.lse2 : p.delta)[rhead + min(r, p.len - 1)];
    past = tid < BQ && r >= p.len;
    if (++f_qt == qt_end) {
      f_qt = qt0;
      ++f_h;
    }
  };
  // (The +inf substitution waits until here so that the fetch never waits
  // on its own loads.)
  auto publish = [&](int blk) {
    const int sq = slot(blk, NBQ), sd = slot(blk, NB);
    qreg.store(Qs[sq], tid);
    dreg.store(Ds[sd], tid);
    if (tid < 2 * BQ) stat_s[sd][tid] = past ? kInf : stat;
  };

  // K (P/dV waves, negated for a negative scale) or V (dS/dK waves) rows of
  // this pair's keys as B fragments; keys past the prefix re-read key L-1.
  frag kv[NKT][DK];
  {
    const T* src = (const T*)(pv_wave ? p.k : p.v) + (size_t)(b * p.hkv + hk) * p.kv_cap * D;
#pragma unroll
    for (int nk = 0; nk < NKT; ++nk) {
      const int key = min(wk0 + nk * 16 + n, L - 1);
#pragma unroll
      for (int kb = 0; kb < DK; ++kb) {
        kv[nk][kb] = ldg8(src + (size_t)key * D + kb * 32 + 8 * g);
        if (pv_wave && p.neg) kv[nk][kb] = negate<T>(kv[nk][kb]);
      }
    }
  }
  f32x4 acc[NKT][MD];  // dV (P/dV waves) or dK (dS/dK waves)
#pragma unroll
  for (int nk = 0; nk < NKT; ++nk)
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[nk][md] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (pv_wave) {
    fetch();
    publish(0);
  }
  wait_loads();
  __syncthreads();

  // The two roles run their phases in different orders so that one's
  // products overlap the other's vector work: in iteration it the P/dV wave
  // computes S = Q K^T of block it (products), P (exponentials) and dV +=
  // P^T dO (products); the dS/dK wave first adds dK += dS^T Q for block it - 2
  // (products, dS kept in registers since the previous iteration), then dP =
  // dO V^T for block it - 1 (products) and dS (vector work). Q blocks stay in
  // LDS for four iterations (four buffers), dO blocks and row statistics for
  // three. Each role has its own loop; both pass the same number of barriers.
  if (pv_wave) {
    int qv = qt0;
    for (int it = 0; it <= iters; ++it) {
      const bool more = it + 1 < iters;
      if (more) fetch();
      if (it < iters) {
        const int q0 = qv * BQ;
        const int q_lo = p.start + q0, q_hi = p.start + min(q0 + BQ, p.len) - 1;
        qv = next_qt(qv);
        if (wk0 <= q_hi) {
          const int sd = slot(it, NB);
          const T* A = Qs[slot(it, NBQ)];
          const T* X = Ds[sd];
          f32x4 s[MQ][NKT];
#pragma unroll
          for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
            for (int nk = 0; nk < NKT; ++nk) s[mq][nk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < DK; ++kb)
#pragma unroll
            for (int mq = 0; mq < MQ; ++mq) {
              const frag a = ld8s<PadLay<T, D>>(A, mq * 16 + n, kb * 32 + 8 * g);
#pragma unroll
              for (int nk = 0; nk < NKT; ++nk) E::mma(s[mq][nk], a, kv[nk][kb]);
            }
#pragma unroll
          for (int mq = 0; mq < MQ; ++mq) {
            const f32x4 l4 = *(const f32x4*)&stat_s[sd][mq * 16 + 4 * g];
#pragma unroll
            for (int nk = 0; nk < NKT; ++nk)
#pragma unroll
              for (int i = 0; i < 4; ++i) s[mq][nk][i] = fexp2(__builtin_fmaf(s[mq][nk][i], c2, -l4[i]));
          }
          if (q_lo < wk0 + NKT * 16 - 1) {  // block crosses this pair's diagonal
#pragma unroll
            for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
              for (int nk = 0; nk < NKT; ++nk)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (wk0 + nk * 16 + n > q_lo + mq * 16 + 4 * g + i) s[mq][nk][i] = 0.f;
          }
          frag wf[KQ][NKT];  // P as A fragments of dV
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
            for (int nk = 0; nk < NKT; ++nk) {
              wf[kq][nk] = pack44<T>(s[2 * kq][nk], s[2 * kq + 1][nk]);
              Ps[slot(it, 2)][pair][kq][nk][lane] = wf[kq][nk];
            }
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
            for (int md = 0; md < MD; ++md) {
              const frag x = ldT8<PadLay<T, D>>(X, kq * 32, md * 16, lane);
#pragma unroll
              for (int nk = 0; nk < NKT; ++nk) E::mma(acc[nk][md], wf[kq][nk], x);
            }
        }
      }
      // Q buffer (it + 1) % 4 last held block it - 3, whose dK product ran in
      // iteration it - 1; dO buffer (it + 1) % 3 held block it - 2, read by
      // iteration it - 1 at the latest.
      if (more) publish(it + 1);
      __syncthreads();
    }
    __syncthreads();  // the dS/dK loop runs one iteration more
  } else {
    int qv = qt0;
    bool have_prev = false;  // dS of block it - 2 is held in dsp
    frag dsp[KQ][NKT];
    for (int it = 0; it <= iters + 1; ++it) {
      if (have_prev) {  // dK += dS^T Q for block it - 2
        const T* X = Qs[slot(it - 2, NBQ)];
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
          for (int md = 0; md < MD; ++md) {
            const frag x = ldT8<PadLay<T, D>>(X, kq * 32, md * 16, lane);
#pragma unroll
            for (int nk = 0; nk < NKT; ++nk) E::mma(acc[nk][md], dsp[kq][nk], x);
          }
      }
      have_prev = false;
      const int blk = it - 1;
      if (blk >= 0 && blk < iters) {
        const int q0 = qv * BQ;
        const int q_hi = p.start + min(q0 + BQ, p.len) - 1;
        qv = next_qt(qv);
        if (wk0 <= q_hi) {
          const int sd = slot(blk, NB);
          const T* A = Ds[sd];
          f32x4 s[MQ][NKT];
#pragma unroll
          for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
            for (int nk = 0; nk < NKT; ++nk) s[mq][nk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < DK; ++kb)
#pragma unroll
            for (int mq = 0; mq < MQ; ++mq) {
              const frag a = ld8s<PadLay<T, D>>(A, mq * 16 + n, kb * 32 + 8 * g);
#pragma unroll
              for (int nk = 0; nk < NKT; ++nk) E::mma(s[mq][nk], a, kv[nk][kb]);
            }
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) {
            const f32x4 d4lo = *(const f32x4*)&stat_s[sd][BQ + kq * 32 + 4 * g];
            const f32x4 d4hi = *(const f32x4*)&stat_s[sd][BQ + kq * 32 + 16 + 4 * g];
#pragma unroll
            for (int nk = 0; nk < NKT; ++nk) {
              const frag pf = Ps[slot(blk, 2)][pair][kq][nk][lane];
              f32x4 lo, hi;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                lo[i] = (float)pf[i] * (s[2 * kq][nk][i] - d4lo[i]);
                hi[i] = (float)pf[4 + i] * (s[2 * kq + 1][nk][i] - d4hi[i]);
              }
              dsp[kq][nk] = pack44<T>(lo, hi);
            }
          }
          have_prev = true;
          // Hand dS to the dQ pass: this lane's slots are keys wk0 + 16 nk + n
          // against query rows q0 + 32 kq + {4g..4g+3, 16+4g..16+4g+3}; they
          // are stored key-major (dS^T) as they are, so column 32 kq + 8 g + s
          // of a key's row holds query row 32 kq + tile_row(8 g + s) and each
          // lane writes one 16-byte run.
          if constexpr (sizeof(T) == 2) {
            static_assert(kDsKeyPad % BKV == 0 && kDsCols % BQ == 0, "dS^T block shape");
            if (p.ds) {
              const int nqb = qt_end - qt0;
              const int hb = hk * G + blk / nqb;
              bf16* dsb = (bf16*)p.ds +
                          ((size_t)((b * p.hq + hb) * p.ds_nqb + q0 / kDsCols) * p.ds_keys + wk0) * kDsCols +
                          q0 % kDsCols;
#pragma unroll
              for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
                for (int nk = 0; nk < NKT; ++nk)
                  *(bf16x8*)(dsb + (size_t)(nk * 16 + n) * kDsCols + kq * 32 + 8 * g) =
                      __builtin_bit_cast(bf16x8, dsp[kq][nk]);
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // Read-modify-write of the fp32 accumulator, 16 keys at a time: all reads
  // are issued before any write (or, for a launch that stores, no reads).
  float* dst = (pv_wave ? p.dv : p.dk) + (size_t)(b * p.hkv + hk) * p.kv_cap * D;
  const float scale = pv_wave ? p.dv_scale : p.dk_scale;
  if (p.acc_store) {
#pragma unroll
    for (int nk = 0; nk < NKT; ++nk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = wk0 + nk * 16 + 4 * g + i;
        if (key < L) {
#pragma unroll
          for (int md = 0; md < MD; ++md) dst[(size_t)key * D + md * 16 + n] = scale * acc[nk][md][i];
        }
      }
    return;
  }
#pragma unroll
  for (int nk = 0; nk < NKT; ++nk) {
    f32x4 old[MD];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(wk0 + nk * 16 + 4 * g + i, L - 1);
#pragma unroll
      for (int md = 0; md < MD; ++md) old[md][i] = dst[(size_t)key * D + md * 16 + n];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = wk0 + nk * 16 + 4 * g + i;
      if (key < L) {
#pragma unroll
        for (int md = 0; md < MD; ++md) dst[(size_t)key * D + md * 16 + n] = old[md][i] + scale * acc[nk][md][i];
      }
    }
  }
}

// dK/dV pass as its own launch (the dS hand-over path, whose dQ pass reads
// what this one stores).
template <typename T, int D, int NKT, int BQ, int NP>
__global__ __launch_bounds__(2 * NP * 64) void dkdv_kernel(BwdParams p) {
  __shared__ DkdvLds<T, D, NKT, BQ, NP> sm;
  dkdv_body<T, D, NKT, BQ, NP>(p, blockIdx.x, gridDim.x, sm);
}

template <typename A, typename B, typename C>
union LdsUnion {
  A a;
  B b;
  C c;
};

// The chunk's dQ (recomputing dS) and dK/dV passes in one launch: a sub-grid
// of n_dq query-tile workgroups, one of n_kv key-tile workgroups over keys
// [0, kv_split) and one of n_kvh half-size key-tile workgroups (NKT = 1) over
// [kv_split, L), and last, next.blocks workgroups computing another chunk's
// row statistics, which nothing in this launch reads. The dQ sub-grid goes
// first or last: first when its longest workgroup carries more work than the
// longest key tile, so that the key tiles fill the compute units it leaves
// idle in its last round. All read the same inputs and write disjoint outputs
// (dQ rows; dK/dV keys, each owned by one workgroup), so the result does not
// depend on how their workgroups interleave. Their LDS layouts share one
// allocation. Each sub-grid is padded to a multiple of the 8 XCDs (padding
// workgroups exit at once) so that each keeps the XCD-aware order of its own
// grid.
template <typename T, int D, int NQT, int BK, int NW, int NKT, int BQ, int NP>
__global__ __launch_bounds__(2 * NW * 64) void bwd_kernel(BwdParams p, int n_dq, int n_kv, int n_kvh, int kv_split,
                                                          int dq_first, StatsArgs next) {
  static_assert(NW == NP, "one workgroup shape for both passes");
  __shared__ LdsUnion<DqLds<T, D, BK>, DkdvLds<T, D, NKT, BQ, NP>, DkdvLds<T, D, 1, BQ, NP>> sm;
  const int pad_dq = (n_dq + 7) / 8 * 8, pad_kv = (n_kv + 7) / 8 * 8, pad_kvh = (n_kvh + 7) / 8 * 8;
  int blk = blockIdx.x;
  int kind;  // 0: dQ, 1: key tiles, 2: half-size key tiles, 3: row statistics
  if (dq_first) {
    if (blk < pad_dq) {
      kind = 0;
    } else if ((blk -= pad_dq) < pad_kv) {
      kind = 1;
    } else if ((blk -= pad_kv) < pad_kvh) {
      kind = 2;
    } else {
      blk -= pad_kvh;
      kind = 3;
    }
  } else {
    if (blk < pad_kv) {
      kind = 1;
    } else if ((blk -= pad_kv) < pad_kvh) {
      kind = 2;
    } else if ((blk -= pad_kvh) < pad_dq) {
      kind = 0;
    } else {
      blk -= pad_dq;
      kind = 3;
    }
  }
  if (kind == 3) {
    row_stats<T, D, 2 * NW * 64>(next, blk, next.blocks);
  } else if (kind == 0) {
    if (blk < n_dq) dq_body<T, D, NQT, BK, NW>(p, blk, n_dq, sm.a);
  } else if (kind == 1) {
    if (blk < n_kv) {
      BwdParams q = p;
      q.kv_end = kv_split;
      dkdv_body<T, D, NKT, BQ, NP>(q, blk, n_kv, sm.b);
    }
  } else if constexpr (NKT > 1) {
    if (blk < n_kvh) {
      BwdParams q = p;
      q.kv_first = kv_split;
      dkdv_body<T, D, 1, BQ, NP>(q, blk, n_kvh, sm.c);
    }
  }
}

// Query row (within a group of 32) held by column p of a stored dS^T row:
// the dK/dV pass writes each lane's fragment slots as they are, so column
// 8 g + s holds row 4 g + s for s < 4 and 16 + 4 g + s - 4 otherwise.
__device__ __forceinline__ int tile_row(int p) {
  const int g = (p & 31) >> 3, s = p & 7;
  return (p & ~31) + (s < 4 ? 4 * g + s : 12 + 4 * g + s);
}

// dQ from the dS^T blocks stored by the dK/dV pass (bf16): dQ^T = K^T dS^T
// per key tile, so each lane owns one (stored) query column. Grid
// (batch, q head, block of kDsCols query rows); two groups of NW waves own the
// same query columns and take the even and odd key tiles; pairs of K and dS^T
// tiles stream into double-buffered LDS by direct global->LDS loads one pair
// ahead, and both operands are read through the transposing path. Entries
// above the diagonal were never written (the dK/dV pass skips them), so
// diagonal tiles select zero there. At the end group 1 hands its partial dQ^T
// to group 0 through LDS.
template <int D, int NQT, int BK, int NW>
__global__ __launch_bounds__(2 * NW * 64) void dqs_kernel(BwdParams p) {
  using T = bf16;
  using E = Elt<T>;
  using frag = typename E::frag;
  using Lk = SwzLay<T, D>;
  constexpr int BQ = NW * NQT * 16, MD = D / 16, KB2 = BK / 32;
  using Ls = SwzLay<T, BQ>;
  static_assert(kDsCols % BQ == 0 && NQT * 16 <= 32, "workgroups cover whole slices of a dS^T block");
  __shared__ __attribute__((aligned(16))) T Kb0[2 * BK * D];
  __shared__ __attribute__((aligned(16))) T Sb0[2 * BK * BQ];
  __shared__ __attribute__((aligned(16))) T Kb1[2 * BK * D];
  __shared__ __attribute__((aligned(16))) T Sb1[2 * BK * BQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / NW, wq = wave % NW;
  const int n = lane & 15, g = lane >> 4;
  const int nqt = (p.len + BQ - 1) / BQ;
  const int work_id = xcd_order(blockIdx.x, gridDim.x);
  const int qt = nqt - 1 - work_id % nqt;  // longest rows first
  const int h = (work_id / nqt) % p.hq, b = work_id / (nqt * p.hq);
  const int hk = h / (p.hq / p.hkv);
  const T* K = (const T*)p.k + (size_t)(b * p.hkv + hk) * p.kv_cap * D;
  // This workgroup's columns [cb, cb + BQ) of stored block qt * BQ / kDsCols,
  // whose column c holds chunk row rb + tile_row(c).
  const int rb = qt * BQ / kDsCols * kDsCols, cb = qt * BQ % kDsCols;
  const T* S = (const T*)p.ds + ((size_t)(b * p.hq + h) * p.ds_nqb + qt * BQ / kDsCols) * p.ds_keys * kDsCols + cb;
  const int L = p.start + p.len;
  const int n_tiles = (p.start + min(rb + tile_row(cb + BQ - 1), p.len - 1)) / BK + 1;
  const int n_pairs = (n_tiles + 1) / 2;
  const int c0 = cb + wq * NQT * 16;  // this wave's first stored column
  const int row_lo = rb + tile_row(c0), row_hi = rb + tile_row(c0 + NQT * 16 - 1);
  const bool active = row_lo < p.len;
  const int wq_lo = p.start + row_lo;
  const int wq_hi = p.start + min(row_hi, p.len - 1);
  int qrow[NQT];  // chunk row of this lane's column in each 16-column tile
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) qrow[nt] = rb + tile_row(c0 + nt * 16 + n);

  auto stage = [&](T* kd, T* sd, int pair) {
    stage_tile<T, 2 * BK, D, 2 * NW>(kd, K, 2 * pair * BK, L, wave, lane);
    stage_tile<T, 2 * BK, BQ, 2 * NW, kDsCols>(sd, S, 2 * pair * BK, p.ds_keys, wave, lane);
  };
  stage(Kb0, Sb0, 0);
  f32x4 acc[MD][NQT];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) acc[md][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_loads();
  __syncthreads();

  auto pair_step = [&](int i, const T* Kc, const T* Sc, T* Kn, T* Sn) {
    if (i + 1 < n_pairs) stage(Kn, Sn, i + 1);
    const int j = 2 * i + grp;
    const int kb0 = j * BK;
    if (active && j < n_tiles && kb0 <= wq_hi) {
      const T* Kt = Kc + grp * BK * D;
      const T* St = Sc + grp * BK * BQ;
      const bool diag = kb0 + BK - 1 > wq_lo;
#pragma unroll
      for (int kb2 = 0; kb2 < KB2; ++kb2) {
        frag sf[NQT];
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
          sf[nt] = ldT8<Ls>(St, kb2 * 32, wq * NQT * 16 + nt * 16, lane);
          if (diag) {
            const int qp = p.start + qrow[nt];
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
              const int key = kb0 + kb2 * 32 + (sl < 4 ? 4 * g + sl : 16 + 4 * g + sl - 4);
              if (key > qp) sf[nt][sl] = (T)0.f;
            }
          }
        }
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const frag a = ldT8<Lk>(Kt, kb2 * 32, md * 16, lane);
#pragma unroll
          for (int nt = 0; nt < NQT; ++nt) E::mma(acc[md][nt], a, sf[nt]);
        }
      }
    }
    wait_loads();
    __syncthreads();
  };
  for (int i = 0; i < n_pairs; i += 2) {
    pair_step(i, Kb0, Sb0, Kb1, Sb1);
    if (i + 1 < n_pairs) pair_step(i + 1, Kb1, Sb1, Kb0, Sb0);
  }

  // Merge: group 1 publishes its dQ^T per lane in two halves of the head
  // dimension (Kb0 and Sb0), group 0 adds and stores.
  constexpr int HALF = MD / 2 * 4;
  static_assert(sizeof(Kb0) >= (size_t)NQT * NW * 64 * HALF * sizeof(float) &&
                    sizeof(Sb0) >= (size_t)NQT * NW * 64 * HALF * sizeof(float),
                "merge area");
  float* xo0 = (float*)Kb0;
  float* xo1 = (float*)Sb0;
  if (grp == 1) {
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      const size_t slot = (size_t)(nt * NW + wq);
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float* x = md < MD / 2 ? xo0 : xo1;
          x[(slot * HALF + (md % (MD / 2)) * 4 + e) * 64 + lane] = acc[md][nt][e];
        }
    }
  }
  __syncthreads();
  if (grp == 1 || !active) return;
  float* DQ = p.dq + ((size_t)(b * p.hq + h) * p.q_cap + p.q_off) * D;
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const size_t slot = (size_t)(nt * NW + wq);
    const int row = qrow[nt];
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const float* x = md < MD / 2 ? xo0 : xo1;
      f32x4 v = acc[md][nt];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += x[(slot * HALF + (md % (MD / 2)) * 4 + e) * 64 + lane];
      if (row < p.len) *(f32x4*)(DQ + (size_t)row * D + md * 16 + 4 * g) = v * p.dq_scale;
    }
  }
}

// ----------------------------------------------------------------------------
// acc += scale * src over the first `rows` rows of every head (float4 lanes).
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void accumulate_kernel(float* acc, const float* src, int heads_total,
                                                         int acc_cap, int src_cap, int hd4, int rows,
                                                         float scale) {
  const size_t per_head = (size_t)rows * hd4;
  const size_t total = per_head * heads_total;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = i / per_head, rem = i % per_head;
    f32x4* a = (f32x4*)acc + bh * (size_t)acc_cap * hd4 + rem;
    const f32x4 s = *((const f32x4*)src + bh * (size_t)src_cap * hd4 + rem);
    *a += scale * s;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, size_t n) {
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    ((f32x4*)p)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (blockIdx.x == 0 && threadIdx.x < n % 4) p[n4 * 4 + threadIdx.x] = 0.f;
}
// ----------------------------------------------------------------------------
// Tile configurations per (type, head_dim).
// ----------------------------------------------------------------------------
template <typename T, int D>
struct Cfg {
  static constexpr int FWD_NQT = 2, FWD_BK = 64, FWD_NW = 4;
  static constexpr int DQ_NQT = 2, DQ_BK = 64, DQ_NW = 4;
  static constexpr int KV_NKT = 2, KV_BQ = 64, KV_NP = 4;
};
// float32 storage (the exactness path) takes smaller tiles: its fragments are
// twice as wide in registers.
template <int D>
struct Cfg<float, D> {
  static constexpr int FWD_NQT = 1, FWD_BK = 32, FWD_NW = 4;
  static constexpr int DQ_NQT = 1, DQ_BK = 32, DQ_NW = 4;
  static constexpr int KV_NKT = 1, KV_BQ = 32, KV_NP = 4;
};

// |scale| * log2(e), kept strictly positive so that a masked score of -inf
// times it stays -inf (a zero scale becomes 1e-30: every score then weighs
// exp(~0) = 1, as it should).
float exp2_coef(float scale) {
  const float c = fabsf(scale) * kLog2e;
  return c > 1e-30f ? c : 1e-30f;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Query-tile workgroups of a forward / recompute-dQ launch with NQT 16-row
// tiles per wave.
template <int NW, int NQT>
int q_tiles(const Shape& s) {
  constexpr int BQ = NW * NQT * 16;
  return ((s.len + BQ - 1) / BQ) * s.hq * s.batch;
}

template <typename T, int D>
hipError_t fwd_impl(const Shape& s, const void* q, const void* k, const void* v, void* o, float* lse,
                    hipStream_t st) {
  using C = Cfg<T, D>;
  FwdParams p{q,     k,     v,       o,        lse,     s.hq,    s.hkv, s.q_cap, s.kv_cap, s.q_off,
              s.start, s.len, exp2_coef(s.scale), s.scale < 0.f ? 1 : 0};
  // A chunk too short to give every compute unit a 128-row tile (e.g. 500
  // rows x 32 heads = 128 tiles) runs 64-row tiles: four groups of two
  // 32-row waves on 32-key tiles.
  if constexpr (C::FWD_NQT > 1) {
    if (q_tiles<C::FWD_NW, C::FWD_NQT>(s) < device_cus()) {
      CA_LAUNCH(CA_KERNEL_FWD, (fwd_kernel<T, D, C::FWD_NQT, 32, 2, 4>), dim3(q_tiles<2, C::FWD_NQT>(s)),
                dim3(4 * 2 * 64), 0, st, p);
      return hipGetLastError();
    }
  }
  CA_LAUNCH(CA_KERNEL_FWD, (fwd_kernel<T, D, C::FWD_NQT, C::FWD_BK, C::FWD_NW>),
            dim3(q_tiles<C::FWD_NW, C::FWD_NQT>(s)), dim3(2 * C::FWD_NW * 64), 0, st, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_impl(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, float gs, float* dq, float* dk, float* dv,
                    float* ws, size_t ws_bytes, hipStream_t st, bool stats_ready, const NextStats& next) {
  using C = Cfg<T, D>;
  constexpr int LPR = D / Elt<T>::VEC;
  const int rows = s.batch * s.hq * s.len;
  const int L = s.start + s.len;
  // dS^T goes through the workspace when it has room (bf16 only).
  const size_t ds_need = bwd_ds_bytes(s.batch, s.hq, s.len, L);
  const bool use_ds = sizeof(T) == 2 && ws_bytes >= bwd_ws_base(rows) + ds_need;
  auto stats_of = [&](int q_off, int len, float* w) {
    const int r = s.batch * s.hq * len;
    return StatsArgs{o, dout, lse, w, w + bwd_ws_stride(r), s.q_cap, q_off, len, r, 0};
  };
  auto stats_launch = [&](const StatsArgs& a) {
    CA_LAUNCH(CA_KERNEL_DELTA, (delta_kernel<T, D>), dim3((a.rows * LPR + 255) / 256), dim3(256), 0, st, a);
    return hipGetLastError();
  };
  const StatsArgs cur = stats_of(s.q_off, s.len, ws);
  hipError_t e = hipSuccess;
  if (!stats_ready && (e = stats_launch(cur)) != hipSuccess) return e;
  StatsArgs nx = stats_of(next.q_off, next.len, next.ws);
  float* const delta = cur.delta;
  float* const lse2 = cur.lse2;
  BwdParams p{q,     k,     v,       dout,     lse,     delta,   lse2,  dq,   dk,
              dv,    s.hq,  s.hkv,   s.q_cap,  s.kv_cap, s.q_off, s.start, s.len,
              exp2_coef(s.scale), s.scale < 0.f ? 1 : 0, gs * s.scale, gs * s.scale, gs,
              use_ds ? (void*)((char*)ws + bwd_ws_base(rows)) : nullptr,
              (s.len + kDsCols - 1) / kDsCols, (L + kDsKeyPad - 1) / kDsKeyPad * kDsKeyPad, 0, L,
              s.acc_store ? 1 : 0};
  constexpr int BKV = C::KV_NP * C::KV_NKT * 16, BKV1 = C::KV_NP * 16;
  const int heads = s.hkv * s.batch;
  const int tiles = (L + BKV - 1) / BKV;
  if (!use_ds) {
    // dQ recomputes dS: both passes in one launch. A dQ workgroup (BQD query
    // rows) walks the whole prefix with three products per key; a dK/dV
    // workgroup (BKV keys) walks up to all G * len query rows of its group
    // with four, so the dQ sub-grid goes first once 3 L >= 4 G len.
    constexpr int BQD = C::DQ_NW * C::DQ_NQT * 16;
    const int n_dq = (s.len + BQD - 1) / BQD * s.hq * s.batch;
    const int dq_first = 3LL * L >= 4LL * (s.hq / s.hkv) * s.len ? 1 : 0;
    // Key tiles in whole rounds of one per compute unit; a remainder that
    // half-size tiles (~3/4 of the time each) cover in one round goes to them.
    const int cus = device_cus();
    int tiles_a = tiles, n_kvh = 0;
    if (C::KV_NKT > 1) {
      const int ta = tiles * heads / cus * cus / heads;
      const int nh = (L - ta * BKV + BKV1 - 1) / BKV1 * heads;
      if (ta < tiles && nh <= cus) {
        tiles_a = ta;
        n_kvh = nh;
      }
    }
    const int n_kv = tiles_a * heads;
    const int kv_split = n_kvh > 0 ? tiles_a * BKV : L;
    // The next chunk's row statistics, if asked for, go to at most one
    // workgroup per compute unit at the end of the grid, where they fill the
    // units the last round leaves idle.
    constexpr int RPB = 2 * C::DQ_NW * 64 / LPR;
    if (next.len > 0) nx.blocks = std::min((nx.rows + RPB - 1) / RPB, cus);
    auto pad8 = [](int n) { return (n + 7) / 8 * 8; };
    const int grid = pad8(n_dq) + pad8(n_kv) + pad8(n_kvh) + nx.blocks;
    CA_LAUNCH(CA_KERNEL_BWD, (bwd_kernel<T, D, C::DQ_NQT, C::DQ_BK, C::DQ_NW, C::KV_NKT, C::KV_BQ, C::KV_NP>),
              dim3(grid), dim3(2 * C::DQ_NW * 64), 0, st, p, n_dq, n_kv, n_kvh, kv_split, dq_first, nx);
    return hipGetLastError();
  }
  if constexpr (sizeof(T) == 2) {
    // dS hand-over: the dK/dV pass stores dS^T, then dQ = dS K streams it.
    // Every workgroup of the dK/dV pass owns one key tile and walks all the
    // chunk's queries that see it, so the pass takes whole "rounds" of one
    // tile per compute unit. Key tiles of half the size (16 keys per wave)
    // take ~3/4 of a round: a prefix that fills at most half the units runs
    // on them alone, and when whole rounds of full tiles leave a remainder
    // that half-size tiles can cover in one round, that remainder (the
    // chunk's own diagonal keys, which the fewest queries see) goes to a
    // second launch of them.
    const int cus = device_cus();
    const int rounds = tiles * heads / cus;
    const int tiles_a = rounds * cus / heads;  // full tiles per head in whole rounds
    const bool split = C::KV_NKT > 1 && rounds >= 1 && tiles_a < tiles &&
                       (L - tiles_a * BKV + BKV1 - 1) / BKV1 * heads <= cus;
    if (C::KV_NKT > 1 && 2 * tiles * heads <= cus) {
      CA_LAUNCH(CA_KERNEL_DKDV, (dkdv_kernel<T, D, 1, C::KV_BQ, C::KV_NP>), dim3((L + BKV1 - 1) / BKV1 * heads),
                dim3(2 * C::KV_NP * 64), 0, st, p);
    } else if (split) {
      p.kv_end = tiles_a * BKV;
      CA_LAUNCH(CA_KERNEL_DKDV, (dkdv_kernel<T, D, C::KV_NKT, C::KV_BQ, C::KV_NP>), dim3(tiles_a * heads),
                dim3(2 * C::KV_NP * 64), 0, st, p);
      p.kv_first = tiles_a * BKV;
      p.kv_end = L;
      CA_LAUNCH(CA_KERNEL_DKDV, (dkdv_kernel<T, D, 1, C::KV_BQ, C::KV_NP>),
                dim3((L - p.kv_first + BKV1 - 1) / BKV1 * heads), dim3(2 * C::KV_NP * 64), 0, st, p);
    } else {
      CA_LAUNCH(CA_KERNEL_DKDV, (dkdv_kernel<T, D, C::KV_NKT, C::KV_BQ, C::KV_NP>), dim3(tiles * heads),
                dim3(2 * C::KV_NP * 64), 0, st, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.ds_nqb * s.hq * s.batch < cus) {  // short chunk: 64-column workgroups
      CA_LAUNCH(CA_KERNEL_DQ, (dqs_kernel<D, 1, 64, 4>), dim3(((s.len + 63) / 64) * s.hq * s.batch), dim3(2 * 4 * 64),
                0, st, p);
    } else {
      CA_LAUNCH(CA_KERNEL_DQ, (dqs_kernel<D, 2, 64, 4>), dim3(p.ds_nqb * s.hq * s.batch), dim3(2 * 4 * 64), 0, st, p);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (next.len > 0) return stats_launch(nx);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const Shape& s, const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t st) {
  if (s.dtype == CA_BF16) {
    return s.head_dim == 128 ? fwd_impl<bf16, 128>(s, q, k, v, o, lse, st)
                             : fwd_impl<bf16, 64>(s, q, k, v, o, lse, st);
  }
  return s.head_dim == 128 ? fwd_impl<float, 128>(s, q, k, v, o, lse, st)
                           : fwd_impl<float, 64>(s, q, k, v, o, lse, st);
}

hipError_t launch_bwd(const Shape& s, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, float gs, float* dq, float* dk, float* dv,
                      float* ws, size_t ws_bytes, hipStream_t st, bool stats_ready, const NextStats& next) {
  if (s.dtype == CA_BF16) {
    return s.head_dim == 128
               ? bwd_impl<bf16, 128>(s, q, k, v, o, lse, dout, gs, dq, dk, dv, ws, ws_bytes, st, stats_ready, next)
               : bwd_impl<bf16, 64>(s, q, k, v, o, lse, dout, gs, dq, dk, dv, ws, ws_bytes, st, stats_ready, next);
  }
  return s.head_dim == 128
             ? bwd_impl<float, 128>(s, q, k, v, o, lse, dout, gs, dq, dk, dv, ws, ws_bytes, st, stats_ready, next)
             : bwd_impl<float, 64>(s, q, k, v, o, lse, dout, gs, dq, dk, dv, ws, ws_bytes, st, stats_ready, next);
}

hipError_t launch_accumulate(float* acc, const float* src, int batch, int heads, int acc_cap, int src_cap,
                             int head_dim, int rows, float scale, hipStream_t st) {
  const size_t total = (size_t)batch * heads * rows * (head_dim / 4);
  if (total == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  CA_LAUNCH(CA_KERNEL_ACCUMULATE, accumulate_kernel, dim3(blocks), dim3(256), 0, st, acc, src, batch * heads, acc_cap,
            src_cap, head_dim / 4, rows, scale);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t want = (n / 4 + 255) / 256;
  const int blocks = (int)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  CA_LAUNCH(CA_KERNEL_ZERO, zero_kernel, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace ca
