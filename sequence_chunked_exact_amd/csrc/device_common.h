// Device-side building blocks shared by the attention and projection kernels
// for gfx950 (CDNA4): element types and their MFMA wrappers, LDS tile layouts
// and the fragment loaders that read them, global->LDS staging helpers.
//
// Matrix products run on v_mfma_f32_16x16x32_bf16 (bf16 storage) or
// v_mfma_f32_16x16x4_f32 (float32 storage, eight of them per 32-deep step),
// always accumulating in float32. For a 16x16 output tile, lane l (n = l % 16,
// g = l / 16) holds rows 4g..4g+3 of column n. A and B operands give each lane
// 8 contraction slots; lane l feeds row/column n. Two slot orders are used:
//   contiguous: slot s <-> index 8g + s (operands read straight from memory)
//   tile order: slot s <-> 4g + s for s < 4, 16 + 4g + (s - 4) for s >= 4,
// the second being what a lane already holds from two stacked output tiles, so
// P and dS feed the next product from registers with no data movement. Both
// operands of a product always use the same order, which is all a k-reduction
// needs.
#pragma once

#include "launch.h"

#include "chunk_attn.h"

#include <math.h>

namespace ca {
namespace {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_huge_valf();
constexpr float kRescale = 8.f;  // lazy-rescale threshold, log2 units

template <typename T>
struct Elt;

template <>
struct Elt<bf16> {
  using frag = bf16x8;  // a lane's 8 contraction slots
  using vec = bf16x8;   // 16-byte memory vector
  using vec8 = bf16x8;  // 8 elements
  using quad = bf16x4;
  static constexpr int VEC = 8;
  static __device__ __forceinline__ void mma(f32x4& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Elt<float> {
  using frag = f32x8;
  using vec = f32x4;
  using vec8 = f32x8;
  using quad = f32x4;
  static constexpr int VEC = 4;
  static __device__ __forceinline__ void mma(f32x4& c, const frag& a, const frag& b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  }
};

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two row-major [rows][D] LDS tile layouts; both keep the two read patterns
// used here free of bank conflicts: 16 lanes reading one 16-byte chunk
// column from 16 consecutive rows (row-major fragments), and the transposing
// read of 16 rows x 32 bytes, which lands on every bank exactly twice (its
// minimum: 512 bytes in two passes).
//
// PadLay: rows padded by 32 bytes (row stride RS = D + 32 / sizeof(T)
// elements, an odd multiple of 8 banks for every head size here), so 16
// consecutive rows start in 16 different bank groups. A lane's address is a
// loop-invariant base plus a constant offset. Used for tiles written from
// registers.
template <typename T, int D>
struct PadLay {
  static constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  static constexpr int RS = D + 2 * EPC;      // row stride in elements
  static_assert(((RS * sizeof(T) / 4 / 8) & 1) == 1, "row stride must be an odd multiple of 8 banks");
  static __device__ __forceinline__ int off(int r, int c) { return r * RS + c; }
};

// SwzLay: unpadded rows (stride D), the 16-byte chunk c of row r stored at
// chunk position c ^ swz(r). The map (r mod 16, with bit 3 ^= bit 0 and bit
// 2 ^= bit 3) was picked by measuring gfx950's LDS bank-conflict counter over
// a family of candidate maps; it is the simplest one under which both read
// patterns run conflict-free. Used for tiles filled by direct global->LDS
// loads, which write each wave's 64 x 16 bytes contiguously.
template <typename T, int D>
struct SwzLay {
  static constexpr int EPC = 16 / sizeof(T);
  static constexpr int CH = D / EPC;  // chunks per row
  static constexpr int RS = D;
  static __device__ __forceinline__ int swz(int r) {
    const int x = (r ^ ((r & 1) << 3) ^ (((r >> 3) & 1) << 2)) & 15;
    return x & (CH - 1);
  }
  static __device__ __forceinline__ int off(int r, int c) {
    return r * D + (((c / EPC) ^ swz(r)) * EPC) + (c % EPC);
  }
};

// 8 consecutive elements of row r from column c (c % 8 == 0), contiguous order.
template <class Lt>
__device__ __forceinline__ bf16x8 ld8s(const bf16* t, int r, int c) {
  return *(const bf16x8*)(t + Lt::off(r, c));
}
template <class Lt>
__device__ __forceinline__ f32x8 ld8s(const float* t, int r, int c) {
  const f32x4 a = *(const f32x4*)(t + Lt::off(r, c));
  const f32x4 b = *(const f32x4*)(t + Lt::off(r, c + 4));
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// This lane's {t[rb + k][c0 + n] : k = 0..3} (n = lane % 16; rb a multiple of 4,
// the same for the 16 lanes of a group). bf16 uses the transposing LDS read:
// lane j of a group points at row rb + j/4, columns c0 + 4(j%4) .. +3, and the
// hardware hands lane i element k of lane 4k + i/4's four.
template <class Lt>
__device__ __forceinline__ bf16x4 ldT4(const bf16* t, int rb, int c0, int lane) {
  const int j = lane & 15;
  const bf16* p = t + Lt::off(rb + (j >> 2), c0 + 4 * (j & 3));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}
template <class Lt>
__device__ __forceinline__ f32x4 ldT4(const float* t, int rb, int c0, int lane) {
  const int n = lane & 15;
  f32x4 v;
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = t[Lt::off(rb + k, c0 + n)];
  return v;
}
// Fragment of t[kbase + tile-order slots][c0 + n] (operand contracted over rows).
template <class Lt>
__device__ __forceinline__ bf16x8 ldT8(const bf16* t, int kbase, int c0, int lane) {
  const int g = lane >> 4;
  const bf16x4 a = ldT4<Lt>(t, kbase + 4 * g, c0, lane), b = ldT4<Lt>(t, kbase + 16 + 4 * g, c0, lane);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <class Lt>
__device__ __forceinline__ f32x8 ldT8(const float* t, int kbase, int c0, int lane) {
  const int g = lane >> 4;
  const f32x4 a = ldT4<Lt>(t, kbase + 4 * g, c0, lane), b = ldT4<Lt>(t, kbase + 16 + 4 * g, c0, lane);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Fragment of row r, columns kbase + tile-order slots (4g + s, 16 + 4g + s - 4).
template <class Lt>
__device__ __forceinline__ bf16x8 ld8t(const bf16* t, int r, int kbase, int g) {
  const bf16x4 a = *(const bf16x4*)(t + Lt::off(r, kbase + 4 * g));
  const bf16x4 b = *(const bf16x4*)(t + Lt::off(r, kbase + 16 + 4 * g));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <class Lt>
__device__ __forceinline__ f32x8 ld8t(const float* t, int r, int kbase, int g) {
  const f32x4 a = *(const f32x4*)(t + Lt::off(r, kbase + 4 * g));
  const f32x4 b = *(const f32x4*)(t + Lt::off(r, kbase + 16 + 4 * g));
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 8 consecutive elements from global memory.
__device__ __forceinline__ bf16x8 ldg8(const bf16* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ f32x8 ldg8(const float* p) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// A fragment of ones: as the A operand of a product with P^T it gives every
// output lane the sum of P over the 32 contracted rows.
template <typename T>
__device__ __forceinline__ typename Elt<T>::frag ones_frag() {
  typename Elt<T>::frag f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (T)1.f;
  return f;
}

// Two stacked output tiles' registers -> fragment in tile slot order.
template <typename T>
__device__ __forceinline__ typename Elt<T>::frag pack44(const f32x4& lo, const f32x4& hi) {
  typename Elt<T>::frag f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = (T)lo[i];
    f[4 + i] = (T)hi[i];
  }
  return f;
}

template <typename T>
__device__ __forceinline__ typename Elt<T>::frag negate(const typename Elt<T>::frag& f) {
  typename Elt<T>::frag r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = -f[i];
  return r;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, const f32x4& x, float mul) {
  typename Elt<T>::quad v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (T)(x[i] * mul);
  *(typename Elt<T>::quad*)dst = v;
}

// Maximum / sum over the 4 lanes l, l^16, l^32, l^48 (the 4 row groups of one
// output column).
__device__ __forceinline__ float max4(float m) {
  m = fmaxf(m, __shfl_xor(m, 16));
  return fmaxf(m, __shfl_xor(m, 32));
}

// Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its
// own L2. This maps the linear id to a logical work index so that every XCD
// receives one contiguous range of the logical order (heads outermost): the
// workgroups streaming the same K/V (forward, dQ) or the same Q/dO (dK/dV)
// then share one L2. Within a range the order is ascending, i.e. each XCD
// starts with the first (longest) tiles of its heads.
__device__ __forceinline__ int xcd_order(int id, int n) {
  constexpr int X = 8;
  const int per = n / X;
  return id < per * X ? (id % X) * per + id / X : id;
}

typedef __attribute__((address_space(3))) void lds_void;

// Stream rows [row0, row0 + ROWS) of a row-major [*, D] head into a SwzLay
// LDS tile with direct global->LDS loads, shared by NW waves: each wave
// instruction fills 64 consecutive 16-byte LDS slots, so lane l fetches the
// global chunk that belongs in its slot (the swizzle is applied on the global
// side, and each instruction still reads whole rows). Rows at or beyond
// `limit` (>= 1) re-read row limit-1; every consumer gives such rows zero
// weight (keys past the prefix are causally masked).
// SRC_STRIDE: elements between consecutive source rows (a tile may be a
// column slice of a wider row-major matrix).
// The loads use the buffer form of the instruction. The compiler tracks that
// form on the vector-memory counter alone; the global form is a flat access,
// and while one is in flight the compiler waits for every outstanding LDS
// read before each use, so no read can run ahead of the products. The buffer
// starts at the first row the tile reads and spans only the rows it reads,
// so offsets stay small for a head of any length.
template <typename T, int ROWS, int D, int NW, int SRC_STRIDE = D>
__device__ __forceinline__ void stage_tile(T* lds, const T* head, int row0, int limit, int wave, int lane) {
  using Lt = SwzLay<T, D>;
  constexpr int CH = Lt::CH, RPI = 64 / CH, PER_WAVE = ROWS / NW;
  static_assert(CH <= 64 && PER_WAVE % RPI == 0, "tile rows per wave must fill whole instructions");
  static_assert((long long)ROWS * SRC_STRIDE * sizeof(T) < (1LL << 31), "tile span fits a 32-bit offset");
#if defined(__HIP_DEVICE_COMPILE__)  // the LDS-loading builtin exists only in the device pass
  const int b0 = min(row0, limit - 1);
  const int nrec = (min(row0 + ROWS, limit) - b0) * SRC_STRIDE * (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(head + (size_t)b0 * SRC_STRIDE), (short)0, nrec, 0x00020000);
  const int rl = lane / CH, slot = lane % CH;
#pragma unroll
  for (int i = 0; i < PER_WAVE / RPI; ++i) {
    const int rb = wave * PER_WAVE + i * RPI;  // wave-uniform first row of this instruction
    const int r = rb + rl;
    const int c = slot ^ Lt::swz(r);
    const int voff = ((min(row0 + r, limit - 1) - b0) * SRC_STRIDE + c * Lt::EPC) * (int)sizeof(T);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + rb * D), 16, voff, 0, 0, 0);
  }
#endif
}

// A [ROWS][D] tile staged through registers: thread tid fetches R rows of
// one 16-byte column vector and later writes them into a PadLay LDS tile
// (threads beyond the tile's ROWS * D / VEC vectors fetch a duplicate and
// store nothing). The loads go through a buffer over the head's first
// `limit` rows, so rows at or beyond it read as zero (with 32-bit offsets and
// no clamp per row); every consumer gives such rows zero weight (query rows
// past the chunk get LSE = +inf). Plain loads into registers let the next
// tile's fetch overlap the current tile's math without any LDS ordering.
template <typename T, int ROWS, int D, int NT>
struct RegTile {
  using V = typename Elt<T>::vec;
  static constexpr int VEC = Elt<T>::VEC;
  static constexpr int NDV = D / VEC;      // column vectors per row
  static constexpr int GROUPS = NT / NDV;  // row groups
  static constexpr bool SPARE = GROUPS > ROWS;
  static constexpr int R = SPARE ? 1 : ROWS / GROUPS;  // rows per thread
  static_assert(NT % NDV == 0 && (SPARE || ROWS % GROUPS == 0), "tile/thread shape");
  V r[R];

  __device__ __forceinline__ void load(const T* head, int row0, int limit, int tid) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer-load builtins exist only in the device pass
    const int dv = tid % NDV, grp = SPARE ? min(tid / NDV, ROWS - 1) : tid / NDV;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)head, (short)0, limit * D * (int)sizeof(T), 0x00020000);
#pragma unroll
    for (int i = 0; i < R; ++i)
      r[i] = __builtin_bit_cast(
          V, __builtin_amdgcn_raw_buffer_load_b128(rsrc, ((row0 + grp * R + i) * D + dv * VEC) * (int)sizeof(T), 0, 0));
#endif
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
    const int dv = tid % NDV, grp = tid / NDV;
    if (SPARE && grp >= ROWS) return;
#pragma unroll
    for (int i = 0; i < R; ++i) *(V*)(lds + PadLay<T, D>::off(grp * R + i, dv * VEC)) = r[i];
  }
};

// Wait for every load this wave has in flight. Called once before a main
// loop: wait counting in the compiler cannot tell the first iteration from
// the others, so a register loaded before the loop and first read inside it
// would otherwise wait, in every iteration, on the in-order load counter for
// the next tile's prefetch as well.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace
}  // namespace ca
