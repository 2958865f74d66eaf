// common.hpp -- gfx950 building blocks shared by the GLA / GSA kernels.
//
// Matrix-core tile convention used everywhere (one wave = 64 lanes, lane = 16*grp + col):
//   D[16x16] += X[16 x 32] * Y[32 x 16]^T-style contraction, written as
//   D[m][n] += sum_k X[m][k] * Y[n][k]
//   X fragment: lane holds X[m = col][k in kset(grp)], 8 values
//   Y fragment: lane holds Y[n = col][k in kset(grp)], 8 values
//   D accumulator (f32x4): lane holds D[m = 4*grp + e][n = col], e = 0..3
// kset(grp) is any fixed set of 8 k-indices per lane group, as long as X and Y use the same
// sets; the plain choice is {8*grp .. 8*grp+7}.  The "split" choice
// {4*grp + 0..3} U {16 + 4*grp + 0..3} lets two stacked accumulator blocks be fed back as a Y
// fragment without moving data between lanes.
//
// bf16: one v_mfma_f32_16x16x32_bf16 per fragment pair.
// fp32: eight v_mfma_f32_16x16x4_f32, the e-th taking element e of each fragment (in that
//       instruction lane group grp contributes k-index kset(grp)[e]).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// 8 consecutive elements p[0..7] (p 16-byte aligned).
__device__ __forceinline__ Frag<bf16> ld8(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> ld8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  Frag<float> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
// split set: p[0..3] and p[16..19] (p 8-byte aligned for bf16, 16-byte for fp32).
__device__ __forceinline__ Frag<bf16> ld8_split(const bf16* p) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> ld8_split(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
  Frag<float> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
// 8 elements down a column: p[0], p[ld], ..., p[7*ld].
template <typename T>
__device__ __forceinline__ Frag<T> ld8_col(const T* p, int ld) {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = p[e * ld];
  return f;
}
// The same column run of a row-major LDS tile, addressed by the corner of its 32 x 16 block:
// lane (grp, col) gets blk[(8 * grp + e) * ld + col], e = 0..7 -- the k-run of a
// matrix-core operand whose k index runs down the tile's rows.  For 16-bit types this is two
// transposing LDS reads (ds_read_b64_tr_b16): within each 16-lane group, lane 4u+t receives
// element t of the 4-element rows read by lanes u, u+4, u+8 and u+12, so lane j reads row
// j / 4 of a 4-row slab at column 4 * (j % 4).  ld * sizeof(T) must be a multiple of 8.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
// lane: this thread's lane in its wave (threadIdx.x & 63)
template <typename T>
__device__ __forceinline__ Frag<T> ld8_colblk(const T* blk, int ld, int lane);
template <>
__device__ __forceinline__ Frag<bf16> ld8_colblk(const bf16* blk, int ld, int lane) {
  typedef i16x4 __attribute__((address_space(3)))* lds_ptr;
  const int grp = lane >> 4, j = lane & 15;
  bf16* a = const_cast<bf16*>(blk) + (8 * grp + (j >> 2)) * ld + 4 * (j & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)a);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(a + 4 * ld));
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}
template <>
__device__ __forceinline__ Frag<float> ld8_colblk(const float* blk, int ld, int lane) {
  const int grp = lane >> 4, col = lane & 15;
  return ld8_col(blk + 8 * grp * ld + col, ld);
}
template <typename T>
__device__ __forceinline__ Frag<T> ld8_colblk(const T* blk, int ld) {
  return ld8_colblk(blk, ld, (int)threadIdx.x & 63);
}

// The thread's index through an opaque register move.  A kernel that loops over work items
// takes it once per item, so that the compiler recomputes the per-lane LDS addresses derived
// from it inside each item instead of hoisting them all out of the loop, where every one of
// them would stay live across the whole loop body.
__device__ __forceinline__ int opaque_thread_index() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

// Split-set fragment taken from two stacked accumulator blocks (rows 4*grp+e of block a and
// of block b): the Y operand of a contraction over the accumulator's row index.
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_acc(const f32x4& a, const f32x4& b) {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = from_f32<T>(a[e]);
    f.v[4 + e] = from_f32<T>(b[e]);
  }
  return f;
}

// An operand carried as hi + lo (hi = T(x), lo = T(x - hi)); for fp32 the lo part is zero
// and unused.  mma3 forms hi.hi + hi.lo + lo.hi, about 2^-17 per term for bf16.
template <typename T>
struct HiLo {
  Frag<T> hi, lo;
};
template <typename T>
__device__ __forceinline__ HiLo<T> hilo(const float (&x)[8]) {
  HiLo<T> r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    r.hi.v[e] = from_f32<T>(x[e]);
    r.lo.v[e] = from_f32<T>(x[e] - to_f32(r.hi.v[e]));
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void mma3(f32x4& acc, const HiLo<T>& a, const HiLo<T>& b) {
  mma(acc, a.hi, b.hi);
  if constexpr (sizeof(T) == 2) {
    mma(acc, a.hi, b.lo);
    mma(acc, a.lo, b.hi);
  }
}
template <typename T>
__device__ __forceinline__ Frag<T> frag_of(const float (&x)[8]) {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = from_f32<T>(x[e]);
  return f;
}

// 16-byte vector of T for coalesced copies.
template <typename T> struct V16;
template <> struct V16<bf16> { static constexpr int N = 8; typedef bf16x8 type; };
template <> struct V16<float> { static constexpr int N = 4; typedef f32x4 type; };

// Four consecutive elements of T, for 8- or 16-byte vector accesses.
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Block-wide max of a non-negative value over NT threads; `red` holds >= NT/64 floats of LDS.
template <int NT = 256>
__device__ __forceinline__ float block_max(float v, float* red, int tid = threadIdx.x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = tid >> 6;
  if ((tid & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Map a flat block index so that consecutive "logical" indices land on the same XCD
// (blocks are dispatched round-robin over the 8 XCDs; each XCD has its own L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  const int per = nblocks / 8;
  return (bid % 8) * per + bid / 8;
}

}  // namespace gla
