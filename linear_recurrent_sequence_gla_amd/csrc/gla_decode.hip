// gla_decode.hip -- one recurrent inference step, S <- Diag(exp g) S + k^T v, o = q S.
//
// This is the O(1)-memory recurrent form (MS-GLA summary, section 1; GSA abstract).  Per
// step the whole fp32 state is read and written once, so the kernel is a pure HBM stream:
// 0.5 flop per byte.  One workgroup per (batch*head, 64 value columns): 16 lanes cover 64
// contiguous columns with 16-byte accesses (256 bytes per state row) and 16 row groups walk
// the key rows, eight rows per thread per pass.  q, k and the decay are requested first and the
// state rows of the first pass right after, so the barrier that publishes the token's inputs
// through LDS waits for those alone and overlaps the state stream; q.S is reduced over the
// row groups in LDS at the end.  No matrix cores: a rank-1 update plus a vector-matrix product
// has nothing to contract.
#include "common.hpp"
#include "kernels.hpp"

namespace gla {

template <typename T>
__global__ __launch_bounds__(256) void gla_decode_kernel(DecodeParams p, int ntile) {
  constexpr int RPP = 8;                       // rows per thread per pass
  __shared__ float sq[256], sk[256], sa[256];
  __shared__ f32x4 sred[16][16];
  const int tile = blockIdx.x % ntile, bh = blockIdx.x / ntile;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int Dk = p.Dk, Dv = p.Dv;
  const int j = tile * 64 + 4 * tx;
  const bool jok = j < Dv;
  const int jc = min(j, Dv - 4);               // in-bounds column for lanes past Dv
  float* S = p.state + (size_t)bh * Dk * Dv + jc;

  // the token's inputs are requested first (clamped, unconditionally): loads complete in issue
  // order, so the wait before the barrier that publishes them does not cover the state rows
  const size_t ot = (size_t)bh * Dk + min(tid, Dk - 1);
  const T qt = reinterpret_cast<const T*>(p.q)[ot];
  const T kt = reinterpret_cast<const T*>(p.k)[ot];
  const T gt = reinterpret_cast<const T*>(p.g)[ot];
  const typename Vec4<T>::type vr =
      *reinterpret_cast<const typename Vec4<T>::type*>(reinterpret_cast<const T*>(p.v) + (size_t)bh * Dv + jc);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s[RPP];
#pragma unroll
  for (int m = 0; m < RPP; ++m) s[m] = *reinterpret_cast<const f32x4*>(S + (size_t)min(ty + 16 * m, Dk - 1) * Dv);
  if (tid < Dk) {
    sq[tid] = to_f32(qt);
    sk[tid] = to_f32(kt);
    sa[tid] = fast_exp2(to_f32(gt) * kLog2e);
  }
  __syncthreads();

  f32x4 acc = zero4();
  for (int base = 0; base < Dk; base += 16 * RPP) {
    if (base > 0) {
#pragma unroll
      for (int m = 0; m < RPP; ++m)
        s[m] = *reinterpret_cast<const f32x4*>(S + (size_t)min(base + ty + 16 * m, Dk - 1) * Dv);
    }
#pragma unroll
    for (int m = 0; m < RPP; ++m) {
      const int i = base + ty + 16 * m;
      if (i < Dk) {
        const float a = sa[i], kv = sk[i], qv = sq[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[m][e] = a * s[m][e] + kv * to_f32(vr[e]);
          acc[e] += qv * s[m][e];
        }
        if (jok) *reinterpret_cast<f32x4*>(S + (size_t)i * Dv) = s[m];
      }
    }
  }
  sred[ty][tx] = acc;
  __syncthreads();
  if (tid < 64) {
    const int c = tid >> 2, e = tid & 3;
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += sred[r][c][e];
    const int jj = tile * 64 + tid;
    if (jj < Dv) reinterpret_cast<T*>(p.o)[(size_t)bh * Dv + jj] = from_f32<T>(sum);
  }
}

template <typename T>
hipError_t launch_gla_decode(const DecodeParams& p, hipStream_t s) {
  const int ntile = (p.Dv + 63) / 64;
  hipLaunchKernelGGL((gla_decode_kernel<T>), dim3(ntile * p.BH), dim3(256), 0, s, p, ntile);
  return hipGetLastError();
}

template hipError_t launch_gla_decode<bf16>(const DecodeParams&, hipStream_t);
template hipError_t launch_gla_decode<float>(const DecodeParams&, hipStream_t);

}  // namespace gla
