// gla_decode.hip -- one recurrent inference step, S <- Diag(exp g) S + k^T v, o = q S.
//
// This is the O(1)-memory recurrent form (MS-GLA summary, section 1; GSA abstract).  Per
// step the whole fp32 state is read and written once, so the kernel is a pure HBM stream:
// 0.5 flop per byte.  One workgroup per (batch*head, 64 value columns): 16 lanes cover 64
// contiguous columns with 16-byte accesses (256 bytes per state row) and 16 row groups walk
// the key rows; q.S is reduced over the row groups in LDS.  No matrix cores: a rank-1 update
// plus a vector-matrix product has nothing to contract.
#include "common.hpp"
#include "kernels.hpp"

namespace gla {

template <typename T>
__global__ __launch_bounds__(256) void gla_decode_kernel(DecodeParams p, int ntile) {
  __shared__ float sq[256], sk[256], sa[256];
  __shared__ f32x4 sred[16][16];
  const int tile = blockIdx.x % ntile, bh = blockIdx.x / ntile;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int Dk = p.Dk, Dv = p.Dv;
  const T* q = reinterpret_cast<const T*>(p.q) + (size_t)bh * Dk;
  const T* k = reinterpret_cast<const T*>(p.k) + (size_t)bh * Dk;
  const T* g = reinterpret_cast<const T*>(p.g) + (size_t)bh * Dk;
  for (int i = tid; i < Dk; i += 256) {
    sq[i] = to_f32(q[i]);
    sk[i] = to_f32(k[i]);
    sa[i] = fast_exp2(to_f32(g[i]) * kLog2e);
  }
  __syncthreads();
  const int j = tile * 64 + 4 * tx;
  f32x4 acc = zero4();
  if (j < Dv) {
    const T* v = reinterpret_cast<const T*>(p.v) + (size_t)bh * Dv + j;
    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f32(v[e]);
    float* S = p.state + (size_t)bh * Dk * Dv + j;
#pragma unroll 4
    for (int i = ty; i < Dk; i += 16) {
      f32x4 s = *reinterpret_cast<const f32x4*>(S + (size_t)i * Dv);
      const float a = sa[i], kv = sk[i], qv = sq[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = a * s[e] + kv * vv[e];
        acc[e] += qv * s[e];
      }
      *reinterpret_cast<f32x4*>(S + (size_t)i * Dv) = s;
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
