// gsa_decode.hip -- one recurrent inference step of gated slot attention (GSA).
//
// GSA's bounded slot memories give recurrent inference a fixed-size state per head (GSA
// abstract: efficient recurrent inference; research-map summary, "Approach").  Per
// (batch, head), with alpha = exp(g) and w = -expm1(g) = 1 - alpha (one value per slot):
//   hk[:, s] <- alpha_s hk[:, s] + w_s k       (slot keys, stored transposed: [Dk][m])
//   hv[s, :] <- alpha_s hv[s, :] + w_s v       (slot values: [m][Dv])
//   z = q hk,  p = softmax(z) over the m slots (or an element-wise read-out),  o = p hv
// Both fp32 memories are read and written once per step: an HBM stream at about 0.5 flop per
// byte, like the GLA decode step, with nothing to contract on matrix cores.  The softmax
// couples every slot, so one workgroup holds one (batch, head), with 16-byte accesses: each
// wave owns whole rows of hk and whole columns of hv.  The first rows of both memories are
// requested before anything else; hv is updated and written back before the softmax, since
// its update does not need p.  z is folded over a wave's rows by shuffles and over the waves
// through LDS (one barrier); every wave then forms the softmax for itself, so o is folded
// over rows by shuffles with no further barrier.  The softmax subtracts the maximum and
// normalises o once at the end.
#include "common.hpp"
#include "kernels.hpp"

namespace gla {

constexpr int kGsaDecThreads = 256;
constexpr int kGsaDecRows = 8;                 // rows per thread per pass, for each memory

__device__ __forceinline__ int pow2_ceil(int x) { return x <= 1 ? 1 : 1 << (32 - __builtin_clz(x - 1)); }

template <typename T>
__global__ __launch_bounds__(kGsaDecThreads) void gsa_decode_kernel(GsaDecodeParams p) {
  constexpr int NT = kGsaDecThreads, R = kGsaDecRows, NW = NT / 64;
  __shared__ float sq[256], sk[256], sa[256], sw[256];
  __shared__ float szp[NW][256];               // per-wave partial z
  __shared__ float sp[NW][256];                // per-wave copy of exp(z - max)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, bh = blockIdx.x;
  const int Dk = p.Dk, Dv = p.Dv, m = p.m;
  // hk: whole rows per wave.  NSGP (a power of two) lanes span the m/4 slot groups of a row, so
  // a wave's row groups differ in the high lane bits and z folds over them by shuffles.
  const int NSG = m >> 2, NSGP = pow2_ceil(NSG), NRK = NT / NSGP;
  const int sgl = tid & (NSGP - 1), rk = tid / NSGP;
  const bool kact = sgl < NSG;
  const int sg = min(sgl, NSG - 1);
  // hv: whole columns per wave.  CGW groups of 4 columns per wave (Dv/16 with four waves),
  // padded to CGWP lanes; o folds over the wave's RVW row groups by shuffles.
  const int CGW = (Dv >> 2) / NW, CGWP = pow2_ceil(CGW), RVW = 64 / CGWP;
  const int cgl = lane & (CGWP - 1), rv = lane / CGWP;
  const bool vact = cgl < CGW;
  const int cg = wave * CGW + min(cgl, CGW - 1);

  // the token's inputs are requested first (from clamped addresses, unconditionally): loads
  // complete in issue order, so their wait then does not cover the memories' rows
  const T qt = reinterpret_cast<const T*>(p.q)[(size_t)bh * Dk + min(tid, Dk - 1)];
  const T kt = reinterpret_cast<const T*>(p.k)[(size_t)bh * Dk + min(tid, Dk - 1)];
  const T gt = reinterpret_cast<const T*>(p.g)[(size_t)bh * m + min(tid, m - 1)];
  const typename Vec4<T>::type vt =
      *reinterpret_cast<const typename Vec4<T>::type*>(reinterpret_cast<const T*>(p.v) + (size_t)bh * Dv + 4 * cg);
  __builtin_amdgcn_sched_barrier(0);          // keep them ahead of the memories' rows
  float* HK = p.hk + (size_t)bh * Dk * m + 4 * sg;
  float* HV = p.hv + (size_t)bh * m * Dv + 4 * cg;
  f32x4 hk[R], hv[R];
#pragma unroll
  for (int u = 0; u < R; ++u) hk[u] = *reinterpret_cast<const f32x4*>(HK + (size_t)min(rk + NRK * u, Dk - 1) * m);
#pragma unroll
  for (int u = 0; u < R; ++u) hv[u] = *reinterpret_cast<const f32x4*>(HV + (size_t)min(rv + RVW * u, m - 1) * Dv);
  if (tid < Dk) sq[tid] = to_f32(qt), sk[tid] = to_f32(kt);
  if (tid < m) {
    const float g = to_f32(gt);
    sa[tid] = expf(g);
    sw[tid] = -expm1f(g);
  }
  __syncthreads();

  // slot keys: update, write back, and z partial sums over this thread's rows
  float ak[4], wk[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ak[e] = sa[4 * sg + e], wk[e] = sw[4 * sg + e];
  f32x4 zacc = zero4();
  for (int base = 0; base < Dk; base += NRK * R) {
    if (base > 0) {
#pragma unroll
      for (int u = 0; u < R; ++u)
        hk[u] = *reinterpret_cast<const f32x4*>(HK + (size_t)min(base + rk + NRK * u, Dk - 1) * m);
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int i = base + rk + NRK * u;
      if (i < Dk) {
        const float kv = sk[i], qv = sq[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hk[u][e] = ak[e] * hk[u][e] + wk[e] * kv;
          zacc[e] += qv * hk[u][e];
        }
        if (kact) *reinterpret_cast<f32x4*>(HK + (size_t)i * m) = hk[u];
      }
    }
  }
  // slot values, first pass: update and write back now; o needs p and waits for the softmax
  float vv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = to_f32(vt[e]);
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int s = rv + RVW * u;
    if (s < m) {
      const float a = sa[s], w = sw[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[u][e] = a * hv[u][e] + w * vv[e];
      if (vact) *reinterpret_cast<f32x4*>(HV + (size_t)s * Dv) = hv[u];
    }
  }
  // z over the wave's rows, then over the waves through LDS
  for (int off = NSGP; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) zacc[e] += __shfl_xor(zacc[e], off, 64);
  }
  if (lane < NSGP && kact) {
#pragma unroll
    for (int e = 0; e < 4; ++e) szp[wave][4 * sg + e] = zacc[e];
  }
  __syncthreads();

  // read-out over the m slots, computed by every wave for itself: lane holds slots lane + 64 j
  float z[4];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = lane + 64 * j;
    z[j] = -INFINITY;
    if (s < m) {
      z[j] = szp[0][s];
#pragma unroll
      for (int w = 1; w < NW; ++w) z[j] += szp[w][s];
    }
    mx = fmaxf(mx, z[j]);
  }
  float sum = 1.f;
  if (p.act == kActSoftmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    sum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = lane + 64 * j;
      if (s < m) {
        const float ez = expf(z[j] - mx);
        sp[wave][s] = ez;
        sum += ez;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = lane + 64 * j;
      if (s < m) sp[wave][s] = gsa_read(z[j], p.act);
    }
  }
  // the wave's own copy of p is read by other lanes of the same wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // o = (sum_s e_s hv[s, :]) / sum_s e_s over the wave's columns (sum = 1 for the element-wise
  // read-outs, whose weights are not normalised)
  f32x4 oacc = zero4();
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int s = rv + RVW * u;
    if (s < m) {
      const float ps = sp[wave][s];
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[e] += ps * hv[u][e];
    }
  }
  for (int base = RVW * R; base < m; base += RVW * R) {
#pragma unroll
    for (int u = 0; u < R; ++u)
      hv[u] = *reinterpret_cast<const f32x4*>(HV + (size_t)min(base + rv + RVW * u, m - 1) * Dv);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int s = base + rv + RVW * u;
      if (s < m) {
        const float a = sa[s], w = sw[s], ps = sp[wave][s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[u][e] = a * hv[u][e] + w * vv[e];
          oacc[e] += ps * hv[u][e];
        }
        if (vact) *reinterpret_cast<f32x4*>(HV + (size_t)s * Dv) = hv[u];
      }
    }
  }
  for (int off = CGWP; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) oacc[e] += __shfl_xor(oacc[e], off, 64);
  }
  if (lane < CGWP && vact) {
    const float inv = 1.f / sum;
    typename Vec4<T>::type ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = from_f32<T>(oacc[e] * inv);
    *reinterpret_cast<typename Vec4<T>::type*>(reinterpret_cast<T*>(p.o) + (size_t)bh * Dv + 4 * cg) = ov;
  }
}

template <typename T>
hipError_t launch_gsa_decode(const GsaDecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((gsa_decode_kernel<T>), dim3(p.BH), dim3(kGsaDecThreads), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_gsa_decode<bf16>(const GsaDecodeParams&, hipStream_t);
template hipError_t launch_gsa_decode<float>(const GsaDecodeParams&, hipStream_t);

}  // namespace gla
