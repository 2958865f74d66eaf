// gsa_decode.hip -- one recurrent inference step of gated slot attention (GSA).
//
// GSA's bounded slot memories give recurrent inference a fixed-size state per head (GSA
// abstract: efficient recurrent inference; research-map summary, "Approach").  Per
// (batch, head), with alpha = exp(g) and w = -expm1(g) = 1 - alpha (one value per slot):
//   hk[:, s] <- alpha_s hk[:, s] + w_s k       (slot keys, stored transposed: [Dk][m])
//   hv[s, :] <- alpha_s hv[s, :] + w_s v       (slot values: [m][Dv])
//   z = q hk,  p = softmax(z) over the m slots,  o = p hv
// Both fp32 memories are read and written once per step: an HBM stream at about 0.5 flop per
// byte, like the GLA decode step, with nothing to contract on matrix cores.  The softmax
// couples every slot, so one workgroup holds one (batch, head): 256 threads tile hk as
// (row group, 4 slots) and hv as (row group, 4 columns), with 16-byte accesses.  The first
// rows of both memories are requested before anything else; hv is updated and written back
// before the softmax, since its update does not need p; z and o are reduced over the row
// groups in LDS.  The softmax subtracts the maximum and normalises o once at the end.
#include "common.hpp"
#include "kernels.hpp"

namespace gla {

constexpr int kGsaDecThreads = 256;
constexpr int kGsaDecRows = 8;                 // rows per thread per pass, for each memory

template <typename T>
__global__ __launch_bounds__(kGsaDecThreads) void gsa_decode_kernel(GsaDecodeParams p) {
  constexpr int NT = kGsaDecThreads, R = kGsaDecRows, NW = NT / 64;
  __shared__ float sq[256], sk[256], sa[256], sw[256], sp[256];
  __shared__ float sred[4 * NT];               // partial sums of z or o: [row group][column]
  __shared__ float swave[2 * NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, bh = blockIdx.x;
  const int Dk = p.Dk, Dv = p.Dv, m = p.m;
  // hk: NSG groups of 4 slots x NRK row groups; lanes past NSG * NRK load but never store
  const int NSG = m >> 2, NRK = NT / NSG;
  const int sg = tid % NSG, rk = min(tid / NSG, NRK - 1);
  const bool kact = tid < NSG * NRK;
  // hv: NCG groups of 4 columns x NRV row groups
  const int NCG = Dv >> 2, NRV = NT / NCG;
  const int cg = tid % NCG, rv = min(tid / NCG, NRV - 1);
  const bool vact = tid < NCG * NRV;

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
  for (int u = 0; u < R; ++u) hv[u] = *reinterpret_cast<const f32x4*>(HV + (size_t)min(rv + NRV * u, m - 1) * Dv);
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
    const int s = rv + NRV * u;
    if (s < m) {
      const float a = sa[s], w = sw[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[u][e] = a * hv[u][e] + w * vv[e];
      if (vact) *reinterpret_cast<f32x4*>(HV + (size_t)s * Dv) = hv[u];
    }
  }
  if (kact) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sred[rk * m + 4 * sg + e] = zacc[e];
  }
  __syncthreads();

  // softmax over the m slots: thread s < m owns z_s
  float z = -INFINITY;
  if (tid < m) {
    z = 0.f;
    for (int r = 0; r < NRK; ++r) z += sred[r * m + tid];
  }
  float mx = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) swave[wave] = mx;
  __syncthreads();
  mx = swave[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, swave[w]);
  const float ez = tid < m ? expf(z - mx) : 0.f;
  if (tid < m) sp[tid] = ez;
  float sum = ez;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane == 0) swave[NW + wave] = sum;
  __syncthreads();
  sum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) sum += swave[NW + w];

  // o = (sum_s e_s hv[s, :]) / sum_s e_s
  f32x4 oacc = zero4();
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int s = rv + NRV * u;
    if (s < m) {
      const float ps = sp[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[e] += ps * hv[u][e];
    }
  }
  for (int base = NRV * R; base < m; base += NRV * R) {
#pragma unroll
    for (int u = 0; u < R; ++u)
      hv[u] = *reinterpret_cast<const f32x4*>(HV + (size_t)min(base + rv + NRV * u, m - 1) * Dv);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int s = base + rv + NRV * u;
      if (s < m) {
        const float a = sa[s], w = sw[s], ps = sp[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[u][e] = a * hv[u][e] + w * vv[e];
          oacc[e] += ps * hv[u][e];
        }
        if (vact) *reinterpret_cast<f32x4*>(HV + (size_t)s * Dv) = hv[u];
      }
    }
  }
  // sred's z partials were all read before the last barrier
  if (vact) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sred[rv * Dv + 4 * cg + e] = oacc[e];
  }
  __syncthreads();
  if (tid < Dv) {
    float o = 0.f;
    for (int r = 0; r < NRV; ++r) o += sred[r * Dv + tid];
    reinterpret_cast<T*>(p.o)[(size_t)bh * Dv + tid] = from_f32<T>(o / sum);
  }
  for (int j = tid + NT; j < Dv; j += NT) {
    float o = 0.f;
    for (int r = 0; r < NRV; ++r) o += sred[r * Dv + j];
    reinterpret_cast<T*>(p.o)[(size_t)bh * Dv + j] = from_f32<T>(o / sum);
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
