// gla_fwd.hip -- chunkwise GLA forward on gfx950.
//
// Two launches per call:
//   1. gla_prep_kernel  (grid N x BH): per chunk, the decayed operands Qs, KdT, Gamma and the
//      masked intra-chunk scores A (prep.hpp).  Fully parallel over chunks.
//   2. gla_fwd_walk     (grid ceil(Dv/64) * BH): one workgroup per (batch*head, 64 value
//      columns) walks the chunks in order with its Dk x 64 slice of the state held in fp32
//      matrix-core accumulators; per chunk it forms
//          O_n     = Qs_n H_n + A_n V_n                       (chunk outputs)
//          H_{n+1} = Diag(2^{Gamma_n}) H_n + KdT_n V_n          (state passing)
//      and writes only O (and the final state).  The state never leaves registers, which is
//      the on-chip reuse the GLA visual companion argues for ("Hardware thesis": fewer HBM
//      writes through chunking).
// Each wave owns 16 of the 64 columns, so the state slice it needs for O_n is exactly the
// slice it updates; the accumulator layout feeds back as the matrix-core operand of Qs H
// through the split k-set (common.hpp), with no LDS round trip for H.
#include "prep.hpp"

namespace gla {

template <typename T, int DKP, int CP>
__global__ __launch_bounds__(256) void gla_fwd_walk(FwdParams p, int ntile) {
  constexpr int PV = 16 / (int)sizeof(T);
  constexpr int LDV = kDvTile + PV;
  constexpr int NBR = CP / 16, NKB = DKP / 32, NCB = CP / 32, NIB = DKP / 16;
  constexpr int V = V16<T>::N;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) T sV[CP * LDV];
  __shared__ float sG[DKP];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = lin % ntile, bh = lin / ntile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int Dv = p.Dv, L = p.L, C = p.C, N = p.N;
  const int j = tile * kDvTile + 16 * wave + col;   // this lane's value column
  const bool jv = j < Dv;

  f32x4 H[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * ib + 4 * grp + e;
      H[ib][e] = (p.h0 && jv && i < p.Dk) ? p.h0[((size_t)bh * p.Dk + i) * Dv + j] : 0.f;
    }
  }
  const T* vg = reinterpret_cast<const T*>(p.v) + (size_t)bh * L * Dv;
  T* og = reinterpret_cast<T*>(p.o) + (size_t)bh * L * Dv;

  for (int n = 0; n < N; ++n) {
    const int row0 = n * C;
    const int len = min(C, L - row0);
    const size_t chunk = (size_t)bh * N + n;
    // stage the V tile [CP][64] (zero outside the chunk and past Dv)
    constexpr int PER_ROW = kDvTile / V;
    for (int idx = tid; idx < CP * PER_ROW; idx += 256) {
      const int r = idx / PER_ROW, cv = (idx - r * PER_ROW) * V;
      const int jj = tile * kDvTile + cv;
      VT val;
      if (r < len && jj < Dv) {
        val = *reinterpret_cast<const VT*>(vg + (size_t)(row0 + r) * Dv + jj);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) val[e] = from_f32<T>(0.f);
      }
      *reinterpret_cast<VT*>(sV + r * LDV + cv) = val;
    }
    if (tid < DKP) sG[tid] = p.ops.Gam[chunk * DKP + tid];
    __syncthreads();

    Frag<T> Yv[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) Yv[cb] = ld8_col(sV + (32 * cb + 8 * grp) * LDV + 16 * wave + col, LDV);

    // O = Qs H + A V
    f32x4 O[NBR];
#pragma unroll
    for (int rb = 0; rb < NBR; ++rb) O[rb] = zero4();
    const T* Qc = reinterpret_cast<const T*>(p.ops.Qs) + chunk * CP * DKP;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Frag<T> Yh = frag_from_acc<T>(H[2 * kb], H[2 * kb + 1]);
#pragma unroll
      for (int rb = 0; rb < NBR; ++rb)
        mma(O[rb], ld8_split(Qc + (16 * rb + col) * DKP + 32 * kb + 4 * grp), Yh);
    }
    const T* Ac = reinterpret_cast<const T*>(p.ops.A) + chunk * CP * CP;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int rb = 0; rb < NBR; ++rb) mma(O[rb], ld8(Ac + (16 * rb + col) * CP + 32 * cb + 8 * grp), Yv[cb]);
    }
    if (jv) {
#pragma unroll
      for (int rb = 0; rb < NBR; ++rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * grp + e;
          if (r < len) og[(size_t)(row0 + r) * Dv + j] = from_f32<T>(O[rb][e]);
        }
      }
    }

    // H <- Diag(2^Gamma) H + KdT V
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) H[ib][e] *= fast_exp2(sG[16 * ib + 4 * grp + e]);
    }
    const T* Kc = reinterpret_cast<const T*>(p.ops.KdT) + chunk * DKP * CP;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) mma(H[ib], ld8(Kc + (16 * ib + col) * CP + 32 * cb + 8 * grp), Yv[cb]);
    }
    __syncthreads();
  }
  if (p.ht && jv) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * ib + 4 * grp + e;
        if (i < p.Dk) p.ht[((size_t)bh * p.Dk + i) * Dv + j] = H[ib][e];
      }
    }
  }
}

template <typename T, int DKP, int CP>
hipError_t launch_gla_fwd(const FwdParams& p, hipStream_t s) {
  PrepParams pp{p.q, p.k, p.g, p.ops, p.L, p.Dk, p.C, p.N};
  hipError_t e = launch_prep<T, DKP, CP, false>(pp, p.BH, s);
  if (e != hipSuccess) return e;
  const int ntile = (p.Dv + kDvTile - 1) / kDvTile;
  hipLaunchKernelGGL((gla_fwd_walk<T, DKP, CP>), dim3(ntile * p.BH), dim3(256), 0, s, p, ntile);
  return hipGetLastError();
}

size_t prep_lds_bytes(int esize, int DKP, int CP) {
  size_t b = 0;
#define GLA_PREP_CASE(TT, D, C_)                                              \
  if (esize == (int)sizeof(TT) && DKP == D && CP == C_) b = PrepCfg<TT, D, C_>::BYTES;
#define GLA_PREP_ALL(TT)                                                       \
  GLA_PREP_CASE(TT, 32, 32) GLA_PREP_CASE(TT, 32, 64) GLA_PREP_CASE(TT, 32, 128) \
  GLA_PREP_CASE(TT, 64, 32) GLA_PREP_CASE(TT, 64, 64) GLA_PREP_CASE(TT, 64, 128) \
  GLA_PREP_CASE(TT, 128, 32) GLA_PREP_CASE(TT, 128, 64) GLA_PREP_CASE(TT, 128, 128) \
  GLA_PREP_CASE(TT, 256, 32) GLA_PREP_CASE(TT, 256, 64) GLA_PREP_CASE(TT, 256, 128)
  GLA_PREP_ALL(bf16)
  GLA_PREP_ALL(float)
#undef GLA_PREP_ALL
#undef GLA_PREP_CASE
  return b <= 160 * 1024 ? b : 0;
}

#define GLA_FWD_INST(TT, D, C_) template hipError_t launch_gla_fwd<TT, D, C_>(const FwdParams&, hipStream_t);
#define GLA_FWD_INST_T(TT)                                                     \
  GLA_FWD_INST(TT, 32, 32) GLA_FWD_INST(TT, 32, 64) GLA_FWD_INST(TT, 32, 128)  \
  GLA_FWD_INST(TT, 64, 32) GLA_FWD_INST(TT, 64, 64) GLA_FWD_INST(TT, 64, 128)  \
  GLA_FWD_INST(TT, 128, 32) GLA_FWD_INST(TT, 128, 64) GLA_FWD_INST(TT, 128, 128) \
  GLA_FWD_INST(TT, 256, 32) GLA_FWD_INST(TT, 256, 64)
GLA_FWD_INST_T(bf16)
GLA_FWD_INST_T(float)

}  // namespace gla
