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

// LDS layout and prefetch shape of the walk.  One stage holds one chunk's operands; the
// stages (and the output staging tile) are double-buffered when two fit a CU's LDS, so a step
// needs one barrier, else single-buffered with two barriers per step.
template <typename T, int DKP, int CP>
struct WalkCfg {
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int LDQ = DKP + V, LDA = CP + V, LDV = kDvTile + V;
  static constexpr size_t QT = (size_t)CP * LDQ * sizeof(T);
  static constexpr size_t AT = (size_t)CP * LDA * sizeof(T);
  static constexpr size_t KT = (size_t)DKP * LDA * sizeof(T);
  static constexpr size_t VT = (size_t)CP * LDV * sizeof(T);
  static constexpr size_t GT = (size_t)DKP * 4;
  static constexpr size_t STAGE = QT + AT + KT + VT + GT;
  static constexpr size_t OT = (size_t)CP * LDV * sizeof(T);
  static constexpr int NB = 2 * (STAGE + OT) <= kMaxLds ? 2 : 1;
  // staging tile for the chunk-start states a saving forward writes (coalesced stores), when
  // it fits beside the rest; otherwise the states leave straight from the accumulators
  static constexpr size_t HT = (size_t)DKP * LDV * sizeof(T);
  static constexpr bool HS_LDS = NB * (STAGE + OT) + HT <= kMaxLds;
  static constexpr size_t BYTES = NB * (STAGE + OT) + (HS_LDS ? HT : 0);
  // 16-byte vectors per chunk and per thread
  static constexpr int NQ = CP * DKP / V, NA = CP * CP / V, NK = DKP * CP / V, NV = CP * kDvTile / V;
  static constexpr int PQ = (NQ + 255) / 256, PA = (NA + 255) / 256, PKd = (NK + 255) / 256, PV = (NV + 255) / 256;
  static constexpr int R = 2;   // chunks whose operands are in flight ahead of the one in use
};

// One chunk's walk operands in flight between global memory and LDS.  Loads are issued
// unconditionally from clamped, in-bounds addresses, with the validity of each value vector
// kept beside it and applied when the registers are written to LDS; no branch or register
// rewrite touches a load in flight, so several chunks' loads can stay outstanding.
template <typename T, int DKP, int CP>
struct WalkStage {
  using W = WalkCfg<T, DKP, CP>;
  typedef typename V16<T>::type VT;
  VT q[W::PQ], a[W::PA], kd[W::PKd], v[W::PV];
  bool vok[W::PV];
  f32x4 gam;

  __device__ __forceinline__ void load(const FwdParams& p, int bh, int n, int tile) {
    const int tid = threadIdx.x;
    const size_t chunk = (size_t)bh * p.N + n;
    const T* Qc = reinterpret_cast<const T*>(p.ops.Qs) + chunk * CP * DKP;
    const T* Ac = reinterpret_cast<const T*>(p.ops.A) + chunk * CP * CP;
    const T* Kc = reinterpret_cast<const T*>(p.ops.KdT) + chunk * DKP * CP;
#pragma unroll
    for (int m = 0; m < W::PQ; ++m) q[m] = *reinterpret_cast<const VT*>(Qc + (size_t)min(tid + 256 * m, W::NQ - 1) * W::V);
#pragma unroll
    for (int m = 0; m < W::PA; ++m) a[m] = *reinterpret_cast<const VT*>(Ac + (size_t)min(tid + 256 * m, W::NA - 1) * W::V);
#pragma unroll
    for (int m = 0; m < W::PKd; ++m)
      kd[m] = *reinterpret_cast<const VT*>(Kc + (size_t)min(tid + 256 * m, W::NK - 1) * W::V);
    const int row0 = n * p.C, len = min(p.C, p.L - row0);
    const T* vg = reinterpret_cast<const T*>(p.v) + ((size_t)bh * p.L + row0) * p.Dv;
    constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
    for (int m = 0; m < W::PV; ++m) {
      const int idx = tid + 256 * m;
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * W::V;
      const int j = tile * kDvTile + c;
      vok[m] = idx < W::NV && r < len && j < p.Dv;
      v[m] = *reinterpret_cast<const VT*>(vg + (size_t)min(r, len - 1) * p.Dv + min(j, p.Dv - W::V));
    }
    gam = *reinterpret_cast<const f32x4*>(p.ops.Gam + chunk * DKP + 4 * (tid % (DKP / 4)));
  }

  __device__ __forceinline__ void store(T* sQ, T* sA, T* sK, T* sV, float* sG) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < W::PQ; ++m) {
      const int idx = tid + 256 * m;
      if (idx < W::NQ) {
        const int r = idx / (DKP / W::V), c = (idx - r * (DKP / W::V)) * W::V;
        *reinterpret_cast<VT*>(sQ + r * W::LDQ + c) = q[m];
      }
    }
#pragma unroll
    for (int m = 0; m < W::PA; ++m) {
      const int idx = tid + 256 * m;
      if (idx < W::NA) {
        const int r = idx / (CP / W::V), c = (idx - r * (CP / W::V)) * W::V;
        *reinterpret_cast<VT*>(sA + r * W::LDA + c) = a[m];
      }
    }
#pragma unroll
    for (int m = 0; m < W::PKd; ++m) {
      const int idx = tid + 256 * m;
      if (idx < W::NK) {
        const int r = idx / (CP / W::V), c = (idx - r * (CP / W::V)) * W::V;
        *reinterpret_cast<VT*>(sK + r * W::LDA + c) = kd[m];
      }
    }
    constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
    for (int m = 0; m < W::PV; ++m) {
      const int idx = tid + 256 * m;
      if (idx < W::NV) {
        const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * W::V;
        *reinterpret_cast<VT*>(sV + r * W::LDV + c) = vok[m] ? v[m] : zero_vec<T>();
      }
    }
    if (tid < DKP / 4) *reinterpret_cast<f32x4*>(sG + 4 * tid) = gam;
  }
};

template <typename T, int DKP, int CP>
__global__ __launch_bounds__(256) void gla_fwd_walk(FwdParams p, int ntile) {
  using W = WalkCfg<T, DKP, CP>;
  constexpr int LDQ = W::LDQ, LDA = W::LDA, LDV = W::LDV, R = W::R, NB = W::NB;
  constexpr int NBR = CP / 16, NKB = DKP / 32, NCB = CP / 32, NIB = DKP / 16;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) char smem[W::BYTES];
  auto base = [&](int b) { return smem + (NB == 2 ? b : 0) * (W::STAGE + W::OT); };
  auto sQ = [&](int b) { return reinterpret_cast<T*>(base(b)); };
  auto sA = [&](int b) { return reinterpret_cast<T*>(base(b) + W::QT); };
  auto sK = [&](int b) { return reinterpret_cast<T*>(base(b) + W::QT + W::AT); };
  auto sV = [&](int b) { return reinterpret_cast<T*>(base(b) + W::QT + W::AT + W::KT); };
  auto sG = [&](int b) { return reinterpret_cast<float*>(base(b) + W::QT + W::AT + W::KT + W::VT); };
  auto sO = [&](int b) { return reinterpret_cast<T*>(base(b) + W::STAGE); };
  T* sHs = reinterpret_cast<T*>(smem + NB * (W::STAGE + W::OT));   // HS_LDS only

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
  __builtin_amdgcn_s_waitcnt(0);                   // initial state in before the pipeline starts
  T* og = reinterpret_cast<T*>(p.o) + (size_t)bh * L * Dv;

  WalkStage<T, DKP, CP> st[R];
#pragma unroll
  for (int r = 0; r < R; ++r) st[r].load(p, bh, min(r, N - 1), tile);
  st[0].store(sQ(0), sA(0), sK(0), sV(0), sG(0));
  __syncthreads();

  for (int k0 = 0; k0 < N; k0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = k0 + r;
      if (n < N) {
        const int b = n & 1, row0 = n * C, len = min(C, L - row0);
        st[r].load(p, bh, min(n + R, N - 1), tile);   // st[r] (chunk n) is already in LDS
        if (p.Hs) {   // H_n for a later backward
          const int DvP = ntile * kDvTile;
          T* hs = reinterpret_cast<T*>(p.Hs) + ((size_t)bh * N + n) * DKP * DvP + tile * kDvTile;
          if constexpr (W::HS_LDS) {   // through LDS: one more barrier, 16-byte stores
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
              for (int e = 0; e < 4; ++e) sHs[(16 * ib + 4 * grp + e) * LDV + 16 * wave + col] = from_f32<T>(H[ib][e]);
            }
            __syncthreads();
            constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
            for (int m = 0; m < (DKP * PER_ROW + 255) / 256; ++m) {
              const int idx = tid + 256 * m;
              if (idx < DKP * PER_ROW) {
                const int rr = idx / PER_ROW, c = (idx - rr * PER_ROW) * W::V;
                *reinterpret_cast<VT*>(hs + (size_t)rr * DvP + c) = *reinterpret_cast<const VT*>(sHs + rr * LDV + c);
              }
            }
            // sHs is rewritten only after this step's closing barrier(s)
          } else {
#pragma unroll
            for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                hs[(size_t)(16 * ib + 4 * grp + e) * DvP + 16 * wave + col] = from_f32<T>(H[ib][e]);
            }
          }
        }
        const T* q_ = sQ(b);
        const T* a_ = sA(b);
        const T* k_ = sK(b);
        const T* v_ = sV(b);
        const float* g_ = sG(b);
        T* o_ = sO(b);

        Frag<T> Yv[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Yv[cb] = ld8_colblk(v_ + (32 * cb) * LDV + 16 * wave, LDV);

        // O = Qs H + A V
        f32x4 O[NBR];
#pragma unroll
        for (int rb = 0; rb < NBR; ++rb) O[rb] = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const Frag<T> Yh = frag_from_acc<T>(H[2 * kb], H[2 * kb + 1]);
#pragma unroll
          for (int rb = 0; rb < NBR; ++rb) mma(O[rb], ld8_split(q_ + (16 * rb + col) * LDQ + 32 * kb + 4 * grp), Yh);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
          for (int rb = 0; rb < NBR; ++rb) mma(O[rb], ld8(a_ + (16 * rb + col) * LDA + 32 * cb + 8 * grp), Yv[cb]);
        }
#pragma unroll
        for (int rb = 0; rb < NBR; ++rb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o_[(16 * rb + 4 * grp + e) * LDV + 16 * wave + col] = from_f32<T>(O[rb][e]);
        }

        // H <- Diag(2^Gamma) H + KdT V
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
          for (int e = 0; e < 4; ++e) H[ib][e] *= fast_exp2(g_[16 * ib + 4 * grp + e]);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
          for (int ib = 0; ib < NIB; ++ib) mma(H[ib], ld8(k_ + (16 * ib + col) * LDA + 32 * cb + 8 * grp), Yv[cb]);
        }
        if constexpr (NB == 2) {
          st[(r + 1) % R].store(sQ(b ^ 1), sA(b ^ 1), sK(b ^ 1), sV(b ^ 1), sG(b ^ 1));
          __syncthreads();   // chunk n+1 staged, chunk n's tiles consumed, O complete
        } else {
          __syncthreads();   // chunk n's tiles consumed, O complete
          st[(r + 1) % R].store(sQ(0), sA(0), sK(0), sV(0), sG(0));
        }
        constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
        for (int m = 0; m < (CP * PER_ROW + 255) / 256; ++m) {
          const int idx = tid + 256 * m;
          const int rr = idx / PER_ROW, c = (idx - rr * PER_ROW) * W::V;
          const int jj = tile * kDvTile + c;
          if (idx < CP * PER_ROW && rr < len && jj < Dv)
            *reinterpret_cast<VT*>(og + (size_t)(row0 + rr) * Dv + jj) = *reinterpret_cast<const VT*>(o_ + rr * LDV + c);
        }
        if constexpr (NB == 1) __syncthreads();   // chunk n+1 staged, O copied out
      }
    }
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
  if constexpr (PrepCfg<T, DKP, CP>::BYTES > kMaxLds || WalkCfg<T, DKP, CP>::BYTES > kMaxLds) {
    return hipErrorNotSupported;
  } else {
    PrepParams pp{p.q, p.k, p.g, p.ops, p.L, p.Dk, p.C, p.N};
    record_event(p.events, 0, s);
    hipError_t e = p.ops.QsT ? launch_prep<T, DKP, CP, true>(pp, p.BH, s) : launch_prep<T, DKP, CP, false>(pp, p.BH, s);
    if (e != hipSuccess) return e;
    record_event(p.events, 1, s);
    const int ntile = (p.Dv + kDvTile - 1) / kDvTile;
    hipLaunchKernelGGL((gla_fwd_walk<T, DKP, CP>), dim3(ntile * p.BH), dim3(256), 0, s, p, ntile);
    record_event(p.events, 2, s);
    return hipGetLastError();
  }
}

bool fwd_config_fits(int esize, int DKP, int CP) {
  bool ok = false;
#define GLA_FIT_CASE(TT, D, C_)                                                       \
  if (esize == (int)sizeof(TT) && DKP == D && CP == C_)                               \
    ok = PrepCfg<TT, D, C_>::BYTES <= kMaxLds && WalkCfg<TT, D, C_>::BYTES <= kMaxLds;
#define GLA_FIT_ALL(TT)                                                                \
  GLA_FIT_CASE(TT, 32, 32) GLA_FIT_CASE(TT, 32, 64) GLA_FIT_CASE(TT, 32, 128)           \
  GLA_FIT_CASE(TT, 64, 32) GLA_FIT_CASE(TT, 64, 64) GLA_FIT_CASE(TT, 64, 128)           \
  GLA_FIT_CASE(TT, 128, 32) GLA_FIT_CASE(TT, 128, 64) GLA_FIT_CASE(TT, 128, 128)        \
  GLA_FIT_CASE(TT, 256, 32) GLA_FIT_CASE(TT, 256, 64)
  GLA_FIT_ALL(bf16)
  GLA_FIT_ALL(float)
#undef GLA_FIT_ALL
#undef GLA_FIT_CASE
  return ok;
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
