// walks.hpp -- the two sequential state walks shared by the GLA and GSA backward (and the
// GSA forward).  Both carry one 64-column tile of a row-gated state S [SP rows][64] in fp32
// matrix-core accumulators while stepping over the chunks of one (batch*head):
//
//   walk_store    S_0 = init;  for n = 0..N-1:  store S_n (bf16/T),
//                              S_{n+1} = Diag(2^{Gamma_n}) S_n + M_n X_n ;  fin = S_N
//   walk_reverse  D_N = init;  for n = N-1..0:  store D_{n+1},
//                              D_n = Diag(2^{Gamma_n}) D_{n+1} + M_n X_n ;  fin = D_0
//
// with M_n = mat[n] a per-chunk [SP][CP] matrix (the decayed keys transposed for the forward
// walk, the decayed queries transposed for the reverse walk) and X_n the chunk's rows of a
// token tensor src [L][Ds] (values for the forward walk, output gradients for the reverse).
// GLA: rows = key channels.  GSA: rows = slots for both passes (pass 1 walks the transposed
// slot-key memory, whose values are the keys).  The chunked structure -- sequential
// inter-chunk updates, state written only at chunk boundaries -- is the chunkwise training
// form of the MS-GLA summary (section 2.1).  The next chunk's operands are loaded into
// registers while the current chunk is processed.
#pragma once
#include "prep.hpp"

namespace gla {

struct WalkIO {
  const void* mat;     // [BH][N][SP][CP] per-chunk matrix (T)
  const void* src;     // [BH][L][Ds] token tensor (T)
  const float* gam;    // [BH][N][SP] chunk log2-decay per state row
  void* states;        // [BH][N][SP][DsP] stored states / state gradients (T)
  const float* init;   // fp32 [BH][rows][Ds] (or [BH][Ds][rows] when trans) or nullptr (= 0)
  float* fin;          // fp32, same layout, or nullptr (= not written)
  int rows, Ds, L, C, N, trans;
};

template <typename T, int SP, int CP>
struct WalkIOCfg {
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int LDA = CP + V, LDV = kDvTile + V;
  static constexpr size_t KT = (size_t)SP * LDA * sizeof(T);
  static constexpr size_t VT = (size_t)CP * LDV * sizeof(T);
  static constexpr size_t HT = (size_t)SP * LDV * sizeof(T);
  static constexpr size_t BYTES = KT + VT + HT + (size_t)SP * 4;
  static constexpr int NK = SP * CP / V, NV = CP * kDvTile / V, NH = SP * kDvTile / V;
  static constexpr int PKd = (NK + 255) / 256, PV = (NV + 255) / 256, PH = (NH + 255) / 256;
};

template <typename T, int SP, int CP>
struct WalkIOStage {
  using W = WalkIOCfg<T, SP, CP>;
  typedef typename V16<T>::type VT;
  VT kt[W::PKd], v[W::PV];
  f32x4 gam;

  // mat: [SP][CP] of this chunk; src: [L][Ds] of this (b,h).
  __device__ __forceinline__ void load(const T* mat, const T* src, int row0, int len, int Ds, int tile,
                                       const float* gam_chunk) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < W::PKd; ++m) {
      const int idx = tid + 256 * m;
      if (idx < W::NK) kt[m] = *reinterpret_cast<const VT*>(mat + (size_t)idx * W::V);
    }
    constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
    for (int m = 0; m < W::PV; ++m) {
      const int idx = tid + 256 * m;
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * W::V;
      const int j = tile * kDvTile + c;
      v[m] = (idx < W::NV && r < len && j < Ds) ? *reinterpret_cast<const VT*>(src + (size_t)(row0 + r) * Ds + j)
                                                : zero_vec<T>();
    }
    if (tid < SP / 4) gam = *reinterpret_cast<const f32x4*>(gam_chunk + 4 * tid);
  }

  __device__ __forceinline__ void store(T* sKT, T* sV, float* sG) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < W::PKd; ++m) {
      const int idx = tid + 256 * m;
      if (idx < W::NK) {
        const int r = idx / (CP / W::V), c = (idx - r * (CP / W::V)) * W::V;
        *reinterpret_cast<VT*>(sKT + r * W::LDA + c) = kt[m];
      }
    }
    constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
    for (int m = 0; m < W::PV; ++m) {
      const int idx = tid + 256 * m;
      if (idx < W::NV) {
        const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * W::V;
        *reinterpret_cast<VT*>(sV + r * W::LDV + c) = v[m];
      }
    }
    if (tid < SP / 4) *reinterpret_cast<f32x4*>(sG + 4 * tid) = gam;
  }
};

// Copy an LDS [SP][64] tile to the state workspace (row stride DsP, already offset).
template <typename T, int SP>
__device__ __forceinline__ void state_tile_out(T* dst, const T* src, int lds, int DsP) {
  constexpr int V = V16<T>::N;
  typedef typename V16<T>::type VT;
  constexpr int PER_ROW = kDvTile / V;
  for (int idx = threadIdx.x; idx < SP * PER_ROW; idx += 256) {
    const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
    *reinterpret_cast<VT*>(dst + (size_t)r * DsP + c) = *reinterpret_cast<const VT*>(src + r * lds + c);
  }
}

__device__ __forceinline__ size_t walk_state_index(const WalkIO& w, int bh, int i, int j) {
  return w.trans ? ((size_t)bh * w.Ds + j) * w.rows + i : ((size_t)bh * w.rows + i) * w.Ds + j;
}

// S_{n+1} = Diag(2^Gamma) S_n + M_n X_n on the accumulators (X from LDS, M from LDS).
template <typename T, int SP, int CP>
__device__ __forceinline__ void walk_step(f32x4 (&S)[SP / 16], const T* sKT, const T* sV, const float* sG) {
  using W = WalkIOCfg<T, SP, CP>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  constexpr int NCB = CP / 32, NIB = SP / 16;
  Frag<T> Yv[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) Yv[cb] = ld8_col(sV + (32 * cb + 8 * grp) * W::LDV + 16 * wave + col, W::LDV);
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
    for (int e = 0; e < 4; ++e) S[ib][e] *= fast_exp2(sG[16 * ib + 4 * grp + e]);
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) mma(S[ib], ld8(sKT + (16 * ib + col) * W::LDA + 32 * cb + 8 * grp), Yv[cb]);
  }
}

template <typename T, int SP, int CP>
__global__ __launch_bounds__(256) void walk_store(WalkIO w, int ntile) {
  using W = WalkIOCfg<T, SP, CP>;
  constexpr int LDV = W::LDV, NIB = SP / 16;
  __shared__ __attribute__((aligned(16))) char smem[W::BYTES];
  T* sKT = reinterpret_cast<T*>(smem);
  T* sV = reinterpret_cast<T*>(smem + W::KT);
  T* sHo = reinterpret_cast<T*>(smem + W::KT + W::VT);
  float* sG = reinterpret_cast<float*>(smem + W::KT + W::VT + W::HT);

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = lin % ntile, bh = lin / ntile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int Ds = w.Ds, L = w.L, C = w.C, N = w.N;
  const int DsP = ntile * kDvTile;
  const int j = tile * kDvTile + 16 * wave + col;
  const bool jv = j < Ds;
  const T* src = reinterpret_cast<const T*>(w.src) + (size_t)bh * L * Ds;
  const T* mat = reinterpret_cast<const T*>(w.mat) + (size_t)bh * N * SP * CP;
  const float* gam = w.gam + (size_t)bh * N * SP;
  T* out = reinterpret_cast<T*>(w.states) + (size_t)bh * N * SP * DsP + tile * kDvTile;

  f32x4 S[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * ib + 4 * grp + e;
      S[ib][e] = (w.init && jv && i < w.rows) ? w.init[walk_state_index(w, bh, i, j)] : 0.f;
    }
  }
  WalkIOStage<T, SP, CP> st;
  st.load(mat, src, 0, min(C, L), Ds, tile, gam);
  st.store(sKT, sV, sG);
  __syncthreads();
  for (int n = 0; n < N; ++n) {
    if (n + 1 < N) {
      const int r1 = (n + 1) * C;
      st.load(mat + (size_t)(n + 1) * SP * CP, src, r1, min(C, L - r1), Ds, tile, gam + (size_t)(n + 1) * SP);
    }
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sHo[(16 * ib + 4 * grp + e) * LDV + 16 * wave + col] = from_f32<T>(S[ib][e]);
    }
    walk_step<T, SP, CP>(S, sKT, sV, sG);
    __syncthreads();
    state_tile_out<T, SP>(out + (size_t)n * SP * DsP, sHo, LDV, DsP);
    if (n + 1 < N) st.store(sKT, sV, sG);
    __syncthreads();
  }
  if (w.fin && jv) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * ib + 4 * grp + e;
        if (i < w.rows) w.fin[walk_state_index(w, bh, i, j)] = S[ib][e];
      }
    }
  }
}

template <typename T, int SP, int CP>
__global__ __launch_bounds__(256) void walk_reverse(WalkIO w, int ntile) {
  using W = WalkIOCfg<T, SP, CP>;
  constexpr int LDV = W::LDV, NIB = SP / 16;
  __shared__ __attribute__((aligned(16))) char smem[W::BYTES];
  T* sKT = reinterpret_cast<T*>(smem);
  T* sV = reinterpret_cast<T*>(smem + W::KT);
  T* sHo = reinterpret_cast<T*>(smem + W::KT + W::VT);
  float* sG = reinterpret_cast<float*>(smem + W::KT + W::VT + W::HT);

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = lin % ntile, bh = lin / ntile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int Ds = w.Ds, L = w.L, C = w.C, N = w.N;
  const int DsP = ntile * kDvTile;
  const int j = tile * kDvTile + 16 * wave + col;
  const bool jv = j < Ds;
  const T* src = reinterpret_cast<const T*>(w.src) + (size_t)bh * L * Ds;
  const T* mat = reinterpret_cast<const T*>(w.mat) + (size_t)bh * N * SP * CP;
  const float* gam = w.gam + (size_t)bh * N * SP;
  T* out = reinterpret_cast<T*>(w.states) + (size_t)bh * N * SP * DsP + tile * kDvTile;

  f32x4 D[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * ib + 4 * grp + e;
      D[ib][e] = (w.init && jv && i < w.rows) ? w.init[walk_state_index(w, bh, i, j)] : 0.f;
    }
  }
  WalkIOStage<T, SP, CP> st;
  {
    const int r1 = (N - 1) * C;
    st.load(mat + (size_t)(N - 1) * SP * CP, src, r1, L - r1, Ds, tile, gam + (size_t)(N - 1) * SP);
    st.store(sKT, sV, sG);
  }
  __syncthreads();
  for (int n = N - 1; n >= 0; --n) {
    if (n > 0) {
      const int r1 = (n - 1) * C;
      st.load(mat + (size_t)(n - 1) * SP * CP, src, r1, C, Ds, tile, gam + (size_t)(n - 1) * SP);
    }
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sHo[(16 * ib + 4 * grp + e) * LDV + 16 * wave + col] = from_f32<T>(D[ib][e]);
    }
    walk_step<T, SP, CP>(D, sKT, sV, sG);
    __syncthreads();
    state_tile_out<T, SP>(out + (size_t)n * SP * DsP, sHo, LDV, DsP);
    if (n > 0) st.store(sKT, sV, sG);
    __syncthreads();
  }
  if (w.fin && jv) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * ib + 4 * grp + e;
        if (i < w.rows) w.fin[walk_state_index(w, bh, i, j)] = D[ib][e];
      }
    }
  }
}

template <typename T, int SP, int CP>
hipError_t launch_walk_store(const WalkIO& w, int BH, hipStream_t s) {
  const int ntile = (w.Ds + kDvTile - 1) / kDvTile;
  hipLaunchKernelGGL((walk_store<T, SP, CP>), dim3(ntile * BH), dim3(256), 0, s, w, ntile);
  return hipGetLastError();
}
template <typename T, int SP, int CP>
hipError_t launch_walk_reverse(const WalkIO& w, int BH, hipStream_t s) {
  const int ntile = (w.Ds + kDvTile - 1) / kDvTile;
  hipLaunchKernelGGL((walk_reverse<T, SP, CP>), dim3(ntile * BH), dim3(256), 0, s, w, ntile);
  return hipGetLastError();
}

}  // namespace gla
