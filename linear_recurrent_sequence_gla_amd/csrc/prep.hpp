// prep.hpp -- chunk preparation kernel shared by the GLA forward and backward.
//
// For one (batch*head, chunk) it forms, from q, k and the log gates g:
//   b      chunk-local inclusive prefix sum of g, in log2 units (b = log2(e) * cumsum g)
//   Gamma  b at the chunk's last row (the chunk's total log2-decay per key channel)
//   Qs     = q * 2^{b}                 (the query seen from the chunk start)
//   KdT    = (k * 2^{Gamma - b})^T     (the key decayed to the chunk end; transposed)
//   A[r,c] = sum_i q_r[i] k_c[i] 2^{b_r[i] - b_c[i]} for c <= r, else 0
// which are the inputs of the state walk (Gamma, KdT), the chunk outputs (Qs, A) and, for
// the backward, the reverse state walk (QsT).  The decomposition into chunks with a
// sequential state pass between them and a parallel causal block inside each chunk follows
// the chunkwise training form (MS-GLA summary, section 2.1; GLA visual companion, "Why
// chunking and SRAM locality matter").
//
// Numerics of A (intra-chunk gated scores).  The exponent b_r - b_c must never be formed as
// 2^{b_r} * 2^{-b_c} when that could overflow or flush.  Two paths:
//   fast path  if every |b| in the chunk is <= kSpanLimit (2^32 either way, far inside
//              bf16/fp32 range): A = mask((q*2^b) (k*2^-b)^T) as one dense MFMA product.
//   safe path  otherwise, secondary sub-chunking into 16-row sub-chunks: an off-diagonal
//              sub-block (x > y) uses the reference row eps = b at the last row of
//              sub-chunk y, A_xy = (q_x * 2^{b_x - eps}) (k_y * 2^{eps - b_y})^T, where both
//              exponents are <= 0 when g <= 0, on MFMA; diagonal sub-blocks are formed
//              element by element in fp32 with exp2(b_r - b_c).
// The key width is processed in slices of 32 channels on the safe path to bound LDS.
//
// Precision of A.  A[r,c] is a dot product over Dk whose terms can cancel heavily (q.k of
// two random vectors); rounding the decayed operands to bf16 would then give an error of
// 2^-9 * sum|terms| instead of 2^-9 * |sum|.  For bf16, each decayed operand X is therefore
// carried as X = hi + lo (hi = bf16(X), lo = bf16(X - hi)) and the product uses
// hi.hi^T + hi.lo^T + lo.hi^T (three MFMAs), good to about 2^-17 per term.  The score
// product is a small share of the chunk's matrix work, so this costs little.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace gla {

constexpr float kSpanLimit = 32.0f;

struct PrepParams {
  const void *q, *k, *g;
  ChunkOps ops;
  int L, Dk, C, N;
};

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

template <typename T, int DKP, int CP>
struct PrepCfg {
  static constexpr int TPC = 256 / DKP;          // threads per key channel
  static constexpr int RPT = CP / TPC;           // chunk rows per thread
  static constexpr int PK = 16 / (int)sizeof(T); // 16-byte row padding, in elements
  static constexpr int LDQ = DKP + PK;           // row stride of the [CP][DKP] tiles
  static constexpr int LDC = CP + PK;            // row stride of the [DKP][CP] tile
  static constexpr int LDP = 32 + PK;            // row stride of the safe-path slice tiles
  static constexpr int NB = CP / 16;             // 16-row sub-chunks per chunk
  static constexpr int NP = NB * (NB - 1) / 2;   // off-diagonal sub-block pairs
  static constexpr int PPW = (NP + 3) / 4;       // pairs per wave
  // bf16 operands of the score product are split hi + lo ("Precision of A"); fp32 is not split
  static constexpr bool SPLIT = sizeof(T) == 2;
  static constexpr size_t TILE = (size_t)CP * LDQ * sizeof(T);
  static constexpr size_t R1 = TILE;
  static constexpr size_t SAFE = (size_t)3 * CP * 33 * 4 + (size_t)(SPLIT ? 2 : 1) * (CP + 16) * LDP * sizeof(T);
  static constexpr size_t R2 = cmax(cmax((SPLIT ? 3 : 1) * TILE, (size_t)DKP * LDC * sizeof(T)), SAFE);
  static constexpr size_t MISC = (size_t)(TPC * DKP + DKP + 8) * 4;
  static constexpr size_t BYTES = R1 + R2 + MISC;
};

// Copy a [rows][cols] tile (LDS row stride lds) to dense global memory, 16 bytes per access.
template <typename T>
__device__ __forceinline__ void tile_out(T* __restrict__ dst, const T* src, int rows, int cols, int lds) {
  constexpr int V = V16<T>::N;
  typedef typename V16<T>::type VT;
  const int per_row = cols / V;
  for (int idx = threadIdx.x; idx < rows * per_row; idx += blockDim.x) {
    const int r = idx / per_row, c = (idx - r * per_row) * V;
    *reinterpret_cast<VT*>(dst + (size_t)r * cols + c) = *reinterpret_cast<const VT*>(src + r * lds + c);
  }
}
// Copy the transpose of a [rows][cols] LDS tile to dense global [cols][rows].
template <typename T>
__device__ __forceinline__ void tile_out_t(T* __restrict__ dst, const T* src, int rows, int cols, int lds) {
  constexpr int V = V16<T>::N;
  typedef typename V16<T>::type VT;
  const int per = rows / V;
  for (int idx = threadIdx.x; idx < cols * per; idx += blockDim.x) {
    const int c = idx / per, r = (idx - c * per) * V;
    VT vec;
#pragma unroll
    for (int e = 0; e < V; ++e) vec[e] = src[(r + e) * lds + c];
    *reinterpret_cast<VT*>(dst + (size_t)c * rows + r) = vec;
  }
}

__device__ __forceinline__ void pair_decode(int p, int& x, int& y) {
  x = 1;
  while ((x * (x + 1)) / 2 <= p) ++x;
  y = p - (x * (x - 1)) / 2;
}

template <typename T, int DKP, int CP, bool WANT_QST>
__global__ __launch_bounds__(256) void gla_prep_kernel(PrepParams p) {
  using Cfg = PrepCfg<T, DKP, CP>;
  constexpr int TPC = Cfg::TPC, RPT = Cfg::RPT, LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDP = Cfg::LDP;
  constexpr int NB = Cfg::NB, NP = Cfg::NP, PPW = Cfg::PPW;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::BYTES];
  T* sQ = reinterpret_cast<T*>(smem);
  char* r2 = smem + Cfg::R1;
  float* segtot = reinterpret_cast<float*>(r2 + Cfg::R2);
  float* sGam = segtot + TPC * DKP;
  float* red = sGam + DKP;

  const int n = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int row0 = n * p.C;
  const int len = min(p.C, p.L - row0);
  const int Dk = p.Dk;
  const int ch = tid % DKP, seg = tid / DKP, r0 = seg * RPT;
  const bool chv = ch < Dk;
  const size_t base = ((size_t)bh * p.L + row0) * Dk;
  const T* qg = reinterpret_cast<const T*>(p.q) + base;
  const T* kg = reinterpret_cast<const T*>(p.k) + base;
  const T* gg = reinterpret_cast<const T*>(p.g) + base;
  const size_t chunk = (size_t)bh * p.N + n;

  // ---- chunk-local prefix sum of the gates (log2 units), segment-wise then combined
  float b[RPT];
  float run = 0.f;
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = r0 + u;
    const float gv = (chv && r < len) ? to_f32(gg[(size_t)r * Dk + ch]) * kLog2e : 0.f;
    run += gv;
    b[u] = run;
  }
  segtot[seg * DKP + ch] = run;
  __syncthreads();
  float pre = 0.f;
  for (int s = 0; s < seg; ++s) pre += segtot[s * DKP + ch];
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    b[u] += pre;
    mx = fmaxf(mx, fabsf(b[u]));
  }
  if (seg == TPC - 1) sGam[ch] = b[RPT - 1];
  const bool fast = block_max256(mx, red) <= kSpanLimit;   // also publishes sGam

  // ---- Qs = q 2^b (and Ks = k 2^-b on the fast path), with bf16 lo parts
  T* sK = reinterpret_cast<T*>(r2);
  T* sQl = sK + CP * LDQ;
  T* sKl = sQl + CP * LDQ;
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = r0 + u;
    const bool rv = chv && r < len;
    const float qv = rv ? to_f32(qg[(size_t)r * Dk + ch]) : 0.f;
    const float qs = qv * fast_exp2(b[u]);
    const T qh = from_f32<T>(qs);
    sQ[r * LDQ + ch] = qh;
    if (fast) {
      const float kv = rv ? to_f32(kg[(size_t)r * Dk + ch]) : 0.f;
      const float ks = kv * fast_exp2(-b[u]);
      const T kh = from_f32<T>(ks);
      sK[r * LDQ + ch] = kh;
      if constexpr (Cfg::SPLIT) {
        sQl[r * LDQ + ch] = from_f32<T>(qs - to_f32(qh));
        sKl[r * LDQ + ch] = from_f32<T>(ks - to_f32(kh));
      }
    }
  }
  __syncthreads();
  tile_out<T>(reinterpret_cast<T*>(p.ops.Qs) + chunk * CP * DKP, sQ, CP, DKP, LDQ);
  if constexpr (WANT_QST) tile_out_t<T>(reinterpret_cast<T*>(p.ops.QsT) + chunk * CP * DKP, sQ, CP, DKP, LDQ);

  // ---- intra-chunk scores A
  T* Ag = reinterpret_cast<T*>(p.ops.A) + chunk * CP * CP;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  if (fast) {
    for (int blk = wave; blk < NB * NB; blk += 4) {
      const int rb = blk / NB, cb = blk % NB;
      f32x4 acc = zero4();
      if (cb <= rb) {
#pragma unroll
        for (int kb = 0; kb < DKP / 32; ++kb) {
          const int oq = (16 * rb + col) * LDQ + 32 * kb + 8 * grp, ok = (16 * cb + col) * LDQ + 32 * kb + 8 * grp;
          const Frag<T> qh = ld8(sQ + oq), kh = ld8(sK + ok);
          mma(acc, qh, kh);
          if constexpr (Cfg::SPLIT) {
            mma(acc, qh, ld8(sKl + ok));
            mma(acc, ld8(sQl + oq), kh);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
        Ag[r * CP + c] = from_f32<T>(c <= r ? acc[e] : 0.f);
      }
    }
  } else {
    float* sqf = reinterpret_cast<float*>(r2);
    float* skf = sqf + CP * 33;
    float* sbs = skf + CP * 33;
    T* sQp = reinterpret_cast<T*>(sbs + CP * 33);
    T* sKp = sQp + CP * LDP;
    T* sQpl = sKp + 16 * LDP;      // lo parts (bf16 only)
    T* sKpl = sQpl + CP * LDP;
    f32x4 acc_off[PPW > 0 ? PPW : 1];
#pragma unroll
    for (int s = 0; s < (PPW > 0 ? PPW : 1); ++s) acc_off[s] = zero4();
    float acc_d[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) acc_d[x] = 0.f;
    const int rr = tid >> 4, cc = tid & 15;
    for (int sl = 0; sl < DKP / 32; ++sl) {
      __syncthreads();
      if (ch >= 32 * sl && ch < 32 * sl + 32) {
#pragma unroll
        for (int u = 0; u < RPT; ++u) sbs[(r0 + u) * 33 + ch - 32 * sl] = b[u];
      }
      for (int e = tid; e < CP * 32; e += 256) {
        const int r = e >> 5, ii = e & 31, c2 = 32 * sl + ii;
        const bool v = c2 < Dk && r < len;
        sqf[r * 33 + ii] = v ? to_f32(qg[(size_t)r * Dk + c2]) : 0.f;
        skf[r * 33 + ii] = v ? to_f32(kg[(size_t)r * Dk + c2]) : 0.f;
      }
      __syncthreads();
      // diagonal sub-blocks, element by element: exponent b_r - b_c <= 0 for c <= r
      if (cc <= rr) {
#pragma unroll
        for (int x = 0; x < NB; ++x) {
          const int r = 16 * x + rr, c = 16 * x + cc;
          float sum = 0.f;
          for (int ii = 0; ii < 32; ++ii)
            sum += sqf[r * 33 + ii] * skf[c * 33 + ii] * fast_exp2(sbs[r * 33 + ii] - sbs[c * 33 + ii]);
          acc_d[x] += sum;
        }
      }
      // off-diagonal sub-blocks against reference row eps_y = b[16y + 15]
      for (int y = 0; y < NB - 1; ++y) {
        __syncthreads();
        for (int e = tid; e < CP * 32; e += 256) {
          const int r = e >> 5, ii = e & 31;
          const float eps = sbs[(16 * y + 15) * 33 + ii];
          if (r >= 16 * (y + 1)) {
            const float xq = sqf[r * 33 + ii] * fast_exp2(sbs[r * 33 + ii] - eps);
            const T h = from_f32<T>(xq);
            sQp[r * LDP + ii] = h;
            if constexpr (Cfg::SPLIT) sQpl[r * LDP + ii] = from_f32<T>(xq - to_f32(h));
          }
          if (r < 16) {
            const int rk = 16 * y + r;
            const float xk = skf[rk * 33 + ii] * fast_exp2(eps - sbs[rk * 33 + ii]);
            const T h = from_f32<T>(xk);
            sKp[r * LDP + ii] = h;
            if constexpr (Cfg::SPLIT) sKpl[r * LDP + ii] = from_f32<T>(xk - to_f32(h));
          }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < PPW; ++s) {
          const int pidx = wave + 4 * s;
          if (pidx < NP) {
            int x, yy;
            pair_decode(pidx, x, yy);
            if (yy == y) {
              const int oq = (16 * x + col) * LDP + 8 * grp, ok = col * LDP + 8 * grp;
              const Frag<T> qh = ld8(sQp + oq), kh = ld8(sKp + ok);
              mma(acc_off[s], qh, kh);
              if constexpr (Cfg::SPLIT) {
                mma(acc_off[s], qh, ld8(sKpl + ok));
                mma(acc_off[s], ld8(sQpl + oq), kh);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < PPW; ++s) {
      const int pidx = wave + 4 * s;
      if (pidx < NP) {
        int x, y;
        pair_decode(pidx, x, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) Ag[(16 * x + 4 * grp + e) * CP + 16 * y + col] = from_f32<T>(acc_off[s][e]);
      }
    }
    for (int blk = wave; blk < NB * NB; blk += 4) {
      const int rb = blk / NB, cb = blk % NB;
      if (cb > rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Ag[(16 * rb + 4 * grp + e) * CP + 16 * cb + col] = from_f32<T>(0.f);
      }
    }
#pragma unroll
    for (int x = 0; x < NB; ++x) Ag[(16 * x + rr) * CP + 16 * x + cc] = from_f32<T>(cc <= rr ? acc_d[x] : 0.f);
  }
  __syncthreads();

  // ---- KdT = (k 2^{Gamma - b})^T
  T* sKdT = reinterpret_cast<T*>(r2);
  const float gam = sGam[ch];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = r0 + u;
    const float kv = (chv && r < len) ? to_f32(kg[(size_t)r * Dk + ch]) : 0.f;
    sKdT[ch * LDC + r] = from_f32<T>(kv * fast_exp2(gam - b[u]));
  }
  __syncthreads();
  tile_out<T>(reinterpret_cast<T*>(p.ops.KdT) + chunk * DKP * CP, sKdT, DKP, CP, LDC);
  if (tid < DKP) p.ops.Gam[chunk * DKP + tid] = sGam[tid];
}

template <typename T, int DKP, int CP, bool WANT_QST>
hipError_t launch_prep(const PrepParams& p, int BH, hipStream_t s) {
  hipLaunchKernelGGL((gla_prep_kernel<T, DKP, CP, WANT_QST>), dim3(p.N, BH), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace gla
