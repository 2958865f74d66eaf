// gsa.hip -- gated slot attention (GSA) on gfx950: two GLA passes linked by a softmax (or by
// one of the element-wise read-outs the GSA summary's ablations use in its place).
//
// GSA ("Gated Slot Attention for Efficient Linear-Time Sequence Modeling": abstract and the
// research-map summary, "Approach") keeps m slot memories per head with a data-dependent
// forget gate per slot.  With alpha_t = exp(g_t) (g_t in R^m) and write weights
// w_t = 1 - alpha_t:
//   pass 1 (slot keys, decay on the slot axis)  S1_t = S1_{t-1} Diag(alpha_t) + k_t^T w_t,
//                                               z_t = q_t S1_t
//   p_t = softmax(z_t) over the m slots  (or p_t = f(z_t) slot by slot: Swish, ReLU, ReLU^2, none)
//   pass 2 (slot values, row-gated GLA)          S2_t = Diag(alpha_t) S2_{t-1} + w_t^T v_t,
//                                               o_t = p_t S2_t
// Pass 2 is exactly GLA with queries p, keys w, values v and the same gates, so it runs on the
// GLA kernels (gla_fwd.hip / gla_bwd.hip) with p and w materialised as [B,H,L,m] tensors.  Pass
// 1 runs here.  Its transposed state S1^T [m x Dk] is row-gated (keys w, values k), so it
// rides the generic state walks of walks.hpp; pass 2's state walk has the same decayed keys
// and decays, so the two forward walks run as one launch (launch_gsa_walks).  In chunk form (b = chunk-local log2 prefix sum
// of g, E = 2^b, Ei = 2^-b, Eg = 2^{Gamma-b}, QK = mask(Q K^T) with c <= r):
//   Z = E * (QK (W*Ei) + Q S1_n)                                    (then P = softmax(Z))
//   dQK = mask((dZ*E)(W*Ei)^T),  dq = dQK K + (dZ*E) S1_n^T
//   dk  = dQK^T Q + (W*Eg) dS1_{n+1}^T
//   dW1 = Ei*(QK^T (dZ*E)) + Eg*(K dS1_{n+1})
// with the same gate-span check as GLA: chunks with |b| > 32 form the intra-chunk terms
// exactly, element by element.  Operands whose dot products can cancel (QK, dZ) go through
// hi/lo bf16 splits.  The gate gradient is assembled without exactly-cancelling pairs:
//   dg_t = sum_{r>=t}(dZ_r Znd_r - W_r dW1'_r) + sum_{c<t} W_c B1_c + Z1_n      (pass 1)
//        + [pass-2 gate gradient from the GLA backward]
//        - alpha_t (dW1_t + dW2_t)                                  (w = 1 - alpha)
// where Znd is Z without its diagonal term QK_rr W_r, dW1' the strictly-upper intra part of
// dW1, B1 = Eg*(K dS1_{n+1}) and Z1_n = 2^Gamma colsum(dS1_{n+1} * S1_n).
#include "walks.hpp"

namespace gla {

template <typename T, int MP, int CP>
struct GsaCfg {
  using M = ChunkMap<T, MP, CP>;
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int LDF = MP + 4;            // fp32 [CP][MP] tiles
  static constexpr int LDS = kDvTile + V;       // 64-wide T slices
  static constexpr int LDM = MP + V;            // T [CP][MP] staging
  static constexpr int LDC = CP + V;            // T [MP][CP] tiles
  static constexpr int NRB = CP / 16, NSB = MP / 16;
  static constexpr size_t FT = (size_t)CP * LDF * 4;
  static constexpr size_t ST_C = (size_t)CP * LDS * sizeof(T);
  static constexpr size_t ST_M = (size_t)MP * LDS * sizeof(T);
  // gsa_pass1_bwd: sB (fp32), the split tiles W Ei and dZ E, then {dQK (T) + slices} aliased by
  // {split QK + three fp32 tiles}; the tail holds the scan totals, Gamma, Z1, the block-max
  // scratch and the dQK and QK diagonals.  Split tiles hold hi and lo parts of T (lo only for
  // 16-bit T) with 32-byte row pads, so that transposing reads of them are free of conflicts.
  static constexpr bool SPLIT = sizeof(T) == 2;
  static constexpr int LDH = MP + 2 * V;        // split [CP][MP] tiles
  static constexpr int LDQ2 = CP + 2 * V;       // split [CP][CP] QK and T dQK tiles
  static constexpr size_t HPAIR = (SPLIT ? 2 : 1) * (size_t)CP * LDH * sizeof(T);
  static constexpr size_t QPAIR = (SPLIT ? 2 : 1) * (size_t)CP * LDQ2 * sizeof(T);
  static constexpr size_t B_REGION = cmax(QPAIR + 4 * ST_C + 2 * ST_M, QPAIR + 3 * FT);
  // gsa_p: sB (fp32), the split tile W Ei, then the slices (q, k, S1^T), which the split QK
  // tile and the P staging tile replace once the Dk loop is done.  Under 80 KB for bf16 at
  // m = 64, so that two workgroups share a CU.
  static constexpr size_t P_REGION = cmax(2 * ST_C + ST_M, QPAIR + (size_t)CP * LDM * sizeof(T));
  static constexpr size_t P_BYTES = FT + HPAIR + P_REGION + (size_t)(M::NSEG * MP + MP + 8) * 4;
  static constexpr size_t B_BYTES = FT + 2 * HPAIR + B_REGION + (size_t)(2 * M::NSEG * MP + 2 * MP + 8 + 2 * CP) * 4;
  // the pass-1 backward walks its tiles in a persistent loop, carrying the next tile's gates
  // and dZ (more slots: one tile per workgroup, where the loop's registers would spill)
  static constexpr bool P1_PERSIST = MP <= 64;
};

// ----------------------------------------------------------------------------- prep
// Per chunk: b, Gamma (log2 units), w = -expm1(g) written as a [L][m] tensor (the keys of
// pass 2), and WdT = (w * 2^{Gamma-b})^T, the decayed write weights both state walks consume.
template <typename T, int MP, int CP>
__global__ __launch_bounds__(256) void gsa_prep_kernel(GsaParams p) {
  using M = ChunkMap<T, MP, CP>;
  constexpr int V = M::V, RPS = M::RPS, LDM = MP + V;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) T sWd[CP * LDM];     // row by row; leaves transposed
  __shared__ float segtot[M::NSEG * MP];
  __shared__ float sGam[MP];
  __shared__ float red[8];
  const int n = blockIdx.x, bh = blockIdx.y, m = p.m;
  const int row0 = n * p.C, len = min(p.C, p.L - row0);
  const size_t gbase = ((size_t)bh * p.L + row0) * m;
  const size_t chunk = (size_t)bh * p.N + n;
  const T* gg = reinterpret_cast<const T*>(p.g) + gbase;
  ChunkScan<T, MP, CP, false> cs;
  cs.run(gg, gg, gg, m, m, len, segtot, sGam, red);
  const int c0 = cs.cg * V, r0 = cs.seg * RPS;
  if (cs.active) {
    T* Wg = p.W ? reinterpret_cast<T*>(p.W) + gbase : nullptr;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const int r = r0 + u;
      VT wv, wd;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float w = -expm1f(cs.qv[u][e]);
        wv[e] = from_f32<T>(w);
        wd[e] = from_f32<T>(w * fast_exp2(sGam[c0 + e] - cs.b[u][e]));
      }
      *reinterpret_cast<VT*>(sWd + r * LDM + c0) = wd;
      if (Wg && r < len && c0 < m) *reinterpret_cast<VT*>(Wg + (size_t)r * m + c0) = wv;
    }
  }
  __syncthreads();
  tile_out_t<T, 4>(reinterpret_cast<T*>(p.WdT) + chunk * MP * CP, sWd, CP, MP, LDM);
  if (threadIdx.x < MP) p.Gam[chunk * MP + threadIdx.x] = sGam[threadIdx.x];
}

// A [ROWS][64] column slice of a row-major [*, ld] tensor held in registers by NT threads,
// 16 bytes per vector: vector j of thread t is item t + NT j, row item / 8 (bf16; / 16 for
// fp32).  Rows < nrows and columns < ncols are valid.  load() clamps its addresses into that
// range, so its loads are unconditional and can be issued one slice ahead of their use;
// store() writes the slice into LDS with zeros outside the valid range.
template <typename T, int ROWS, int NT = 256>
struct SliceRegs {
  static constexpr int V = V16<T>::N, PER_ROW = kDvTile / V, ITEMS = ROWS * PER_ROW;
  static constexpr int N = (ITEMS + NT - 1) / NT;
  typedef typename V16<T>::type VT;
  VT x[N];
  // item j of this thread exists (always, when the items divide evenly over the threads)
  // tid: the thread's index (threadIdx.x, or an opaque copy of it in a persistent loop)
  __device__ __forceinline__ static bool has(int j, int tid = threadIdx.x) { return ITEMS % NT == 0 || tid + NT * j < ITEMS; }
  __device__ __forceinline__ void load(const T* src, size_t ld, int nrows, int col0, int ncols, int tid = threadIdx.x) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = min(tid + NT * j, ITEMS - 1), r = idx / PER_ROW;
      const int c = col0 + (idx % PER_ROW) * V;
      x[j] = *reinterpret_cast<const VT*>(src + (size_t)min(r, nrows - 1) * ld + min(c, ncols - V));
    }
  }
  __device__ __forceinline__ void store(T* dst, int lds, int nrows, int col0, int ncols, int tid = threadIdx.x) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + NT * j, r = idx / PER_ROW, c = (idx % PER_ROW) * V;
      if (has(j, tid))
        *reinterpret_cast<VT*>(dst + r * lds + c) = (r < nrows && col0 + c < ncols) ? x[j] : zero_vec<T>();
    }
  }
};

// An fp32 [rows][ld] tile kept in LDS as hi = T(x) and, for 16-bit T, lo = T(x - hi): the
// matrix-core operands come from it whole, by rows (ld8) or by columns (transposing reads),
// with no splitting at the point of use; a single value reads back as hi + lo.
template <typename T>
struct SplitTile {
  static constexpr bool SPLIT = sizeof(T) == 2;
  T* hi;
  T* lo;
  int ld;
  __device__ __forceinline__ float get(int r, int c) const {
    float x = to_f32(hi[r * ld + c]);
    if constexpr (SPLIT) x += to_f32(lo[r * ld + c]);
    return x;
  }
  // the 8 values of row r from column c0 (c0 a multiple of 8)
  __device__ __forceinline__ void get8(int r, int c0, float (&x)[8]) const {
    const Frag<T> h = ld8(hi + r * ld + c0);
    Frag<T> l;
    if constexpr (SPLIT) l = ld8(lo + r * ld + c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = to_f32(h.v[e]) + (SPLIT ? to_f32(l.v[e]) : 0.f);
  }
  // V consecutive values of row r from column c0, as 16-byte stores
  template <int NV>
  __device__ __forceinline__ void put(int r, int c0, const float (&x)[NV]) const {
    typedef typename V16<T>::type VT;
    static_assert(NV == V16<T>::N, "one 16-byte vector");
    VT h, l;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      h[e] = from_f32<T>(x[e]);
      l[e] = from_f32<T>(x[e] - to_f32(h[e]));
    }
    *reinterpret_cast<VT*>(hi + r * ld + c0) = h;
    if constexpr (SPLIT) *reinterpret_cast<VT*>(lo + r * ld + c0) = l;
  }
  __device__ __forceinline__ void put1(int r, int c, float x) const {
    const T h = from_f32<T>(x);
    hi[r * ld + c] = h;
    if constexpr (SPLIT) lo[r * ld + c] = from_f32<T>(x - to_f32(h));
  }
  // operand row r, k-run from column k0 (lane layout of ld8)
  __device__ __forceinline__ HiLo<T> row(int r, int k0) const {
    HiLo<T> f;
    f.hi = ld8(hi + r * ld + k0);
    if constexpr (SPLIT) f.lo = ld8(lo + r * ld + k0);
    return f;
  }
  // operand column n0 + col, k-run down rows k0 .. k0 + 31 (lane layout of ld8_colblk)
  __device__ __forceinline__ HiLo<T> col(int k0, int n0, int lane = threadIdx.x & 63) const {
    HiLo<T> f;
    f.hi = ld8_colblk(hi + k0 * ld + n0, ld, lane);
    if constexpr (SPLIT) f.lo = ld8_colblk(lo + k0 * ld + n0, ld, lane);
    return f;
  }
};

// ----------------------------------------------------------------------------- pass 1 forward
// Z = E * (QK (W Ei) + Q S1_n), P = softmax_slots(Z), written as the [L][m] queries of pass 2,
// together with pass 2's chunk operands, which are what the GLA preparation would form from
// the queries P (as stored), the keys w and the same gates:
//   Qs2 = P 2^b,   A2[r][c] = sum_s P[r][s] w[c][s] 2^{b_r[s] - b_c[s]}  (c <= r, else 0)
// on the factorised path as (P E)(W Ei)^T on hi/lo matrix-core products, on the exact path
// element by element.  Pass 2's decayed keys and chunk decays are WdT and Gamma themselves.
template <typename T, int MP, int CP>
__global__ __launch_bounds__(256, 2) void gsa_p_kernel(GsaParams p) {
  using G = GsaCfg<T, MP, CP>;
  using M = ChunkMap<T, MP, CP>;
  constexpr int V = M::V, RPS = M::RPS;
  constexpr int LDF = G::LDF, LDS = G::LDS, LDM = G::LDM, LDC = G::LDC, NRB = G::NRB, NSB = G::NSB;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) char smem[G::P_BYTES];
  float* sB = reinterpret_cast<float*>(smem);
  auto split_at = [&](char* base, int rows, int ld) {
    return SplitTile<T>{reinterpret_cast<T*>(base), reinterpret_cast<T*>(base) + rows * ld, ld};
  };
  const SplitTile<T> tW = split_at(smem + G::FT, CP, G::LDH);   // Ws = W 2^-b (fast) or W (exact path)
  char* reg = smem + G::FT + G::HPAIR;
  T* sq = reinterpret_cast<T*>(reg);          // during the Dk loop
  T* sk = sq + CP * LDS;
  T* sS1 = sk + CP * LDS;
  const SplitTile<T> tQK = split_at(reg, CP, G::LDQ2);   // after it: masked QK
  T* sP = reinterpret_cast<T*>(reg + G::QPAIR);
  T* sA2 = reinterpret_cast<T*>(reg);          // once the scores are formed: A2 [CP][LDC]
  float* segtot = reinterpret_cast<float*>(smem + G::FT + G::HPAIR + G::P_REGION);
  float* sGam = segtot + M::NSEG * MP;
  float* red = sGam + MP;

  const int n = blockIdx.x, bh = blockIdx.y, m = p.m, Dk = p.Dk, DkP = p.DkP;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int row0 = n * p.C, len = min(p.C, p.L - row0);
  const size_t chunk = (size_t)bh * p.N + n;
  const size_t gbase = ((size_t)bh * p.L + row0) * m;
  const T* gg = reinterpret_cast<const T*>(p.g) + gbase;
  const T* qg = reinterpret_cast<const T*>(p.q) + ((size_t)bh * p.L + row0) * Dk;
  const T* kg = reinterpret_cast<const T*>(p.k) + ((size_t)bh * p.L + row0) * Dk;
  const T* s1 = reinterpret_cast<const T*>(p.S1s) + chunk * MP * DkP;
  ChunkScan<T, MP, CP, false> cs;
  cs.load(gg, gg, gg, m, m, len);
  // the first Dk slice is in flight while the gates are scanned
  SliceRegs<T, CP> rq, rk;
  SliceRegs<T, MP> rs;
  rq.load(qg, Dk, len, 0, Dk);
  rk.load(kg, Dk, len, 0, Dk);
  rs.load(s1, DkP, MP, 0, DkP);
  const bool fast = cs.finish(segtot, sGam, red) <= kSpanLimit;
  if (cs.active) {
    const int c0 = cs.cg * V, r0 = cs.seg * RPS;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      float xw[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float bb = cs.b[u][e];
        const float w = -expm1f(cs.qv[u][e]);
        sB[(r0 + u) * LDF + c0 + e] = bb;
        xw[e] = fast ? w * fast_exp2(-bb) : w;
      }
      tW.put(r0 + u, c0, xw);
    }
  }
  const int rb = wave;                        // this wave's 16 chunk rows
  const bool rbv = rb < NRB;
  f32x4 accQK[NRB], accZe[NSB];
#pragma unroll
  for (int c = 0; c < NRB; ++c) accQK[c] = zero4();
#pragma unroll
  for (int s = 0; s < NSB; ++s) accZe[s] = zero4();
  const int nds = DkP / kDvTile;
  for (int ds = 0; ds < nds; ++ds) {
    __syncthreads();
    rq.store(sq, LDS, len, ds * kDvTile, Dk);
    rk.store(sk, LDS, len, ds * kDvTile, Dk);
    rs.store(sS1, LDS, MP, ds * kDvTile, DkP);
    if (ds + 1 < nds) {
      rq.load(qg, Dk, len, (ds + 1) * kDvTile, Dk);
      rk.load(kg, Dk, len, (ds + 1) * kDvTile, Dk);
      rs.load(s1, DkP, MP, (ds + 1) * kDvTile, DkP);
    }
    __syncthreads();
    if (rbv) {
#pragma unroll
      for (int kb = 0; kb < kDvTile / 32; ++kb) {
        const Frag<T> X = ld8(sq + (16 * rb + col) * LDS + 32 * kb + 8 * grp);
#pragma unroll
        for (int cb = 0; cb < NRB; ++cb)
          if (cb <= rb) mma(accQK[cb], X, ld8(sk + (16 * cb + col) * LDS + 32 * kb + 8 * grp));
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) mma(accZe[sb], X, ld8(sS1 + (16 * sb + col) * LDS + 32 * kb + 8 * grp));
      }
    }
  }
  __syncthreads();   // the QK tile and sP take the slices' bytes
  if (rbv) {
#pragma unroll
    for (int cb = 0; cb < NRB; ++cb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
        tQK.put1(r, c, c <= r ? accQK[cb][e] : 0.f);
      }
    }
  }
  __syncthreads();
  float z[NSB][4];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) z[sb][0] = z[sb][1] = z[sb][2] = z[sb][3] = 0.f;
  if (rbv) {
    if (fast) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kc = 0; kc < CP / 32; ++kc) mma3(acc, tQK.row(16 * rb + col, 32 * kc + 8 * grp), tW.col(32 * kc, 16 * sb));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * grp + e, s = 16 * sb + col;
          z[sb][e] = fast_exp2(sB[r * LDF + s]) * (acc[e] + accZe[sb][e]);
        }
      }
    } else {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * grp + e, s = 16 * sb + col;
          const float br = sB[r * LDF + s];
          float zi = 0.f;
          for (int c = 0; c <= r; ++c) zi += tQK.get(r, c) * tW.get(c, s) * fast_exp2(br - sB[c * LDF + s]);
          z[sb][e] = zi + fast_exp2(br) * accZe[sb][e];
        }
      }
    }
  }
  if (rbv && p.act != kActSoftmax) {
    // element-wise read-out; the backward keeps the scores Z, from which it forms f'(Z)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rb + 4 * grp + e;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const bool ok = 16 * sb + col < m;
        sP[r * LDM + 16 * sb + col] = from_f32<T>(ok ? gsa_read(z[sb][e], p.act) : 0.f);
        if (p.Pf && r < len && ok) p.Pf[gbase + (size_t)r * m + 16 * sb + col] = z[sb][e];
      }
    }
  } else if (rbv) {
    // softmax over the m valid slots of each row (rows spread over e, slots over sb and col)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
        if (16 * sb + col < m) mx = fmaxf(mx, z[sb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
      float ex[NSB], sum = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        ex[sb] = (16 * sb + col < m) ? fast_exp2((z[sb][e] - mx) * kLog2e) : 0.f;
        sum += ex[sb];
      }
      sum += __shfl_xor(sum, 1, 64);
      sum += __shfl_xor(sum, 2, 64);
      sum += __shfl_xor(sum, 4, 64);
      sum += __shfl_xor(sum, 8, 64);
      const float inv = 1.f / sum;
      const int r = 16 * rb + 4 * grp + e;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const float pr = ex[sb] * inv;
        sP[r * LDM + 16 * sb + col] = from_f32<T>(pr);
        if (p.Pf && r < len && 16 * sb + col < m) p.Pf[gbase + (size_t)r * m + 16 * sb + col] = pr;
      }
    }
  }
  __syncthreads();   // P staged; the QK tile dead

  // ---- A2 (rows past the chunk's end are zero, as are columns there: w = 0)
  if (rbv) {
    HiLo<T> fpe[MP / 32];                     // P E on this lane's operand row, once per wave
    if (fast) {
#pragma unroll
      for (int ks = 0; ks < MP / 32; ++ks) {
        float xa[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 16 * rb + col, sl = 32 * ks + 8 * grp + e;
          xa[e] = to_f32(sP[r * LDM + sl]) * fast_exp2(sB[r * LDF + sl]);
        }
        fpe[ks] = hilo<T>(xa);
      }
    }
#pragma unroll
    for (int cb = 0; cb < NRB; ++cb) {
      f32x4 acc = zero4();
      if (cb <= rb) {
        if (fast) {
#pragma unroll
          for (int ks = 0; ks < MP / 32; ++ks) mma3(acc, fpe[ks], tW.row(16 * cb + col, 32 * ks + 8 * grp));   // W Ei
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
            float x = 0.f;
            if (c <= r)
              for (int sl = 0; sl < m; ++sl)
                x += to_f32(sP[r * LDM + sl]) * tW.get(c, sl) * fast_exp2(sB[r * LDF + sl] - sB[c * LDF + sl]);
            acc[e] = x;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
        sA2[r * LDC + c] = from_f32<T>(c <= r && r < len ? acc[e] : 0.f);
      }
    }
  }
  T* Pg = p.P ? reinterpret_cast<T*>(p.P) + gbase : nullptr;   // null: the forward alone
  T* Qg2 = reinterpret_cast<T*>(p.ops2.Qs) + chunk * CP * MP;
  constexpr int PER_ROW = MP / V;
  for (int idx = tid; idx < CP * PER_ROW; idx += 256) {
    const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
    const VT pv = *reinterpret_cast<const VT*>(sP + r * LDM + c);
    if (Pg && r < len && c < m) *reinterpret_cast<VT*>(Pg + (size_t)r * m + c) = pv;
    VT qs;
#pragma unroll
    for (int e = 0; e < V; ++e) qs[e] = from_f32<T>(r < len ? to_f32(pv[e]) * fast_exp2(sB[r * LDF + c + e]) : 0.f);
    *reinterpret_cast<VT*>(Qg2 + (size_t)r * MP + c) = qs;
  }
  __syncthreads();
  tile_out<T>(reinterpret_cast<T*>(p.ops2.A) + chunk * CP * CP, sA2, CP, CP, LDC);
}

// ----------------------------------------------------------------------------- read-out backward
// dZ = P (dP - <dP, P>) per row for the softmax, dZ = f'(Z) dP for the element-wise read-outs;
// written in fp32, and (dZ * 2^b)^T per chunk for the pass-1 reverse walk.
template <typename T, int MP, int CP>
__global__ __launch_bounds__(256) void gsa_dz_kernel(GsaParams p) {
  using M = ChunkMap<T, MP, CP>;
  constexpr int V = M::V, RPS = M::RPS, LDM = MP + V;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) T sZs[CP * LDM];     // dZ 2^b, staged to leave in 16-byte rows
  __shared__ float segtot[M::NSEG * MP];
  __shared__ float sGam[MP];
  __shared__ float red[8];
  __shared__ float rpart[M::NCG * CP];
  const int n = blockIdx.x, bh = blockIdx.y, m = p.m;
  const int row0 = n * p.C, len = min(p.C, p.L - row0);
  const size_t gbase = ((size_t)bh * p.L + row0) * m;
  const size_t chunk = (size_t)bh * p.N + n;
  const T* gg = reinterpret_cast<const T*>(p.g) + gbase;
  ChunkScan<T, MP, CP, false> cs;
  cs.load(gg, gg, gg, m, m, len);
  const int c0 = cs.cg * V, r0 = cs.seg * RPS;
  // P (fp32: the softmax's Jacobian keeps sum_s dZ = 0; Z for the element-wise read-outs) and
  // dP (fp32: dP - <dP, P> cancels when the slot memories are alike, so dP is not rounded to
  // the input type first), from clamped rows, in flight while the gates are scanned
  f32x4 pl[RPS][V / 4], dl[RPS][V / 4];
  {
    const int cc = (cs.active && c0 < m) ? c0 : 0;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const size_t off = gbase + (size_t)min(r0 + u, len - 1) * m + cc;
#pragma unroll
      for (int e4 = 0; e4 < V / 4; ++e4) {
        pl[u][e4] = *reinterpret_cast<const f32x4*>(p.Pf + off + 4 * e4);
        dl[u][e4] = *reinterpret_cast<const f32x4*>(p.dP + off + 4 * e4);
      }
    }
  }
  cs.finish(segtot, sGam, red);
  float pv[RPS][V], dpv[RPS][V];
  if (cs.active) {
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const int r = r0 + u;
      const bool ok = r < len && c0 < m;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        pv[u][e] = ok ? pl[u][e >> 2][e & 3] : 0.f;
        dpv[u][e] = ok ? dl[u][e >> 2][e & 3] : 0.f;
        s += pv[u][e] * dpv[u][e];
      }
      rpart[cs.cg * CP + r] = s;
    }
  }
  __syncthreads();
  if (cs.active) {
    float* dZg = p.dZ + gbase;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const int r = r0 + u;
      float rs = 0.f;
      for (int c = 0; c < M::NCG; ++c) rs += rpart[c * CP + r];
      float dz[V];
      VT zs;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        dz[e] = p.act == kActSoftmax ? pv[u][e] * (dpv[u][e] - rs) : gsa_read_grad(pv[u][e], dpv[u][e], p.act);
        zs[e] = from_f32<T>(dz[e] * fast_exp2(cs.b[u][e]));
      }
      *reinterpret_cast<VT*>(sZs + r * LDM + c0) = zs;
      if (r < len && c0 < m) {
#pragma unroll
        for (int e = 0; e < V; e += 4)
          *reinterpret_cast<f32x4*>(dZg + (size_t)r * m + c0 + e) = f32x4{dz[e], dz[e + 1], dz[e + 2], dz[e + 3]};
      }
    }
  }
  __syncthreads();
  tile_out<T>(reinterpret_cast<T*>(p.dZs) + chunk * CP * MP, sZs, CP, MP, LDM);
}

// ----------------------------------------------------------------------------- pass 1 backward
// Eight waves: the two waves (rb, 0) and (rb, 1) of 16-row block rb split its column blocks by
// parity, so each holds half the accumulators and a CU runs two waves per SIMD.  The scans
// keep the 256-thread layout (the upper 256 threads sit them out).
constexpr int kP1Threads = 512;

template <typename T, int MP, int CP>
__global__ __launch_bounds__(kP1Threads) void gsa_pass1_bwd_kernel(GsaParams p, int ntk, int ntiles) {
  using G = GsaCfg<T, MP, CP>;
  using M = ChunkMap<T, MP, CP>;
  constexpr int NT = kP1Threads;
  constexpr int V = M::V, RPS = M::RPS, NSEG = M::NSEG, NCG = M::NCG;
  constexpr int LDF = G::LDF, LDS = G::LDS, NRB = G::NRB, NSB = G::NSB;
  constexpr int NRH = (NRB + 1) / 2, NSH = NSB / 2, NIH = kDvTile / 32;   // column blocks per half
  typedef typename V16<T>::type VT;
  using SC = SliceRegs<T, CP, NT>;
  using SM = SliceRegs<T, MP, NT>;
  __shared__ __attribute__((aligned(16))) char smem[G::B_BYTES];
  constexpr int LDH = G::LDH, LDQ2 = G::LDQ2;
  float* sB = reinterpret_cast<float*>(smem);
  auto split_at = [&](char* base, int rows, int ld) {
    return SplitTile<T>{reinterpret_cast<T*>(base), reinterpret_cast<T*>(base) + rows * ld, ld};
  };
  const SplitTile<T> tW = split_at(smem + G::FT, CP, LDH);                 // W Ei (fast) or W
  const SplitTile<T> tZ = split_at(smem + G::FT + G::HPAIR, CP, LDH);      // dZ E (fast) or dZ
  char* reg = smem + G::FT + 2 * G::HPAIR;
  T* sdQK = reinterpret_cast<T*>(reg);                     // until the Dk loop
  T* sq = reinterpret_cast<T*>(reg + G::QPAIR);
  T* sk = sq + CP * LDS;
  T* sS1 = sk + CP * LDS;
  T* sdS1 = sS1 + MP * LDS;
  T* sDQ = sdS1 + MP * LDS;
  T* sDK = sDQ + CP * LDS;
  const SplitTile<T> tQK = split_at(reg, CP, LDQ2);        // after the Dk loop: strictly lower QK
  float* sU = reinterpret_cast<float*>(reg + G::QPAIR);
  float* sY = sU + CP * LDF;
  float* sD = sY + CP * LDF;
  float* segtot = reinterpret_cast<float*>(smem + G::FT + 2 * G::HPAIR + G::B_REGION);
  float* sGam = segtot + 2 * NSEG * MP;
  float* sZ1 = sGam + MP;
  float* red = sZ1 + MP;
  float* sDiag = red + 8;
  float* sQKd = sDiag + CP;                                 // diagonal of QK

  const int m = p.m, Dk = p.Dk, DkP = p.DkP;

  // The grid is persistent: workgroup w takes tiles w, w + gridDim.x, ... (tile = chunk
  // tile % N of sequence tile / N).  A tile's gates and dZ, which its gate scan and first phase
  // wait for, go out during the previous tile's gate-gradient phase; past the last tile they
  // still go out, unconditionally, but read one cached row of that tile.
  ChunkScan<T, MP, CP, false> cs;
  f32x4 dzv[RPS][V / 4];                 // dZ in the scan's layout
  auto issue = [&](int tt, bool past, int tid) {
    const int nn = tt % p.N, rr0 = nn * p.C;
    const int ll = past ? 1 : min(p.C, p.L - rr0);
    const size_t gb = ((size_t)(tt / p.N) * p.L + rr0) * m;
    const T* g0 = reinterpret_cast<const T*>(p.g) + gb;
    cs.load(g0, g0, g0, m, m, ll, tid);
    const int cc = (cs.active && cs.cg * V < m) ? cs.cg * V : 0;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const float* src = p.dZ + gb + (size_t)min(cs.seg * RPS + u, ll - 1) * m + cc;
#pragma unroll
      for (int e4 = 0; e4 < V / 4; ++e4) dzv[u][e4] = *reinterpret_cast<const f32x4*>(src + 4 * e4);
    }
  };
  // With more than 64 slots the persistent loop would spill: there each workgroup takes one
  // tile (the launch gives one workgroup per tile) and the loop body runs once.
  constexpr bool PERSIST = GsaCfg<T, MP, CP>::P1_PERSIST;
  int tile_t = blockIdx.x;
  issue(tile_t, false, threadIdx.x);
  for (;;) {
  // the thread index through an opaque move, once per tile: per-lane addresses are then formed
  // inside each tile instead of being hoisted out of the loop and held across it
  const int tid = opaque_thread_index(), wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int tile_n = tile_t + gridDim.x;
  const int n = tile_t % p.N, bh = tile_t / p.N;
  const int row0 = n * p.C, len = min(p.C, p.L - row0);
  const size_t chunk = (size_t)bh * p.N + n;
  const size_t gbase = ((size_t)bh * p.L + row0) * m;
  const size_t kbase = ((size_t)bh * p.L + row0) * Dk;
  const T* qg = reinterpret_cast<const T*>(p.q) + kbase;
  const T* kg = reinterpret_cast<const T*>(p.k) + kbase;
  const T* s1 = reinterpret_cast<const T*>(p.S1s) + chunk * MP * DkP;
  const T* ds1 = reinterpret_cast<const T*>(p.dS1s) + chunk * MP * DkP;
  T* dqg = reinterpret_cast<T*>(p.dq) + kbase;
  T* dkg = reinterpret_cast<T*>(p.dk) + kbase;
  const int c0 = cs.cg * V, r0 = cs.seg * RPS;
  // the first Dk slice: in flight while the gates are scanned
  SC rq, rk;
  SM rs, rd;
  rq.load(qg, Dk, len, 0, Dk, tid);
  rk.load(kg, Dk, len, 0, Dk, tid);
  rs.load(s1, DkP, MP, 0, DkP, tid);
  rd.load(ds1, DkP, MP, 0, DkP, tid);
  const bool fast = cs.finish(segtot, sGam, red, tid) <= kSpanLimit;
  // diagonal of dQK, sum_s dZ w per row.  For the softmax it equals -sum_s dZ alpha, since
  // sum_s dZ = 0 (its Jacobian); that form scales with alpha instead of cancelling.
  float dsum[RPS];
#pragma unroll
  for (int u = 0; u < RPS; ++u) dsum[u] = 0.f;
  if (cs.active) {
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const int r = r0 + u;
      const bool ok = r < len && c0 < m;
      float xw[V], xz[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float w = -expm1f(cs.qv[u][e]);
        const float dz = ok ? dzv[u][e >> 2][e & 3] : 0.f;
        // on the factorised path the tiles hold the decayed operands W Ei and dZ E, which every
        // product there takes; the exact path reads the raw values
        const float bb = cs.b[u][e];
        sB[r * LDF + c0 + e] = bb;
        xw[e] = fast ? w * fast_exp2(-bb) : w;
        xz[e] = fast ? dz * fast_exp2(bb) : dz;
        dsum[u] += p.act == kActSoftmax ? -dz * (1.f - w) : dz * w;
      }
      tW.put(r, c0, xw);
      tZ.put(r, c0, xz);
    }
  }
#pragma unroll
  for (int u = 0; u < RPS; ++u) {
#pragma unroll
    for (int o = 1; o < NCG; o <<= 1) dsum[u] += __shfl_xor(dsum[u], o, 64);
  }
  if (cs.active && cs.cg == 0) {
#pragma unroll
    for (int u = 0; u < RPS; ++u) sDiag[r0 + u] = dsum[u];
  }
  __syncthreads();
  const int rb = wave & 3, hf = wave >> 2;   // row block; which parity of column blocks
  const bool rbv = rb < NRB;

  // (dZ E) on this lane's operand row 16 rb + col: the row operand of dQK and of dq's state term
  HiLo<T> dze[MP / 32];
  if (rbv) {
#pragma unroll
    for (int ks = 0; ks < MP / 32; ++ks) {
      const int r = 16 * rb + col, s0 = 32 * ks + 8 * grp;
      if (fast) {
        dze[ks] = tZ.row(r, s0);
      } else {
        float x[8];
        tZ.get8(r, s0, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= fast_exp2(sB[r * LDF + s0 + e]);
        dze[ks] = hilo<T>(x);
      }
    }
  }

  // ---- dQK = mask_{c<=r}((dZ E)(W Ei)^T), with the diagonal from sDiag
  if (rbv) {
#pragma unroll
    for (int ch = 0; ch < NRH; ++ch) {
      const int cb = 2 * ch + hf;
      if (cb >= NRB) break;
      f32x4 acc = zero4();
      if (cb <= rb) {
        if (fast) {
#pragma unroll
          for (int ks = 0; ks < MP / 32; ++ks) mma3(acc, dze[ks], tW.row(16 * cb + col, 32 * ks + 8 * grp));   // W Ei
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
            float x = 0.f;
            if (c < r)
              for (int s = 0; s < m; ++s)
                x += tZ.get(r, s) * tW.get(c, s) * fast_exp2(sB[r * LDF + s] - sB[c * LDF + s]);
            acc[e] = x;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
        sdQK[r * LDQ2 + c] = from_f32<T>(c < r ? acc[e] : c == r ? sDiag[r] : 0.f);
      }
    }
  }
  __syncthreads();

  // Operands that stay fixed over the Dk slices, built once: dQK rows and columns, dZ E and
  // W Eg (Eg = 2^{Gamma-b}), all on this wave's 16 rows
  Frag<T> fA[CP / 32], fT[CP / 32], fZ[MP / 32], fG[MP / 32];
  if (rbv) {
#pragma unroll
    for (int kc = 0; kc < CP / 32; ++kc) {
      fA[kc] = ld8(sdQK + (16 * rb + col) * LDQ2 + 32 * kc + 8 * grp);
      fT[kc] = ld8_colblk(sdQK + (32 * kc) * LDQ2 + 16 * rb, LDQ2, lane);
    }
#pragma unroll
    for (int ks = 0; ks < MP / 32; ++ks) {
      const int r = 16 * rb + col, s0 = 32 * ks + 8 * grp;
      float xw[8];
      tW.get8(r, s0, xw);
#pragma unroll
      for (int e = 0; e < 8; ++e) xw[e] *= fast ? fast_exp2(sGam[s0 + e]) : fast_exp2(sGam[s0 + e] - sB[r * LDF + s0 + e]);
      fZ[ks] = dze[ks].hi;
      fG[ks] = frag_of<T>(xw);
    }
  }

  // ---- Dk slices: QK, Ze, B1 accumulate; dq, dk slices written; the next slice is loaded
  // while this one is used
  f32x4 accQK[NRH], accZe[NSH], accB1[NSH];   // column blocks 2 i + hf
#pragma unroll
  for (int c = 0; c < NRH; ++c) accQK[c] = zero4();
#pragma unroll
  for (int s = 0; s < NSH; ++s) accZe[s] = accB1[s] = zero4();
  float z1[SM::N];                       // partial colsum(dS1 * S1) over this thread's slice rows
#pragma unroll
  for (int j = 0; j < SM::N; ++j) z1[j] = 0.f;
  for (int ds = 0; ds < ntk; ++ds) {
    __syncthreads();
    rq.store(sq, LDS, len, ds * kDvTile, Dk, tid);
    rk.store(sk, LDS, len, ds * kDvTile, Dk, tid);
    rs.store(sS1, LDS, MP, ds * kDvTile, DkP, tid);
    rd.store(sdS1, LDS, MP, ds * kDvTile, DkP, tid);
#pragma unroll
    for (int j = 0; j < SM::N; ++j) {
      if (SM::has(j, tid)) {
#pragma unroll
        for (int e = 0; e < V; ++e) z1[j] += to_f32(rs.x[j][e]) * to_f32(rd.x[j][e]);
      }
    }
    if (ds + 1 < ntk) {
      rq.load(qg, Dk, len, (ds + 1) * kDvTile, Dk, tid);
      rk.load(kg, Dk, len, (ds + 1) * kDvTile, Dk, tid);
      rs.load(s1, DkP, MP, (ds + 1) * kDvTile, DkP, tid);
      rd.load(ds1, DkP, MP, (ds + 1) * kDvTile, DkP, tid);
    }
    __syncthreads();
    if (rbv) {
#pragma unroll
      for (int kb = 0; kb < kDvTile / 32; ++kb) {
        const Frag<T> Xq = ld8(sq + (16 * rb + col) * LDS + 32 * kb + 8 * grp);
        const Frag<T> Xk = ld8(sk + (16 * rb + col) * LDS + 32 * kb + 8 * grp);
#pragma unroll
        for (int ch = 0; ch < NRH; ++ch) {
          const int cb = 2 * ch + hf;
          if (cb <= rb) mma(accQK[ch], Xq, ld8(sk + (16 * cb + col) * LDS + 32 * kb + 8 * grp));
        }
#pragma unroll
        for (int sh = 0; sh < NSH; ++sh) {
          const int sb = 2 * sh + hf;
          mma(accZe[sh], Xq, ld8(sS1 + (16 * sb + col) * LDS + 32 * kb + 8 * grp));
          mma(accB1[sh], Xk, ld8(sdS1 + (16 * sb + col) * LDS + 32 * kb + 8 * grp));
        }
      }
      // dq slice = dQK K + (dZ E) S1^T ; dk slice = dQK^T Q + (W Eg) dS1^T
#pragma unroll
      for (int ih = 0; ih < NIH; ++ih) {
        const int ib = 2 * ih + hf;
        f32x4 aq = zero4(), ak = zero4();
#pragma unroll
        for (int kc = 0; kc < CP / 32; ++kc) {
          mma(aq, fA[kc], ld8_colblk(sk + (32 * kc) * LDS + 16 * ib, LDS, lane));
          mma(ak, fT[kc], ld8_colblk(sq + (32 * kc) * LDS + 16 * ib, LDS, lane));
        }
#pragma unroll
        for (int ks = 0; ks < MP / 32; ++ks) {
          mma(aq, fZ[ks], ld8_colblk(sS1 + (32 * ks) * LDS + 16 * ib, LDS, lane));
          mma(ak, fG[ks], ld8_colblk(sdS1 + (32 * ks) * LDS + 16 * ib, LDS, lane));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sDQ[(16 * rb + 4 * grp + e) * LDS + 16 * ib + col] = from_f32<T>(aq[e]);
          sDK[(16 * rb + 4 * grp + e) * LDS + 16 * ib + col] = from_f32<T>(ak[e]);
        }
      }
    }
    __syncthreads();
    constexpr int PER_ROW = kDvTile / V;
    for (int idx = tid; idx < CP * PER_ROW; idx += NT) {
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
      const int cc = ds * kDvTile + c;
      if (r < len && cc < Dk) {
        *reinterpret_cast<VT*>(dqg + (size_t)r * Dk + cc) = *reinterpret_cast<const VT*>(sDQ + r * LDS + c);
        *reinterpret_cast<VT*>(dkg + (size_t)r * Dk + cc) = *reinterpret_cast<const VT*>(sDK + r * LDS + c);
      }
    }
  }
  // the pass-2 gradients the gate gradient adds at the end, fetched while the rest runs
  VT w2v[RPS];
  f32x4 g2v[RPS][V / 4];
  {
    const int cc = (cs.active && c0 < m) ? c0 : 0;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const size_t off = gbase + (size_t)min(r0 + u, len - 1) * m + cc;
      w2v[u] = *reinterpret_cast<const VT*>(reinterpret_cast<const T*>(p.dW2) + off);
#pragma unroll
      for (int e4 = 0; e4 < V / 4; ++e4) g2v[u][e4] = *reinterpret_cast<const f32x4*>(p.dg2 + off + 4 * e4);
    }
  }
  // Z1_n = 2^Gamma colsum(dS1_{n+1} * S1_n): slot row (tid + NT j) / PER_ROW, summed over the
  // PER_ROW consecutive lanes that share it
#pragma unroll
  for (int j = 0; j < SM::N; ++j) {
#pragma unroll
    for (int o = 1; o < SM::PER_ROW; o <<= 1) z1[j] += __shfl_xor(z1[j], o, 64);
    const int idx = tid + NT * j, zs = idx / SM::PER_ROW;
    if (SM::has(j, tid) && idx % SM::PER_ROW == 0) sZ1[zs] = zs < m ? z1[j] * fast_exp2(sGam[zs]) : 0.f;
  }
  __syncthreads();   // slices and dQK dead: the QK tile and the dg tiles take their bytes
  if (rbv) {
#pragma unroll
    for (int ch = 0; ch < NRH; ++ch) {
      const int cb = 2 * ch + hf;
      if (cb >= NRB) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the strictly lower part (what the intra products take), the diagonal apart
        const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
        tQK.put1(r, c, c < r ? accQK[ch][e] : 0.f);
        if (c == r) sQKd[r] = accQK[ch][e];
      }
    }
  }
  __syncthreads();

  // ---- per element (rows of this wave): Znd, dW1', B1 -> u, y, dW1 total
  if (rbv) {
#pragma unroll
    for (int sh = 0; sh < NSH; ++sh) {
      const int sb = 2 * sh + hf;
      f32x4 zi = zero4(), w1 = zero4();
      if (fast) {
#pragma unroll
        for (int kc = 0; kc < CP / 32; ++kc) {
          // QK' row r against (W Ei) column s; QK' column r against (dZ E) column s
          mma3(zi, tQK.row(16 * rb + col, 32 * kc + 8 * grp), tW.col(32 * kc, 16 * sb, lane));
          mma3(w1, tQK.col(32 * kc, 16 * rb, lane), tZ.col(32 * kc, 16 * sb, lane));
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * grp + e, s = 16 * sb + col;
        const float br = sB[r * LDF + s];
        const float eb = fast_exp2(br), eib = fast_exp2(-br);
        float zip, dw1p;
        if (fast) {
          zip = eb * zi[e];
          dw1p = eib * w1[e];
        } else {
          zip = 0.f;
          dw1p = 0.f;
          for (int c = 0; c < r; ++c) zip += tQK.get(r, c) * tW.get(c, s) * fast_exp2(br - sB[c * LDF + s]);
          for (int c = r + 1; c < CP; ++c)
            dw1p += tQK.get(c, r) * tZ.get(c, s) * fast_exp2(sB[c * LDF + s] - br);
        }
        const float znd = zip + eb * accZe[sh][e];
        const float b1 = fast_exp2(sGam[s] - br) * accB1[sh][e];
        const float dz = fast ? tZ.get(r, s) * eib : tZ.get(r, s);
        const float w = fast ? tW.get(r, s) * eb : tW.get(r, s);
        sU[r * LDF + s] = dz * znd - w * dw1p;
        sY[r * LDF + s] = w * b1;
        sD[r * LDF + s] = dw1p + sQKd[r] * dz + b1;
      }
    }
  }
  __syncthreads();
  // the gates and dZ of this workgroup's next tile (dzv and the raw gates are dead here)
  if constexpr (PERSIST) issue(tile_n < ntiles ? tile_n : tile_t, tile_n >= ntiles, tid);

  // ---- dg: in-chunk suffix of u, exclusive prefix of y, Z1, pass-2 part, -alpha dW
  float up[RPS][V], yk[RPS][V];
  if (cs.active) {
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        up[u][e] = sU[(r0 + u) * LDF + c0 + e];
        yk[u][e] = sY[(r0 + u) * LDF + c0 + e];
      }
    }
    float sp[V], sk2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) sp[e] = sk2[e] = 0.f;
#pragma unroll
    for (int u = RPS - 1; u >= 0; --u) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        sp[e] += up[u][e];
        up[u][e] = sp[e];
      }
    }
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float x = yk[u][e];
        yk[u][e] = sk2[e];
        sk2[e] += x;
      }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      segtot[cs.seg * MP + c0 + e] = sp[e];
      segtot[(NSEG + cs.seg) * MP + c0 + e] = sk2[e];
    }
  }
  __syncthreads();
  // later segments' suffix totals of u, earlier segments' prefix totals of y
  for (int t = tid; t < 2 * MP; t += 256)
    seg_scan_channel<NSEG>(segtot + (t < MP ? 0 : NSEG * MP), MP, t < MP ? t : t - MP, t < MP);
  __syncthreads();
  if (cs.active) {
    float add[V];
#pragma unroll
    for (int e = 0; e < V; ++e) add[e] = sZ1[c0 + e];
#pragma unroll
    for (int e = 0; e < V; ++e) add[e] += segtot[cs.seg * MP + c0 + e] + segtot[(NSEG + cs.seg) * MP + c0 + e];
    float* dgg = p.dg + gbase;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const int r = r0 + u;
      if (r < len && c0 < m) {
#pragma unroll
        for (int e = 0; e < V; e += 4) {
          const f32x4 g2 = g2v[u][e >> 2];
          f32x4 o;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const float alpha = fast_exp2(cs.qv[u][e + x] * kLog2e);
            const float dwt = sD[r * LDF + c0 + e + x] + to_f32(w2v[u][e + x]);
            o[x] = up[u][e + x] + yk[u][e + x] + add[e + x] + g2[x] - alpha * dwt;
          }
          *reinterpret_cast<f32x4*>(dgg + (size_t)r * m + c0 + e) = o;
        }
      }
    }
  }
  if (!PERSIST || tile_n >= ntiles) break;
  tile_t = tile_n;
  __syncthreads();                       // the next tile's scan reuses the tail and the tiles
  }
  __builtin_amdgcn_s_waitcnt(0);         // the last tile's repeated loads have landed
}

// Resident workgroups of the pass-1 backward on the current device (its persistent grid),
// cached per device id.
template <typename T, int MP, int CP>
int p1_slots() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gsa_pass1_bwd_kernel<T, MP, CP>, kP1Threads, 0) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  const int cus = device_cu_count();
  const int n = (cus > 0 ? cus : 256) * per_cu;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// ----------------------------------------------------------------------------- launchers
// The forward needs the read-out kernel's LDS and the walks; the backward also the pass-1
// backward kernel's, whose three fp32 [CP][MP] tiles and phase region rule out m > 64 at
// C = 64 (about 237 KB at m = 128).
template <typename T, int MP, int CP>
constexpr bool gsa_fwd_fits() {
  return GsaCfg<T, MP, CP>::P_BYTES <= kMaxLds && walk_fits<T, MP, CP>();
}
template <typename T, int MP, int CP>
constexpr bool gsa_fits() {
  return gsa_fwd_fits<T, MP, CP>() && GsaCfg<T, MP, CP>::B_BYTES <= kMaxLds;
}

// Both passes' state walks in one launch.  Pass 2's decayed keys are the pass-1 walk's matrix
// WdT = (w 2^{Gamma-b})^T and its chunk decays are Gamma, so the two walks share the matrix and
// differ only in their source (k for pass 1's transposed slot keys, v for pass 2's slot
// values), their states and their end states.
template <typename T, int MP, int CP>
hipError_t launch_gsa_walks(const GsaParams& p, float* hkt, float* hvt, hipStream_t s) {
  Batches<WalkIO> b{};
  b.n = 2;
  b.p[0] = WalkIO{p.WdT, p.k, p.Gam, p.S1s, p.hk0, hkt, p.m, p.Dk, p.L, p.C, p.N, 1};
  b.p[1] = WalkIO{p.WdT, p.v, p.Gam, p.Hs2, p.hv0, hvt, p.m, p.Dv, p.L, p.C, p.N, 0};
  const int BH[2] = {p.BH, p.BH};
  return launch_walk_store_batches<T, MP, CP>(b, BH, s);
}

template <typename T, int MP, int CP>
hipError_t launch_gsa_fwd(const GsaParams& p, hipStream_t s) {
  if constexpr (!gsa_fwd_fits<T, MP, CP>()) {
    return hipErrorNotSupported;
  } else {
    hipError_t e;
    hipLaunchKernelGGL((gsa_prep_kernel<T, MP, CP>), dim3(p.N, p.BH), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_gsa_walks<T, MP, CP>(p, p.hkt, p.hvt, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((gsa_p_kernel<T, MP, CP>), dim3(p.N, p.BH), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // pass 2's outputs from the chunk operands gsa_p left and the states the walk above left
    FwdParams f;
    f.q = p.P; f.k = p.W; f.v = p.v; f.g = p.g; f.h0 = p.hv0; f.o = p.o; f.ht = p.hvt;
    f.BH = p.BH; f.L = p.L; f.Dk = p.m; f.Dv = p.Dv; f.C = p.C; f.N = p.N;
    f.ops = p.ops2; f.Hs = p.Hs2; f.states_ready = true; f.ops_ready = true; f.events = LaunchEvents{nullptr, 0};
    return launch_gla_fwd<T, MP, CP>(f, s);
  }
}

template <typename T, int MP, int CP>
hipError_t launch_gsa_bwd(const GsaParams& p, hipStream_t s) {
  if constexpr (!gsa_fits<T, MP, CP>()) {
    return hipErrorNotSupported;
  } else {
    hipError_t e;
    if (!p.saved) {   // recompute the forward's tensors, as the saving forward leaves them
      hipLaunchKernelGGL((gsa_prep_kernel<T, MP, CP>), dim3(p.N, p.BH), dim3(256), 0, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = launch_gsa_walks<T, MP, CP>(p, nullptr, nullptr, s)) != hipSuccess) return e;
      hipLaunchKernelGGL((gsa_p_kernel<T, MP, CP>), dim3(p.N, p.BH), dim3(256), 0, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    BwdParams b;
    b.q = p.P; b.k = p.W; b.v = p.v; b.g = p.g; b.do_ = p.do_; b.h0 = p.hv0; b.dht = p.dhvt;
    b.dq = p.dP; b.dk = p.dW2; b.dv = p.dv; b.dg = p.dg2; b.dh0 = p.dhv0;
    b.BH = p.BH; b.L = p.L; b.Dk = p.m; b.Dv = p.Dv; b.C = p.C; b.N = p.N;
    b.ops = p.ops2; b.Hs = p.Hs2; b.dHs = p.dHs2; b.saved = true; b.events = LaunchEvents{nullptr, 0};
    // the read-out's backward needs each row's whole slot width: in the chunk kernel's epilogue
    // when one tile holds it, else in its own kernel on the fp32 dP
    const bool fuse_dz = gla_bwd_key_slices((int)sizeof(T), MP, CP) == 1;
    if (fuse_dz) {
      b.rd = p.Pf; b.dz = p.dZ; b.dzs = p.dZs; b.act = p.act;
    } else {
      b.dq32 = p.dP;   // dP stays fp32 for the read-out's backward
    }
    if ((e = launch_gla_bwd<T, MP, CP>(b, s)) != hipSuccess) return e;
    if (!fuse_dz) {
      hipLaunchKernelGGL((gsa_dz_kernel<T, MP, CP>), dim3(p.N, p.BH), dim3(256), 0, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    WalkIO w1r{p.dZs, p.q, p.Gam, p.dS1s, p.dhkt, p.dhk0, p.m, p.Dk, p.L, p.C, p.N, 1};
    if ((e = launch_walk_reverse<T, MP, CP>(w1r, p.BH, s)) != hipSuccess) return e;
    const int ntk = p.DkP / kDvTile, ntiles = p.N * p.BH;
    const int grid = GsaCfg<T, MP, CP>::P1_PERSIST ? imin(ntiles, p1_slots<T, MP, CP>()) : ntiles;
    hipLaunchKernelGGL((gsa_pass1_bwd_kernel<T, MP, CP>), dim3(grid), dim3(kP1Threads), 0, s, p, ntk, ntiles);
    return hipGetLastError();
  }
}

bool gsa_config_fits(int esize, int MP, int CP, bool bwd) {
  bool ok = false;
#define GSA_FIT(TT, M_, C_) \
  if (esize == (int)sizeof(TT) && MP == M_ && CP == C_) ok = bwd ? gsa_fits<TT, M_, C_>() : gsa_fwd_fits<TT, M_, C_>();
  GSA_FIT(bf16, 32, 32) GSA_FIT(bf16, 32, 64) GSA_FIT(bf16, 64, 32) GSA_FIT(bf16, 64, 64)
  GSA_FIT(bf16, 128, 32) GSA_FIT(bf16, 128, 64)
  GSA_FIT(float, 32, 32) GSA_FIT(float, 32, 64) GSA_FIT(float, 64, 32) GSA_FIT(float, 64, 64)
  GSA_FIT(float, 128, 32) GSA_FIT(float, 128, 64)
#undef GSA_FIT
  return ok;
}

#define GSA_INST(TT, M_, C_)                                                          \
  template hipError_t launch_gsa_fwd<TT, M_, C_>(const GsaParams&, hipStream_t); \
  template hipError_t launch_gsa_bwd<TT, M_, C_>(const GsaParams&, hipStream_t);
GSA_INST(bf16, 32, 32) GSA_INST(bf16, 32, 64) GSA_INST(bf16, 64, 32) GSA_INST(bf16, 64, 64)
GSA_INST(bf16, 128, 32) GSA_INST(bf16, 128, 64)
GSA_INST(float, 32, 32) GSA_INST(float, 32, 64) GSA_INST(float, 64, 32) GSA_INST(float, 64, 64)
GSA_INST(float, 128, 32) GSA_INST(float, 128, 64)

}  // namespace gla
