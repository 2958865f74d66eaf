// gla_bwd.hip -- chunkwise GLA backward on gfx950.
//
// Gradients of sum(o * do) + sum(ht * dht), recomputing everything from the forward inputs.
// With Qs = q 2^b, Ks = k 2^-b, Kd = k 2^{Gamma-b} (prep.hpp), H_n the state at the start of
// chunk n and dH_{n+1} the gradient of the state at its end, per chunk:
//   dA  = mask(dO V^T)
//   dq  = 2^b     * (dA Ks + dO H_n^T)
//   dk  = 2^-b    * (dA^T Qs) + 2^{Gamma-b} * (V dH_{n+1}^T)
//   dv  = A^T dO + Kd dH_{n+1}
//   dH_n = Diag(2^{Gamma_n}) dH_{n+1} + Qs_n^T dO_n,   dH_N = dht,  dh0 = dH_0
// The gate gradient.  q_t only appears as q_t 2^{G_t} and k_t only as k_t 2^{-G_t} (G the
// prefix sum of g), so dg_t = sum_{s >= t} (q_s dq_s - k_s dk_s) (+ rowsum(dht * ht)).  Taken
// literally that sum cancels: its diagonal intra-chunk terms (q_s dA_ss k_s - k_s dA_ss q_s)
// and the state-update terms cancel exactly in exact arithmetic, and when the true dg is
// small (strong forgetting, a tiny initial state) the rounding left over from those
// cancelling O(1) terms would dominate.  The kernels therefore evaluate the same quantity
// with every exactly-cancelling pair removed.  For t in chunk n:
//   dg_t = sum_{s >= t, s in n} (q_s dq^nd_s - k_s dk'_s)  +  sum_{c < t, c in n} k_c B_c  +  Z_n
// where dq^nd = dq minus its diagonal term (dA_ss k_s), dk' = the strictly-upper intra part
// of dk, B_c = 2^{Gamma - b_c} (V dH_{n+1}^T)_c (the inter part of dk), and
// Z_n = 2^{Gamma_n} rowsum(dH_{n+1} * H_n) is the gradient through the chunk's state decay
// (everything beyond the chunk is folded into dH_{n+1}).  Every surviving term carries the
// decay factors that contain alpha_t, so its rounding scales with dg itself.  The chunk
// kernel forms Z_n from the H_n and dH_{n+1} tiles it stages anyway, and does the two
// in-chunk prefix sums.
//
// Launches:
//   1. gla_prep_kernel                                        grid N x BH
//   2. walk_store: forward state walk storing H_n               grid ceil(Dv/64) * BH
//   3. walk_reverse: reverse walk storing dH_{n+1}              grid ceil(Dv/64) * BH
//      (walks.hpp; state slices in fp32 MFMA accumulators)
//   4. gla_bwd_chunk: dA, dq, dk (+ dv when the whole key width fits one workgroup) on MFMA
//      over 64-column slices of Dv, then an element-wise epilogue (gate scaling, diagonal
//      terms, Z_n, the two in-chunk prefix sums of dg) with 16-byte stores
//                               N x BH x (Dk slices) tiles over a persistent grid, one per CU
//   5. gla_bwd_dv (only when dv did not fit step 4)           grid N x BH
// Intra-chunk terms use the factorised form only on chunks whose gate span passes the same
// check as the forward; other chunks form them exactly, element by element, in fp32.
#include "walks.hpp"

namespace gla {

// ======================================================================= chunk gradients
// The chunk-gradient kernel runs 512 threads (8 waves): one workgroup fills a CU's LDS, and
// two waves per SIMD let one wave's LDS and matrix-core latencies hide behind the other's.
constexpr int kBwdThreads = 512;

// LDS phases of the chunk kernel:
//   front   sdA [CP][CP] (written after the Dv loop, read to the end), diag of dA (fp32)
//   phase 1 (Dv loop)    sKd, sA (with dv) and the Dv slice tiles dO, V, H, dH
//   phase 2 (intra)      Qs, Ks [CP][DKS] for the intra-chunk products
//   phase 3 (epilogue)   three fp32 [CP][DKS] gradient tiles; on the exact path b takes the
//                        place of the (unused) intra dk tile
constexpr size_t chunk_bwd_bytes(int es, int DKS, int CP, bool dv, int nseg) {   // nseg for kBwdThreads
  const size_t V = 16 / es;
  const size_t LDQ = DKS + 2 * V, LDC = CP + 2 * V, LDV = kDvTile + 2 * V, LDF = DKS + 4;
  const size_t QT = CP * LDQ * es, CT = CP * LDC * es, VT = CP * LDV * es, HT = DKS * LDV * es;
  const size_t FT = CP * LDF * 4;
  const size_t ph1 = (dv ? QT + CT : 0) + 2 * VT + 2 * HT;
  const size_t ph2 = 2 * QT;
  const size_t ph3 = 3 * FT;
  const size_t mx = ph1 > ph2 ? (ph1 > ph3 ? ph1 : ph3) : (ph2 > ph3 ? ph2 : ph3);
  return CT + mx + (size_t)(2 * nseg * DKS + 2 * DKS + CP + 8) * 4;
}

template <typename T, int DKS, int CP, bool WITH_DV>
struct BwdChunkCfg {
  static constexpr int NT = kBwdThreads;
  using M = ChunkMap<T, DKS, CP, NT>;
  static constexpr int V = 16 / (int)sizeof(T);
  // 32-byte row pads: the four rows a transposing LDS read touches per 16 lanes then fall in
  // disjoint bank windows, which the 16-byte pads of the other kernels do not give here
  static constexpr int LDQ = DKS + 2 * V, LDC = CP + 2 * V, LDV = kDvTile + 2 * V, LDF = DKS + 4;
  static constexpr size_t QT = (size_t)CP * LDQ * sizeof(T);
  static constexpr size_t CT = (size_t)CP * LDC * sizeof(T);
  static constexpr size_t VT = (size_t)CP * LDV * sizeof(T);
  static constexpr size_t HT = (size_t)DKS * LDV * sizeof(T);
  static constexpr size_t FT = (size_t)CP * LDF * 4;
  static constexpr size_t PH1 = (WITH_DV ? QT + CT : 0) + 2 * VT + 2 * HT;
  static constexpr size_t PH2 = 2 * QT;
  static constexpr size_t PH3 = 3 * FT;
  static constexpr size_t MAIN = CT + cmax(cmax(PH1, PH2), PH3);
  static constexpr size_t BYTES = chunk_bwd_bytes(sizeof(T), DKS, CP, WITH_DV, M::NSEG);
  static constexpr int NV = CP * kDvTile / V, NH = DKS * kDvTile / V;
  static constexpr int PV = (NV + NT - 1) / NT, PH = (NH + NT - 1) / NT;
};

// One 64-column Dv slice of dO, V (chunk rows) and of H_n, dH_{n+1} (key rows) in flight.
// Loads are unconditional from clamped in-bounds addresses; each vector's validity is kept
// beside it and applied once the data is used, so no branch or register rewrite touches a
// load in flight and the next slice's loads overlap the current slice's matrix work.
// where the chunk kernel's lanes outside a ragged chunk or the value width write their dv
__device__ __attribute__((aligned(16))) char g_dv_sink[16];

template <typename T, int DKS, int CP, bool WITH_DV>
struct SliceStage {
  using Cf = BwdChunkCfg<T, DKS, CP, WITH_DV>;
  typedef typename V16<T>::type VT;
  VT dov[Cf::PV], vv[Cf::PV], hv[Cf::PH], dhv[Cf::PH];
  bool vok[Cf::PV], hok[Cf::PH];

  // dog/vg: rows of this chunk ([len][Dv]); hs/dhs: [DKS rows][DVP] state tiles of this chunk
  __device__ __forceinline__ void load(const T* dog, const T* vg, const T* hs, const T* dhs, int len, int Dv,
                                       int DVP, int js, int kvalid, int tid) {
    constexpr int PER_ROW = kDvTile / Cf::V;
#pragma unroll
    for (int m = 0; m < Cf::PV; ++m) {
      const int idx = tid + Cf::NT * m;
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * Cf::V;
      const int jj = js * kDvTile + c;
      vok[m] = idx < Cf::NV && r < len && jj < Dv;
      const size_t off = (size_t)min(r, len - 1) * Dv + min(jj, Dv - Cf::V);
      dov[m] = *reinterpret_cast<const VT*>(dog + off);
      vv[m] = *reinterpret_cast<const VT*>(vg + off);
    }
#pragma unroll
    for (int m = 0; m < Cf::PH; ++m) {
      const int idx = tid + Cf::NT * m;
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * Cf::V;
      hok[m] = idx < Cf::NH && r < kvalid;
      const size_t off = (size_t)min(r, kvalid - 1) * DVP + js * kDvTile + c;
      hv[m] = *reinterpret_cast<const VT*>(hs + off);
      dhv[m] = *reinterpret_cast<const VT*>(dhs + off);
    }
  }
  // z[m] += this thread's share of rowsum(H * dH) for the state tile it stages
  __device__ __forceinline__ void zdot(float (&z)[Cf::PH], bool take = true) const {
#pragma unroll
    for (int m = 0; m < Cf::PH; ++m) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < Cf::V; ++e) t += to_f32(hv[m][e]) * to_f32(dhv[m][e]);
      z[m] += hok[m] && take ? t : 0.f;
    }
  }
  __device__ __forceinline__ void store(T* sdO, T* sV, T* sH, T* sdH, int tid) const {
    constexpr int PER_ROW = kDvTile / Cf::V;
#pragma unroll
    for (int m = 0; m < Cf::PV; ++m) {
      const int idx = tid + Cf::NT * m;
      if (idx < Cf::NV) {
        const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * Cf::V;
        *reinterpret_cast<VT*>(sdO + r * Cf::LDV + c) = vok[m] ? dov[m] : zero_vec<T>();
        *reinterpret_cast<VT*>(sV + r * Cf::LDV + c) = vok[m] ? vv[m] : zero_vec<T>();
      }
    }
#pragma unroll
    for (int m = 0; m < Cf::PH; ++m) {
      const int idx = tid + Cf::NT * m;
      if (idx < Cf::NH) {
        const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * Cf::V;
        *reinterpret_cast<VT*>(sH + r * Cf::LDV + c) = hok[m] ? hv[m] : zero_vec<T>();
        *reinterpret_cast<VT*>(sdH + r * Cf::LDV + c) = hok[m] ? dhv[m] : zero_vec<T>();
      }
    }
  }
};

// The chunk's A tile [CP][CP] in flight to LDS (16-byte vectors, issued early).
template <typename T, int CP, int NT>
struct ATileStage {
  static constexpr int V = 16 / (int)sizeof(T), N = CP * CP / V, P = (N + NT - 1) / NT;
  typedef typename V16<T>::type VT;
  VT a[P];
  __device__ __forceinline__ void load(const T* src, int tid) {
#pragma unroll
    for (int m = 0; m < P; ++m) a[m] = *reinterpret_cast<const VT*>(src + (size_t)min(tid + NT * m, N - 1) * V);
  }
  __device__ __forceinline__ void store(T* dst, int lds, int tid) const {
#pragma unroll
    for (int m = 0; m < P; ++m) {
      const int idx = tid + NT * m;
      if (idx < N) {
        const int r = idx / (CP / V), c = (idx - r * (CP / V)) * V;
        *reinterpret_cast<VT*>(dst + r * lds + c) = a[m];
      }
    }
  }
};

// Where tile t of the chunk kernel lies.  With the whole key width in one tile (NS = 1):
// chunk fastest, then b*h.  With NS key-width slices, the slices of one chunk are 8 tiles
// apart: workgroups are dealt to the 8 XCDs in turn, so the persistent grid's workgroups w and
// w + 8 sit on one XCD and take their tiles at the same time; a chunk's dO and V rows, which
// every slice reads, then come from HBM once and from that XCD's L2 for the other slices.
struct BwdTile {
  int n, bh, ch0, row0, len, kvalid;
  size_t chunk, qbase, vbase;
  __device__ __forceinline__ BwdTile(const BwdParams& p, int t, int DKS, int NS) {
    const int nc = p.N * p.BH, whole = nc / 8 * 8;
    int c = t, s = 0;
    if (NS > 1) {
      if (t < whole * NS) {               // groups of 8 chunks: tile 8 (NS a + s) + x
        const int x = t % 8, r = t / 8;
        s = r % NS;
        c = (r / NS) * 8 + x;
      } else {                            // the last nc % 8 chunks, slice by slice
        const int u = t - whole * NS, rem = nc - whole;
        s = u / rem;
        c = whole + u % rem;
      }
    }
    n = c % p.N;
    bh = c / p.N;
    ch0 = s * DKS;
    row0 = n * p.C;
    len = min(p.C, p.L - row0);
    kvalid = min(DKS, p.Dk - ch0);
    chunk = (size_t)bh * p.N + n;
    qbase = ((size_t)bh * p.L + row0) * p.Dk + ch0;
    vbase = ((size_t)bh * p.L + row0) * p.Dv;
  }
};

// RD: GSA's pass 2 with the read-out's backward in the epilogue (p.dz, p.rd, p.dzs, p.act set);
// a separate instance, so that the plain GLA backward carries none of its registers
template <typename T, int DKS, int CP, bool WITH_DV, bool RD>
__global__ __launch_bounds__(kBwdThreads) void gla_bwd_chunk(BwdParams p, int DKP, int ntile, int ntiles) {
  using Cf = BwdChunkCfg<T, DKS, CP, WITH_DV>;
  constexpr int NT = Cf::NT, NW = NT / 64;
  using M = ChunkMap<T, DKS, CP, NT>;
  constexpr int V = M::V, RPS = M::RPS, NSEG = M::NSEG;
  constexpr int LDQ = Cf::LDQ, LDC = Cf::LDC, LDV = Cf::LDV, LDF = Cf::LDF;
  constexpr int NBR = CP / 16, NIB = DKS / 16, NJB = kDvTile / 16;
  constexpr int NA_BLK = NBR * NBR, NQ_BLK = NBR * NIB, NV_BLK = NBR * NJB;
  constexpr int PA = (NA_BLK + NW - 1) / NW, PQ = (NQ_BLK + NW - 1) / NW, PVb = (NV_BLK + NW - 1) / NW;
  // Square blocking: where the [C][DKS] products split into 2 x 2 blocks per wave (two row blocks,
  // two key blocks) and dA into the same two row blocks, a wave reads two dO, two V, two H and two
  // dH fragments per k step for its eight products instead of four, four, one and one -- and
  // its dA blocks reuse the two dO fragments.  Otherwise a wave owns one key block and every row.
  constexpr bool SQ2 = NBR % 2 == 0 && NIB % 2 == 0 && (NBR / 2) * (NIB / 2) == NW && PQ == 4 && PA == 2 &&
                       NIB / 2 == NBR;
  // Row sharing: where a wave's dQ and dKI blocks are its row blocks rb0, rb0 + NW / NIB, ... of
  // one key block and its dA blocks the same row blocks of one column block (NIB == NBR), the
  // three products run in one k loop and read each dO and V row fragment once
  constexpr bool ROWS = !SQ2 && NIB == NBR && PQ == PA && NQ_BLK % NW == 0 && NW % NIB == 0 &&
                        NA_BLK % NW == 0;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) char smem[Cf::BYTES];
  T* sdA = reinterpret_cast<T*>(smem);                            // strictly lower dA
  char* rmain = smem + Cf::CT;
  // phase 1
  T* sKd = reinterpret_cast<T*>(rmain);                           // WITH_DV only
  T* sA = sKd + (WITH_DV ? CP * LDQ : 0);                         // WITH_DV only
  T* sdO = sA + (WITH_DV ? CP * LDC : 0);
  T* sV = sdO + CP * LDV;
  T* sH = sV + CP * LDV;
  T* sdH = sH + DKS * LDV;
  // phase 2 (aliases phase 1)
  T* sQs = reinterpret_cast<T*>(rmain);                           // q 2^b   [CP][DKS]
  T* sKs = sQs + CP * LDQ;                                        // k 2^-b
  // phase 3 (aliases phases 1 and 2)
  float* sDQ = reinterpret_cast<float*>(rmain);                   // dq^nd / 2^b
  float* sDK = sDQ + CP * LDF;                                    // dk'  / 2^-b (fast path)
  float* sDKI = sDK + CP * LDF;                                   // V dH^T
  float* sB = sDK;                                                // b [CP][DKS] (exact path)
  float* segtot = reinterpret_cast<float*>(smem + Cf::MAIN);      // [2][NSEG][DKS]
  float* sGam = segtot + 2 * NSEG * DKS;
  float* sZ = sGam + DKS;
  float* sDiag = sZ + DKS;
  float* red = sDiag + CP;

  const int Dk = p.Dk, Dv = p.Dv, L = p.L;
  const int DVP = ntile * kDvTile;
  int tid = threadIdx.x;

  // The grid is persistent: workgroup w takes tiles w, w + gridDim.x, ...  A tile's q, k and
  // g, which its gate scan waits for, go out during the previous tile's epilogue, which leaves
  // HBM idle otherwise; the first tile's go out here.
  ChunkScan<T, DKS, CP, true, NT> cs;
  auto issue = [&](const BwdTile& u) {
    cs.load(reinterpret_cast<const T*>(p.q) + u.qbase, reinterpret_cast<const T*>(p.k) + u.qbase,
            reinterpret_cast<const T*>(p.g) + u.qbase, Dk, Dk - u.ch0, u.len, tid);
  };
  int t = blockIdx.x;
  issue(BwdTile(p, t, DKS, DKP / DKS));
  for (;;) {
    tid = opaque_thread_index();  // per-lane addresses are formed anew for each tile
    const int wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
    // block s of this wave's [C][DKS] products and of its dA (rows rb, key or column block)
    const int rp = wave / (NIB > 1 ? NIB / 2 : 1), ip = wave % (NIB > 1 ? NIB / 2 : 1);   // SQ2 only
    auto q_rb = [&](int s) { return SQ2 ? 2 * rp + (s >> 1) : (wave + NW * s) / NIB; };
    auto q_ib = [&](int s) { return SQ2 ? 2 * ip + (s & 1) : (wave + NW * s) % NIB; };
    auto a_rb = [&](int s) { return SQ2 ? 2 * rp + s : (wave + NW * s) / NBR; };
    auto a_cb = [&](int s) { return SQ2 ? ip : (wave + NW * s) % NBR; };
    const BwdTile tile(p, t, DKS, DKP / DKS);
    const int tn = t + gridDim.x;  // this workgroup's next tile
    const int ch0 = tile.ch0, row0 = tile.row0, len = tile.len, kvalid = tile.kvalid;
    const size_t chunk = tile.chunk, qbase = tile.qbase;
    const T* qg = reinterpret_cast<const T*>(p.q) + qbase;
    const T* kg = reinterpret_cast<const T*>(p.k) + qbase;
    const T* dog = reinterpret_cast<const T*>(p.do_) + tile.vbase;
    const T* vg = reinterpret_cast<const T*>(p.v) + tile.vbase;
    // dv goes out straight from the accumulators, four consecutive columns of one row per lane;
    // a lane outside the chunk or the value width writes to a sink instead, so that every lane
    // stores and the wait for the next slice's loads can leave these stores in flight
    typedef typename Vec4<T>::type DV4;
    auto dv_dst = [&](int r, int c) -> DV4* {
      T* dvg = reinterpret_cast<T*>(p.dv) + tile.vbase;
      return r < len && c < Dv ? reinterpret_cast<DV4*>(dvg + (size_t)r * Dv + c) : reinterpret_cast<DV4*>(g_dv_sink);
    };
    const T* hs = reinterpret_cast<const T*>(p.Hs) + (chunk * DKP + ch0) * DVP;
    const T* dhs = reinterpret_cast<const T*>(p.dHs) + (chunk * DKP + ch0) * DVP;
    // the first Dv slice and (with dv) the chunk's A tile load while the gates are scanned
    SliceStage<T, DKS, CP, WITH_DV> st;
    st.load(dog, vg, hs, dhs, len, Dv, DVP, 0, kvalid, tid);
    ATileStage<T, CP, NT> at;
    if constexpr (WITH_DV) at.load(reinterpret_cast<const T*>(p.ops.A) + chunk * CP * CP, tid);
    const float maxb = cs.finish(segtot, sGam, red, tid);
    cs.kvals();                            // q is converted after the Dv loop, where it is first needed
    const bool fast = maxb <= kSpanLimit;
    const int c0 = cs.cg * V, r0 = cs.seg * RPS;

    if constexpr (WITH_DV) {
      if (cs.active) {
#pragma unroll
        for (int u = 0; u < RPS; ++u) {
          VT kd;
#pragma unroll
          for (int e = 0; e < V; ++e) kd[e] = from_f32<T>(cs.kv[u][e] * fast_exp2(sGam[c0 + e] - cs.b[u][e]));
          *reinterpret_cast<VT*>(sKd + (r0 + u) * LDQ + c0) = kd;
        }
      }
      at.store(sA, LDC, tid);
    }
    float zp[Cf::PH];
#pragma unroll
    for (int m = 0; m < Cf::PH; ++m) zp[m] = 0.f;
    st.zdot(zp);
    st.store(sdO, sV, sH, sdH, tid);
    __syncthreads();

    // The accumulators hold their blocks transposed (the products are formed with the operands
    // swapped), so a lane owns four consecutive columns of one row and moves them to LDS with a
    // single 8- or 16-byte write
    f32x4 accA[PA], accQ[PQ], accK[PQ], accKI[PQ];
#pragma unroll
    for (int s = 0; s < PA; ++s) accA[s] = zero4();
#pragma unroll
    for (int s = 0; s < PQ; ++s) accQ[s] = accK[s] = accKI[s] = zero4();

    for (int js = 0; js < ntile; ++js) {
      st.load(dog, vg, hs, dhs, len, Dv, DVP, min(js + 1, ntile - 1), kvalid, tid);   // last: harmless reload
      // Where every wave owns the same number of blocks, its blocks of one product share one
      // operand block (dA: the V block, dQ and dKI: the H and dH blocks, dV: the dO and dH
      // column blocks), which is then read from LDS once per k step instead of once per block.
      // Each accumulator still sums its k steps in the same order.
      if constexpr (SQ2) {                 // dA += dO V^T ; dQ += dO H^T ; dKI += V dH^T
#pragma unroll
        for (int kb = 0; kb < kDvTile / 32; ++kb) {
          const int ko = 32 * kb + 8 * grp;
          const Frag<T> o0 = ld8(sdO + (32 * rp + col) * LDV + ko), o1 = ld8(sdO + (32 * rp + 16 + col) * LDV + ko);
          const Frag<T> v0 = ld8(sV + (32 * rp + col) * LDV + ko), v1 = ld8(sV + (32 * rp + 16 + col) * LDV + ko);
          const Frag<T> h0 = ld8(sH + (32 * ip + col) * LDV + ko), h1 = ld8(sH + (32 * ip + 16 + col) * LDV + ko);
          const Frag<T> d0 = ld8(sdH + (32 * ip + col) * LDV + ko), d1 = ld8(sdH + (32 * ip + 16 + col) * LDV + ko);
          const Frag<T> vc = ld8(sV + (16 * ip + col) * LDV + ko);
          mma(accA[0], vc, o0);
          mma(accA[1], vc, o1);
          mma(accQ[0], h0, o0);
          mma(accQ[1], h1, o0);
          mma(accQ[2], h0, o1);
          mma(accQ[3], h1, o1);
          mma(accKI[0], d0, v0);
          mma(accKI[1], d1, v0);
          mma(accKI[2], d0, v1);
          mma(accKI[3], d1, v1);
        }
      } else if constexpr (ROWS) {          // dA += dO V^T ; dQ += dO H^T ; dKI += V dH^T
        const int ib = wave % NIB, rb0 = wave / NIB;
#pragma unroll
        for (int kb = 0; kb < kDvTile / 32; ++kb) {
          const int ko = 32 * kb + 8 * grp;
          const Frag<T> fh = ld8(sH + (16 * ib + col) * LDV + ko);
          const Frag<T> fdh = ld8(sdH + (16 * ib + col) * LDV + ko);
          const Frag<T> vc = ld8(sV + (16 * ib + col) * LDV + ko);     // dA's column block is ib
#pragma unroll
          for (int s = 0; s < PQ; ++s) {
            const int o = (16 * (rb0 + (NW / NIB) * s) + col) * LDV + ko;
            const Frag<T> fo = ld8(sdO + o);
            mma(accA[s], vc, fo);
            mma(accQ[s], fh, fo);
            mma(accKI[s], fdh, ld8(sV + o));
          }
        }
      } else if constexpr (NA_BLK % NW == 0 && NW % NBR == 0) {   // dA += dO V^T
        const int cb = wave % NBR, rb0 = wave / NBR;
#pragma unroll
        for (int kb = 0; kb < kDvTile / 32; ++kb) {
          const Frag<T> fv = ld8(sV + (16 * cb + col) * LDV + 32 * kb + 8 * grp);
#pragma unroll
          for (int s = 0; s < PA; ++s)
            mma(accA[s], fv, ld8(sdO + (16 * (rb0 + (NW / NBR) * s) + col) * LDV + 32 * kb + 8 * grp));
        }
      } else {
#pragma unroll
        for (int s = 0; s < PA; ++s) {       // dA += dO V^T
          const int blk = wave + NW * s;
          if (blk < NA_BLK) {
            const int rb = blk / NBR, cb = blk % NBR;
#pragma unroll
            for (int kb = 0; kb < kDvTile / 32; ++kb)
              mma(accA[s], ld8(sV + (16 * cb + col) * LDV + 32 * kb + 8 * grp), ld8(sdO + (16 * rb + col) * LDV + 32 * kb + 8 * grp));
          }
        }
      }
      if constexpr (SQ2 || ROWS) {
        // done above
      } else if constexpr (NQ_BLK % NW == 0 && NW % NIB == 0) {   // dQ += dO H^T ; dKI += V dH^T
        const int ib = wave % NIB, rb0 = wave / NIB;
#pragma unroll
        for (int kb = 0; kb < kDvTile / 32; ++kb) {
          const Frag<T> fh = ld8(sH + (16 * ib + col) * LDV + 32 * kb + 8 * grp);
          const Frag<T> fdh = ld8(sdH + (16 * ib + col) * LDV + 32 * kb + 8 * grp);
#pragma unroll
          for (int s = 0; s < PQ; ++s) {
            const int o = (16 * (rb0 + (NW / NIB) * s) + col) * LDV + 32 * kb + 8 * grp;
            mma(accQ[s], fh, ld8(sdO + o));
            mma(accKI[s], fdh, ld8(sV + o));
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < PQ; ++s) {       // dQ += dO H^T ; dKI += V dH^T
          const int blk = wave + NW * s;
          if (blk < NQ_BLK) {
            const int rb = blk / NIB, ib = blk % NIB;
#pragma unroll
            for (int kb = 0; kb < kDvTile / 32; ++kb) {
              mma(accQ[s], ld8(sH + (16 * ib + col) * LDV + 32 * kb + 8 * grp), ld8(sdO + (16 * rb + col) * LDV + 32 * kb + 8 * grp));
              mma(accKI[s], ld8(sdH + (16 * ib + col) * LDV + 32 * kb + 8 * grp), ld8(sV + (16 * rb + col) * LDV + 32 * kb + 8 * grp));
            }
          }
        }
      }
      if constexpr (WITH_DV) {             // dV = A^T dO + Kd dH for this slice
        if constexpr (NV_BLK % NW == 0 && NW % NJB == 0) {
          const int jb = wave % NJB, cb0 = wave / NJB;
          f32x4 acc[PVb];
#pragma unroll
          for (int s = 0; s < PVb; ++s) acc[s] = zero4();
#pragma unroll
          for (int kr = 0; kr < CP / 32; ++kr) {
            const Frag<T> fo = ld8_colblk(sdO + (32 * kr) * LDV + 16 * jb, LDV, lane);
#pragma unroll
            for (int s = 0; s < PVb; ++s)
              mma(acc[s], fo, ld8_colblk(sA + (32 * kr) * LDC + 16 * (cb0 + (NW / NJB) * s), LDC, lane));
          }
#pragma unroll
          for (int ki = 0; ki < DKS / 32; ++ki) {
            const Frag<T> fd = ld8_colblk(sdH + (32 * ki) * LDV + 16 * jb, LDV, lane);
#pragma unroll
            for (int s = 0; s < PVb; ++s)
              mma(acc[s], fd, ld8(sKd + (16 * (cb0 + (NW / NJB) * s) + col) * LDQ + 32 * ki + 8 * grp));
          }
#pragma unroll
          for (int s = 0; s < PVb; ++s) {
            // transposed block: this lane holds dV[16 cb + col][16 jb + 4 grp + e]
            const int cb = cb0 + (NW / NJB) * s;
            typename Vec4<T>::type dv4;
#pragma unroll
            for (int e = 0; e < 4; ++e) dv4[e] = from_f32<T>(acc[s][e]);
            *dv_dst(16 * cb + col, js * kDvTile + 16 * jb + 4 * grp) = dv4;
          }
        } else {
#pragma unroll
          for (int s = 0; s < PVb; ++s) {
            const int blk = wave + NW * s;
            if (blk < NV_BLK) {
              const int cb = blk / NJB, jb = blk % NJB;
              f32x4 acc = zero4();
#pragma unroll
              for (int kr = 0; kr < CP / 32; ++kr)
                mma(acc, ld8_colblk(sdO + (32 * kr) * LDV + 16 * jb, LDV, lane),
                    ld8_colblk(sA + (32 * kr) * LDC + 16 * cb, LDC, lane));
#pragma unroll
              for (int ki = 0; ki < DKS / 32; ++ki)
                mma(acc, ld8_colblk(sdH + (32 * ki) * LDV + 16 * jb, LDV, lane),
                    ld8(sKd + (16 * cb + col) * LDQ + 32 * ki + 8 * grp));
              // transposed block: this lane holds dV[16 cb + col][16 jb + 4 grp + e]
              typename Vec4<T>::type dv4;
#pragma unroll
              for (int e = 0; e < 4; ++e) dv4[e] = from_f32<T>(acc[e]);
              *dv_dst(16 * cb + col, js * kDvTile + 16 * jb + 4 * grp) = dv4;
            }
          }
        }
      }
      __syncthreads();
      // The next slice is staged on every path: after the last slice the reloaded copy goes to
      // LDS that the intra phase overwrites, and adds nothing to Z.  Its loads are older than
      // this slice's dv stores, so the wait for them leaves the stores in flight.
      st.zdot(zp, js + 1 < ntile);
      st.store(sdO, sV, sH, sdH, tid);
      __syncthreads();
    }
    // GSA's pass 2 with the read-out's backward fused: the read-out's input (fp32) for the
    // epilogue, in flight through the intra phase
    f32x4 rdl[RPS][V / 4];
    if constexpr (RD) {
      const int cc = (cs.active && c0 < kvalid) ? c0 : 0;
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
        const float* src = p.rd + qbase + (size_t)min(r0 + u, len - 1) * Dk + cc;
#pragma unroll
        for (int e4 = 0; e4 < V / 4; ++e4) rdl[u][e4] = *reinterpret_cast<const f32x4*>(src + 4 * e4);
      }
    }
    {  // Z_n = 2^Gamma rowsum(dH_{n+1} * H_n): reduce over the lanes that staged one state row
      constexpr int PER_ROW = kDvTile / V;
#pragma unroll
      for (int m = 0; m < Cf::PH; ++m) {
        float z = zp[m];
#pragma unroll
        for (int off = 1; off < PER_ROW; off <<= 1) z += __shfl_xor(z, off, 64);
        const int idx = tid + NT * m, r = idx / PER_ROW;
        if (idx < Cf::NH && idx % PER_ROW == 0) sZ[r] = r < kvalid ? z * fast_exp2(sGam[r]) : 0.f;
      }
    }

    cs.qvals();

    // strictly lower dA -> LDS, the diagonal kept apart in fp32; on the factorised path also
    // Qs and Ks (the phase-1 tiles are dead here).  The intra products read dA^T, Qs^T and Ks^T
    // as column runs of these tiles through transposing LDS reads.
#pragma unroll
    for (int s = 0; s < PA; ++s) {
      if (SQ2 || wave + NW * s < NA_BLK) {
        const int rb = a_rb(s), cb = a_cb(s);
        // transposed block: this lane holds dA[16 rb + col][16 cb + 4 grp + e]
        const int r = 16 * rb + col;
        typename Vec4<T>::type a4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * cb + 4 * grp + e;
          a4[e] = from_f32<T>(c < r ? accA[s][e] : 0.f);
          if (c == r) sDiag[r] = accA[s][e];
        }
        *reinterpret_cast<typename Vec4<T>::type*>(sdA + r * LDC + 16 * cb + 4 * grp) = a4;
      }
    }
    if (fast && cs.active) {
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
        VT qs, ks;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          qs[e] = from_f32<T>(cs.qv[u][e] * fast_exp2(cs.b[u][e]));
          ks[e] = from_f32<T>(cs.kv[u][e] * fast_exp2(-cs.b[u][e]));
        }
        *reinterpret_cast<VT*>(sQs + (r0 + u) * LDQ + c0) = qs;
        *reinterpret_cast<VT*>(sKs + (r0 + u) * LDQ + c0) = ks;
      }
    }
    __syncthreads();
    if (fast) {                            // off-diagonal intra terms on MFMA
      if constexpr (SQ2) {
        // the wave's two key blocks' Ks and Qs column blocks and its two row blocks' dA rows
        // and dA columns, each read once per k step
#pragma unroll
        for (int kc = 0; kc < CP / 32; ++kc) {
          const Frag<T> ks0 = ld8_colblk(sKs + (32 * kc) * LDQ + 32 * ip, LDQ, lane);
          const Frag<T> ks1 = ld8_colblk(sKs + (32 * kc) * LDQ + 32 * ip + 16, LDQ, lane);
          const Frag<T> qs0 = ld8_colblk(sQs + (32 * kc) * LDQ + 32 * ip, LDQ, lane);
          const Frag<T> qs1 = ld8_colblk(sQs + (32 * kc) * LDQ + 32 * ip + 16, LDQ, lane);
          const Frag<T> ar0 = ld8(sdA + (32 * rp + col) * LDC + 32 * kc + 8 * grp);
          const Frag<T> ar1 = ld8(sdA + (32 * rp + 16 + col) * LDC + 32 * kc + 8 * grp);
          const Frag<T> ac0 = ld8_colblk(sdA + (32 * kc) * LDC + 32 * rp, LDC, lane);
          const Frag<T> ac1 = ld8_colblk(sdA + (32 * kc) * LDC + 32 * rp + 16, LDC, lane);
          mma(accQ[0], ks0, ar0);
          mma(accQ[1], ks1, ar0);
          mma(accQ[2], ks0, ar1);
          mma(accQ[3], ks1, ar1);
          mma(accK[0], qs0, ac0);
          mma(accK[1], qs1, ac0);
          mma(accK[2], qs0, ac1);
          mma(accK[3], qs1, ac1);
        }
      } else if constexpr (NQ_BLK % NW == 0 && NW % NIB == 0) {
        // as in the slice loop: the key block ib is fixed per wave, so its Ks and Qs column
        // blocks are read once per k step
        const int ib = wave % NIB, rb0 = wave / NIB;
#pragma unroll
        for (int kc = 0; kc < CP / 32; ++kc) {
          const Frag<T> fks = ld8_colblk(sKs + (32 * kc) * LDQ + 16 * ib, LDQ, lane);
          const Frag<T> fqs = ld8_colblk(sQs + (32 * kc) * LDQ + 16 * ib, LDQ, lane);
#pragma unroll
          for (int s = 0; s < PQ; ++s) {
            const int rb = rb0 + (NW / NIB) * s;
            mma(accQ[s], fks, ld8(sdA + (16 * rb + col) * LDC + 32 * kc + 8 * grp));
            mma(accK[s], fqs, ld8_colblk(sdA + (32 * kc) * LDC + 16 * rb, LDC, lane));
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < PQ; ++s) {
          const int blk = wave + NW * s;
          if (blk < NQ_BLK) {
            const int rb = blk / NIB, ib = blk % NIB;
#pragma unroll
            for (int kc = 0; kc < CP / 32; ++kc) {
              mma(accQ[s], ld8_colblk(sKs + (32 * kc) * LDQ + 16 * ib, LDQ, lane),
                  ld8(sdA + (16 * rb + col) * LDC + 32 * kc + 8 * grp));
              mma(accK[s], ld8_colblk(sQs + (32 * kc) * LDQ + 16 * ib, LDQ, lane),
                  ld8_colblk(sdA + (32 * kc) * LDC + 16 * rb, LDC, lane));
            }
          }
        }
      }
    }
    __syncthreads();                       // phase-1 tiles are dead from here on
#pragma unroll
    for (int s = 0; s < PQ; ++s) {
      if (SQ2 || wave + NW * s < NQ_BLK) {
        const int rb = q_rb(s), ib = q_ib(s);
        const int o = (16 * rb + col) * LDF + 16 * ib + 4 * grp;   // four consecutive channels
        *reinterpret_cast<f32x4*>(sDQ + o) = accQ[s];
        if (fast) *reinterpret_cast<f32x4*>(sDK + o) = accK[s];
        *reinterpret_cast<f32x4*>(sDKI + o) = accKI[s];
      }
    }
    if (!fast && cs.active) {
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
#pragma unroll
        for (int e = 0; e < V; ++e) sB[(r0 + u) * DKS + c0 + e] = cs.b[u][e];
      }
    }
    // q, k and g of this tile are in registers as fp32 from here on: the next tile's go out.
    // Past the last tile the loads still go out, so that none is conditional, but read only
    // this tile's first row (cached) instead of a whole chunk.
    {
      BwdTile nx(p, tn < ntiles ? tn : t, DKS, DKP / DKS);
      if (tn >= ntiles) nx.len = 1;
      issue(nx);
    }
    __syncthreads();

    // ---- epilogue: dq, dk; dg from the two in-chunk prefix sums and Z
    float up[RPS][V], uk[RPS][V];          // q dq^nd - k dk'  (suffix-summed) ; k B (prefix-summed)
    if (cs.active) {
      T* dqg = reinterpret_cast<T*>(p.dq) + qbase;
      T* dkg = reinterpret_cast<T*>(p.dk) + qbase;
      // dq^nd and dk' per element; the path test is uniform and kept outside the element loops
      // so that the fast path's LDS reads issue together
      float dqn[RPS][V], dkp[RPS][V];
      if (fast) {
#pragma unroll
        for (int u = 0; u < RPS; ++u) {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const int o = (r0 + u) * LDF + c0 + e;
            dqn[u][e] = sDQ[o] * fast_exp2(cs.b[u][e]);
            dkp[u][e] = sDK[o] * fast_exp2(-cs.b[u][e]);
          }
        }
      } else {
        // exact off-diagonal intra terms: every exponent b_r - b_c has r > c
        const int cend = c0 < kvalid ? len : 0;            // padded channels: q = k = 0
#pragma unroll
        for (int u = 0; u < RPS; ++u) {
          const int r = r0 + u;
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const int i = c0 + e;
            const float bb = cs.b[u][e];
            float iq = 0.f, ik = 0.f;
            for (int c = 0; c < cend; ++c) {
              if (c < r) iq += to_f32(sdA[r * LDC + c]) * to_f32(kg[(size_t)c * Dk + i]) * fast_exp2(bb - sB[c * DKS + i]);
              if (c > r) ik += to_f32(sdA[c * LDC + r]) * to_f32(qg[(size_t)c * Dk + i]) * fast_exp2(sB[c * DKS + i] - bb);
            }
            dqn[u][e] = sDQ[r * LDF + i] * fast_exp2(bb) + iq;
            dkp[u][e] = ik;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
        const int r = r0 + u;
        const float dgn = sDiag[r];
        VT dkv;
        float dqf[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int i = c0 + e;
          const float bb = cs.b[u][e];
          const float bk = sDKI[r * LDF + i] * fast_exp2(sGam[i] - bb);
          const float qv = cs.qv[u][e], kv = cs.kv[u][e];
          dqf[e] = dqn[u][e] + dgn * kv;
          dkv[e] = from_f32<T>(dkp[u][e] + dgn * qv + bk);
          up[u][e] = qv * dqn[u][e] - kv * dkp[u][e];
          uk[u][e] = kv * bk;
        }
        if constexpr (RD) {
          // the read-out's backward: dq here is dP, the gradient of the read-out's output, and
          // dZ = P (dP - <dP, P>) over the row's slots for the softmax (the row's channel groups
          // are NCG consecutive lanes), else f'(Z) dP; dZ 2^b also goes out chunk-padded for
          // the pass-1 reverse walk
          const bool ok = r < len && c0 < kvalid;
          float rv[V], sdot = 0.f;
#pragma unroll
          for (int e = 0; e < V; ++e) {
            rv[e] = ok ? rdl[u][e >> 2][e & 3] : 0.f;
            sdot += rv[e] * dqf[e];
          }
#pragma unroll
          for (int o = 1; o < M::NCG; o <<= 1) sdot += __shfl_xor(sdot, o, 64);
          float dzv[V];
          VT zs;
#pragma unroll
          for (int e = 0; e < V; ++e) {
            dzv[e] = p.act == kActSoftmax ? rv[e] * (dqf[e] - sdot) : gsa_read_grad(rv[e], dqf[e], p.act);
            zs[e] = from_f32<T>(dzv[e] * fast_exp2(cs.b[u][e]));
          }
          *reinterpret_cast<VT*>(reinterpret_cast<T*>(p.dzs) + (chunk * CP + r) * DKP + ch0 + c0) = zs;
          if (ok) {
            float* d = p.dz + qbase + (size_t)r * Dk + c0;
#pragma unroll
            for (int e = 0; e < V; e += 4) *reinterpret_cast<f32x4*>(d + e) = f32x4{dzv[e], dzv[e + 1], dzv[e + 2], dzv[e + 3]};
          }
        }
        if (r < len && c0 < kvalid) {
          if constexpr (RD) {
            // dq itself is not kept
          } else if (p.dq32) {
            float* d32 = p.dq32 + qbase + (size_t)r * Dk + c0;
#pragma unroll
            for (int e = 0; e < V; e += 4) *reinterpret_cast<f32x4*>(d32 + e) = f32x4{dqf[e], dqf[e + 1], dqf[e + 2], dqf[e + 3]};
          } else {
            VT dqv;
#pragma unroll
            for (int e = 0; e < V; ++e) dqv[e] = from_f32<T>(dqf[e]);
            *reinterpret_cast<VT*>(dqg + (size_t)r * Dk + c0) = dqv;
          }
          *reinterpret_cast<VT*>(dkg + (size_t)r * Dk + c0) = dkv;
        }
      }
      // in-segment scans: inclusive suffix of up, exclusive prefix of uk
      float sp[V], sk[V];
#pragma unroll
      for (int e = 0; e < V; ++e) sp[e] = sk[e] = 0.f;
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
          const float x = uk[u][e];
          uk[u][e] = sk[e];
          sk[e] += x;
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        segtot[cs.seg * DKS + c0 + e] = sp[e];
        segtot[(NSEG + cs.seg) * DKS + c0 + e] = sk[e];
      }
    }
    __syncthreads();
    // later segments' suffix totals of u, earlier segments' prefix totals of y
    for (int t = tid; t < 2 * DKS; t += NT)
      seg_scan_channel<NSEG>(segtot + (t < DKS ? 0 : NSEG * DKS), DKS, t < DKS ? t : t - DKS, t < DKS);
    __syncthreads();
    if (cs.active) {
      float add[V];
#pragma unroll
      for (int e = 0; e < V; ++e)
        add[e] = sZ[c0 + e] + segtot[cs.seg * DKS + c0 + e] + segtot[(NSEG + cs.seg) * DKS + c0 + e];
      float* dgg = p.dg + qbase;
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
        const int r = r0 + u;
        if (r < len && c0 < kvalid) {
#pragma unroll
          for (int e = 0; e < V; e += 4) {
            f32x4 w;
#pragma unroll
            for (int x = 0; x < 4; ++x) w[x] = up[u][e + x] + uk[u][e + x] + add[e + x];
            *reinterpret_cast<f32x4*>(dgg + (size_t)r * Dk + c0 + e) = w;
          }
        }
      }
    }
    if (tn >= ntiles) break;
    t = tn;
    __syncthreads();                       // the next tile's scan reuses segtot, sGam and red
  }
  __builtin_amdgcn_s_waitcnt(0);         // the last tile's repeated loads have landed
}

// ======================================================================= dv (separate)
// When the chunk-gradient kernel splits the key width (it does when dv does not fit its LDS:
// Dk = 256, or C = 128), dv = A^T dO + Kd dH_{n+1} runs here.  One workgroup of 8 waves per
// (chunk, b*h) stages the chunk's A and KdT tiles once, from which each wave keeps the A^T and
// Kd fragments of its blocks in registers, and walks the 64-column Dv slices; each slice's dO
// and dH loads are in flight while the previous slice's products run, as in the chunk-gradient
// kernel.  Column operands are read with transposing LDS reads (tiles with 32-byte row pads),
// and the accumulators hold dV transposed, so that each lane stores four consecutive columns of
// a row straight to memory.
constexpr int kDvThreads = 512;

template <typename T, int DKP, int CP>
struct BwdDvCfg {
  static constexpr int NT = kDvThreads, NW = NT / 64;
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int LDC = CP + 2 * V, LDV = kDvTile + 2 * V;
  static constexpr size_t AT = (size_t)CP * LDC * sizeof(T);     // A   [CP][CP]
  static constexpr size_t KT = (size_t)DKP * LDC * sizeof(T);    // KdT [DKP][CP]
  static constexpr size_t OT = (size_t)CP * LDV * sizeof(T);     // dO slice [CP][64]
  static constexpr size_t HT = (size_t)DKP * LDV * sizeof(T);    // dH slice [DKP][64]
  static constexpr size_t BYTES = AT + KT + OT + HT;
  static constexpr int PER_ROW = kDvTile / V;
  static constexpr int NO = CP * PER_ROW, NH = DKP * PER_ROW;    // 16-byte vectors per slice
  static constexpr int PO = (NO + NT - 1) / NT, PH = (NH + NT - 1) / NT;
  static constexpr int NA = CP * CP / V, NK = DKP * CP / V;
  static constexpr int PA = (NA + NT - 1) / NT, PK = (NK + NT - 1) / NT;
  static constexpr int NBR = CP / 16, NJB = kDvTile / 16, PVB = NBR * NJB / NW;   // dV blocks per wave
  static_assert(NBR * NJB % NW == 0 && NW % NJB == 0, "every wave owns the same dV blocks of one column block");
};

// One Dv slice of dO (chunk rows) and dH_{n+1} (key rows) in flight: loads from clamped
// in-bounds addresses, validity kept beside them and applied when the slice goes to LDS.
template <typename T, int DKP, int CP>
struct DvSlice {
  using Cf = BwdDvCfg<T, DKP, CP>;
  typedef typename V16<T>::type VT;
  VT o[Cf::PO], h[Cf::PH];
  bool ook[Cf::PO];
  __device__ __forceinline__ void load(const T* dog, const T* dhs, int len, int Dv, int DVP, int js, int tid) {
#pragma unroll
    for (int m = 0; m < Cf::PO; ++m) {
      const int idx = tid + Cf::NT * m, r = idx / Cf::PER_ROW, c = (idx % Cf::PER_ROW) * Cf::V;
      const int jj = js * kDvTile + c;
      ook[m] = idx < Cf::NO && r < len && jj < Dv;
      o[m] = *reinterpret_cast<const VT*>(dog + (size_t)min(r, len - 1) * Dv + min(jj, Dv - Cf::V));
    }
#pragma unroll
    for (int m = 0; m < Cf::PH; ++m) {
      const int idx = min(tid + Cf::NT * m, Cf::NH - 1), r = idx / Cf::PER_ROW, c = (idx % Cf::PER_ROW) * Cf::V;
      h[m] = *reinterpret_cast<const VT*>(dhs + (size_t)r * DVP + js * kDvTile + c);
    }
  }
  __device__ __forceinline__ void store(T* sdO, T* sdH, int tid) const {
#pragma unroll
    for (int m = 0; m < Cf::PO; ++m) {
      const int idx = tid + Cf::NT * m, r = idx / Cf::PER_ROW, c = (idx % Cf::PER_ROW) * Cf::V;
      if (Cf::NO % Cf::NT == 0 || idx < Cf::NO) *reinterpret_cast<VT*>(sdO + r * Cf::LDV + c) = ook[m] ? o[m] : zero_vec<T>();
    }
#pragma unroll
    for (int m = 0; m < Cf::PH; ++m) {
      const int idx = tid + Cf::NT * m, r = idx / Cf::PER_ROW, c = (idx % Cf::PER_ROW) * Cf::V;
      if (Cf::NH % Cf::NT == 0 || idx < Cf::NH) *reinterpret_cast<VT*>(sdH + r * Cf::LDV + c) = h[m];
    }
  }
};

// grid N * BH: chunk n = blockIdx.x % N of sequence bh = blockIdx.x / N
template <typename T, int DKP, int CP>
__global__ __launch_bounds__(kDvThreads) void gla_bwd_dv(BwdParams p, int ntile) {
  using Cf = BwdDvCfg<T, DKP, CP>;
  constexpr int NT = Cf::NT, NW = Cf::NW, V = Cf::V, LDC = Cf::LDC, LDV = Cf::LDV;
  constexpr int NJB = Cf::NJB, PVB = Cf::PVB;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) char smem[Cf::BYTES];
  T* sA = reinterpret_cast<T*>(smem);
  T* sKdT = reinterpret_cast<T*>(smem + Cf::AT);
  T* sdO = reinterpret_cast<T*>(smem + Cf::AT + Cf::KT);
  T* sdH = reinterpret_cast<T*>(smem + Cf::AT + Cf::KT + Cf::OT);

  const int n = blockIdx.x % p.N, bh = blockIdx.x / p.N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int Dv = p.Dv, L = p.L;
  const int DVP = ntile * kDvTile;
  const int row0 = n * p.C, len = min(p.C, L - row0);
  const size_t chunk = (size_t)bh * p.N + n;
  const T* dhs = reinterpret_cast<const T*>(p.dHs) + chunk * DKP * DVP;
  const T* dog = reinterpret_cast<const T*>(p.do_) + ((size_t)bh * L + row0) * Dv;
  T* dvg = reinterpret_cast<T*>(p.dv) + ((size_t)bh * L + row0) * Dv;

  // the chunk's A and KdT tiles and the first slice, all in flight together
  const T* Ag = reinterpret_cast<const T*>(p.ops.A) + chunk * CP * CP;
  const T* Kg = reinterpret_cast<const T*>(p.ops.KdT) + chunk * DKP * CP;
  VT av[Cf::PA], kv[Cf::PK];
#pragma unroll
  for (int m = 0; m < Cf::PA; ++m) av[m] = *reinterpret_cast<const VT*>(Ag + (size_t)min(tid + NT * m, Cf::NA - 1) * V);
#pragma unroll
  for (int m = 0; m < Cf::PK; ++m) kv[m] = *reinterpret_cast<const VT*>(Kg + (size_t)min(tid + NT * m, Cf::NK - 1) * V);
  DvSlice<T, DKP, CP> st;
  st.load(dog, dhs, len, Dv, DVP, 0, tid);
#pragma unroll
  for (int m = 0; m < Cf::PA; ++m) {
    const int idx = tid + NT * m, r = idx / (CP / V), c = (idx % (CP / V)) * V;
    if (Cf::NA % NT == 0 || idx < Cf::NA) *reinterpret_cast<VT*>(sA + r * LDC + c) = av[m];
  }
#pragma unroll
  for (int m = 0; m < Cf::PK; ++m) {
    const int idx = tid + NT * m, r = idx / (CP / V), c = (idx % (CP / V)) * V;
    if (Cf::NK % NT == 0 || idx < Cf::NK) *reinterpret_cast<VT*>(sKdT + r * LDC + c) = kv[m];
  }
  st.store(sdO, sdH, tid);
  __syncthreads();

  // wave w owns column block jb = w % NJB of the slice and row blocks cb0 + (NW / NJB) s.  Its
  // A^T and Kd fragments are the same for every slice: they stay in registers, and each slice
  // reads only its dO and dH column fragments from LDS
  const int jb = wave % NJB, cb0 = wave / NJB;
  Frag<T> fa[CP / 32][PVB], fk[DKP / 32][PVB];
#pragma unroll
  for (int kr = 0; kr < CP / 32; ++kr) {
#pragma unroll
    for (int s = 0; s < PVB; ++s) fa[kr][s] = ld8_colblk(sA + (32 * kr) * LDC + 16 * (cb0 + (NW / NJB) * s), LDC, lane);
  }
#pragma unroll
  for (int ki = 0; ki < DKP / 32; ++ki) {
#pragma unroll
    for (int s = 0; s < PVB; ++s) fk[ki][s] = ld8_colblk(sKdT + (32 * ki) * LDC + 16 * (cb0 + (NW / NJB) * s), LDC, lane);
  }
  for (int js = 0; js < ntile; ++js) {
    st.load(dog, dhs, len, Dv, DVP, min(js + 1, ntile - 1), tid);   // last: harmless reload
    f32x4 acc[PVB];
#pragma unroll
    for (int s = 0; s < PVB; ++s) acc[s] = zero4();
#pragma unroll
    for (int kr = 0; kr < CP / 32; ++kr) {            // A^T dO
      const Frag<T> fo = ld8_colblk(sdO + (32 * kr) * LDV + 16 * jb, LDV, lane);
#pragma unroll
      for (int s = 0; s < PVB; ++s) mma(acc[s], fo, fa[kr][s]);
    }
#pragma unroll
    for (int ki = 0; ki < DKP / 32; ++ki) {           // Kd dH
      const Frag<T> fd = ld8_colblk(sdH + (32 * ki) * LDV + 16 * jb, LDV, lane);
#pragma unroll
      for (int s = 0; s < PVB; ++s) mma(acc[s], fd, fk[ki][s]);
    }
    // dv straight from the accumulators (this lane holds dV[16 cb + col][16 jb + 4 grp + e]);
    // lanes outside the chunk or the value width write to a sink, so every lane stores and the
    // wait for the next slice's loads, which are older, leaves these stores in flight
#pragma unroll
    for (int s = 0; s < PVB; ++s) {
      const int r = 16 * (cb0 + (NW / NJB) * s) + col, c = js * kDvTile + 16 * jb + 4 * grp;
      typename Vec4<T>::type dv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dv4[e] = from_f32<T>(acc[s][e]);
      *reinterpret_cast<typename Vec4<T>::type*>(r < len && c < Dv ? dvg + (size_t)r * Dv + c
                                                                   : reinterpret_cast<T*>(g_dv_sink)) = dv4;
    }
    __syncthreads();
    st.store(sdO, sdH, tid);
    __syncthreads();
  }
}

// ======================================================================= plan + launch
// Workgroups of the persistent chunk kernel that the device runs at once (CUs times the
// workgroups one CU holds), cached per device; 0 cannot happen (at least one per CU).
template <typename T, int DKS, int CP, bool WITH_DV, bool RD>
int bwd_chunk_slots() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gla_bwd_chunk<T, DKS, CP, WITH_DV, RD>, kBwdThreads, 0) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  const int cus = device_cu_count();
  const int n = (cus > 0 ? cus : 256) * per_cu;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Key-width slice of the chunk kernel: the whole key width with dv fused when it fits the
// LDS of a CU, otherwise slices of at most 128 channels with dv in its own kernel.
template <typename T, int DKP, int CP>
struct BwdPlan {
  static constexpr int es = sizeof(T);
  static constexpr int nseg(int dks) { return imin(kBwdThreads / (dks / (16 / es)), CP); }
  static constexpr bool fits(int dks, bool dv) { return chunk_bwd_bytes(es, dks, CP, dv, nseg(dks)) <= kMaxLds; }
  static constexpr bool FUSED = fits(DKP, true);
  static constexpr int DKS = FUSED ? DKP
                           : (DKP >= 128 && fits(128, false)) ? 128
                           : (DKP >= 64 && fits(64, false)) ? 64 : 32;
  static constexpr bool OK = (FUSED || fits(DKS, false)) && PrepCfg<T, DKP, CP>::BYTES <= kMaxLds &&
                             walk_fits<T, DKP, CP>() &&
                             (FUSED || BwdDvCfg<T, DKP, CP>::BYTES <= kMaxLds);
};

template <typename T, int DKP, int CP>
constexpr int bwd_key_slices() {
  return BwdPlan<T, DKP, CP>::OK ? DKP / BwdPlan<T, DKP, CP>::DKS : 0;
}

int gla_bwd_key_slices(int esize, int DKP, int CP) {
#define GLA_BWD_SLICES(TT, D, C_) \
  if (esize == (int)sizeof(TT) && DKP == D && CP == C_) return bwd_key_slices<TT, D, C_>();
  GLA_BWD_SLICES(bf16, 32, 32) GLA_BWD_SLICES(bf16, 32, 64) GLA_BWD_SLICES(bf16, 64, 32)
  GLA_BWD_SLICES(bf16, 64, 64) GLA_BWD_SLICES(bf16, 128, 32) GLA_BWD_SLICES(bf16, 128, 64)
  GLA_BWD_SLICES(float, 32, 32) GLA_BWD_SLICES(float, 32, 64) GLA_BWD_SLICES(float, 64, 32)
  GLA_BWD_SLICES(float, 64, 64) GLA_BWD_SLICES(float, 128, 32) GLA_BWD_SLICES(float, 128, 64)
#undef GLA_BWD_SLICES
  return 0;
}

template <typename T, int DKP, int CP>
hipError_t launch_gla_bwd(const BwdParams& p, hipStream_t s) {
  using P = BwdPlan<T, DKP, CP>;
  if constexpr (!P::OK) {
    return hipErrorNotSupported;
  } else {
    hipError_t e;
    int ev = 0;
    record_event(p.events, ev++, s);
    const int ntile = (p.Dv + kDvTile - 1) / kDvTile;
    if (!p.saved) {   // recompute the chunk operands and the forward states
      PrepParams pp{p.q, p.k, p.g, p.ops, p.L, p.Dk, p.C, p.N};
      if ((e = launch_prep<T, DKP, CP>(pp, p.BH, s)) != hipSuccess) return e;
      record_event(p.events, ev++, s);
      WalkIO wf{p.ops.KdT, p.v, p.ops.Gam, p.Hs, p.h0, nullptr, p.Dk, p.Dv, p.L, p.C, p.N, 0};
      if ((e = launch_walk_store<T, DKP, CP>(wf, p.BH, s)) != hipSuccess) return e;
      record_event(p.events, ev++, s);
    }
    WalkIO wr{p.ops.Qs, p.do_, p.ops.Gam, p.dHs, p.dht, p.dh0, p.Dk, p.Dv, p.L, p.C, p.N, 0};
    if ((e = launch_walk_reverse<T, DKP, CP>(wr, p.BH, s)) != hipSuccess) return e;
    record_event(p.events, ev++, s);
    const int ntiles = p.N * p.BH * (DKP / P::DKS);
    if (p.dz) {   // GSA's pass 2 with the read-out's backward: one key-width slice only
      if constexpr (P::DKS == DKP && DKP <= 128) {   // GSA pads at most 128 slots
        hipLaunchKernelGGL((gla_bwd_chunk<T, P::DKS, CP, P::FUSED, true>),
                           dim3(imin(ntiles, bwd_chunk_slots<T, P::DKS, CP, P::FUSED, true>())), dim3(kBwdThreads), 0, s,
                           p, DKP, ntile, ntiles);
      } else {
        return hipErrorInvalidValue;
      }
    } else {
      hipLaunchKernelGGL((gla_bwd_chunk<T, P::DKS, CP, P::FUSED, false>),
                         dim3(imin(ntiles, bwd_chunk_slots<T, P::DKS, CP, P::FUSED, false>())), dim3(kBwdThreads), 0, s,
                         p, DKP, ntile, ntiles);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    record_event(p.events, ev++, s);
    if constexpr (!P::FUSED) {
      hipLaunchKernelGGL((gla_bwd_dv<T, DKP, CP>), dim3(p.N * p.BH), dim3(kDvThreads), 0, s, p, ntile);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      record_event(p.events, ev++, s);
    }
    return hipSuccess;
  }
}

int bwd_launch_count(int esize, int DKP, int CP) {
  int c = 0;
#define GLA_BCNT_CASE(TT, D, C_) \
  if (esize == (int)sizeof(TT) && DKP == D && CP == C_) c = BwdPlan<TT, D, C_>::FUSED ? 4 : 5;
#define GLA_BCNT_ALL(TT)                                                                 \
  GLA_BCNT_CASE(TT, 32, 32) GLA_BCNT_CASE(TT, 32, 64) GLA_BCNT_CASE(TT, 32, 128)           \
  GLA_BCNT_CASE(TT, 64, 32) GLA_BCNT_CASE(TT, 64, 64) GLA_BCNT_CASE(TT, 64, 128)           \
  GLA_BCNT_CASE(TT, 128, 32) GLA_BCNT_CASE(TT, 128, 64) GLA_BCNT_CASE(TT, 128, 128)        \
  GLA_BCNT_CASE(TT, 256, 32) GLA_BCNT_CASE(TT, 256, 64)
  GLA_BCNT_ALL(bf16)
  GLA_BCNT_ALL(float)
#undef GLA_BCNT_ALL
#undef GLA_BCNT_CASE
  return c;
}

bool bwd_config_fits(int esize, int DKP, int CP) {
  bool ok = false;
#define GLA_BFIT_CASE(TT, D, C_) \
  if (esize == (int)sizeof(TT) && DKP == D && CP == C_) ok = BwdPlan<TT, D, C_>::OK;
#define GLA_BFIT_ALL(TT)                                                                 \
  GLA_BFIT_CASE(TT, 32, 32) GLA_BFIT_CASE(TT, 32, 64) GLA_BFIT_CASE(TT, 32, 128)           \
  GLA_BFIT_CASE(TT, 64, 32) GLA_BFIT_CASE(TT, 64, 64) GLA_BFIT_CASE(TT, 64, 128)           \
  GLA_BFIT_CASE(TT, 128, 32) GLA_BFIT_CASE(TT, 128, 64) GLA_BFIT_CASE(TT, 128, 128)        \
  GLA_BFIT_CASE(TT, 256, 32) GLA_BFIT_CASE(TT, 256, 64)
  GLA_BFIT_ALL(bf16)
  GLA_BFIT_ALL(float)
#undef GLA_BFIT_ALL
#undef GLA_BFIT_CASE
  return ok;
}

#define GLA_BWD_INST(TT, D, C_) template hipError_t launch_gla_bwd<TT, D, C_>(const BwdParams&, hipStream_t);
#define GLA_BWD_INST_T(TT)                                                     \
  GLA_BWD_INST(TT, 32, 32) GLA_BWD_INST(TT, 32, 64) GLA_BWD_INST(TT, 32, 128)  \
  GLA_BWD_INST(TT, 64, 32) GLA_BWD_INST(TT, 64, 64) GLA_BWD_INST(TT, 64, 128)  \
  GLA_BWD_INST(TT, 128, 32) GLA_BWD_INST(TT, 128, 64) GLA_BWD_INST(TT, 128, 128) \
  GLA_BWD_INST(TT, 256, 32) GLA_BWD_INST(TT, 256, 64)
GLA_BWD_INST_T(bf16)
GLA_BWD_INST_T(float)

}  // namespace gla
