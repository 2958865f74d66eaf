// walk_out.hpp -- the forward state walk fused with the chunk outputs.
//
// The unfused forward writes every chunk-start state H_n to memory in its walk and reads it
// back in the output kernel, O_n = Qs_n H_n + A_n V_n (gla_fwd.hip).  Here one workgroup per
// (b*h, 32 value columns) carries the whole key width of its state columns ([DKP][32], fp32,
// in matrix-core accumulators) and, at each chunk, forms that chunk's outputs from the bf16
// copy of H_n it stages in LDS anyway, so the states reach memory only when a caller keeps
// them (the saving forward, whose backward reads them) and are never read back.  The
// chunked structure -- a sequential inter-chunk state pass and a parallel intra-chunk part --
// is the chunkwise training form (MS-GLA summary, section 2.1).
//
// Per chunk n, in order within one step:
//   T_n   = Kd_n^T V_n                 (from LDS: the chunk's staged KdT and V tiles)
//   O_n   = Qs_n H_n + A_n V_n         (H_n, and the chunk's staged Qs and A tiles, from LDS;
//                                       O_n leaves through LDS, 8 bytes per thread)
//   H_n+1 = Diag(2^Gamma_n) H_n + T_n  (fp32 accumulators; its bf16 copy goes to LDS for the
//                                       next chunk's O and, if kept, to memory)
// O_n needs every key row of H_n, which four waves write, so the bf16 copy of H_n is written
// one step earlier (after the fold that produces it), and the staged tiles, the copy and the
// output tile are double-buffered: one barrier per chunk.  Every tile moves between memory and
// LDS in whole runs of consecutive threads.  A first form read each lane's Qs and A row
// fragments straight from memory (as the unfused output kernel does) and stored the outputs
// from the accumulators, four elements of one row per lane: 84 us at the 340M shape against
// 58 us as built, since every step waits for those loads.
//
// Layout: 8 waves; wave w owns state columns 16 (w % 2) .. +15 and rows DKP/4 (w / 2) .. +
// DKP/4 - 1, and the 16 x 16 output block (rows 16 (w / 2), columns 16 (w % 2)).  The
// accumulators hold their blocks transposed (products formed as X^T M^T), so a lane owns four
// consecutive columns of one row: one decay factor per row, and 8-byte writes of the state
// copy and of the outputs.
#pragma once
#include "walks.hpp"

namespace gla {

constexpr int kWoCols = 32;      // value columns per workgroup
constexpr int kWoThreads = 512;

template <typename T, int DKP, int CP>
struct WalkOutCfg {
  static constexpr int NT = kWoThreads, NW = NT / 64, V = 16 / (int)sizeof(T);
  // row pitches: a 32-byte pad on the 32-column tiles puts the four rows a transposing read
  // touches per 16 lanes in disjoint bank windows
  static constexpr int LDA = CP + V, LDV = kWoCols + 2 * V, LDH = kWoCols + 2 * V, LDQ = DKP + V, LDC = CP + V;
  static constexpr size_t KT = (size_t)DKP * LDA * sizeof(T);   // KdT [DKP][CP]
  static constexpr size_t VT = (size_t)CP * LDV * sizeof(T);    // V   [CP][32]
  static constexpr size_t QT = (size_t)CP * LDQ * sizeof(T);    // Qs  [CP][DKP]
  static constexpr size_t AT = (size_t)CP * LDC * sizeof(T);    // A   [CP][CP]
  static constexpr size_t GT = (size_t)DKP * 4;                 // Gamma [DKP]
  static constexpr size_t SLOT = KT + VT + QT + AT + GT;
  static constexpr size_t HT = (size_t)DKP * LDH * sizeof(T);   // bf16 H [DKP][32]
  static constexpr size_t OT = (size_t)CP * LDV * sizeof(T);    // O [CP][32]
  static constexpr size_t BYTES = 2 * SLOT + 2 * HT + 2 * OT;
  static constexpr int NK = DKP * CP / V, NV = CP * kWoCols / V, NHV = DKP * kWoCols / V;
  static constexpr int NQ = CP * DKP / V, NA = CP * CP / V;
  static constexpr int PK = NK / NT, PQ = NQ / NT, PA = NA / NT;
  static constexpr int RW = DKP / 4, NIB = RW / 16, NKB = DKP / 32, NCB = CP / 32;
  // what the kernel is written for: every thread stages whole vectors of the KdT tile and of
  // the state copy, four row groups of whole 16-row blocks, and one 16 x 16 output block per
  // wave
  static constexpr bool OK = sizeof(T) == 2 && CP == 64 && DKP % 64 == 0 && DKP <= 128 && NK % NT == 0 &&
                             NQ % NT == 0 && NA % NT == 0 && NHV == NT && NV <= NT && BYTES <= kMaxLds;
};

// One chunk's operands in flight to LDS: the KdT, V, Qs and A tiles and Gamma.  Loads are
// issued unconditionally from clamped addresses; validity is applied when the tiles go to
// LDS.
template <typename T, int DKP, int CP>
struct WalkOutStage {
  using W = WalkOutCfg<T, DKP, CP>;
  typedef typename V16<T>::type VT;
  VT kt[W::PK], qs[W::PQ], a[W::PA], v;
  bool vok;
  f32x4 gam;

  // n: chunk; row0/len: its rows; vg: this sequence's V [L][Dv]; tile: the 32-column tile
  __device__ __forceinline__ void load(const FwdParams& p, size_t chunk, const T* vg, int row0, int len, int tile,
                                       int tid) {
    const T* kt_g = reinterpret_cast<const T*>(p.ops.KdT) + chunk * DKP * CP;
    const T* qs_g = reinterpret_cast<const T*>(p.ops.Qs) + chunk * CP * DKP;
    const T* a_g = reinterpret_cast<const T*>(p.ops.A) + chunk * CP * CP;
#pragma unroll
    for (int m = 0; m < W::PK; ++m) kt[m] = *reinterpret_cast<const VT*>(kt_g + (size_t)(tid + W::NT * m) * W::V);
#pragma unroll
    for (int m = 0; m < W::PQ; ++m) qs[m] = *reinterpret_cast<const VT*>(qs_g + (size_t)(tid + W::NT * m) * W::V);
#pragma unroll
    for (int m = 0; m < W::PA; ++m) a[m] = *reinterpret_cast<const VT*>(a_g + (size_t)(tid + W::NT * m) * W::V);
    constexpr int PER_ROW = kWoCols / W::V;
    const int idx = min(tid, W::NV - 1), r = idx / PER_ROW, c = (idx - r * PER_ROW) * W::V;
    vok = tid < W::NV && r < len;
    v = *reinterpret_cast<const VT*>(vg + (size_t)(row0 + min(r, len - 1)) * p.Dv + tile * kWoCols + c);
    gam = *reinterpret_cast<const f32x4*>(p.ops.Gam + chunk * DKP + 4 * (tid % (DKP / 4)));
  }
  __device__ __forceinline__ void store(T* sKT, T* sV, T* sQ, T* sA, float* sG, int tid) const {
    constexpr int KPR = CP / W::V, QPR = DKP / W::V;  // vectors per row: KdT and A, Qs
#pragma unroll
    for (int m = 0; m < W::PK; ++m) {
      const int idx = tid + W::NT * m, r = idx / KPR, c = (idx - r * KPR) * W::V;
      *reinterpret_cast<VT*>(sKT + r * W::LDA + c) = kt[m];
    }
#pragma unroll
    for (int m = 0; m < W::PQ; ++m) {
      const int idx = tid + W::NT * m, r = idx / QPR, c = (idx - r * QPR) * W::V;
      *reinterpret_cast<VT*>(sQ + r * W::LDQ + c) = qs[m];
    }
#pragma unroll
    for (int m = 0; m < W::PA; ++m) {
      const int idx = tid + W::NT * m, r = idx / KPR, c = (idx - r * KPR) * W::V;
      *reinterpret_cast<VT*>(sA + r * W::LDC + c) = a[m];
    }
    constexpr int PER_ROW = kWoCols / W::V;
    if (W::NV == W::NT || tid < W::NV) {
      const int r = tid / PER_ROW, c = (tid - r * PER_ROW) * W::V;
      *reinterpret_cast<VT*>(sV + r * W::LDV + c) = vok ? v : zero_vec<T>();
    }
    if (tid < DKP / 4) *reinterpret_cast<f32x4*>(sG + 4 * tid) = gam;
  }
};

// where the threads whose rows lie past a ragged last chunk write their outputs: a slot per
// thread, so that no two threads of a workgroup store to one address
__device__ __attribute__((aligned(16))) char g_wo_sink[kWoThreads * 8];

// grid (Dv / 32) * BH, remapped so that a sequence's column tiles share an XCD (and its L2 for
// the KdT, Qs and A they all read).  Hs null: the states are not kept.
template <typename T, int DKP, int CP>
__global__ __launch_bounds__(kWoThreads) void walk_out_kernel(FwdParams p, int ntile) {
  using W = WalkOutCfg<T, DKP, CP>;
  using Stage = WalkOutStage<T, DKP, CP>;
  constexpr int NT = W::NT, LDA = W::LDA, LDV = W::LDV, LDH = W::LDH, LDQ = W::LDQ, LDC = W::LDC, NIB = W::NIB;
  constexpr int R = kWalkDepth;
  static_assert(R == 2, "two register stages, one per step of a round");
  typedef typename Vec4<T>::type V4T;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) char smem[W::BYTES];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = lin % ntile, bh = lin / ntile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int jo = wave & 1, cw = 16 * jo, ri = W::RW * (wave >> 1), rbo = wave >> 1;
  const int Dv = p.Dv, L = p.L, C = p.C, N = p.N, DvP = (Dv + kDvTile - 1) / kDvTile * kDvTile;
  const T* vg = reinterpret_cast<const T*>(p.v) + (size_t)p.in(bh) * L * Dv;
  T* og = reinterpret_cast<T*>(p.o) + (size_t)bh * L * Dv + tile * kWoCols;
  T* hs = p.Hs ? reinterpret_cast<T*>(p.Hs) + (size_t)bh * N * DKP * DvP + tile * kWoCols : nullptr;

  auto sKT = [&](int b) { return reinterpret_cast<T*>(smem + b * W::SLOT); };
  auto sV = [&](int b) { return reinterpret_cast<T*>(smem + b * W::SLOT + W::KT); };
  auto sQ = [&](int b) { return reinterpret_cast<T*>(smem + b * W::SLOT + W::KT + W::VT); };
  auto sA = [&](int b) { return reinterpret_cast<T*>(smem + b * W::SLOT + W::KT + W::VT + W::QT); };
  auto sG = [&](int b) { return reinterpret_cast<float*>(smem + b * W::SLOT + W::KT + W::VT + W::QT + W::AT); };
  auto sH = [&](int b) { return reinterpret_cast<T*>(smem + 2 * W::SLOT + b * W::HT); };
  auto sO = [&](int b) { return reinterpret_cast<T*>(smem + 2 * W::SLOT + 2 * W::HT + b * W::OT); };
  auto chunk_of = [&](int k) { return (size_t)bh * N + min(k, N - 1); };

  f32x4 S[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = ri + 16 * ib + col, j = tile * kWoCols + cw + 4 * grp + e;
      S[ib][e] = (p.h0 && i < p.Dk) ? p.h0[((size_t)bh * p.Dk + i) * Dv + j] : 0.f;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);                   // initial state in before the pipeline starts

  Stage st[R];
  auto load = [&](Stage& s, int k) {               // past the end: reload the last chunk
    const int n = min(k, N - 1), row0 = n * C;
    s.load(p, chunk_of(n), vg, row0, min(C, L - row0), tile, tid);
  };
  // the bf16 copy of the state (rows of this wave, four columns per lane) into sH(b)
  auto put_state = [&](int b) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      V4T hv;
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = from_f32<T>(S[ib][e]);
      *reinterpret_cast<V4T*>(sH(b) + (ri + 16 * ib + col) * LDH + cw + 4 * grp) = hv;
    }
  };
  // the staged copy of H_k to Hs[k]: one 16-byte vector per thread
  auto state_out = [&](int b, int k) {
    constexpr int PER_ROW = kWoCols / W::V;
    const int r = tid / PER_ROW, c = (tid - r * PER_ROW) * W::V;
    *reinterpret_cast<VT*>(hs + ((size_t)k * DKP + r) * DvP + c) = *reinterpret_cast<const VT*>(sH(b) + r * LDH + c);
  };

  // the staged O_k: rows 0 .. len-1 of the chunk, four elements (8 bytes) per thread, so that
  // every thread stores a piece of the tile ([64][32] bf16 is 512 such pieces); a row past a
  // ragged chunk's end goes to the thread's sink slot.  (16-byte pieces would leave half the
  // threads storing to a shared sink address every step: 5.5 us at the 340M shape.)
  static_assert(CP * kWoCols == 4 * NT, "one 4-element piece of the output tile per thread");
  auto out_tile = [&](int b, int k) {
    constexpr int PER_ROW = kWoCols / 4;
    const int r = tid / PER_ROW, c = (tid % PER_ROW) * 4, row0 = k * C;
    const V4T x = *reinterpret_cast<const V4T*>(sO(b) + r * LDV + c);
    V4T* dst = r < min(C, L - row0) ? reinterpret_cast<V4T*>(og + (size_t)(row0 + r) * Dv + c)
                                    : reinterpret_cast<V4T*>(g_wo_sink + 8 * tid);
    *dst = x;
  };

  load(st[0], 0);
  load(st[1], 1);
  put_state(0);
  st[0].store(sKT(0), sV(0), sQ(0), sA(0), sG(0), tid);
  __syncthreads();
  if (hs) state_out(0, 0);

  // Step k (register stage r = k % 2, LDS buffers b = k % 2): the next-but-one chunk's loads
  // into the register stage whose tiles went to LDS in the previous step, T_k from the staged
  // tiles, the fold into H_{k+1} (its bf16 copy into the other buffer), O_k from the staged
  // tiles and H_k's copy (into its LDS tile), chunk k+1's tiles into the other buffer, one
  // barrier, O_k and H_{k+1} out.  LAST: the final step, whose H_N is not a chunk-start state.
  auto body = [&](auto rc, int k, auto lc) {
    constexpr int r = decltype(rc)::value;
    constexpr bool LAST = decltype(lc)::value;
    const int b = k & 1;
    load(st[r], k + R);
    Frag<T> Yv[W::NCB];
#pragma unroll
    for (int cb = 0; cb < W::NCB; ++cb) Yv[cb] = ld8_colblk(sV(b) + (32 * cb) * LDV + cw, LDV, lane);
    f32x4 Tm[NIB];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      Tm[ib] = zero4();
#pragma unroll
      for (int cb = 0; cb < W::NCB; ++cb)
        mma(Tm[ib], Yv[cb], ld8(sKT(b) + (ri + 16 * ib + col) * LDA + 32 * cb + 8 * grp));
    }
    const float* gg = sG(b);
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      const float dec = fast_exp2(gg[ri + 16 * ib + col]);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[ib][e] = dec * S[ib][e] + Tm[ib][e];
    }
    put_state(b ^ 1);
    // O_k^T block: X = H_k column run (out column), Y = Qs_k / A_k row (out row)
    f32x4 O = zero4();
    const int ro = 16 * rbo + col;
#pragma unroll
    for (int kb = 0; kb < W::NKB; ++kb)
      mma(O, ld8_colblk(sH(b) + (32 * kb) * LDH + cw, LDH, lane), ld8(sQ(b) + ro * LDQ + 32 * kb + 8 * grp));
#pragma unroll
    for (int cb = 0; cb < W::NCB; ++cb) mma(O, Yv[cb], ld8(sA(b) + ro * LDC + 32 * cb + 8 * grp));
    {
      V4T o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = from_f32<T>(O[e]);
      *reinterpret_cast<V4T*>(sO(b) + ro * LDV + cw + 4 * grp) = o4;
    }
    st[r ^ 1].store(sKT(b ^ 1), sV(b ^ 1), sQ(b ^ 1), sA(b ^ 1), sG(b ^ 1), tid);
    __syncthreads();
    out_tile(b, k);
    if (!LAST && hs) state_out(b ^ 1, k + 1);
  };
  // two steps per round, one per register stage; the final step is peeled
  int k = 0;
  for (; k + 2 < N; k += 2) {
    body(std::integral_constant<int, 0>{}, k, std::false_type{});
    body(std::integral_constant<int, 1>{}, k + 1, std::false_type{});
  }
  if (k + 1 < N) {
    body(std::integral_constant<int, 0>{}, k, std::false_type{});
    body(std::integral_constant<int, 1>{}, k + 1, std::true_type{});
  } else {
    body(std::integral_constant<int, 0>{}, k, std::true_type{});
  }
  if (p.ht) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      const int i = ri + 16 * ib + col;
      if (i < p.Dk) {
        const int j = tile * kWoCols + cw + 4 * grp;
        *reinterpret_cast<f32x4*>(p.ht + ((size_t)bh * p.Dk + i) * Dv + j) = S[ib];
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);                   // the last reloads have landed
}

template <typename T, int DKP, int CP>
constexpr bool walk_out_fits() {
  return WalkOutCfg<T, DKP, CP>::OK;
}

// Whether a forward of BH sequences of Dv value columns runs the fused kernel (on a shape it
// fits): when its 32-column tiles give every CU of the current device a workgroup.  Kept
// states need whole 64-column tiles: their padding columns, which the backward reads, are not
// written.
inline bool walk_out_applies(int BH, int Dv, bool keep_states) {
  const int cus = device_cu_count();
  const int cols = keep_states ? kDvTile : kWoCols;
  return Dv % cols == 0 && cus > 0 && (long long)(Dv / kWoCols) * BH >= cus;
}

// The fused walk and outputs for p (p.Hs null: states not kept); the caller has checked
// walk_out_fits and that Dv is a multiple of 32.
template <typename T, int DKP, int CP>
hipError_t launch_walk_out(const FwdParams& p, hipStream_t s) {
  if constexpr (!walk_out_fits<T, DKP, CP>()) {
    return hipErrorNotSupported;
  } else {
    const int ntile = p.Dv / kWoCols;
    hipLaunchKernelGGL((walk_out_kernel<T, DKP, CP>), dim3(ntile * p.BH), dim3(kWoThreads), 0, s, p, ntile);
    return hipGetLastError();
  }
}

}  // namespace gla
