// walks.hpp -- the sequential state walks shared by the GLA and GSA backward (and the GSA
// forward).  A walk carries a [RT rows][64 columns] tile of a row-gated state in fp32
// matrix-core accumulators while stepping over the chunks of one (batch*head):
//
//   forward walk   S_0 = init;  for n = 0..N-1:      store S_n,
//                               S_{n+1} = Diag(2^{Gamma_n}) S_n + M_n X_n ;    fin = S_N
//   reverse walk   D_N = init;  for n = N-1..0:      store D_{n+1} (at index n),
//                               D_n = Diag(2^{Gamma_n}) D_{n+1} + M_n X_n ;    fin = D_0
//
// with M_n = mat[n] a per-chunk [SP][CP] matrix and X_n the chunk's rows of a token tensor
// src [L][Ds] (values for the forward walk, output gradients for the reverse).  The forward
// walk reads M_n as stored ([SP][CP]: the decayed keys transposed); the reverse walk reads its
// transpose as stored ([CP][SP]: the decayed queries, chunk rows first, exactly as the output
// kernels use them) and takes M_n from it with transposing LDS reads, so no transposed copy of
// the queries is ever written.
// GLA: rows = key channels.  GSA: rows = slots for both passes (pass 1 walks the transposed
// slot-key memory, whose values are the keys).  The chunked structure -- sequential
// inter-chunk updates, state written only at chunk boundaries -- is the chunkwise training
// form of the MS-GLA summary (section 2.1).
//
// Both walks are one kernel.  Row i of the update needs only row i of M_n, so the state is
// tiled over rows as well as columns: one workgroup per (row tile, 64-column tile, b*h).
// Per chunk the walk's own arithmetic is tiny, so its speed is set by the latency of each
// sequential step (LDS round trip, barrier, matrix-core chain) rather than by bandwidth.  A
// step therefore takes a group of G chunks: the G products T_g = M_g X_g are independent and
// go on the matrix cores back to back, and the sequential part is only the element-wise fold
// S <- Diag(2^Gamma_g) S + T_g, which also yields each stored state.  Group operands are
// loaded into registers kWalkDepth groups ahead of use and LDS is double-buffered, so a step
// needs one barrier per G chunks.  The accumulators hold the transposed tile (the product is
// formed as X^T M^T): a lane then owns four consecutive columns of one state row, so it needs
// one decay factor per row and stages each stored state with one 8-byte LDS write per 16-row
// block; the staged tile leaves in full 128-byte rows.
#pragma once
#include <atomic>
#include <type_traits>
#include <utility>
#include "prep.hpp"

namespace gla {

struct WalkIO {
  const void* mat;     // [BH][N][SP][CP] per-chunk matrix (T); reverse walks: [BH][N][CP][SP]
  const void* src;     // [BH][L][Ds] token tensor (T)
  const float* gam;    // [BH][N][SP] chunk log2-decay per state row
  void* states;        // [BH][N][SP][DsP] stored states / state gradients (T)
  const float* init;   // fp32 [BH][rows][Ds] (or [BH][Ds][rows] when trans) or nullptr (= 0)
  float* fin;          // fp32, same layout, or nullptr (= not written)
  int rows, Ds, L, C, N, trans;
  SeqView in;          // input sequences of src
  // Forward walks only: nseg > 1 splits the chunks into segments of seg_len chunks walked in
  // parallel, the first from init and the others from zero.  Each segment then leaves its end
  // state in seg_end ([BH][nseg][SP][DsP] fp32) instead of writing fin; the stored states of
  // later segments lack the part carried in from before the segment (the segment kernels
  // further down add it).  The first column tile's workgroups also write, per row, the
  // segment's log2-decay before each chunk (seg_prefix [BH][N][SP]) and in all
  // (seg_total [BH][nseg][SP]).
  int nseg = 1, seg_len = 0;
  float* seg_end = nullptr;
  float* seg_prefix = nullptr;
  float* seg_total = nullptr;
};

constexpr int kWalkDepth = 2;   // chunk groups whose operands are in flight ahead of use

template <typename T, int RT, int CP, int G = 1, int NT = 256>
struct WalkIOCfg {
  static constexpr int V = 16 / (int)sizeof(T);
  // per-chunk matrix tile: [RT][LDA] as stored for a forward walk, [CP][LDM] (chunk rows
  // first) for a reverse walk; the slot has room for either, so both directions share a plan
  static constexpr int LDA = CP + V, LDM = RT + V, LDV = kDvTile + V;
  static constexpr size_t KT = (size_t)(RT * LDA > CP * LDM ? RT * LDA : CP * LDM) * sizeof(T);
  static constexpr size_t VT = (size_t)CP * LDV * sizeof(T);
  static constexpr size_t GT = (size_t)RT * 4;
  static constexpr size_t SLOT = KT + VT + GT;            // one chunk's operands
  static constexpr size_t STAGE = G * SLOT;               // one group's operands
  static constexpr size_t HT = (size_t)RT * LDV * sizeof(T);   // one staged state tile
  static constexpr size_t BYTES = 2 * STAGE + 2 * G * HT;
  static constexpr int NK = RT * CP / V, NV = CP * kDvTile / V;
  static constexpr int PKd = (NK + NT - 1) / NT, PV = (NV + NT - 1) / NT;   // vectors per thread
};

// Row tile RT (32 rows, at most SP; 16 if nothing fits) and group size G (4, 2 or 1 chunks):
// the largest group whose double-buffered tiles leave room for two workgroups per CU (the
// grid has two row tiles per 64 columns, so every workgroup is resident at once), else the
// largest that fits at all.
template <typename T, int SP, int CP>
struct WalkPlan {
  static constexpr int cand(int r) { return r < SP ? r : SP; }
  template <int RT_>
  static constexpr int group() {
    return WalkIOCfg<T, RT_, CP, 4>::BYTES <= kMaxLds / 2   ? 4
           : WalkIOCfg<T, RT_, CP, 2>::BYTES <= kMaxLds / 2 ? 2
           : WalkIOCfg<T, RT_, CP, 2>::BYTES <= kMaxLds     ? 2
                                                             : 1;
  }
  static constexpr int RT = WalkIOCfg<T, cand(32), CP, 1>::BYTES <= kMaxLds ? cand(32) : cand(16);
  static constexpr int G = group<RT>();
  static constexpr bool OK = WalkIOCfg<T, RT, CP, G>::BYTES <= kMaxLds;
  // 64-row tiles of 8 waves (two 32-row halves sharing each chunk's source rows), two chunks
  // per group, one workgroup per CU: each source row is fetched by half as many workgroups.
  // Worth it only while the grid still gives every CU a workgroup; below that, more and
  // smaller tiles shorten each sequential step: 16-row tiles when even the 32-row grid leaves
  // CUs idle (few sequences).
  static constexpr bool WIDE = OK && RT == 32 && SP % 64 == 0 && WalkIOCfg<T, 64, CP, 2>::BYTES <= kMaxLds;
  static constexpr bool NARROW = OK && RT == 32 && WalkIOCfg<T, 16, CP, 2>::BYTES <= kMaxLds;
};

template <typename T, int SP, int CP>
constexpr bool walk_fits() {
  return WalkPlan<T, SP, CP>::OK;
}

// One chunk's walk operands in flight between global memory and LDS.  Loads are issued
// unconditionally from clamped, in-bounds addresses and the validity of each vector is kept
// beside it; masking happens when the registers are written to LDS, after the data has
// arrived.  This keeps branches and register rewrites away from loads in flight, so the
// compiler can leave several chunks' loads outstanding.
// ROWM: the chunk's matrix is stored chunk rows first ([CP][SP]; mat points at this tile's
// first column and the rows are SP apart), else as [RT][CP] rows (row stride CP).
template <typename T, int RT, int CP, int NT, bool ROWM, int SP>
struct WalkIOStage {
  using W = WalkIOCfg<T, RT, CP, 1, NT>;
  typedef typename V16<T>::type VT;
  static constexpr int MPR = ROWM ? RT / W::V : CP / W::V;   // matrix vectors per stored row
  VT kt[W::PKd], v[W::PV];
  bool vok[W::PV];
  f32x4 gam;

  // mat: this tile's part of the chunk's matrix; src: [L][Ds] of this (b,h); gam_chunk: this
  // tile's RT decay values.
  __device__ __forceinline__ void load(const T* mat, const T* src, int row0, int len, int Ds, int tile,
                                       const float* gam_chunk) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < W::PKd; ++m) {
      const int idx = min(tid + NT * m, W::NK - 1);
      if constexpr (ROWM) {
        const int r = idx / MPR, c = (idx - r * MPR) * W::V;
        kt[m] = *reinterpret_cast<const VT*>(mat + (size_t)r * SP + c);
      } else {
        kt[m] = *reinterpret_cast<const VT*>(mat + (size_t)idx * W::V);
      }
    }
    constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
    for (int m = 0; m < W::PV; ++m) {
      const int idx = tid + NT * m;
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * W::V;
      const int j = tile * kDvTile + c;
      vok[m] = idx < W::NV && r < len && j < Ds;
      const int rr = min(r, len - 1), jj = min(j, Ds - W::V);
      v[m] = *reinterpret_cast<const VT*>(src + (size_t)(row0 + rr) * Ds + jj);
    }
    gam = *reinterpret_cast<const f32x4*>(gam_chunk + 4 * (tid % (RT / 4)));
  }

  __device__ __forceinline__ void store(T* sKT, T* sV, float* sG) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < W::PKd; ++m) {
      const int idx = tid + NT * m;
      if (W::NK % NT == 0 || idx < W::NK) {
        const int r = idx / MPR, c = (idx - r * MPR) * W::V;
        *reinterpret_cast<VT*>(sKT + r * (ROWM ? W::LDM : W::LDA) + c) = kt[m];
      }
    }
    constexpr int PER_ROW = kDvTile / W::V;
#pragma unroll
    for (int m = 0; m < W::PV; ++m) {
      const int idx = tid + NT * m;
      if (W::NV % NT == 0 || idx < W::NV) {
        const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * W::V;
        *reinterpret_cast<VT*>(sV + r * W::LDV + c) = vok[m] ? v[m] : zero_vec<T>();
      }
    }
    if (tid < RT / 4) *reinterpret_cast<f32x4*>(sG + 4 * tid) = gam;
  }
};

// Copy an LDS [RT][64] tile to the state workspace (row stride DsP, already offset).
template <typename T, int RT, int NT>
__device__ __forceinline__ void state_tile_out(T* dst, const T* src, int lds, int DsP) {
  // 16-byte pieces, or 4-element (8-byte for bf16) pieces where a 16-row bf16 tile would
  // leave half the threads without one
  constexpr bool HALF = sizeof(T) == 2 && RT * kDvTile * (int)sizeof(T) < 16 * NT;
  constexpr int V = HALF ? 4 : V16<T>::N;
  typedef typename std::conditional<HALF, typename Vec4<T>::type, typename V16<T>::type>::type VT;
  constexpr int PER_ROW = kDvTile / V;
#pragma unroll
  for (int m = 0; m < (RT * PER_ROW + NT - 1) / NT; ++m) {
    const int idx = threadIdx.x + NT * m;
    // a guard only where the tile does not divide evenly: a store the compiler must treat as
    // optional would make it wait for the stores before it at the next operand wait
    if (RT * PER_ROW % NT == 0 || idx < RT * PER_ROW) {
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
      *reinterpret_cast<VT*>(dst + (size_t)r * DsP + c) = *reinterpret_cast<const VT*>(src + r * lds + c);
    }
  }
}

// f(integral_constant<int, r>) for r = 0 .. R-1, unrolled at compile time
template <typename F, int... r>
__device__ __forceinline__ void for_each_stage(F&& f, std::integer_sequence<int, r...>) {
  (f(std::integral_constant<int, r>{}), ...);
}

__device__ __forceinline__ size_t walk_state_index(const WalkIO& w, int bh, int i, int j) {
  return w.trans ? ((size_t)bh * w.Ds + j) * w.rows + i : ((size_t)bh * w.rows + i) * w.Ds + j;
}

// T^T = X^T M^T on fresh accumulators (M and X from LDS): one chunk's state increment over
// the RW rows from row ri and the 16 columns from cj, with lane (col, grp) holding
// T[ri + 16 ib + col][cj + 4 grp + e] in Tm[ib][e].  ROWM: sKT holds M^T ([CP][LDM]).
template <typename T, int RT, int CP, int RW, bool ROWM>
__device__ __forceinline__ void walk_product(f32x4 (&Tm)[RW / 16], const T* sKT, const T* sV, int ri, int cj) {
  using W = WalkIOCfg<T, RT, CP>;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  constexpr int NCB = CP / 32, NIB = RW / 16;
  Frag<T> Yv[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) Yv[cb] = ld8_colblk(sV + (32 * cb) * W::LDV + cj, W::LDV);
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) Tm[ib] = zero4();
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      if constexpr (ROWM)
        mma(Tm[ib], Yv[cb], ld8_colblk(sKT + (32 * cb) * W::LDM + ri + 16 * ib, W::LDM));
      else
        mma(Tm[ib], Yv[cb], ld8(sKT + (ri + 16 * ib + col) * W::LDA + 32 * cb + 8 * grp));
    }
  }
}

// grid: ntile * (SP / RT) * BH workgroups of 64 NW threads.  Wave w owns columns 16 (w % 4)
// .. +15 of the 64 and rows RW (w / 4) .. +RW-1 of the RT, RW = 4 RT / NW.
template <typename T, int SP, int RT, int CP, int G, bool REV, int NW>
__device__ __forceinline__ void walk_tile(const WalkIO& w, int ntile, int lin) {
  constexpr int NT = 64 * NW, RW = RT * 4 / NW;
  static_assert(NW == 4 || NW == 8, "four column waves, one or two row groups");
  using W = WalkIOCfg<T, RT, CP, G, NT>;
  using Stage = WalkIOStage<T, RT, CP, NT, REV, SP>;
  constexpr int LDV = W::LDV, NIB = RW / 16, NRT = SP / RT, R = kWalkDepth;
  __shared__ __attribute__((aligned(16))) char smem[W::BYTES];

  int seg = 0;                                   // segment (the launch grid is nseg equal parts)
  if (w.nseg > 1) {
    const int per_seg = gridDim.x / w.nseg;
    seg = lin / per_seg;
    lin -= seg * per_seg;
  }
  const int tile = lin % ntile, rt = (lin / ntile) % NRT, bh = lin / (ntile * NRT);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int cw = 16 * (wave & 3), ri = RW * (wave >> 2);    // this wave's columns and rows
  const int Ds = w.Ds, L = w.L, C = w.C, NT_ = w.N;
  // this segment's chunks: c0 .. c0 + N - 1 (the whole sequence when not segmented)
  const int c0 = w.nseg > 1 ? seg * w.seg_len : 0;
  const int N = w.nseg > 1 ? min(w.seg_len, NT_ - c0) : NT_;
  const int NG = (N + G - 1) / G;
  const int DsP = ntile * kDvTile, i0 = rt * RT;
  const int j0 = tile * kDvTile + cw + 4 * grp;             // this lane's four columns
  typedef typename Vec4<T>::type V4T;
  const T* src = reinterpret_cast<const T*>(w.src) + (size_t)w.in(bh) * L * Ds;
  const T* mat = reinterpret_cast<const T*>(w.mat) + (size_t)bh * NT_ * SP * CP + (REV ? i0 : i0 * CP);
  const float* gam = w.gam + (size_t)bh * NT_ * SP + i0;
  T* out = reinterpret_cast<T*>(w.states) + ((size_t)bh * NT_ * SP + i0) * DsP + tile * kDvTile;

  auto slot = [&](int b, int g) { return smem + b * W::STAGE + g * W::SLOT; };
  auto sKT = [&](int b, int g) { return reinterpret_cast<T*>(slot(b, g)); };
  auto sV = [&](int b, int g) { return reinterpret_cast<T*>(slot(b, g) + W::KT); };
  auto sG = [&](int b, int g) { return reinterpret_cast<float*>(slot(b, g) + W::KT + W::VT); };
  auto sHo = [&](int b, int g) { return reinterpret_cast<T*>(smem + 2 * W::STAGE + (b * G + g) * W::HT); };
  auto chunk_of = [&](int k) { return REV ? N - 1 - k : c0 + k; };   // the k-th chunk visited

  // segmented walk: the lanes of the first column wave of the first column tile keep the
  // running log2-decay of their rows over the segment's chunks
  const bool keep_pre = !REV && w.nseg > 1 && tile == 0 && (wave & 3) == 0 && grp == 0;
  float run[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) run[ib] = 0.f;
  f32x4 S[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + ri + 16 * ib + col, j = j0 + e;
      S[ib][e] = (w.init && seg == 0 && j < Ds && i < w.rows) ? w.init[walk_state_index(w, bh, i, j)] : 0.f;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);                   // initial state in before the pipeline starts

  Stage st[R][G];
  auto load = [&](Stage (&s)[G], int kg) {   // past the end: reload the last chunk
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int n = chunk_of(min(kg * G + g, N - 1)), row0 = n * C;
      s[g].load(mat + (size_t)n * SP * CP, src, row0, min(C, L - row0), Ds, tile, gam + (size_t)n * SP);
    }
  };
  auto store = [&](const Stage (&s)[G], int b) {
#pragma unroll
    for (int g = 0; g < G; ++g) s[g].store(sKT(b, g), sV(b, g), sG(b, g));
  };
#pragma unroll
  for (int r = 0; r < R; ++r) load(st[r], r);
  store(st[0], 0);
  __syncthreads();

  // One chunk group: its products from LDS, the sequential fold (which stages each state in
  // LDS), the next group's operands into the other LDS buffer, one barrier, the states out.  CHECK guards
  // the ragged end; the bulk of the walk runs unguarded, so the compiler can count the loads
  // and stores in flight exactly and never waits on the prefetch it has just issued.
  auto body = [&](auto rc, int kg, auto cc) {
    constexpr int r = decltype(rc)::value;
    constexpr bool CHECK = decltype(cc)::value;
    const int b = kg & 1;
    load(st[r], kg + R);                         // st[r] (group kg) is already in LDS
    f32x4 Tm[G][NIB];
#pragma unroll
    for (int g = 0; g < G; ++g) walk_product<T, RT, CP, RW, REV>(Tm[g], sKT(b, g), sV(b, g), ri, cw);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int k = kg * G + g;
      if (!CHECK || k < N) {
        const float* gg = sG(b, g);
        T* ho = sHo(b, g) + (ri + col) * LDV + cw + 4 * grp;
        if (!REV && keep_pre) {
#pragma unroll
          for (int ib = 0; ib < NIB; ++ib) {
            w.seg_prefix[((size_t)bh * NT_ + chunk_of(k)) * SP + i0 + ri + 16 * ib + col] = run[ib];
            run[ib] += gg[ri + 16 * ib + col];
          }
        }
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) {
          V4T hv;
          const float dec = fast_exp2(gg[ri + 16 * ib + col]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hv[e] = from_f32<T>(S[ib][e]);
            S[ib][e] = dec * S[ib][e] + Tm[g][ib][e];
          }
          *reinterpret_cast<V4T*>(ho + 16 * ib * LDV) = hv;
        }
      }
    }
    store(st[(r + 1) % R], b ^ 1);
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int k = kg * G + g;
      if (!CHECK || k < N) state_tile_out<T, RT, NT>(out + (size_t)chunk_of(k) * SP * DsP, sHo(b, g), LDV, DsP);
    }
  };
  // R consecutive groups, one per register stage (the r-th group in stage r)
  auto round = [&](int kg0, auto cc) {
    for_each_stage([&](auto rc) { body(rc, kg0 + decltype(rc)::value, cc); }, std::make_integer_sequence<int, R>{});
  };
  auto round_checked = [&](int kg0) {           // the ragged end: stop at the last group
    for_each_stage([&](auto rc) { if (kg0 + decltype(rc)::value < NG) body(rc, kg0 + decltype(rc)::value, std::true_type{}); },
                   std::make_integer_sequence<int, R>{});
  };
  const int full = (N / G) / R * R;              // groups walked without bounds checks
  int kg = 0;
  // The first round runs ahead of the loop, and the loop is reached only through it: every path
  // into a group's operand wait then has the previous group's state stores between that
  // group's loads and the wait, so the compiler's count leaves those stores in flight instead
  // of waiting for them.
  if (full >= R) {
    round(0, std::false_type{});
    for (kg = R; kg < full; kg += R) round(kg, std::false_type{});
  }
  for (; kg < NG; kg += R) round_checked(kg);
  if (w.nseg > 1) {
    if (keep_pre) {
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) w.seg_total[((size_t)bh * w.nseg + seg) * SP + i0 + ri + 16 * ib + col] = run[ib];
    }
    float* e_out = w.seg_end + (((size_t)bh * w.nseg + seg) * SP + i0 + ri) * DsP;
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib)
      *reinterpret_cast<f32x4*>(e_out + (size_t)(16 * ib + col) * DsP + j0) = S[ib];
  } else if (w.fin) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + ri + 16 * ib + col, j = j0 + e;
        if (i < w.rows && j < Ds) w.fin[walk_state_index(w, bh, i, j)] = S[ib][e];
      }
    }
  }
}

template <typename T, int SP, int RT, int CP, int G, bool REV, int NW>
__global__ __launch_bounds__(64 * NW) void walk_kernel(WalkIO w, int ntile) {
  walk_tile<T, SP, RT, CP, G, REV, NW>(w, ntile, xcd_remap(blockIdx.x, gridDim.x));
}

// several batches in one launch (see Batches): batch i owns blocks first[i] .. first[i+1] - 1;
// each batch has its own source width Ds (so its own count of 64-column tiles)
template <typename T, int SP, int RT, int CP, int G, bool REV, int NW>
__global__ __launch_bounds__(64 * NW) void walk_batches(Batches<WalkIO> b) {
  const int gi = b.find(blockIdx.x);
  walk_tile<T, SP, RT, CP, G, REV, NW>(b.p[gi], (b.p[gi].Ds + kDvTile - 1) / kDvTile, blockIdx.x - b.first[gi]);
}

template <typename T, int SP, int CP, bool REV>
hipError_t launch_walk(const WalkIO& w, int BH, hipStream_t s) {
  using P = WalkPlan<T, SP, CP>;
  if constexpr (!P::OK) {
    return hipErrorNotSupported;
  } else {
    const int ntile = (w.Ds + kDvTile - 1) / kDvTile;
    if constexpr (P::WIDE) {
      const int cus = device_cu_count();
      if (cus > 0 && ntile * (SP / 64) * BH >= cus) {
        hipLaunchKernelGGL((walk_kernel<T, SP, 64, CP, 2, REV, 8>), dim3(ntile * (SP / 64) * BH), dim3(512), 0, s,
                           w, ntile);
        return hipGetLastError();
      }
    }
    if constexpr (P::NARROW) {
      const int cus = device_cu_count();
      if (cus > 0 && ntile * (SP / 32) * BH < cus) {
        hipLaunchKernelGGL((walk_kernel<T, SP, 16, CP, 2, REV, 4>), dim3(ntile * (SP / 16) * BH), dim3(256), 0, s, w,
                           ntile);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((walk_kernel<T, SP, P::RT, CP, P::G, REV, 4>), dim3(ntile * (SP / P::RT) * BH), dim3(256), 0,
                       s, w, ntile);
    return hipGetLastError();
  }
}
// b.p[i] with BH[i] sequences each; the launch sets b.first
template <typename T, int SP, int CP>
hipError_t launch_walk_store_batches(Batches<WalkIO> b, const int* BH, hipStream_t s) {
  using P = WalkPlan<T, SP, CP>;
  if constexpr (!P::OK) {
    return hipErrorNotSupported;
  } else {
    b.first[0] = 0;
    for (int i = 0; i < b.n; ++i)
      b.first[i + 1] = b.first[i] + (b.p[i].Ds + kDvTile - 1) / kDvTile * (SP / P::RT) * BH[i];
    hipLaunchKernelGGL((walk_batches<T, SP, P::RT, CP, P::G, false, 4>), dim3(b.first[b.n]), dim3(256), 0, s, b);
    return hipGetLastError();
  }
}
template <typename T, int SP, int CP>
hipError_t launch_walk_store(const WalkIO& w, int BH, hipStream_t s) {
  return launch_walk<T, SP, CP, false>(w, BH, s);
}

// ----------------------------------------------------------------------------- segmented walk
// With few sequences the forward walk is a long chain of dependent steps on a fraction of the
// CUs.  Splitting each sequence's chunks into segments walked in parallel, each from a zero
// state (the first from the initial state), makes it nseg times shorter.  For chunk n of
// segment s the true chunk-start state is
//     H_n = H_n^seg + Diag(2^{P_n}) X_s,
// with H_n^seg what the segment's own walk stored, P_n the log2-decay of the segment's chunks
// before n (per row) and X_s the true state at the segment's start:
//     X_1 = E_0,   X_{s+1} = Diag(2^{D_s}) X_s + E_s,   final state = X_nseg,
// E_s being the segment's own end state and D_s its total log2-decay.  The segmented walk
// itself forms P and D, seg_carry_kernel X and the final state, and seg_fixup_kernel adds the
// carried part to the stored states.
struct SegParams {
  const float* gam;       // [BH][N][SP] chunk log2-decay per row
  const float* seg_end;   // [BH][nseg][SP][DsP] each segment's own end state (fp32)
  float* carry;           // [BH][nseg][SP][DsP] X_s (s >= 1)
  float* prefix;          // [BH][N][SP] P_n
  float* total;           // [BH][nseg][SP] D_s
  void* states;           // [BH][N][SP][DsP] chunk-start states (T), fixed up in place
  float* fin;             // [BH][rows][Ds] final state, or null
  int N, nseg, seg_len, rows, Ds, DsP;
};
constexpr int kMaxSeg = 8;

// grid (BH, SP / 16, DsP / 64): the carries for 16 rows and 64 columns, four columns a thread
template <int SP>
__global__ __launch_bounds__(256) void seg_carry_kernel(SegParams q) {
  const int bh = blockIdx.x, i = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int j = blockIdx.z * 64 + 4 * (threadIdx.x & 15);
  const size_t sstride = (size_t)SP * q.DsP;
  const size_t e0 = ((size_t)bh * q.nseg * SP + i) * q.DsP + j;
  f32x4 e[kMaxSeg];
  float d[kMaxSeg];
#pragma unroll
  for (int sg = 0; sg < kMaxSeg; ++sg) {
    if (sg < q.nseg) {
      e[sg] = *reinterpret_cast<const f32x4*>(q.seg_end + e0 + sg * sstride);
      d[sg] = fast_exp2(q.total[((size_t)bh * q.nseg + sg) * SP + i]);
    }
  }
  f32x4 x = e[0];
#pragma unroll
  for (int sg = 1; sg < kMaxSeg; ++sg) {
    if (sg < q.nseg) {
      *reinterpret_cast<f32x4*>(q.carry + e0 + sg * sstride) = x;
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = d[sg] * x[c] + e[sg][c];
    }
  }
  if (q.fin && i < q.rows) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (j + c < q.Ds) q.fin[((size_t)bh * q.rows + i) * q.Ds + j + c] = x[c];
  }
}

// grid (N - seg_len, BH): chunk seg_len + blockIdx.x (segments 1 ..) of sequence bh
template <typename T, int SP>
__global__ __launch_bounds__(256) void seg_fixup_kernel(SegParams q) {
  typedef typename V16<T>::type VT;
  constexpr int V = V16<T>::N;
  const int n = q.seg_len + blockIdx.x, bh = blockIdx.y, sg = n / q.seg_len;
  T* h = reinterpret_cast<T*>(q.states) + ((size_t)bh * q.N + n) * SP * q.DsP;
  const float* x = q.carry + ((size_t)bh * q.nseg + sg) * SP * q.DsP;
  const float* pre = q.prefix + ((size_t)bh * q.N + n) * SP;
  const int per_row = q.DsP / V;
  for (int idx = threadIdx.x; idx < SP * per_row; idx += 256) {
    const int i = idx / per_row, c = (idx - i * per_row) * V;
    const float sc = fast_exp2(pre[i]);
    VT hv = *reinterpret_cast<const VT*>(h + (size_t)i * q.DsP + c);
#pragma unroll
    for (int e4 = 0; e4 < V / 4; ++e4) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(x + (size_t)i * q.DsP + c + 4 * e4);
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[4 * e4 + e] = from_f32<T>(to_f32(hv[4 * e4 + e]) + sc * xv[e]);
    }
    *reinterpret_cast<VT*>(h + (size_t)i * q.DsP + c) = hv;
  }
}

// Tile height of a segmented walk.  The segments supply the parallelism, so the tile is the
// tallest that fits: for the same number of resident workgroups the chunks then split into more
// segments, each a shorter chain of sequential steps, and each chunk's source rows are fetched
// by fewer workgroups.  64-row tiles run 8 waves, 32- and 16-row tiles 4; PER_CU is how many
// workgroups a CU's LDS holds.
template <typename T, int SP, int CP, int RT>
struct SegTileCfg {
  static constexpr int NW = RT == 64 ? 8 : 4;
  static constexpr size_t BYTES = WalkIOCfg<T, RT, CP, 2, 64 * NW>::BYTES;
  static constexpr bool OK = RT <= SP && SP % RT == 0 && BYTES <= kMaxLds;
  static constexpr int PER_CU = OK ? (int)(kMaxLds / BYTES) : 0;
};
template <typename T, int SP, int CP>
struct SegTile {
  static constexpr int RT = SegTileCfg<T, SP, CP, 64>::OK ? 64 : SegTileCfg<T, SP, CP, 32>::OK ? 32 : 16;
  using Cf = SegTileCfg<T, SP, CP, RT>;
};

// Segments of a sequence for a forward walk of BH sequences of N chunks, given room for up to
// seg_max: split only when even the 16-row plain walk leaves CUs idle; then as many segments as
// the resident workgroups of the segmented tile allow, at least 8 chunks each.  1 = no split.
template <typename T, int SP, int CP>
int walk_segments(int BH, int Ds, int N, int seg_max) {
  using P = WalkPlan<T, SP, CP>;
  using S = typename SegTile<T, SP, CP>::Cf;
  if constexpr (!P::NARROW || !S::OK) {
    return 1;
  } else {
    const int cus = device_cu_count();
    const int ntile = (Ds + kDvTile - 1) / kDvTile;
    const int grid16 = ntile * (SP / 16) * BH;
    if (cus <= 0 || seg_max < 2 || grid16 >= cus) return 1;
    const int grid = ntile * (SP / SegTile<T, SP, CP>::RT) * BH;    // one segment's workgroups
    int ns = min(min(seg_max, kMaxSeg), max(1, S::PER_CU * cus / grid));
    ns = min(ns, N / 8);
    if (ns < 2) return 1;
    const int len = (N + ns - 1) / ns;
    return (N + len - 1) / len;            // no empty trailing segment
  }
}

// The forward walk in nseg segments (nseg from walk_segments, >= 2; it also leaves the decay
// prefixes and totals), then the carries and the fix-up: w.states and w.fin end as the plain walk would leave them.
// Scratch: seg_end and carry [BH][nseg][SP][DsP] fp32, prefix [BH][N][SP] fp32, total
// [BH][nseg][SP] fp32.
// fixup = false leaves the stored states without their carried part, for a consumer that adds
// it itself (the forward's output kernel).
template <typename T, int SP, int CP>
hipError_t launch_walk_store_segmented(WalkIO w, int BH, int nseg, float* seg_end, float* carry, float* prefix,
                                       float* total, bool fixup, hipStream_t s) {
  using P = WalkPlan<T, SP, CP>;
  constexpr int RT = SegTile<T, SP, CP>::RT, NW = SegTile<T, SP, CP>::Cf::NW;
  if constexpr (!P::NARROW || !SegTile<T, SP, CP>::Cf::OK) {
    return hipErrorNotSupported;
  } else {
    const int ntile = (w.Ds + kDvTile - 1) / kDvTile, DsP = ntile * kDvTile;
    w.nseg = nseg;
    w.seg_len = (w.N + nseg - 1) / nseg;
    w.seg_end = seg_end;
    w.seg_prefix = prefix;
    w.seg_total = total;
    hipLaunchKernelGGL((walk_kernel<T, SP, RT, CP, 2, false, NW>), dim3(ntile * (SP / RT) * BH * nseg), dim3(64 * NW),
                       0, s, w, ntile);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SegParams q{w.gam, seg_end, carry, prefix, total, w.states, w.fin, w.N, nseg, w.seg_len, w.rows, w.Ds, DsP};
    hipLaunchKernelGGL((seg_carry_kernel<SP>), dim3(BH, SP / 16, ntile), dim3(256), 0, s, q);
    if ((e = hipGetLastError()) != hipSuccess || !fixup) return e;
    hipLaunchKernelGGL((seg_fixup_kernel<T, SP>), dim3(w.N - w.seg_len, BH), dim3(256), 0, s, q);
    return hipGetLastError();
  }
}
template <typename T, int SP, int CP>
hipError_t launch_walk_reverse(const WalkIO& w, int BH, hipStream_t s) {
  return launch_walk<T, SP, CP, true>(w, BH, s);
}

}  // namespace gla
