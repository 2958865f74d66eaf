// gla_fwd.hip -- chunkwise GLA forward on gfx950.
//
// Three kernel phases per call:
//   1. gla_prep_kernel  (grid N x BH): per chunk, the decayed operands Qs, KdT, Gamma and the
//      masked intra-chunk scores A (prep.hpp).  Fully parallel over chunks.
//   2. state walk       (walks.hpp): the only sequential part -- H_{n+1} = Diag(2^Gamma_n) H_n
//      + KdT_n V_n over the chunks of each (batch*head), held in fp32 matrix-core
//      accumulators, writing the chunk-start states H_n (and the final state).
//   3. gla_fwd_out      (grid N x BH x ceil(Dv/64)): the chunk outputs
//          O_n = Qs_n H_n + A_n V_n
//      fully parallel over chunks and value tiles.
// This follows the chunkwise training form (MS-GLA summary, section 2.1): sequential
// inter-chunk updates, parallel intra-chunk computation.  The chunk-start states cost one
// write and one read of B*H*N*Dk*Dv elements; in exchange the sequential walk carries only
// the state update, so it is short per step and every matrix product of the outputs runs at
// full occupancy.  Where 32-column tiles give every CU a workgroup, phases 2 and 3 run as one
// kernel instead (walk_out.hpp), which never reads the states back.  A forward that keeps its
// activations for the backward leaves the states where the backward finds them.
#include "walk_out.hpp"

namespace gla {

// One output workgroup: O [CP rows][64 columns] of one chunk.  Wave w owns the 16-row blocks
// w, w+4, ... of O across all 64 columns.  Its row operands (Qs, A rows) are loaded straight
// from global memory into registers -- each row block is read by exactly one wave -- while the
// column operands every wave shares (H_n [DKP][64], V [CP][64]) are staged in LDS and read
// with transposing LDS reads.
template <typename T, int DKP, int CP>
struct OutCfg {
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int LDV = kDvTile + V;
  static constexpr size_t HT = (size_t)DKP * LDV * sizeof(T);
  static constexpr size_t VT = (size_t)CP * LDV * sizeof(T);
  static constexpr size_t OT = (size_t)CP * LDV * sizeof(T);
  static constexpr size_t BYTES = HT + VT > OT ? HT + VT : OT;   // O staging reuses H, V
  static constexpr int NH = DKP * kDvTile / V, NV = CP * kDvTile / V;
  static constexpr int PH = (NH + 255) / 256, PV = (NV + 255) / 256;
  static constexpr int NBR = CP / 16, RBW = (NBR + 3) / 4;       // row blocks, per wave
};

// SEGC: the states come from a segmented walk without their carried part (FwdParams::seg_carry)
// HOLD: O is written to the tokens that hold it (FwdParams::hold_o) instead of to p.o
template <typename T, int DKP, int CP, bool SEGC = false, bool HOLD = false>
__device__ __forceinline__ void fwd_out_block(const FwdParams& p, int ntile, int lin) {
  using W = OutCfg<T, DKP, CP>;
  constexpr int LDV = W::LDV, V = W::V, NBR = W::NBR, RBW = W::RBW;
  constexpr int NKB = DKP / 32, NCB = CP / 32, NJB = kDvTile / 16;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) char smem[W::BYTES];
  T* sH = reinterpret_cast<T*>(smem);
  T* sV = reinterpret_cast<T*>(smem + W::HT);

  const int tile = lin % ntile, n = (lin / ntile) % p.N, bh = lin / (ntile * p.N);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int Dv = p.Dv, L = p.L, DvP = ntile * kDvTile;
  const int row0 = n * p.C, len = min(p.C, L - row0);
  const size_t chunk = (size_t)bh * p.N + n;
  const T* Qc = reinterpret_cast<const T*>(p.ops.Qs) + chunk * CP * DKP;
  const T* Ac = reinterpret_cast<const T*>(p.ops.A) + chunk * CP * CP;
  const T* Hc = reinterpret_cast<const T*>(p.Hs) + chunk * DKP * DvP + tile * kDvTile;
  const T* vg = reinterpret_cast<const T*>(p.v) + ((size_t)p.in(bh) * L + row0) * Dv;

  // all loads first: shared tiles (16-byte vectors; value rows past the chunk end and columns
  // past Dv come from clamped addresses and are zeroed when stored), then this wave's row
  // operands as matrix-core fragments
  VT h[W::PH], v[W::PV];
  bool vok[W::PV];
  constexpr int PER_ROW = kDvTile / V;
#pragma unroll
  for (int m = 0; m < W::PH; ++m) {
    const int idx = min(tid + 256 * m, W::NH - 1), r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
    h[m] = *reinterpret_cast<const VT*>(Hc + (size_t)r * DvP + c);
  }
#pragma unroll
  for (int m = 0; m < W::PV; ++m) {
    const int idx = tid + 256 * m, r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
    const int j = tile * kDvTile + c;
    vok[m] = idx < W::NV && r < len && j < Dv;
    v[m] = *reinterpret_cast<const VT*>(vg + (size_t)min(r, len - 1) * Dv + min(j, Dv - V));
  }
  // a segmented walk stored this state without the part carried in from before its segment:
  // its rows of X_s and the decay 2^{P_n} are fetched with the rest
  f32x4 xc[SEGC ? W::PH : 1][V / 4];
  float sc[SEGC ? W::PH : 1];
  const bool carried = SEGC && n >= p.seg_len;
  if constexpr (SEGC) {
    const int sg = carried ? n / p.seg_len : 0;
    const float* X = p.seg_carry + ((size_t)bh * p.seg_n + sg) * DKP * DvP + tile * kDvTile;
    const float* Pn = p.seg_prefix + chunk * DKP;
#pragma unroll
    for (int m = 0; m < W::PH; ++m) {
      const int idx = min(tid + 256 * m, W::NH - 1), r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
      sc[m] = Pn[r];
#pragma unroll
      for (int e4 = 0; e4 < V / 4; ++e4) xc[m][e4] = *reinterpret_cast<const f32x4*>(X + (size_t)r * DvP + c + 4 * e4);
    }
  }
  Frag<T> xq[RBW][NKB], xa[RBW][NCB];
#pragma unroll
  for (int s = 0; s < RBW; ++s) {
    const int rb = min(wave + 4 * s, NBR - 1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) xq[s][kb] = ld8(Qc + (16 * rb + col) * DKP + 32 * kb + 8 * grp);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) xa[s][cb] = ld8(Ac + (16 * rb + col) * CP + 32 * cb + 8 * grp);
  }
  if constexpr (SEGC) {
    if (carried) {   // H_n += Diag(2^{P_n}) X_s
#pragma unroll
      for (int m = 0; m < W::PH; ++m) {
        const float f = fast_exp2(sc[m]);
#pragma unroll
        for (int e4 = 0; e4 < V / 4; ++e4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) h[m][4 * e4 + e] = from_f32<T>(to_f32(h[m][4 * e4 + e]) + f * xc[m][e4][e]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < W::PH; ++m) {
    const int idx = tid + 256 * m;
    if (idx < W::NH) {
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
      *reinterpret_cast<VT*>(sH + r * LDV + c) = h[m];
    }
  }
#pragma unroll
  for (int m = 0; m < W::PV; ++m) {
    const int idx = tid + 256 * m;
    if (idx < W::NV) {
      const int r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
      *reinterpret_cast<VT*>(sV + r * LDV + c) = vok[m] ? v[m] : zero_vec<T>();
    }
  }
  __syncthreads();

  // O = Qs H + A V
  f32x4 O[RBW][NJB];
#pragma unroll
  for (int s = 0; s < RBW; ++s) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) O[s][jb] = zero4();
  }
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Frag<T> Yh = ld8_colblk(sH + (32 * kb) * LDV + 16 * jb, LDV);
#pragma unroll
      for (int s = 0; s < RBW; ++s) mma(O[s][jb], xq[s][kb], Yh);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const Frag<T> Yv = ld8_colblk(sV + (32 * cb) * LDV + 16 * jb, LDV);
#pragma unroll
      for (int s = 0; s < RBW; ++s) mma(O[s][jb], xa[s][cb], Yv);
    }
  }
  __syncthreads();   // H and V are consumed: stage O in their place for 16-byte stores
  T* sO = reinterpret_cast<T*>(smem);
#pragma unroll
  for (int s = 0; s < RBW; ++s) {
    const int rb = wave + 4 * s;
    if (rb < NBR) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sO[(16 * rb + 4 * grp + e) * LDV + 16 * jb + col] = from_f32<T>(O[s][jb][e]);
      }
    }
  }
  __syncthreads();
  if constexpr (HOLD) {
    // rows row0 .. row0 + len - 1 go to the tokens t with (t + 1) / s - 1 among them, scaled by
    // the token's weight; chunk 0 also writes the zeros of the tokens before the first block
    const int s = p.hold_s, Lf = p.hold_L;
    const int t_beg = n == 0 ? 0 : (row0 + 1) * s - 1;
    const int t_end = min((row0 + len + 1) * s - 1, Lf);
    const int b = bh / p.hold_nh, h = p.hold_h0 + bh % p.hold_nh;
    T* og = reinterpret_cast<T*>(p.hold_o) + ((size_t)b * p.hold_H + h) * Lf * Dv;
    const float* wg = p.hold_w ? p.hold_w + (size_t)b * Lf * p.hold_ng + p.hold_gi : nullptr;
    // the weights of 256 tokens at a time go to LDS with one load per thread, so that no
    // store waits on a load of its own
    __shared__ float sW[256];
    for (int tb = t_beg; tb < t_end; tb += 256) {
      const int nt = min(256, t_end - tb);
      if (tb > t_beg) __syncthreads();   // the previous tokens' weights are read
      if (tid < nt) sW[tid] = wg ? wg[(size_t)(tb + tid) * p.hold_ng] : 1.f;
      __syncthreads();
      for (int idx = tid; idx < nt * PER_ROW; idx += 256) {
        const int q = idx / PER_ROW, c = (idx - q * PER_ROW) * V;
        const int t = tb + q, r = (t + 1) / s - 1 - row0, jj = tile * kDvTile + c;
        if (jj < Dv) {
          VT y = zero_vec<T>();
          if (r >= 0) {
            const float wt = sW[q];
            const VT x = *reinterpret_cast<const VT*>(sO + r * LDV + c);
#pragma unroll
            for (int e = 0; e < V; ++e) y[e] = from_f32<T>(wt * to_f32(x[e]));
          }
          *reinterpret_cast<VT*>(og + (size_t)t * Dv + jj) = y;
        }
      }
    }
  } else {
    T* og = reinterpret_cast<T*>(p.o) + ((size_t)bh * L + row0) * Dv;
#pragma unroll
    for (int m = 0; m < (CP * PER_ROW + 255) / 256; ++m) {
      const int idx = tid + 256 * m, r = idx / PER_ROW, c = (idx - r * PER_ROW) * V;
      const int j = tile * kDvTile + c;
      if (idx < CP * PER_ROW && r < len && j < Dv)
        *reinterpret_cast<VT*>(og + (size_t)r * Dv + j) = *reinterpret_cast<const VT*>(sO + r * LDV + c);
    }
  }
}

// grid ntile * N * BH; the ntile value tiles of one chunk are consecutive after the XCD
// remapping, so they share an XCD's L2 for Qs and A
template <typename T, int DKP, int CP, bool SEGC = false>
__global__ __launch_bounds__(256) void gla_fwd_out(FwdParams p, int ntile) {
  fwd_out_block<T, DKP, CP, SEGC>(p, ntile, xcd_remap(blockIdx.x, gridDim.x));
}

// several batches in one launch (see Batches): batch i owns blocks first[i] .. first[i+1] - 1
template <typename T, int DKP, int CP, bool HOLD>
__global__ __launch_bounds__(256) void gla_fwd_out_batches(Batches<FwdParams> b, int ntile) {
  const int gi = b.find(blockIdx.x);
  fwd_out_block<T, DKP, CP, false, HOLD>(b.p[gi], ntile, blockIdx.x - b.first[gi]);
}

template <typename T, int DKP, int CP>
constexpr bool fwd_fits() {
  return PrepCfg<T, DKP, CP>::BYTES <= kMaxLds && walk_fits<T, DKP, CP>() && OutCfg<T, DKP, CP>::BYTES <= kMaxLds;
}

template <typename T, int DKP, int CP>
hipError_t launch_gla_fwd(const FwdParams& p, hipStream_t s) {
  if constexpr (!fwd_fits<T, DKP, CP>()) {
    return hipErrorNotSupported;
  } else {
    PrepParams pp{p.q, p.k, p.g, p.ops, p.L, p.Dk, p.C, p.N, p.in};
    record_event(p.events, 0, s);
    hipError_t e = p.ops_ready ? hipSuccess : launch_prep<T, DKP, CP>(pp, p.BH, s);
    if (e != hipSuccess) return e;
    record_event(p.events, 1, s);
    // Enough sequences to give every CU a workgroup of 32 value columns: the walk and the
    // outputs run as one kernel (walk_out.hpp), which writes the states only if they are kept;
    // its time is recorded as the walk's and the output kernel's as zero
    if constexpr (walk_out_fits<T, DKP, CP>()) {
      if (!p.states_ready && !p.hold_o && walk_out_applies(p.BH, p.Dv, p.keep_states)) {
        FwdParams pf = p;
        if (!p.keep_states) pf.Hs = nullptr;
        if ((e = launch_walk_out<T, DKP, CP>(pf, s)) != hipSuccess) return e;
        record_event(p.events, 2, s);
        record_event(p.events, 3, s);
        return hipSuccess;
      }
    }
    WalkIO wf{p.ops.KdT, p.v, p.ops.Gam, p.Hs, p.h0, p.ht, p.Dk, p.Dv, p.L, p.C, p.N, 0, p.in};
    // few, long sequences: the walk runs in segments and the output kernel adds each state's
    // carried part as it stages it (these states serve only that kernel)
    const int nseg = p.seg_ws && !p.states_ready ? walk_segments<T, DKP, CP>(p.BH, p.Dv, p.N, p.seg_max) : 1;
    FwdParams po = p;
    if (p.states_ready) {
      // the caller's walk already left the chunk-start states (GSA's pass 2)
    } else if (nseg >= 2) {
      const size_t part = (size_t)p.BH * p.seg_max * DKP * ((p.Dv + kDvTile - 1) / kDvTile * kDvTile);
      float* prefix = p.seg_ws + 2 * part;
      float* total = prefix + (size_t)p.BH * p.N * DKP;
      if ((e = launch_walk_store_segmented<T, DKP, CP>(wf, p.BH, nseg, p.seg_ws, p.seg_ws + part, prefix, total, false,
                                                       s)) != hipSuccess)
        return e;
      po.seg_carry = p.seg_ws + part;
      po.seg_prefix = prefix;
      po.seg_len = (p.N + nseg - 1) / nseg;
      po.seg_n = nseg;
    } else if ((e = launch_walk_store<T, DKP, CP>(wf, p.BH, s)) != hipSuccess) {
      return e;
    }
    record_event(p.events, 2, s);
    const int ntile = (p.Dv + kDvTile - 1) / kDvTile;
    if (po.seg_carry)
      hipLaunchKernelGGL((gla_fwd_out<T, DKP, CP, true>), dim3(ntile * p.N * p.BH), dim3(256), 0, s, po, ntile);
    else
      hipLaunchKernelGGL((gla_fwd_out<T, DKP, CP>), dim3(ntile * p.N * p.BH), dim3(256), 0, s, po, ntile);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    record_event(p.events, 3, s);
    return hipSuccess;
  }
}

// The forward of nb independent batches (same T, Dk, Dv, C; each with its own inputs, sequence
// view, workspace and outputs) with three launches in all.
template <typename T, int DKP, int CP>
hipError_t launch_gla_fwd_batches(const FwdParams* ps, int nb, hipStream_t s) {
  if constexpr (!fwd_fits<T, DKP, CP>()) {
    return hipErrorNotSupported;
  } else {
    if (nb < 1 || nb > kMaxBatches) return hipErrorInvalidValue;
    Batches<PrepParams> bp{};
    Batches<WalkIO> bw{};
    Batches<FwdParams> bo{};
    bp.n = bw.n = bo.n = nb;
    int BH[kMaxBatches], maxN = 0;
    const int ntile = (ps[0].Dv + kDvTile - 1) / kDvTile;
    bp.first[0] = bo.first[0] = 0;
    for (int i = 0; i < nb; ++i) {
      const FwdParams& p = ps[i];
      if (p.Dk != ps[0].Dk || p.Dv != ps[0].Dv || p.C != ps[0].C || !p.hold_o != !ps[0].hold_o)
        return hipErrorInvalidValue;
      bp.p[i] = PrepParams{p.q, p.k, p.g, p.ops, p.L, p.Dk, p.C, p.N, p.in};
      bw.p[i] = WalkIO{p.ops.KdT, p.v, p.ops.Gam, p.Hs, p.h0, p.ht, p.Dk, p.Dv, p.L, p.C, p.N, 0, p.in};
      bo.p[i] = p;
      BH[i] = p.BH;
      maxN = p.N > maxN ? p.N : maxN;
      bp.first[i + 1] = bp.first[i] + p.BH;
      bo.first[i + 1] = bo.first[i] + ntile * p.N * p.BH;
    }
    hipError_t e;
    if ((e = launch_prep_batches<T, DKP, CP>(bp, maxN, s)) != hipSuccess) return e;
    if ((e = launch_walk_store_batches<T, DKP, CP>(bw, BH, s)) != hipSuccess) return e;
    if (ps[0].hold_o)
      hipLaunchKernelGGL((gla_fwd_out_batches<T, DKP, CP, true>), dim3(bo.first[nb]), dim3(256), 0, s, bo, ntile);
    else
      hipLaunchKernelGGL((gla_fwd_out_batches<T, DKP, CP, false>), dim3(bo.first[nb]), dim3(256), 0, s, bo, ntile);
    return hipGetLastError();
  }
}

bool fwd_fused(int esize, int DKP, int CP, int BH, int Dv, bool keep_states) {
  bool fits = false;
#define GLA_FUSED_CASE(D, C_) \
  if (esize == (int)sizeof(bf16) && DKP == D && CP == C_) fits = walk_out_fits<bf16, D, C_>();
  GLA_FUSED_CASE(128, 64)
#undef GLA_FUSED_CASE
  return fits && walk_out_applies(BH, Dv, keep_states);
}

bool fwd_config_fits(int esize, int DKP, int CP) {
  bool ok = false;
#define GLA_FIT_CASE(TT, D, C_)                                                       \
  if (esize == (int)sizeof(TT) && DKP == D && CP == C_)                               \
    ok = fwd_fits<TT, D, C_>();
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

#define GLA_FWD_INST(TT, D, C_)                                                     \
  template hipError_t launch_gla_fwd<TT, D, C_>(const FwdParams&, hipStream_t); \
  template hipError_t launch_gla_fwd_batches<TT, D, C_>(const FwdParams*, int, hipStream_t);
#define GLA_FWD_INST_T(TT)                                                     \
  GLA_FWD_INST(TT, 32, 32) GLA_FWD_INST(TT, 32, 64) GLA_FWD_INST(TT, 32, 128)  \
  GLA_FWD_INST(TT, 64, 32) GLA_FWD_INST(TT, 64, 64) GLA_FWD_INST(TT, 64, 128)  \
  GLA_FWD_INST(TT, 128, 32) GLA_FWD_INST(TT, 128, 64) GLA_FWD_INST(TT, 128, 128) \
  GLA_FWD_INST(TT, 256, 32) GLA_FWD_INST(TT, 256, 64)
GLA_FWD_INST_T(bf16)
GLA_FWD_INST_T(float)

}  // namespace gla
