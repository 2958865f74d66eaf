// prep.hpp -- chunk preparation kernel shared by the GLA forward and backward.
//
// For one (batch*head, chunk) it forms, from q, k and the log gates g:
//   b      chunk-local inclusive prefix sum of g, in log2 units (b = log2(e) * cumsum g)
//   Gamma  b at the chunk's last row (the chunk's total log2-decay per key channel)
//   Qs     = q * 2^{b}                 (the query seen from the chunk start)
//   KdT    = (k * 2^{Gamma - b})^T     (the key decayed to the chunk end; transposed)
//   A[r,c] = sum_i q_r[i] k_c[i] 2^{b_r[i] - b_c[i]} for c <= r, else 0
// which are the inputs of the state walk (Gamma, KdT), the chunk outputs (Qs, A) and, for
// the backward, the reverse state walk (Gamma, Qs).  The decomposition into chunks with a
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
//
// Memory access: every thread owns V = 16/sizeof(T) adjacent key channels of a few chunk
// rows, loads its q, k, g vectors with 16-byte accesses issued together, and scans its rows
// locally; segment totals are combined through LDS.  Qs leaves straight from registers with
// 16-byte stores; KdT and A are staged in LDS so their stores are 16-byte and coalesced.
#pragma once
#include <atomic>
#include "common.hpp"
#include "kernels.hpp"

namespace gla {

constexpr float kSpanLimit = 32.0f;

struct PrepParams {
  const void *q, *k, *g;
  ChunkOps ops;
  int L, Dk, C, N;
  SeqView in;     // input sequences of q, k, g
};

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
constexpr int imin(int a, int b) { return a < b ? a : b; }

// Thread -> (channel group, row segment) map for the element-wise phase of a chunk, for a
// workgroup of NT threads.
template <typename T, int DKP, int CP, int NT = 256>
struct ChunkMap {
  static constexpr int V = 16 / (int)sizeof(T);        // channels per thread (one 16-byte vector)
  static constexpr int NCG = DKP / V;                  // channel groups
  static constexpr int NSEG = imin(NT / NCG, CP);      // row segments
  static constexpr int RPS = CP / NSEG;                // rows per segment
  static constexpr int ACTIVE = NCG * NSEG;            // threads with work (<= NT)
};

// Threads of the preparation kernel: 256 (4 waves), two workgroups to a CU; 512 (8 waves) for
// 16-bit inputs with 256-channel keys and chunks of at most 64 rows, whose 136 KB of LDS leave
// room for one workgroup per CU: 256 threads would then keep only four waves on a CU, each
// carrying eight rows of the chunk (1.3B-layer shape: 61 -> 47 us).  At 128 channels the
// 512-thread form measured no faster than two 256-thread workgroups per CU.
template <typename T, int DKP, int CP>
constexpr int prep_threads() { return sizeof(T) == 2 && CP <= 64 && DKP >= 256 ? 512 : 256; }

template <typename T, int DKP, int CP>
struct PrepCfg {
  static constexpr int NT = prep_threads<T, DKP, CP>(), NW = NT / 64;
  using M = ChunkMap<T, DKP, CP, NT>;
  static constexpr int PK = 16 / (int)sizeof(T);       // 16-byte row padding, in elements
  static constexpr int LDQ = DKP + PK;                 // row stride of the [CP][DKP] tiles
  static constexpr int LDC = CP + PK;                  // row stride of the [CP][CP] score tile
  static constexpr int LDP = 32 + PK;                  // row stride of the safe-path slice tiles
  static constexpr int NB = CP / 16;                   // 16-row sub-chunks per chunk
  static constexpr int NP = NB * (NB - 1) / 2;         // off-diagonal sub-block pairs
  static constexpr int PPW = (NP + NW - 1) / NW;       // pairs per wave
  static constexpr bool SPLIT = sizeof(T) == 2;        // hi/lo operands ("Precision of A")
  static constexpr size_t TILE = (size_t)CP * LDQ * sizeof(T);
  static constexpr size_t KD = TILE;                   // Kd [CP][DKP], copied out transposed
  static constexpr size_t ATILE = (size_t)CP * LDC * sizeof(T);
  // fast path: sQ, sK (+ sQl, sKl); after the score product the same bytes hold Kd and A
  static constexpr size_t FAST = (SPLIT ? 4 : 2) * TILE;
  static constexpr size_t SAFE = TILE + (size_t)3 * CP * 33 * 4 +
                                 (size_t)(SPLIT ? 2 : 1) * (CP + 16) * LDP * sizeof(T);
  // the gate scan's segment totals ([NSEG][DKP] fp32) use the main region, which is free
  // while a chunk's gates are scanned; Gamma and the block-max scratch stay apart
  static constexpr size_t MAIN = cmax(cmax(cmax(FAST, SAFE), TILE + KD + ATILE), (size_t)M::NSEG * DKP * 4);
  static constexpr size_t MISC = (size_t)(DKP + 8) * 4;
  static constexpr size_t BYTES = MAIN + MISC;
  // A persistent grid (each chunk's loads in flight during the previous chunk's work) for
  // 256-thread workgroups, except fp32 with the widest keys, whose registers cannot carry the
  // next chunk's loads; and for 512-thread workgroups only where a CU holds one of them: two
  // share a CU otherwise and overlap one another's loads and work, in 128 registers that leave
  // no room for a second chunk's loads.
  static constexpr bool PERSIST = NT == 512 ? BYTES > kMaxLds / 2 : (sizeof(T) == 2 || DKP <= 128);
  static constexpr int MIN_WAVES = NT == 512 && !PERSIST ? 4 : 2;   // per SIMD, for the registers
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
// Copy a dense global [rows][cols] tile into LDS (row stride lds), 16 bytes per access.
template <typename T>
__device__ __forceinline__ void tile_in_dense(T* dst, const T* __restrict__ src, int rows, int cols, int lds) {
  constexpr int V = V16<T>::N;
  typedef typename V16<T>::type VT;
  const int per_row = cols / V;
  for (int idx = threadIdx.x; idx < rows * per_row; idx += blockDim.x) {
    const int r = idx / per_row, c = (idx - r * per_row) * V;
    *reinterpret_cast<VT*>(dst + r * lds + c) = *reinterpret_cast<const VT*>(src + (size_t)r * cols + c);
  }
}
// Copy the transpose of a [rows][cols] LDS tile to dense global [cols][rows] with transposing
// LDS reads: each lane gathers eight consecutive rows of one column (a matrix-core column
// fragment, ld8_colblk) and writes them as one contiguous run.  Element-wise column reads
// and column writes of such tiles hit few LDS banks.  NW waves; rows % 32 == 0,
// cols % 16 == 0, lds * sizeof(T) % 8 == 0.
template <typename T, int NW>
__device__ __forceinline__ void tile_out_t(T* __restrict__ dst, const T* src, int rows, int cols, int lds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int nrb = rows / 32, nblk = nrb * (cols / 16);
  for (int blk = wave; blk < nblk; blk += NW) {
    const int rb = blk % nrb, cb = blk / nrb;
    const Frag<T> f = ld8_colblk(src + (32 * rb) * lds + 16 * cb, lds);
    *reinterpret_cast<decltype(f.v)*>(dst + (size_t)(16 * cb + col) * rows + 32 * rb + 8 * grp) = f.v;
  }
}

__device__ __forceinline__ void pair_decode(int p, int& x, int& y) {
  x = 1;
  while ((x * (x + 1)) / 2 <= p) ++x;
  y = p - (x * (x - 1)) / 2;
}

template <typename T>
__device__ __forceinline__ typename V16<T>::type zero_vec() {
  typename V16<T>::type z;
#pragma unroll
  for (int e = 0; e < V16<T>::N; ++e) z[e] = from_f32<T>(0.f);
  return z;
}

// In-place exclusive scan along the NSEG segment totals of each channel of an [NSEG][width]
// array: prefix (sum over earlier segments) or suffix (sum over later segments).  One thread
// per channel, all NSEG values read into registers first, so the cost is one LDS round trip
// instead of a per-thread loop over segments.  The caller synchronises before and after.
template <int NSEG>
__device__ __forceinline__ void seg_scan_channel(float* a, int width, int ch, bool suffix) {
  float v[NSEG];
#pragma unroll
  for (int s = 0; s < NSEG; ++s) v[s] = a[s * width + ch];
  float run = 0.f;
  if (suffix) {
#pragma unroll
    for (int s = NSEG - 1; s >= 0; --s) {
      const float x = v[s];
      a[s * width + ch] = run;
      run += x;
    }
  } else {
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const float x = v[s];
      a[s * width + ch] = run;
      run += x;
    }
  }
}

// Chunk-local gate scan for the thread's (channel group, row segment): loads g, k, q
// vectors (16-byte, all issued before first use, g first), keeps b (log2 units) and the raw q
// and k of its rows and channels, publishes Gamma in sGam and returns the block-wide max |b|.
// load() only issues the loads -- unconditionally, from clamped in-bounds addresses, with the
// validity kept beside them -- so a kernel can put other independent loads in flight before
// finish() consumes the gates; kvals() and qvals() convert k and q when they are needed.
// run() is load(), finish(), kvals() and qvals().  finish() must be called by all NT threads.
// With LOAD_QK = false only g is loaded, and qv holds the raw gate values.
template <typename T, int DKP, int CP, bool LOAD_QK = true, int NT = 256>
struct ChunkScan {
  using M = ChunkMap<T, DKP, CP, NT>;
  static constexpr int V = M::V, RPS = M::RPS;
  typedef typename V16<T>::type VT;
  float b[RPS][V];
  float qv[RPS][V];
  float kv[RPS][V];
  int cg, seg;
  bool active;
  VT gvec[RPS], qvec[RPS], kvec[RPS];
  bool ok[RPS];

  // ld: row stride of q, k, g (elements); width: valid channels from the base pointer
  // tid: the thread's index (threadIdx.x)
  __device__ __forceinline__ void load(const T* qg, const T* kg, const T* gg, int ld, int width, int len,
                                       int tid = threadIdx.x) {
    cg = tid % M::NCG;
    seg = tid / M::NCG;
    active = tid < M::ACTIVE;
    const bool chv = active && cg * V < width;
    const int cc = chv ? cg * V : 0;
    // g first: the scan needs only the gates, and loads complete in issue order
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const int r = seg * RPS + u;
      ok[u] = chv && r < len;
      gvec[u] = *reinterpret_cast<const VT*>(gg + (size_t)min(r, len - 1) * ld + cc);
    }
    if constexpr (LOAD_QK) {
#pragma unroll
      for (int u = 0; u < RPS; ++u)
        kvec[u] = *reinterpret_cast<const VT*>(kg + (size_t)min(seg * RPS + u, len - 1) * ld + cc);
#pragma unroll
      for (int u = 0; u < RPS; ++u)
        qvec[u] = *reinterpret_cast<const VT*>(qg + (size_t)min(seg * RPS + u, len - 1) * ld + cc);
    }
  }

  // k and q as fp32 (zero outside the chunk and the channel range); separate from finish() so
  // that the scan does not wait for them
  __device__ __forceinline__ void kvals() {
    if constexpr (LOAD_QK) {
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
#pragma unroll
        for (int e = 0; e < V; ++e) kv[u][e] = ok[u] ? to_f32(kvec[u][e]) : 0.f;
      }
    }
  }
  __device__ __forceinline__ void qvals() {
    if constexpr (LOAD_QK) {
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
#pragma unroll
        for (int e = 0; e < V; ++e) qv[u][e] = ok[u] ? to_f32(qvec[u][e]) : 0.f;
      }
    }
  }

  __device__ __forceinline__ float finish(float* segtot, float* sGam, float* red, int tid = threadIdx.x) {
    float run_[V];
#pragma unroll
    for (int e = 0; e < V; ++e) run_[e] = 0.f;
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float gv = ok[u] ? to_f32(gvec[u][e]) : 0.f;
        run_[e] += gv * kLog2e;
        b[u][e] = run_[e];
        if constexpr (!LOAD_QK) {
          qv[u][e] = gv;
          kv[u][e] = 0.f;
        }
      }
    }
    if (active) {
#pragma unroll
      for (int e = 0; e < V; ++e) segtot[seg * DKP + cg * V + e] = run_[e];
    }
    __syncthreads();
    for (int ch = tid; ch < DKP; ch += NT) seg_scan_channel<M::NSEG>(segtot, DKP, ch, false);
    __syncthreads();
    float mx = 0.f;
    if (active) {
      float pre[V];
#pragma unroll
      for (int e = 0; e < V; ++e) pre[e] = segtot[seg * DKP + cg * V + e];
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          b[u][e] += pre[e];
          mx = fmaxf(mx, fabsf(b[u][e]));
        }
      }
      if (seg == M::NSEG - 1) {
#pragma unroll
        for (int e = 0; e < V; ++e) sGam[cg * V + e] = b[RPS - 1][e];
      }
    }
    return block_max<NT>(mx, red, tid);   // also makes sGam visible to all threads
  }

  __device__ __forceinline__ float run(const T* qg, const T* kg, const T* gg, int ld, int width, int len,
                                       float* segtot, float* sGam, float* red) {
    load(qg, kg, gg, ld, width, len);
    const float mx = finish(segtot, sGam, red);
    kvals();
    qvals();
    return mx;
  }
};

// Compute units of the current device, cached per device id.
inline int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}
// Issue the loads of chunk n of sequence bh (q, k, g) into cs; past = true reads only the
// chunk's first row (a harmless, cached reload: the loads of a persistent loop's last round are
// issued unconditionally)
template <typename T, int DKP, int CP>
__device__ __forceinline__ void prep_issue(const PrepParams& p, int n, int bh, ChunkScan<T, DKP, CP, true, prep_threads<T, DKP, CP>()>& cs,
                                           bool past) {
  const int row0 = n * p.C;
  const int len = past ? 1 : min(p.C, p.L - row0);
  const size_t base = ((size_t)p.in(bh) * p.L + row0) * p.Dk;
  cs.load(reinterpret_cast<const T*>(p.q) + base, reinterpret_cast<const T*>(p.k) + base,
          reinterpret_cast<const T*>(p.g) + base, p.Dk, p.Dk, len);
}

// One chunk, whose loads the caller has issued into cs.  Once q and k are converted (the raw
// vectors dead), next() runs: a persistent caller issues its next chunk's loads there, so they
// are in flight while this chunk is computed.
template <typename T, int DKP, int CP, typename Next>
__device__ __forceinline__ void prep_chunk(const PrepParams& p, int n, int bh,
                                           ChunkScan<T, DKP, CP, true, prep_threads<T, DKP, CP>()>& cs, Next&& next) {
  using Cfg = PrepCfg<T, DKP, CP>;
  using M = typename Cfg::M;
  constexpr int V = M::V, RPS = M::RPS, NT = Cfg::NT, NW = Cfg::NW;
  constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDP = Cfg::LDP;
  constexpr int NB = Cfg::NB, NP = Cfg::NP, PPW = Cfg::PPW;
  typedef typename V16<T>::type VT;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::BYTES];
  float* segtot = reinterpret_cast<float*>(smem);              // during the scan only
  float* sGam = reinterpret_cast<float*>(smem + Cfg::MAIN);
  float* red = sGam + DKP;

  const int tid = threadIdx.x;
  const int row0 = n * p.C;
  const int len = min(p.C, p.L - row0);
  const int Dk = p.Dk;
  const size_t base = ((size_t)p.in(bh) * p.L + row0) * Dk;
  const size_t chunk = (size_t)bh * p.N + n;

  const float maxb = cs.finish(segtot, sGam, red);
  cs.kvals();
  cs.qvals();
  next();
  const bool fast = maxb <= kSpanLimit;
  const int c0 = cs.cg * V, r0 = cs.seg * RPS;

  // LDS regions: [0, TILE) sQ; then fast: sK, sQl, sKl; safe: its scratch
  T* sQ = reinterpret_cast<T*>(smem);
  T* sK = sQ + CP * LDQ;
  T* sQl = sK + CP * LDQ;
  T* sKl = sQl + CP * LDQ;
  T* Qg = reinterpret_cast<T*>(p.ops.Qs) + chunk * CP * DKP;

  // ---- Qs = q 2^b (global + LDS), Ks = k 2^-b (fast path), bf16 lo parts
  if (cs.active) {
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      const int r = r0 + u;
      VT qh, ql, kh, kl;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float qs = cs.qv[u][e] * fast_exp2(cs.b[u][e]);
        qh[e] = from_f32<T>(qs);
        ql[e] = from_f32<T>(qs - to_f32(qh[e]));
        const float ks = fast ? cs.kv[u][e] * fast_exp2(-cs.b[u][e]) : 0.f;
        kh[e] = from_f32<T>(ks);
        kl[e] = from_f32<T>(ks - to_f32(kh[e]));
      }
      *reinterpret_cast<VT*>(sQ + r * LDQ + c0) = qh;
      *reinterpret_cast<VT*>(Qg + (size_t)r * DKP + c0) = qh;
      if (fast) {
        *reinterpret_cast<VT*>(sK + r * LDQ + c0) = kh;
        if constexpr (Cfg::SPLIT) {
          *reinterpret_cast<VT*>(sQl + r * LDQ + c0) = ql;
          *reinterpret_cast<VT*>(sKl + r * LDQ + c0) = kl;
        }
      }
    }
  }
  __syncthreads();

  // ---- intra-chunk scores A, kept in registers until the LDS operands are released
  const int wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  constexpr int NBLK = NB * NB;
  constexpr int BPW = (NBLK + NW - 1) / NW;  // score blocks per wave
  f32x4 accA[BPW];
#pragma unroll
  for (int s = 0; s < BPW; ++s) accA[s] = zero4();
  T* sKd = reinterpret_cast<T*>(smem + Cfg::TILE);
  T* sA = reinterpret_cast<T*>(smem + Cfg::TILE + Cfg::KD);
  if (fast) {
#pragma unroll
    for (int s = 0; s < BPW; ++s) {
      const int blk = wave + NW * s;
      const int rb = blk / NB, cb = blk % NB;
      if (blk < NBLK && cb <= rb) {
#pragma unroll
        for (int kb = 0; kb < DKP / 32; ++kb) {
          const int oq = (16 * rb + col) * LDQ + 32 * kb + 8 * grp, ok = (16 * cb + col) * LDQ + 32 * kb + 8 * grp;
          const Frag<T> qh = ld8(sQ + oq), kh = ld8(sK + ok);
          mma(accA[s], qh, kh);
          if constexpr (Cfg::SPLIT) {
            mma(accA[s], qh, ld8(sKl + ok));
            mma(accA[s], ld8(sQl + oq), kh);
          }
        }
      }
    }
    __syncthreads();   // score operands released: KdT and A reuse their bytes
#pragma unroll
    for (int s = 0; s < BPW; ++s) {
      const int blk = wave + NW * s;
      if (blk < NBLK) {
        const int rb = blk / NB, cb = blk % NB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * grp + e, c = 16 * cb + col;
          sA[r * LDC + c] = from_f32<T>(c <= r ? accA[s][e] : 0.f);
        }
      }
    }
  } else {
    // safe path scratch lives after sQ
    float* sqf = reinterpret_cast<float*>(smem + Cfg::TILE);
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
    const int rr = tid >> 4, cc = tid & 15;   // diagonal sub-block element (the first 256 threads)
    const bool dgl = tid < 256;
    for (int sl = 0; sl < DKP / 32; ++sl) {
      __syncthreads();
      if (cs.active && c0 >= 32 * sl && c0 < 32 * sl + 32) {
#pragma unroll
        for (int u = 0; u < RPS; ++u) {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const int r = r0 + u, ii = c0 - 32 * sl + e;
            sbs[r * 33 + ii] = cs.b[u][e];
            sqf[r * 33 + ii] = cs.qv[u][e];
            skf[r * 33 + ii] = cs.kv[u][e];
          }
        }
      }
      __syncthreads();
      // diagonal sub-blocks, element by element: exponent b_r - b_c <= 0 for c <= r
      if (dgl && cc <= rr) {
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
        for (int e = tid; e < CP * 32; e += NT) {
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
          const int pidx = wave + NW * s;
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
    __syncthreads();   // safe-path scratch released: KdT and A reuse its bytes
#pragma unroll
    for (int s = 0; s < PPW; ++s) {
      const int pidx = wave + NW * s;
      if (pidx < NP) {
        int x, y;
        pair_decode(pidx, x, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) sA[(16 * x + 4 * grp + e) * LDC + 16 * y + col] = from_f32<T>(acc_off[s][e]);
      }
    }
    for (int blk = wave; blk < NBLK; blk += NW) {
      const int rb = blk / NB, cb = blk % NB;
      if (cb > rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sA[(16 * rb + 4 * grp + e) * LDC + 16 * cb + col] = from_f32<T>(0.f);
      }
    }
    if (dgl) {
#pragma unroll
      for (int x = 0; x < NB; ++x) sA[(16 * x + rr) * LDC + 16 * x + cc] = from_f32<T>(cc <= rr ? acc_d[x] : 0.f);
    }
  }

  // ---- Kd = k 2^{Gamma - b} into LDS row by row; it leaves transposed (KdT)
  if (cs.active) {
#pragma unroll
    for (int u = 0; u < RPS; ++u) {
      VT kd;
#pragma unroll
      for (int e = 0; e < V; ++e) kd[e] = from_f32<T>(cs.kv[u][e] * fast_exp2(sGam[c0 + e] - cs.b[u][e]));
      *reinterpret_cast<VT*>(sKd + (r0 + u) * LDQ + c0) = kd;
    }
  }
  __syncthreads();
  tile_out_t<T, NW>(reinterpret_cast<T*>(p.ops.KdT) + chunk * DKP * CP, sKd, CP, DKP, LDQ);
  tile_out<T>(reinterpret_cast<T*>(p.ops.A) + chunk * CP * CP, sA, CP, CP, LDC);
  if (tid < DKP) p.ops.Gam[chunk * DKP + tid] = sGam[tid];
}

// Persistent grid over the ntiles = N * BH chunks (tile t: chunk t % N of sequence t / N):
// workgroup w takes tiles w, w + gridDim.x, ..., each tile's loads in flight during the
// previous tile's computation
template <typename T, int DKP, int CP>
__global__ __launch_bounds__((PrepCfg<T, DKP, CP>::NT), (PrepCfg<T, DKP, CP>::MIN_WAVES)) void gla_prep_kernel(PrepParams p, int ntiles) {
  ChunkScan<T, DKP, CP, true, prep_threads<T, DKP, CP>()> cs;
  int t = blockIdx.x;
  prep_issue(p, t % p.N, t / p.N, cs, false);
  if constexpr (!PrepCfg<T, DKP, CP>::PERSIST) {    // one chunk per workgroup
    prep_chunk<T, DKP, CP>(p, t % p.N, t / p.N, cs, [] {});
    return;
  }
  for (;;) {
    const int tn = t + gridDim.x;
    prep_chunk<T, DKP, CP>(p, t % p.N, t / p.N, cs, [&] {
      const int u = tn < ntiles ? tn : t;
      prep_issue(p, u % p.N, u / p.N, cs, tn >= ntiles);
    });
    if (tn >= ntiles) break;
    t = tn;
    __syncthreads();                     // the next chunk's scan reuses the LDS
  }
  __builtin_amdgcn_s_waitcnt(0);         // the last round's repeated loads have landed
}

// grid (max N, total sequences): blockIdx.y runs over the batches' sequences back to back;
// blocks past a batch's own chunk count return at once
template <typename T, int DKP, int CP>
__global__ __launch_bounds__((PrepCfg<T, DKP, CP>::NT), (PrepCfg<T, DKP, CP>::MIN_WAVES)) void gla_prep_batches(Batches<PrepParams> b) {
  const int gi = b.find(blockIdx.y);
  const PrepParams& p = b.p[gi];
  if ((int)blockIdx.x >= p.N) return;
  ChunkScan<T, DKP, CP, true, prep_threads<T, DKP, CP>()> cs;
  prep_issue(p, blockIdx.x, blockIdx.y - b.first[gi], cs, false);
  prep_chunk<T, DKP, CP>(p, blockIdx.x, blockIdx.y - b.first[gi], cs, [] {});
}

// Workgroups of the persistent preparation kernel the device runs at once (CUs times the
// workgroups one CU holds), cached per device
template <typename T, int DKP, int CP>
int prep_slots() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gla_prep_kernel<T, DKP, CP>, PrepCfg<T, DKP, CP>::NT, 0) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  const int cus = device_cu_count();
  const int n = (cus > 0 ? cus : 256) * per_cu;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <typename T, int DKP, int CP>
hipError_t launch_prep(const PrepParams& p, int BH, hipStream_t s) {
  if constexpr (PrepCfg<T, DKP, CP>::BYTES > kMaxLds) {
    return hipErrorNotSupported;
  } else {
    const int ntiles = p.N * BH;
    const int grid = PrepCfg<T, DKP, CP>::PERSIST ? imin(ntiles, prep_slots<T, DKP, CP>()) : ntiles;
    hipLaunchKernelGGL((gla_prep_kernel<T, DKP, CP>), dim3(grid), dim3(PrepCfg<T, DKP, CP>::NT), 0, s, p, ntiles);
    return hipGetLastError();
  }
}

template <typename T, int DKP, int CP>
hipError_t launch_prep_batches(const Batches<PrepParams>& b, int maxN, hipStream_t s) {
  if constexpr (PrepCfg<T, DKP, CP>::BYTES > kMaxLds) {
    return hipErrorNotSupported;
  } else {
    hipLaunchKernelGGL((gla_prep_batches<T, DKP, CP>), dim3(maxN, b.first[b.n]), dim3(PrepCfg<T, DKP, CP>::NT), 0, s, b);
    return hipGetLastError();
  }
}

}  // namespace gla
