// kernels.hpp -- launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gla {

// Which input sequence the bh-th sequence of a launch reads: (bh / n) * stride + off + bh % n.
// The default is the contiguous [BH] batch itself.  With n = nh, stride = H, off = h0 a launch
// over B * nh sequences reads heads h0 .. h0 + nh - 1 of caller tensors laid out [B][H][L][D]
// in place (the multi-scale front end runs its scale-1 head group this way).  Only the token
// inputs (q, k, g, v) are read through it; workspaces and outputs stay indexed by bh.
struct SeqView {
  int n = 1, stride = 1, off = 0;
  __host__ __device__ int operator()(int bh) const { return (bh / n) * stride + off + bh % n; }
};

// Up to kMaxBatches independent sequence batches with the same widths and chunk size, run by
// one launch per kernel: batch i owns blocks first[i] .. first[i + 1] - 1 of the launch's
// batch axis (its sequences for the preparation kernel, its blocks for the others).  The
// multi-scale front end runs its head groups this way, so that the small groups fill the CUs
// the large one leaves idle.
constexpr int kMaxBatches = 8;
template <typename P>
struct Batches {
  P p[kMaxBatches];
  int first[kMaxBatches + 1];
  int n;
  __host__ __device__ int find(int i) const {
    int g = 0;
    while (g + 1 < n && i >= first[g + 1]) ++g;
    return g;
  }
};

// Per-chunk operands written by the chunk-preparation kernel, all chunk-padded so that the
// consumers need no bounds checks: CP = padded chunk rows, DKP = padded key width.
struct ChunkOps {
  void* Qs;     // [BH][N][CP][DKP]  q * 2^{b}            (T)
  void* KdT;    // [BH][N][DKP][CP]  (k * 2^{Gamma - b})^T (T)
  void* A;      // [BH][N][CP][CP]   masked intra-chunk scores (T)
  float* Gam;   // [BH][N][DKP]      chunk log2-decay Gamma (f32)
};

// Optional launch-boundary events (profiling): events[0] is recorded before the first
// kernel and events[i] after the i-th kernel, on the launch stream; nullptr = none.
struct LaunchEvents {
  void** ev;
  int n;
};
inline void record_event(const LaunchEvents& e, int i, hipStream_t s) {
  if (e.ev && i < e.n && e.ev[i]) (void)hipEventRecord(static_cast<hipEvent_t>(e.ev[i]), s);
}

struct FwdParams {
  const void *q, *k, *v, *g;
  const float* h0;
  void* o;
  float* ht;
  int BH, L, Dk, Dv, C, N;
  ChunkOps ops;
  void* Hs;       // [BH][N][DKP][DvP] chunk-start states (T), written by the state walk
  bool states_ready = false;   // Hs (and ht) already hold the walk's result: no walk is run
  bool ops_ready = false;      // ops.Qs and ops.A already hold the chunk operands: no preparation
  bool keep_states = true;     // Hs must hold the chunk-start states afterwards (else it is scratch)
  LaunchEvents events;
  SeqView in;     // input sequences read by the launch
  // optional scratch for a segmented state walk (walks.hpp), room for seg_max segments:
  // [BH][seg_max][DKP][DvP] fp32 twice, [BH][N][DKP] fp32, [BH][seg_max][DKP] fp32; null =
  // never segment
  float* seg_ws = nullptr;
  int seg_max = 0;
  // set by the launcher for the output kernel when the walk ran in seg_n segments of seg_len
  // chunks and left the carried part out of the stored states: it adds Diag(2^{P_n}) X_s to
  // H_n as it stages it (carry [BH][seg_n][DKP][DvP], prefix [BH][N][DKP], fp32)
  const float* seg_carry = nullptr;
  const float* seg_prefix = nullptr;
  int seg_len = 0, seg_n = 0;
  // set for the batched output kernel by the multi-scale front end: instead of o, row j of
  // this (pooled) sequence goes to the hold_s tokens t of hold_o with (t + 1) / hold_s - 1 == j,
  // times hold_w[(b * hold_L + t) * hold_ng + hold_gi] (1 without weights), and the first
  // hold_s - 1 tokens get zeros.  Sequence bh is batch bh / hold_nh, head hold_h0 + bh % hold_nh
  // of hold_o [B][hold_H][hold_L][Dv].
  void* hold_o = nullptr;
  const float* hold_w = nullptr;
  int hold_s = 1, hold_L = 0, hold_H = 0, hold_h0 = 0, hold_nh = 1, hold_ng = 1, hold_gi = 0;
};

struct BwdParams {
  const void *q, *k, *v, *g, *do_;
  const float *h0, *dht;
  void *dq, *dk, *dv;
  float *dg, *dh0;
  int BH, L, Dk, Dv, C, N;
  ChunkOps ops;
  void* Hs;       // [BH][N][DKP][DvP] state at chunk starts (T)
  void* dHs;      // [BH][N][DKP][DvP] state gradient at chunk ends (T)
  bool saved;     // ops and Hs were left by a forward: skip recomputing them
  LaunchEvents events;
  // if set, dq goes here in fp32 [BH][L][Dk] instead of to dq: GSA's pass 2, whose dq is the
  // gradient of the read-out, which the softmax's Jacobian then reduces with cancellation
  float* dq32 = nullptr;
  // if set (GSA's pass 2 with its whole slot width in one chunk tile: gla_bwd_key_slices == 1),
  // the read-out's backward runs in the chunk kernel's epilogue: from dq = dP and the fp32
  // read-out input rd (P for the softmax, the scores Z otherwise) it writes dz = dZ (fp32
  // [BH][L][Dk]) and dzs = dZ 2^b ([BH][N][CP][DKP], T, chunk-padded), and no dq
  const float* rd = nullptr;
  float* dz = nullptr;
  void* dzs = nullptr;
  int act = 0;
};

// Gated slot attention: pass 1 runs on its own kernels, pass 2 on the GLA kernels.
struct GsaParams {
  const void *q, *k, *v, *g, *do_;
  const float *hk0, *hv0, *dhkt, *dhvt;
  void* o;
  float *hkt, *hvt;
  void *dq, *dk, *dv;
  float *dg, *dhk0, *dhv0;
  int BH, L, Dk, DkP, Dv, m, C, N;
  int act;        // read-out between the passes (GsaAct)
  int saved;      // backward: W, P, Pf, WdT, Gam, S1s, ops2 and Hs2 were left by a
                  // saving forward, so the backward does not recompute them
  // workspace
  void* W;        // [BH][L][m] write weights 1 - exp(g)   (keys of pass 2)   (T), or null
  void* P;        // [BH][L][m] slot softmax              (queries of pass 2) (T), or null
                  // (W and P serve only pass 2's backward: the forward alone writes neither)
  float* Pf;      // [BH][L][m] fp32, backward only: the softmax P (its Jacobian needs P) or,
                  // for the element-wise read-outs, the scores Z (their derivative needs Z)
  float* dP;      // [BH][L][m] gradient of P (backward), fp32
  void* dW2;      // [BH][L][m] pass-2 gradient of W (backward)                (T)
  float* dg2;     // [BH][L][m] pass-2 decay gradient (backward)
  float* dZ;      // [BH][L][m] gradient of the softmax input (backward)
  void* WdT;      // [BH][N][MP][CP] (W 2^{Gamma-b})^T                         (T)
  float* Gam;     // [BH][N][MP]
  void* S1s;      // [BH][N][MP][DkP] pass-1 state S1^T at chunk starts        (T)
  void* dS1s;     // [BH][N][MP][DkP] its gradient at chunk ends (backward)    (T)
  void* dZs;      // [BH][N][CP][MP] dZ 2^b, chunk-padded (backward)           (T)
  ChunkOps ops2;  // pass-2 GLA chunk operands: Qs and A from gsa_p; KdT and Gam are WdT and Gam
  void *Hs2, *dHs2;
};

struct DecodeParams {
  const void *q, *k, *v, *g;
  float* state;
  void* o;
  int BH, Dk, Dv;
};

// Padded sizes shared by host and kernels.
constexpr int kDvTile = 64;                       // Dv columns per walk workgroup
inline int pad_dk(int Dk) { return Dk <= 32 ? 32 : Dk <= 64 ? 64 : Dk <= 128 ? 128 : 256; }
inline int pad_c(int C) { return C <= 32 ? 32 : C; }
inline int pad_dv(int Dv) { return (Dv + kDvTile - 1) / kDvTile * kDvTile; }

template <typename T, int DKP, int CP>
hipError_t launch_gla_fwd(const FwdParams& p, hipStream_t s);
template <typename T, int DKP, int CP>
hipError_t launch_gla_fwd_batches(const FwdParams* ps, int nb, hipStream_t s);
template <typename T, int DKP, int CP>
hipError_t launch_gla_bwd(const BwdParams& p, hipStream_t s);
// key-width slices of the backward's chunk tiles for a (type size, padded key width, padded
// chunk) configuration; 0 = unsupported
int gla_bwd_key_slices(int esize, int DKP, int CP);
template <typename T>
hipError_t launch_gla_decode(const DecodeParams& p, hipStream_t s);

// Read-out between GSA's two passes.  Softmax over the slots is the method's own; the GSA
// summary's ablations ("Measured effects") also replace it with Swish, ReLU or ReLU^2, or drop
// it, each applied to every slot score alone.  Values match gla.h's GSA_ACT_* constants.
enum GsaAct { kActSoftmax = 0, kActSwish = 1, kActRelu = 2, kActRelu2 = 3, kActNone = 4 };

// p = f(z) for the element-wise read-outs
__device__ __forceinline__ float gsa_read(float z, int act) {
  switch (act) {
    case kActSwish: return z / (1.f + __expf(-z));
    case kActRelu: return fmaxf(z, 0.f);
    case kActRelu2: { const float r = fmaxf(z, 0.f); return r * r; }
    default: return z;
  }
}

// dLoss/dz = f'(z) dLoss/dp for the element-wise read-outs
__device__ __forceinline__ float gsa_read_grad(float z, float dp, int act) {
  switch (act) {
    case kActSwish: {
      const float sg = 1.f / (1.f + __expf(-z));
      return dp * (sg + z * sg * (1.f - sg));
    }
    case kActRelu: return z > 0.f ? dp : 0.f;
    case kActRelu2: return z > 0.f ? 2.f * z * dp : 0.f;
    default: return dp;
  }
}

struct GsaDecodeParams {
  const void *q, *k, *v, *g;
  float *hk, *hv;                 // [BH][Dk][m], [BH][m][Dv], updated in place
  void* o;
  int BH, Dk, Dv, m, act;
};
template <typename T>
hipError_t launch_gsa_decode(const GsaDecodeParams& p, hipStream_t s);

// MS-GLA front end: head groups, one per temporal scale
constexpr int kMsMaxGroups = 8;
static_assert(kMsMaxGroups <= kMaxBatches, "the head groups run as one batched launch");
struct MsglaGroup {
  int h0, nh, s;                  // first head, number of heads, pooling scale
  void *qp, *kp, *gp, *vp;        // pooled inputs [B][nh][ceil(L/s)][Dk or Dv] (T)
};
struct MsglaParams {
  const void *q, *k, *v, *g;      // [B][H][L][Dk or Dv] (T)
  int B, H, L, Dk, Dv, ngroups;
  int pooled_heads;               // heads in groups with scale > 1
  int max_pooled_len;             // longest pooled sequence among those groups
  MsglaGroup grp[kMsMaxGroups];
};
template <typename T>
hipError_t launch_msgla_pool(const MsglaParams& p, hipStream_t s);

constexpr size_t kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950

template <typename T, int MP, int CP>
hipError_t launch_gsa_fwd(const GsaParams& p, hipStream_t s);
template <typename T, int MP, int CP>
hipError_t launch_gsa_bwd(const GsaParams& p, hipStream_t s);
bool gsa_config_fits(int esize, int MP, int CP, bool bwd);   // bwd: the backward's kernels too

// Kernel phases per call (for the profiled entry points; the forward's walk and outputs may be
// one kernel, whose events then bracket both phases).
constexpr int GLA_FWD_LAUNCHES = 3;
constexpr int GLA_BWD_MAX_LAUNCHES = 5;
int bwd_launch_count(int esize, int DKP, int CP);   // self-contained backward; 2 fewer when saved

// Whether every kernel of the forward fits the LDS of a CU for this (dtype size, DKP, CP).
bool fwd_config_fits(int esize, int DKP, int CP);
// whether the forward runs its state walk and chunk outputs as one kernel (walk_out.hpp)
bool fwd_fused(int esize, int DKP, int CP, int BH, int Dv, bool keep_states);
// Same for the backward kernels.
bool bwd_config_fits(int esize, int DKP, int CP);

}  // namespace gla
