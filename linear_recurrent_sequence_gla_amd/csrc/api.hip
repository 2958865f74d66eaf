// api.hip -- the extern "C" entry points declared in include/gla.h: synchronous argument
// validation, workspace carving and kernel dispatch.  Nothing is enqueued unless every check
// passes, so a failing call leaves all outputs untouched.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <initializer_list>
#include <mutex>

#include "../../include/gla.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace gla;

namespace {

constexpr int kAbiVersion = 3;
constexpr size_t kAlign = 256;

bool valid_act(int act) { return act >= GSA_ACT_SOFTMAX && act <= GSA_ACT_NONE; }

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int esize_of(int dtype) { return dtype == GLA_BF16 ? 2 : 4; }

// Kernels use 16-byte vector accesses on every tensor.
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}

bool valid_c(int C) { return C == 16 || C == 32 || C == 64 || C == 128; }

// Shape checks shared by the chunked entry points.  Returns GLA_OK or an error status.
int check_dims(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  if (dtype != GLA_F32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 1 || Dk < 1 || Dv < 1 || C < 1) return GLA_ERR_SHAPE;
  if (!valid_c(C)) return GLA_ERR_UNSUPPORTED;
  if (Dk % 16 != 0 || Dk > 256 || Dv % 16 != 0 || Dv > 512) return GLA_ERR_UNSUPPORTED;
  const int DKP = pad_dk(Dk), CP = pad_c(C);
  if (DKP == 256 && CP == 128) return GLA_ERR_UNSUPPORTED;   // chunk tile exceeds LDS
  if (!fwd_config_fits(esize_of(dtype), DKP, CP)) return GLA_ERR_UNSUPPORTED;
  // element counts must fit the kernels' 64-bit offsets and int row indices
  if ((int64_t)B * H > 65535) return GLA_ERR_UNSUPPORTED;   // grid y-dimension of the chunk kernels
  if ((int64_t)B * H > INT32_MAX / 2 || (int64_t)L * Dv > INT32_MAX / 2 || (int64_t)L * Dk > INT32_MAX / 2)
    return GLA_ERR_UNSUPPORTED;
  return GLA_OK;
}

// The chunk size the kernels tile a call with.  The operator's result does not depend on the
// chunk size (chunks only regroup the same recurrence: sequential state passing between them,
// the parallel form inside), so where the requested size's tiles do not fit a CU's LDS the call
// runs with the largest smaller supported size whose tiles do, and computes the same outputs to
// rounding.  bwd: the backward's kernels must fit too (backward, saving forward and their
// sizes, so that a saving forward and its backward agree).  A size nothing fits under comes
// back unchanged, for the checks to refuse.
int gla_tile_c(int Dk, int C, int dtype, bool bwd) {
  if (!valid_c(C) || (dtype != GLA_F32 && dtype != GLA_BF16) || Dk < 1 || Dk > 256) return C;
  const int es = esize_of(dtype), DKP = pad_dk(Dk);
  for (int c = C; c >= 16; c /= 2) {
    const int CP = pad_c(c);
    if (DKP == 256 && CP == 128) continue;
    if (!fwd_config_fits(es, DKP, CP) || (bwd && !bwd_config_fits(es, DKP, CP))) continue;
    return c;
  }
  return C;
}

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Outputs must not overlap inputs, each other, or the workspace.
bool any_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

// Chunk-operand region of the workspace (shared by forward and backward).
struct OpsLayout {
  size_t qs, kdt, a, gam, total;
};

// kd_gam = false: no room for KdT and Gam (GSA's pass 2 uses pass 1's WdT and Gamma)
OpsLayout ops_layout(size_t BH, size_t N, size_t CP, size_t DKP, size_t es, bool kd_gam = true) {
  OpsLayout l{};
  size_t off = 0;
  l.qs = off;  off += align_up(BH * N * CP * DKP * es);
  l.kdt = off; if (kd_gam) off += align_up(BH * N * CP * DKP * es);
  l.a = off;   off += align_up(BH * N * CP * CP * es);
  l.gam = off; if (kd_gam) off += align_up(BH * N * DKP * 4);
  l.total = off;
  return l;
}

ChunkOps carve_ops(char* ws, const OpsLayout& l) {
  ChunkOps o;
  o.Qs = ws + l.qs;
  o.KdT = ws + l.kdt;
  o.A = ws + l.a;
  o.Gam = reinterpret_cast<float*>(ws + l.gam);
  return o;
}

#define GLA_DISPATCH_DKCP(LAUNCH, TT, DKP, CP, ...)                                        \
  do {                                                                                    \
    if (DKP == 32 && CP == 32) return LAUNCH<TT, 32, 32>(__VA_ARGS__);                    \
    if (DKP == 32 && CP == 64) return LAUNCH<TT, 32, 64>(__VA_ARGS__);                    \
    if (DKP == 32 && CP == 128) return LAUNCH<TT, 32, 128>(__VA_ARGS__);                  \
    if (DKP == 64 && CP == 32) return LAUNCH<TT, 64, 32>(__VA_ARGS__);                    \
    if (DKP == 64 && CP == 64) return LAUNCH<TT, 64, 64>(__VA_ARGS__);                    \
    if (DKP == 64 && CP == 128) return LAUNCH<TT, 64, 128>(__VA_ARGS__);                  \
    if (DKP == 128 && CP == 32) return LAUNCH<TT, 128, 32>(__VA_ARGS__);                  \
    if (DKP == 128 && CP == 64) return LAUNCH<TT, 128, 64>(__VA_ARGS__);                  \
    if (DKP == 128 && CP == 128) return LAUNCH<TT, 128, 128>(__VA_ARGS__);                \
    if (DKP == 256 && CP == 32) return LAUNCH<TT, 256, 32>(__VA_ARGS__);                  \
    if (DKP == 256 && CP == 64) return LAUNCH<TT, 256, 64>(__VA_ARGS__);                  \
  } while (0)

hipError_t dispatch_fwd(int dtype, int DKP, int CP, const FwdParams& p, hipStream_t s) {
  if (dtype == GLA_BF16) GLA_DISPATCH_DKCP(launch_gla_fwd, bf16, DKP, CP, p, s);
  else GLA_DISPATCH_DKCP(launch_gla_fwd, float, DKP, CP, p, s);
  return hipErrorInvalidValue;
}

hipError_t dispatch_fwd_batches(int dtype, int DKP, int CP, const FwdParams* ps, int nb, hipStream_t s) {
  if (dtype == GLA_BF16) GLA_DISPATCH_DKCP(launch_gla_fwd_batches, bf16, DKP, CP, ps, nb, s);
  else GLA_DISPATCH_DKCP(launch_gla_fwd_batches, float, DKP, CP, ps, nb, s);
  return hipErrorInvalidValue;
}

hipError_t dispatch_bwd(int dtype, int DKP, int CP, const BwdParams& p, hipStream_t s) {
  if (dtype == GLA_BF16) GLA_DISPATCH_DKCP(launch_gla_bwd, bf16, DKP, CP, p, s);
  else GLA_DISPATCH_DKCP(launch_gla_bwd, float, DKP, CP, p, s);
  return hipErrorInvalidValue;
}

// Forward workspace: the chunk operands, then the chunk-start states.
// Segments gla_fwd keeps room for, to split its state walk when there are few sequences
// (walks.hpp, walk_segments): up to 8 while the 16-row walk grid is under 256 workgroups
// and the sequence has at least 16 chunks, else none.
int fwd_seg_max(int B, int H, int L, int Dk, int Dv, int C) {
  const int64_t grid16 = (int64_t)((Dv + kDvTile - 1) / kDvTile) * (pad_dk(Dk) / 16) * B * H;
  const int N = (L + C - 1) / C;
  return (grid16 < 256 && N >= 16) ? std::min(8, N / 8) : 0;
}

size_t fwd_seg_bytes(int B, int H, int L, int Dk, int Dv, int C) {
  const int S = fwd_seg_max(B, H, L, Dk, Dv, C);
  if (S < 2) return 0;
  const size_t BH = (size_t)B * H, DKP = pad_dk(Dk), N = (L + C - 1) / C;
  return align_up((2 * BH * S * DKP * pad_dv(Dv) + BH * N * DKP + BH * S * DKP) * 4);
}

// seg: keep room for a segmented walk (gla_fwd); the batched forwards of MS-GLA never segment
size_t fwd_ws_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype, bool seg = true) {
  const size_t BH = (size_t)B * H, CP = pad_c(C), DKP = pad_dk(Dk), N = (L + C - 1) / C;
  const size_t es = esize_of(dtype);
  return ops_layout(BH, N, CP, DKP, es).total + align_up(BH * N * DKP * pad_dv(Dv) * es) +
         (seg ? fwd_seg_bytes(B, H, L, Dk, Dv, C) : 0);
}

struct BwdLayout {
  OpsLayout ops;
  size_t hs, dhs, total;
};

// What gla_fwd_save leaves for gla_bwd_saved: the chunk operands and the chunk-start
// states.  The saved-state backward's own workspace holds only dH.
struct SavedLayout {
  OpsLayout ops;
  size_t hs, total;
};

SavedLayout saved_layout(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  const size_t BH = (size_t)B * H, CP = pad_c(C), DKP = pad_dk(Dk), N = (L + C - 1) / C;
  const size_t es = esize_of(dtype), DVP = pad_dv(Dv);
  SavedLayout l;
  l.ops = ops_layout(BH, N, CP, DKP, es);
  l.hs = l.ops.total;
  l.total = l.hs + align_up(BH * N * DKP * DVP * es);
  return l;
}

size_t bwd_saved_ws_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  const size_t BH = (size_t)B * H, DKP = pad_dk(Dk), N = (L + C - 1) / C;
  return align_up(BH * N * DKP * pad_dv(Dv) * esize_of(dtype));
}

BwdLayout bwd_layout(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  const size_t BH = (size_t)B * H, CP = pad_c(C), DKP = pad_dk(Dk), N = (L + C - 1) / C;
  const size_t es = esize_of(dtype), DVP = pad_dv(Dv);
  BwdLayout l;
  l.ops = ops_layout(BH, N, CP, DKP, es);
  size_t off = l.ops.total;
  l.hs = off;    off += align_up(BH * N * DKP * DVP * es);
  l.dhs = off;   off += align_up(BH * N * DKP * DVP * es);
  l.total = off;
  return l;
}

}  // namespace

extern "C" {

int gla_abi_version(void) { return kAbiVersion; }

const char* gla_status_str(int s) {
  switch (s) {
    case GLA_OK: return "GLA_OK: success";
    case GLA_ERR_NULL_ARG: return "GLA_ERR_NULL_ARG: a required pointer is NULL";
    case GLA_ERR_SHAPE: return "GLA_ERR_SHAPE: a size is smaller than 1";
    case GLA_ERR_DTYPE: return "GLA_ERR_DTYPE: dtype must be GLA_F32 (0) or GLA_BF16 (1)";
    case GLA_ERR_UNSUPPORTED:
      return "GLA_ERR_UNSUPPORTED: C must be 16/32/64/128, Dk a multiple of 16 up to 256, "
             "Dv a multiple of 16 up to 512, GSA slots m a multiple of 16 up to 128, B*H <= 65535, "
             "16-byte aligned tensors; tiles that exceed a CU's LDS are not supported (bf16: "
             "Dk > 128 with C = 128; fp32: Dk > 128 with C = 64, Dk > 64 with C = 128, and every "
             "backward with C = 128; chunked GSA: C <= 64, and its backward C <= 32 when m > 64, "
             "fp32 m <= 64 with C <= 32)";
    case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE: workspace NULL or smaller than the query returned";
    case GLA_ERR_ALIAS: return "GLA_ERR_ALIAS: an output overlaps an input, another output or the workspace";
    case GLA_ERR_HIP: return "GLA_ERR_HIP: a HIP kernel launch failed";
    case GLA_ERR_SCRATCH:
      return "GLA_ERR_SCRATCH: these sizes need more scratch memory than gla_fwd_noalloc's fixed "
             "per-device buffer holds (64 MiB; gla_fwd_workspace_bytes gives the need)";
    default: return "unknown status";
  }
}

size_t gla_fwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  C = gla_tile_c(Dk, C, dtype, false);
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  return fwd_ws_bytes(B, H, L, Dk, Dv, C, dtype);
}

size_t gla_bwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  C = gla_tile_c(Dk, C, dtype, true);
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  if (!bwd_config_fits(esize_of(dtype), pad_dk(Dk), pad_c(C))) return 0;
  return bwd_layout(B, H, L, Dk, Dv, C, dtype).total;
}

}  // extern "C"

namespace {

int fwd_impl(const void* q, const void* k, const void* v, const void* g, const float* h0,
             void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype,
             void* workspace, size_t workspace_bytes, void* stream, LaunchEvents ev) {
  C = gla_tile_c(Dk, C, dtype, false);
  int st = check_dims(B, H, L, Dk, Dv, C, dtype);
  if (st != GLA_OK) return st;
  if (!q || !k || !v || !g || !o) return GLA_ERR_NULL_ARG;
  if (!all_aligned({q, k, v, g, h0, o, ht, workspace})) return GLA_ERR_UNSUPPORTED;
  const size_t need = fwd_ws_bytes(B, H, L, Dk, Dv, C, dtype);
  if (!workspace || workspace_bytes < need) return GLA_ERR_WORKSPACE;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const size_t nk = BH * L * Dk * es, nv = BH * L * Dv * es, ns = BH * Dk * Dv * 4;
  const Range ins[] = {{q, nk}, {k, nk}, {v, nv}, {g, nk}, {h0, h0 ? ns : 0}};
  const Range outs[] = {{o, nv}, {ht, ht ? ns : 0}, {workspace, need}};
  if (any_alias(outs, 3, ins, 5)) return GLA_ERR_ALIAS;

  const int DKP = pad_dk(Dk), CP = pad_c(C), N = (L + C - 1) / C;
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.g = g; p.h0 = h0; p.o = o; p.ht = ht;
  p.BH = (int)BH; p.L = L; p.Dk = Dk; p.Dv = Dv; p.C = C; p.N = N;
  const OpsLayout ol = ops_layout(BH, N, CP, DKP, es);
  p.ops = carve_ops(static_cast<char*>(workspace), ol);
  p.Hs = static_cast<char*>(workspace) + ol.total;
  p.keep_states = false;
  if (fwd_seg_bytes(B, H, L, Dk, Dv, C) > 0) {
    p.seg_ws = reinterpret_cast<float*>(static_cast<char*>(p.Hs) + align_up(BH * N * DKP * pad_dv(Dv) * es));
    p.seg_max = fwd_seg_max(B, H, L, Dk, Dv, C);
  }
  p.events = ev;
  if (dispatch_fwd(dtype, DKP, CP, p, static_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

int fwd_save_impl(const void* q, const void* k, const void* v, const void* g, const float* h0,
                  void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype,
                  void* saved, size_t saved_bytes, void* stream, LaunchEvents ev) {
  C = gla_tile_c(Dk, C, dtype, true);
  int st = check_dims(B, H, L, Dk, Dv, C, dtype);
  if (st != GLA_OK) return st;
  if (!bwd_config_fits(esize_of(dtype), pad_dk(Dk), pad_c(C))) return GLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !o) return GLA_ERR_NULL_ARG;
  if (!all_aligned({q, k, v, g, h0, o, ht, saved})) return GLA_ERR_UNSUPPORTED;
  const SavedLayout lay = saved_layout(B, H, L, Dk, Dv, C, dtype);
  if (!saved || saved_bytes < lay.total) return GLA_ERR_WORKSPACE;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const size_t nk = BH * L * Dk * es, nv = BH * L * Dv * es, ns = BH * Dk * Dv * 4;
  const Range ins[] = {{q, nk}, {k, nk}, {v, nv}, {g, nk}, {h0, h0 ? ns : 0}};
  const Range outs[] = {{o, nv}, {ht, ht ? ns : 0}, {saved, lay.total}};
  if (any_alias(outs, 3, ins, 5)) return GLA_ERR_ALIAS;

  const int DKP = pad_dk(Dk), CP = pad_c(C), N = (L + C - 1) / C;
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.g = g; p.h0 = h0; p.o = o; p.ht = ht;
  p.BH = (int)BH; p.L = L; p.Dk = Dk; p.Dv = Dv; p.C = C; p.N = N;
  p.ops = carve_ops(static_cast<char*>(saved), lay.ops);
  p.Hs = static_cast<char*>(saved) + lay.hs;
  p.events = ev;
  if (dispatch_fwd(dtype, DKP, CP, p, static_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

int bwd_impl(const void* q, const void* k, const void* v, const void* g, const float* h0,
             const void* do_, const float* dht, void* dq, void* dk, void* dv, float* dg,
             float* dh0, int B, int H, int L, int Dk, int Dv, int C, int dtype,
             void* workspace, size_t workspace_bytes, void* stream, LaunchEvents ev) {
  C = gla_tile_c(Dk, C, dtype, true);
  int st = check_dims(B, H, L, Dk, Dv, C, dtype);
  if (st != GLA_OK) return st;
  if (!bwd_config_fits(esize_of(dtype), pad_dk(Dk), pad_c(C))) return GLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !do_ || !dq || !dk || !dv || !dg) return GLA_ERR_NULL_ARG;
  if (!all_aligned({q, k, v, g, h0, do_, dht, dq, dk, dv, dg, dh0, workspace})) return GLA_ERR_UNSUPPORTED;
  const BwdLayout lay = bwd_layout(B, H, L, Dk, Dv, C, dtype);
  if (!workspace || workspace_bytes < lay.total) return GLA_ERR_WORKSPACE;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const size_t nk = BH * L * Dk * es, nv = BH * L * Dv * es, ns = BH * Dk * Dv * 4;
  const Range ins[] = {{q, nk}, {k, nk}, {v, nv}, {g, nk}, {h0, h0 ? ns : 0}, {do_, nv}, {dht, dht ? ns : 0}};
  const Range outs[] = {{dq, nk}, {dk, nk}, {dv, nv}, {dg, BH * L * Dk * 4}, {dh0, dh0 ? ns : 0},
                        {workspace, lay.total}};
  if (any_alias(outs, 6, ins, 7)) return GLA_ERR_ALIAS;

  const int DKP = pad_dk(Dk), CP = pad_c(C), N = (L + C - 1) / C;
  char* ws = static_cast<char*>(workspace);
  BwdParams p;
  p.q = q; p.k = k; p.v = v; p.g = g; p.do_ = do_; p.h0 = h0; p.dht = dht;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.dh0 = dh0;
  p.BH = (int)BH; p.L = L; p.Dk = Dk; p.Dv = Dv; p.C = C; p.N = N;
  p.ops = carve_ops(ws, lay.ops);
  p.Hs = ws + lay.hs;
  p.dHs = ws + lay.dhs;
  p.saved = false;
  p.events = ev;
  if (dispatch_bwd(dtype, DKP, CP, p, static_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

int bwd_saved_impl(const void* q, const void* k, const void* v, const void* g, const float* h0,
                   const void* do_, const float* dht, void* dq, void* dk, void* dv, float* dg,
                   float* dh0, int B, int H, int L, int Dk, int Dv, int C, int dtype,
                   const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                   void* stream, LaunchEvents ev) {
  C = gla_tile_c(Dk, C, dtype, true);
  int st = check_dims(B, H, L, Dk, Dv, C, dtype);
  if (st != GLA_OK) return st;
  if (!bwd_config_fits(esize_of(dtype), pad_dk(Dk), pad_c(C))) return GLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !do_ || !dq || !dk || !dv || !dg) return GLA_ERR_NULL_ARG;
  if (!all_aligned({q, k, v, g, h0, do_, dht, dq, dk, dv, dg, dh0, saved, workspace})) return GLA_ERR_UNSUPPORTED;
  const SavedLayout lay = saved_layout(B, H, L, Dk, Dv, C, dtype);
  if (!saved || saved_bytes < lay.total) return GLA_ERR_WORKSPACE;
  const size_t wsb = bwd_saved_ws_bytes(B, H, L, Dk, Dv, C, dtype);
  if (!workspace || workspace_bytes < wsb) return GLA_ERR_WORKSPACE;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const size_t nk = BH * L * Dk * es, nv = BH * L * Dv * es, ns = BH * Dk * Dv * 4;
  const Range ins[] = {{q, nk},   {k, nk},           {v, nv},   {g, nk},
                       {h0, h0 ? ns : 0}, {do_, nv}, {dht, dht ? ns : 0}, {saved, lay.total}};
  const Range outs[] = {{dq, nk}, {dk, nk}, {dv, nv}, {dg, BH * L * Dk * 4}, {dh0, dh0 ? ns : 0},
                        {workspace, wsb}};
  if (any_alias(outs, 6, ins, 8)) return GLA_ERR_ALIAS;

  const int DKP = pad_dk(Dk), CP = pad_c(C), N = (L + C - 1) / C;
  BwdParams p;
  p.q = q; p.k = k; p.v = v; p.g = g; p.do_ = do_; p.h0 = h0; p.dht = dht;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.dh0 = dh0;
  p.BH = (int)BH; p.L = L; p.Dk = Dk; p.Dv = Dv; p.C = C; p.N = N;
  char* sv = const_cast<char*>(static_cast<const char*>(saved));   // read only on this path
  p.ops = carve_ops(sv, lay.ops);
  p.Hs = sv + lay.hs;
  p.dHs = workspace;
  p.saved = true;
  p.events = ev;
  if (dispatch_bwd(dtype, DKP, CP, p, static_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

// ---------------------------------------------------------------- no-allocation forward
// gla_fwd_noalloc's scratch: the forward workspace (chunk operands, chunk-start states and the
// segmented walk's carries) lives in this fixed array of the library's own device memory
// instead of a caller buffer.  Each device the library runs on holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel: the name is a host-side
// stand-in, and the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

}  // namespace

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, or null if it cannot be had.  The first call
// on a device looks it up with that device current; later calls read the cached address.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int gla_fwd(const void* q, const void* k, const void* v, const void* g, const float* h0,
            void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype,
            void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, g, h0, o, ht, B, H, L, Dk, Dv, C, dtype, workspace, workspace_bytes, stream,
                  LaunchEvents{nullptr, 0});
}

int gla_fwd_profiled(const void* q, const void* k, const void* v, const void* g, const float* h0,
                     void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream, void** events, int nevents) {
  if (!events || nevents < GLA_FWD_LAUNCHES + 1) return GLA_ERR_NULL_ARG;
  return fwd_impl(q, k, v, g, h0, o, ht, B, H, L, Dk, Dv, C, dtype, workspace, workspace_bytes, stream,
                  LaunchEvents{events, nevents});
}

size_t gla_fwd_noalloc_max_workspace_bytes(void) { return kNoAllocScratchBytes; }

int gla_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const float* h0,
                    void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype,
                    void* stream) {
  C = gla_tile_c(Dk, C, dtype, false);
  const int st = check_dims(B, H, L, Dk, Dv, C, dtype);
  if (st != GLA_OK) return st;
  if (fwd_ws_bytes(B, H, L, Dk, Dv, C, dtype) > kNoAllocScratchBytes) return GLA_ERR_SCRATCH;
  void* ws = noalloc_scratch();
  if (!ws) return GLA_ERR_HIP;
  return fwd_impl(q, k, v, g, h0, o, ht, B, H, L, Dk, Dv, C, dtype, ws, kNoAllocScratchBytes, stream,
                  LaunchEvents{nullptr, 0});
}

int gla_bwd(const void* q, const void* k, const void* v, const void* g, const float* h0,
            const void* do_, const float* dht, void* dq, void* dk, void* dv, float* dg,
            float* dh0, int B, int H, int L, int Dk, int Dv, int C, int dtype,
            void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, g, h0, do_, dht, dq, dk, dv, dg, dh0, B, H, L, Dk, Dv, C, dtype, workspace,
                  workspace_bytes, stream, LaunchEvents{nullptr, 0});
}

int gla_bwd_profiled(const void* q, const void* k, const void* v, const void* g, const float* h0,
                     const void* do_, const float* dht, void* dq, void* dk, void* dv, float* dg,
                     float* dh0, int B, int H, int L, int Dk, int Dv, int C, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream, void** events, int nevents) {
  if (!events || nevents < GLA_BWD_MAX_LAUNCHES + 1) return GLA_ERR_NULL_ARG;
  return bwd_impl(q, k, v, g, h0, do_, dht, dq, dk, dv, dg, dh0, B, H, L, Dk, Dv, C, dtype, workspace,
                  workspace_bytes, stream, LaunchEvents{events, nevents});
}

size_t gla_saved_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  C = gla_tile_c(Dk, C, dtype, true);
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  if (!bwd_config_fits(esize_of(dtype), pad_dk(Dk), pad_c(C))) return 0;
  return saved_layout(B, H, L, Dk, Dv, C, dtype).total;
}

size_t gla_bwd_saved_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  C = gla_tile_c(Dk, C, dtype, true);
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  if (!bwd_config_fits(esize_of(dtype), pad_dk(Dk), pad_c(C))) return 0;
  return bwd_saved_ws_bytes(B, H, L, Dk, Dv, C, dtype);
}

int gla_fwd_save(const void* q, const void* k, const void* v, const void* g, const float* h0,
                 void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype,
                 void* saved, size_t saved_bytes, void* stream, void** events, int nevents) {
  if (events && nevents < GLA_FWD_LAUNCHES + 1) return GLA_ERR_NULL_ARG;
  return fwd_save_impl(q, k, v, g, h0, o, ht, B, H, L, Dk, Dv, C, dtype, saved, saved_bytes, stream,
                       LaunchEvents{events, events ? nevents : 0});
}

int gla_bwd_saved(const void* q, const void* k, const void* v, const void* g, const float* h0,
                  const void* do_, const float* dht, void* dq, void* dk, void* dv, float* dg,
                  float* dh0, int B, int H, int L, int Dk, int Dv, int C, int dtype,
                  const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                  void* stream, void** events, int nevents) {
  if (events && nevents < GLA_BWD_MAX_LAUNCHES - 1) return GLA_ERR_NULL_ARG;
  return bwd_saved_impl(q, k, v, g, h0, do_, dht, dq, dk, dv, dg, dh0, B, H, L, Dk, Dv, C, dtype, saved,
                        saved_bytes, workspace, workspace_bytes, stream, LaunchEvents{events, events ? nevents : 0});
}

int gla_bwd_launch_count(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  C = gla_tile_c(Dk, C, dtype, true);
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  return bwd_launch_count(esize_of(dtype), pad_dk(Dk), pad_c(C));
}

int gla_fwd_launch_count(int B, int H, int L, int Dk, int Dv, int C, int dtype, int keep_states) {
  C = gla_tile_c(Dk, C, dtype, keep_states != 0);
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  const int es = esize_of(dtype), DKP = pad_dk(Dk), CP = pad_c(C);
  if (keep_states && !bwd_config_fits(es, DKP, CP)) return 0;
  return fwd_fused(es, DKP, CP, B * H, Dv, keep_states != 0) ? 2 : 3;
}

int gla_decode_step(const void* q, const void* k, const void* v, const void* g, float* state,
                    void* o, int B, int H, int Dk, int Dv, int dtype, void* stream) {
  if (dtype != GLA_F32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  if (B < 1 || H < 1 || Dk < 1 || Dv < 1) return GLA_ERR_SHAPE;
  if (Dk % 16 != 0 || Dk > 256 || Dv % 16 != 0 || Dv > 512) return GLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !state || !o) return GLA_ERR_NULL_ARG;
  if ((int64_t)B * H > INT32_MAX / 64) return GLA_ERR_UNSUPPORTED;
  if (!all_aligned({q, k, v, g, state, o})) return GLA_ERR_UNSUPPORTED;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const Range ins[] = {{q, BH * Dk * es}, {k, BH * Dk * es}, {v, BH * Dv * es}, {g, BH * Dk * es},
                       {state, BH * Dk * Dv * 4}};
  const Range outs[] = {{o, BH * Dv * es}};
  if (any_alias(outs, 1, ins, 5)) return GLA_ERR_ALIAS;
  // the in-place state must not overlap the read-only token inputs either
  const Range st_[] = {{state, BH * Dk * Dv * 4}};
  if (any_alias(st_, 1, ins, 4)) return GLA_ERR_ALIAS;
  DecodeParams p{q, k, v, g, state, o, (int)BH, Dk, Dv};
  hipError_t e = dtype == GLA_BF16 ? launch_gla_decode<bf16>(p, static_cast<hipStream_t>(stream))
                                   : launch_gla_decode<float>(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

int gsa_decode_step(const void* q, const void* k, const void* v, const void* g, float* hk, float* hv,
                    void* o, int B, int H, int Dk, int Dv, int m, int dtype, int act, void* stream) {
  if (dtype != GLA_F32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  if (B < 1 || H < 1 || Dk < 1 || Dv < 1 || m < 1) return GLA_ERR_SHAPE;
  if (!valid_act(act)) return GLA_ERR_UNSUPPORTED;
  if (Dk % 16 != 0 || Dk > 256 || Dv % 16 != 0 || Dv > 512 || m % 16 != 0 || m > 256)
    return GLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !hk || !hv || !o) return GLA_ERR_NULL_ARG;
  if ((int64_t)B * H > INT32_MAX) return GLA_ERR_UNSUPPORTED;
  if (!all_aligned({q, k, v, g, hk, hv, o})) return GLA_ERR_UNSUPPORTED;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const Range ins[] = {{q, BH * Dk * es}, {k, BH * Dk * es}, {v, BH * Dv * es}, {g, BH * m * es},
                       {hk, BH * Dk * m * 4}, {hv, BH * m * Dv * 4}};
  const Range outs[] = {{o, BH * Dv * es}};
  if (any_alias(outs, 1, ins, 6)) return GLA_ERR_ALIAS;
  // the two in-place memories overlap neither the token inputs nor each other
  const Range mem[] = {{hk, BH * Dk * m * 4}, {hv, BH * m * Dv * 4}};
  if (any_alias(mem, 2, ins, 4)) return GLA_ERR_ALIAS;
  GsaDecodeParams p{q, k, v, g, hk, hv, o, (int)BH, Dk, Dv, m, act};
  hipError_t e = dtype == GLA_BF16 ? launch_gsa_decode<bf16>(p, static_cast<hipStream_t>(stream))
                                   : launch_gsa_decode<float>(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- MS-GLA front end
struct MsglaLayout {
  size_t pooled[kMsMaxGroups];   // per group: pooled q, k, g, then v (none at scale 1)
  size_t h0g[kMsMaxGroups];      // per group: initial / final states, gathered from and
  size_t htg[kMsMaxGroups];      //   scattered to the group's heads of h0 / ht
  size_t gla[kMsMaxGroups];      // per group: GLA forward workspace (the groups run together)
  size_t total;
};

int pooled_len(int L, int s) { return (L + s - 1) / s; }

int check_msgla(int B, int H, int L, int Dk, int Dv, int C, int dtype, int ngroups, const int* scales,
                const int* heads) {
  int st = check_dims(B, H, L, Dk, Dv, C, dtype);
  if (st != GLA_OK) return st;
  if (ngroups < 1 || ngroups > kMsMaxGroups) return GLA_ERR_UNSUPPORTED;
  if (!scales || !heads) return GLA_ERR_NULL_ARG;
  int total = 0;
  for (int i = 0; i < ngroups; ++i) {
    if (scales[i] < 1 || heads[i] < 1) return GLA_ERR_SHAPE;
    if (scales[i] > 65536) return GLA_ERR_UNSUPPORTED;
    total += heads[i];
    if (total > H) return GLA_ERR_SHAPE;
    if ((st = check_dims(B, heads[i], pooled_len(L, scales[i]), Dk, Dv, C, dtype)) != GLA_OK) return st;
  }
  return total == H ? GLA_OK : GLA_ERR_SHAPE;
}

MsglaLayout msgla_layout(int B, int L, int Dk, int Dv, int C, int dtype, int ngroups, const int* scales,
                         const int* heads) {
  MsglaLayout l{};
  const size_t es = esize_of(dtype);
  size_t off = 0;
  for (int i = 0; i < ngroups; ++i) {
    const size_t rows = (size_t)B * heads[i] * pooled_len(L, scales[i]);
    const size_t st = align_up((size_t)B * heads[i] * Dk * Dv * 4);
    l.pooled[i] = off;
    if (scales[i] > 1) off += 3 * align_up(rows * Dk * es) + align_up(rows * Dv * es);
    l.h0g[i] = off;
    off += st;
    l.htg[i] = off;
    off += st;
    l.gla[i] = off;
    off += align_up(fwd_ws_bytes(B, heads[i], pooled_len(L, scales[i]), Dk, Dv, C, dtype, false));
  }
  l.total = off;
  return l;
}

// ---------------------------------------------------------------- gated slot attention
// As gla_tile_c, for GSA, whose kernels tile chunks of at most 64 rows: a requested C whose
// tiles do not fit (C = 128 always; more than 64 slots with C = 64 in the backward) runs at the
// largest smaller chunk size that fits, with the same results to rounding.
int gsa_tile_c(int m, int C, int dtype, bool bwd) {
  if (!valid_c(C) || (dtype != GLA_F32 && dtype != GLA_BF16) || m < 16 || m > 128 || m % 16 != 0) return C;
  const int es = esize_of(dtype), MP = pad_dk(m);
  for (int c = C; c >= 16; c /= 2) {
    if (c > 64) continue;
    const int CP = pad_c(c);
    if (!gsa_config_fits(es, MP, CP, bwd) || !fwd_config_fits(es, MP, CP) || (bwd && !bwd_config_fits(es, MP, CP)))
      continue;
    return c;
  }
  return C;
}

int check_gsa(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, bool bwd) {
  if (dtype != GLA_F32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 1 || Dk < 1 || Dv < 1 || m < 1 || C < 1) return GLA_ERR_SHAPE;
  if (C != 16 && C != 32 && C != 64) return GLA_ERR_UNSUPPORTED;
  if (m % 16 != 0 || m > 128 || Dk % 16 != 0 || Dk > 256 || Dv % 16 != 0 || Dv > 512) return GLA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > 65535 || (int64_t)L * Dv > INT32_MAX / 2 || (int64_t)L * Dk > INT32_MAX / 2)
    return GLA_ERR_UNSUPPORTED;
  const int es = esize_of(dtype), MP = pad_dk(m), CP = pad_c(C);
  if (!gsa_config_fits(es, MP, CP, bwd) || !fwd_config_fits(es, MP, CP)) return GLA_ERR_UNSUPPORTED;
  if (bwd && !bwd_config_fits(es, MP, CP)) return GLA_ERR_UNSUPPORTED;
  return GLA_OK;
}

struct GsaLayout {
  size_t W, P, Pf, dP, dW2, dg2, dZ, WdT, Gam, S1s, dS1s, dZs, ops2base, Hs2, dHs2, total;
  OpsLayout ops2;
};

// Parts of the GSA device memory.  FWD: the forward's own tensors.  SAVED: those plus what only
// the backward reads (the fp32 read-out Pf) -- what gsa_fwd_save leaves
// for gsa_bwd_saved.  GRAD: the backward's gradient buffers.  gsa_bwd keeps SAVED and GRAD in
// one workspace.
enum { kGsaFwd = 1, kGsaSaved = 2, kGsaGrad = 4 };

GsaLayout gsa_layout_of(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, int parts) {
  const size_t BH = (size_t)B * H, es = esize_of(dtype), MP = pad_dk(m), CP = pad_c(C);
  const size_t N = (L + C - 1) / C, DkP = pad_dv(Dk), DvP = pad_dv(Dv);
  const size_t tok = BH * L * m;
  const bool fwd = parts & (kGsaFwd | kGsaSaved), saved = parts & kGsaSaved, grad = parts & kGsaGrad;
  GsaLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
  if (fwd) {
    if (saved) {   // W and P as [L][m] tensors serve only pass 2's backward
      l.W = take(tok * es);
      l.P = take(tok * es);
    }
    l.WdT = take(BH * N * MP * CP * es);
    l.Gam = take(BH * N * MP * 4);
    l.S1s = take(BH * N * MP * DkP * es);
    if (saved) l.Pf = take(tok * 4);
    l.ops2 = ops_layout(BH, N, CP, MP, es, false);
    l.ops2base = take(l.ops2.total);
    l.Hs2 = take(BH * N * MP * DvP * es);
  }
  if (grad) {
    l.dP = take(tok * 4);
    l.dW2 = take(tok * es);
    l.dg2 = take(tok * 4);
    l.dZ = take(tok * 4);
    l.dS1s = take(BH * N * MP * DkP * es);
    l.dZs = take(BH * N * CP * MP * es);
    l.dHs2 = take(BH * N * MP * DvP * es);
  }
  l.total = off;
  return l;
}

GsaLayout gsa_layout(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, bool bwd) {
  return gsa_layout_of(B, H, L, Dk, Dv, m, C, dtype, bwd ? (kGsaSaved | kGsaGrad) : kGsaFwd);
}

// lf/fb: the forward tensors (FWD or SAVED layout) and their base; lg/gb: the gradient buffers
// (GRAD layout) and their base, or null for a forward
GsaParams gsa_params(const GsaLayout& lf, char* fb, bool saved, const GsaLayout& lg, char* gb, int B, int H, int L,
                     int Dk, int Dv, int m, int C) {
  GsaParams p{};
  p.BH = B * H; p.L = L; p.Dk = Dk; p.DkP = pad_dv(Dk); p.Dv = Dv; p.m = m; p.C = C; p.N = (L + C - 1) / C;
  p.W = saved ? fb + lf.W : nullptr;   // the forward alone needs neither
  p.P = saved ? fb + lf.P : nullptr;
  p.WdT = fb + lf.WdT; p.Gam = reinterpret_cast<float*>(fb + lf.Gam);
  p.S1s = fb + lf.S1s;
  if (saved) p.Pf = reinterpret_cast<float*>(fb + lf.Pf);
  p.ops2 = carve_ops(fb + lf.ops2base, lf.ops2);
  p.ops2.KdT = p.WdT;   // pass 2's decayed keys and chunk decays are pass 1's
  p.ops2.Gam = p.Gam;
  p.Hs2 = fb + lf.Hs2;
  if (gb) {
    p.dP = reinterpret_cast<float*>(gb + lg.dP); p.dW2 = gb + lg.dW2;
    p.dg2 = reinterpret_cast<float*>(gb + lg.dg2); p.dZ = reinterpret_cast<float*>(gb + lg.dZ);
    p.dS1s = gb + lg.dS1s; p.dZs = gb + lg.dZs;
    p.dHs2 = gb + lg.dHs2;
  }
  return p;
}

#define GSA_DISPATCH(LAUNCH, TT, MP, CP, ...)                                                   \
  do {                                                                                         \
    if (MP == 32 && CP == 32) return LAUNCH<TT, 32, 32>(__VA_ARGS__);                          \
    if (MP == 32 && CP == 64) return LAUNCH<TT, 32, 64>(__VA_ARGS__);                          \
    if (MP == 64 && CP == 32) return LAUNCH<TT, 64, 32>(__VA_ARGS__);                          \
    if (MP == 64 && CP == 64) return LAUNCH<TT, 64, 64>(__VA_ARGS__);                          \
    if (MP == 128 && CP == 32) return LAUNCH<TT, 128, 32>(__VA_ARGS__);                        \
    if (MP == 128 && CP == 64) return LAUNCH<TT, 128, 64>(__VA_ARGS__);                        \
  } while (0)

hipError_t dispatch_gsa(bool bwd, int dtype, int MP, int CP, const GsaParams& p, hipStream_t s) {
  if (bwd) {
    if (dtype == GLA_BF16) GSA_DISPATCH(launch_gsa_bwd, bf16, MP, CP, p, s);
    else GSA_DISPATCH(launch_gsa_bwd, float, MP, CP, p, s);
  } else {
    if (dtype == GLA_BF16) GSA_DISPATCH(launch_gsa_fwd, bf16, MP, CP, p, s);
    else GSA_DISPATCH(launch_gsa_fwd, float, MP, CP, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

extern "C" {

size_t gsa_fwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype) {
  C = gsa_tile_c(m, C, dtype, false);
  if (check_gsa(B, H, L, Dk, Dv, m, C, dtype, false) != GLA_OK) return 0;
  return gsa_layout(B, H, L, Dk, Dv, m, C, dtype, false).total;
}

size_t gsa_bwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype) {
  C = gsa_tile_c(m, C, dtype, true);
  if (check_gsa(B, H, L, Dk, Dv, m, C, dtype, true) != GLA_OK) return 0;
  return gsa_layout(B, H, L, Dk, Dv, m, C, dtype, true).total;
}

size_t gsa_saved_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype) {
  C = gsa_tile_c(m, C, dtype, true);
  if (check_gsa(B, H, L, Dk, Dv, m, C, dtype, true) != GLA_OK) return 0;
  return gsa_layout_of(B, H, L, Dk, Dv, m, C, dtype, kGsaSaved).total;
}

size_t gsa_bwd_saved_workspace_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype) {
  C = gsa_tile_c(m, C, dtype, true);
  if (check_gsa(B, H, L, Dk, Dv, m, C, dtype, true) != GLA_OK) return 0;
  return gsa_layout_of(B, H, L, Dk, Dv, m, C, dtype, kGsaGrad).total;
}

}  // extern "C"

namespace {

// gsa_fwd (saving = false: workspace of the FWD layout) and gsa_fwd_save (saving = true: `mem`
// is the caller's saved buffer, SAVED layout)
int gsa_fwd_impl(const void* q, const void* k, const void* v, const void* g, const float* hk0, const float* hv0,
                 void* o, float* hkt, float* hvt, int B, int H, int L, int Dk, int Dv, int m, int C, int dtype,
                 int act, void* mem, size_t mem_bytes, void* stream, bool saving) {
  C = gsa_tile_c(m, C, dtype, saving);
  int st = check_gsa(B, H, L, Dk, Dv, m, C, dtype, saving);
  if (st != GLA_OK) return st;
  if (!valid_act(act)) return GLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !o) return GLA_ERR_NULL_ARG;
  if (!all_aligned({q, k, v, g, hk0, hv0, o, hkt, hvt, mem})) return GLA_ERR_UNSUPPORTED;
  const GsaLayout lay = gsa_layout_of(B, H, L, Dk, Dv, m, C, dtype, saving ? kGsaSaved : kGsaFwd);
  if (!mem || mem_bytes < lay.total) return GLA_ERR_WORKSPACE;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const size_t nk = BH * L * Dk * es, nv = BH * L * Dv * es, ng = BH * L * m * es;
  const size_t sk = BH * Dk * m * 4, sv = BH * m * Dv * 4;
  const Range ins[] = {{q, nk}, {k, nk}, {v, nv}, {g, ng}, {hk0, hk0 ? sk : 0}, {hv0, hv0 ? sv : 0}};
  const Range outs[] = {{o, nv}, {hkt, hkt ? sk : 0}, {hvt, hvt ? sv : 0}, {mem, lay.total}};
  if (any_alias(outs, 4, ins, 6)) return GLA_ERR_ALIAS;
  GsaParams p = gsa_params(lay, static_cast<char*>(mem), saving, lay, nullptr, B, H, L, Dk, Dv, m, C);
  p.q = q; p.k = k; p.v = v; p.g = g; p.hk0 = hk0; p.hv0 = hv0; p.o = o; p.hkt = hkt; p.hvt = hvt;
  p.act = act;
  if (dispatch_gsa(false, dtype, pad_dk(m), pad_c(C), p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

// gsa_bwd (saved = null: `workspace` holds SAVED then GRAD, and the forward tensors are
// recomputed) and gsa_bwd_saved (saved: what gsa_fwd_save left; workspace: GRAD)
int gsa_bwd_impl(const void* q, const void* k, const void* v, const void* g, const float* hk0, const float* hv0,
                 const void* do_, const float* dhkt, const float* dhvt, void* dq, void* dk, void* dv, float* dg,
                 float* dhk0, float* dhv0, int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, int act,
                 const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  C = gsa_tile_c(m, C, dtype, true);
  int st = check_gsa(B, H, L, Dk, Dv, m, C, dtype, true);
  if (st != GLA_OK) return st;
  if (!valid_act(act)) return GLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !do_ || !dq || !dk || !dv || !dg) return GLA_ERR_NULL_ARG;
  if (!all_aligned({q, k, v, g, hk0, hv0, do_, dhkt, dhvt, dq, dk, dv, dg, dhk0, dhv0, workspace, saved}))
    return GLA_ERR_UNSUPPORTED;
  const bool use_saved = saved != nullptr;
  const GsaLayout ls = gsa_layout_of(B, H, L, Dk, Dv, m, C, dtype, kGsaSaved);
  const GsaLayout lg = gsa_layout_of(B, H, L, Dk, Dv, m, C, dtype, kGsaGrad);
  const GsaLayout lw = use_saved ? lg : gsa_layout(B, H, L, Dk, Dv, m, C, dtype, true);
  if (use_saved && saved_bytes < ls.total) return GLA_ERR_WORKSPACE;
  if (!workspace || workspace_bytes < lw.total) return GLA_ERR_WORKSPACE;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const size_t nk = BH * L * Dk * es, nv = BH * L * Dv * es, ng = BH * L * m * es;
  const size_t sk = BH * Dk * m * 4, sv = BH * m * Dv * 4;
  const Range ins[] = {{q, nk}, {k, nk}, {v, nv}, {g, ng}, {hk0, hk0 ? sk : 0}, {hv0, hv0 ? sv : 0},
                       {do_, nv}, {dhkt, dhkt ? sk : 0}, {dhvt, dhvt ? sv : 0}, {saved, use_saved ? ls.total : 0}};
  const Range outs[] = {{dq, nk}, {dk, nk}, {dv, nv}, {dg, BH * L * m * 4}, {dhk0, dhk0 ? sk : 0},
                        {dhv0, dhv0 ? sv : 0}, {workspace, lw.total}};
  if (any_alias(outs, 7, ins, 10)) return GLA_ERR_ALIAS;
  char* ws = static_cast<char*>(workspace);
  // read only on the saved path
  GsaParams p = use_saved ? gsa_params(ls, const_cast<char*>(static_cast<const char*>(saved)), true, lg, ws, B, H,
                                       L, Dk, Dv, m, C)
                          : gsa_params(lw, ws, true, lw, ws, B, H, L, Dk, Dv, m, C);
  p.q = q; p.k = k; p.v = v; p.g = g; p.do_ = do_; p.hk0 = hk0; p.hv0 = hv0; p.dhkt = dhkt; p.dhvt = dhvt;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.dhk0 = dhk0; p.dhv0 = dhv0;
  p.act = act;
  p.saved = use_saved ? 1 : 0;
  if (dispatch_gsa(true, dtype, pad_dk(m), pad_c(C), p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

}  // namespace

extern "C" {

int gsa_fwd(const void* q, const void* k, const void* v, const void* g, const float* hk0, const float* hv0,
            void* o, float* hkt, float* hvt, int B, int H, int L, int Dk, int Dv, int m, int C, int dtype,
            int act, void* workspace, size_t workspace_bytes, void* stream) {
  return gsa_fwd_impl(q, k, v, g, hk0, hv0, o, hkt, hvt, B, H, L, Dk, Dv, m, C, dtype, act, workspace,
                      workspace_bytes, stream, false);
}

int gsa_fwd_save(const void* q, const void* k, const void* v, const void* g, const float* hk0, const float* hv0,
                 void* o, float* hkt, float* hvt, int B, int H, int L, int Dk, int Dv, int m, int C, int dtype,
                 int act, void* saved, size_t saved_bytes, void* stream) {
  return gsa_fwd_impl(q, k, v, g, hk0, hv0, o, hkt, hvt, B, H, L, Dk, Dv, m, C, dtype, act, saved, saved_bytes,
                      stream, true);
}

int gsa_bwd(const void* q, const void* k, const void* v, const void* g, const float* hk0, const float* hv0,
            const void* do_, const float* dhkt, const float* dhvt, void* dq, void* dk, void* dv, float* dg,
            float* dhk0, float* dhv0, int B, int H, int L, int Dk, int Dv, int m, int C, int dtype,
            int act, void* workspace, size_t workspace_bytes, void* stream) {
  return gsa_bwd_impl(q, k, v, g, hk0, hv0, do_, dhkt, dhvt, dq, dk, dv, dg, dhk0, dhv0, B, H, L, Dk, Dv, m, C,
                      dtype, act, nullptr, 0, workspace, workspace_bytes, stream);
}

int gsa_bwd_saved(const void* q, const void* k, const void* v, const void* g, const float* hk0, const float* hv0,
                  const void* do_, const float* dhkt, const float* dhvt, void* dq, void* dk, void* dv, float* dg,
                  float* dhk0, float* dhv0, int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, int act,
                  const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  if (!saved) return GLA_ERR_NULL_ARG;
  return gsa_bwd_impl(q, k, v, g, hk0, hv0, do_, dhkt, dhvt, dq, dk, dv, dg, dhk0, dhv0, B, H, L, Dk, Dv, m, C,
                      dtype, act, saved, saved_bytes, workspace, workspace_bytes, stream);
}

size_t msgla_fwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype, int ngroups,
                                 const int* scales, const int* heads) {
  C = gla_tile_c(Dk, C, dtype, false);
  if (check_msgla(B, H, L, Dk, Dv, C, dtype, ngroups, scales, heads) != GLA_OK) return 0;
  return msgla_layout(B, L, Dk, Dv, C, dtype, ngroups, scales, heads).total;
}

int msgla_fwd(const void* q, const void* k, const void* v, const void* g, const float* h0, const float* w,
              void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype, int ngroups,
              const int* scales, const int* heads, void* workspace, size_t workspace_bytes, void* stream) {
  C = gla_tile_c(Dk, C, dtype, false);
  int st = check_msgla(B, H, L, Dk, Dv, C, dtype, ngroups, scales, heads);
  if (st != GLA_OK) return st;
  if (!q || !k || !v || !g || !o) return GLA_ERR_NULL_ARG;
  if (!all_aligned({q, k, v, g, h0, o, ht, workspace}) || (reinterpret_cast<uintptr_t>(w) & 3))
    return GLA_ERR_UNSUPPORTED;
  const MsglaLayout lay = msgla_layout(B, L, Dk, Dv, C, dtype, ngroups, scales, heads);
  if (!workspace || workspace_bytes < lay.total) return GLA_ERR_WORKSPACE;
  const size_t es = esize_of(dtype), BH = (size_t)B * H;
  const size_t nk = BH * L * Dk * es, nv = BH * L * Dv * es, ns = BH * Dk * Dv * 4;
  const Range ins[] = {{q, nk}, {k, nk}, {v, nv}, {g, nk}, {h0, h0 ? ns : 0},
                       {w, w ? (size_t)B * L * ngroups * 4 : 0}};
  const Range outs[] = {{o, nv}, {ht, ht ? ns : 0}, {workspace, lay.total}};
  if (any_alias(outs, 3, ins, 6)) return GLA_ERR_ALIAS;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  MsglaParams mp{};
  mp.q = q; mp.k = k; mp.v = v; mp.g = g;
  mp.B = B; mp.H = H; mp.L = L; mp.Dk = Dk; mp.Dv = Dv; mp.ngroups = ngroups;
  int hbeg = 0;
  bool pooled = false;
  mp.pooled_heads = 0;
  mp.max_pooled_len = 0;
  for (int i = 0; i < ngroups; ++i) {
    const size_t rows = (size_t)B * heads[i] * pooled_len(L, scales[i]);
    MsglaGroup& G = mp.grp[i];
    G.h0 = hbeg; G.nh = heads[i]; G.s = scales[i];
    if (G.s > 1) {
      G.qp = ws + lay.pooled[i];
      G.kp = static_cast<char*>(G.qp) + align_up(rows * Dk * es);
      G.gp = static_cast<char*>(G.kp) + align_up(rows * Dk * es);
      G.vp = static_cast<char*>(G.gp) + align_up(rows * Dk * es);
      pooled = true;
      mp.pooled_heads += G.nh;
      mp.max_pooled_len = std::max(mp.max_pooled_len, pooled_len(L, G.s));
    }
    hbeg += heads[i];
  }
  hipError_t e = hipSuccess;
  if (pooled && (e = dtype == GLA_BF16 ? launch_msgla_pool<bf16>(mp, hs) : launch_msgla_pool<float>(mp, hs)) !=
                    hipSuccess)
    return GLA_ERR_HIP;

  // The head groups' GLA forwards on their pooled sequences (scale 1: on the caller's tensors,
  // through a strided view of the group's heads), all groups in each of three launches, so the
  // small groups fill the CUs the large one leaves idle.  A group's heads are a strided slice
  // of [B][H]: its states are gathered into / scattered from contiguous buffers.
  const size_t head_bytes = (size_t)Dk * Dv * 4;
  const int DKP = pad_dk(Dk), CP = pad_c(C);
  FwdParams ps[kMsMaxGroups];
  for (int i = 0; i < ngroups; ++i) {
    const MsglaGroup& G = mp.grp[i];
    float* h0g = reinterpret_cast<float*>(ws + lay.h0g[i]);
    float* htg = reinterpret_cast<float*>(ws + lay.htg[i]);
    const int Ls = pooled_len(L, G.s), N = (Ls + C - 1) / C;
    if (h0 && hipMemcpy2DAsync(h0g, G.nh * head_bytes, h0 + (size_t)G.h0 * Dk * Dv, (size_t)H * head_bytes,
                               G.nh * head_bytes, B, hipMemcpyDeviceToDevice, hs) != hipSuccess)
      return GLA_ERR_HIP;
    FwdParams& p = ps[i];
    if (G.s == 1) {
      p.q = q; p.k = k; p.v = v; p.g = g;
      p.in = SeqView{G.nh, H, G.h0};
    } else {
      p.q = G.qp; p.k = G.kp; p.v = G.vp; p.g = G.gp;
    }
    p.h0 = h0 ? h0g : nullptr;
    p.o = nullptr; p.ht = ht ? htg : nullptr;
    // the output kernel holds each pooled row over its tokens and applies the fusion weights
    p.hold_o = o; p.hold_w = w;
    p.hold_s = G.s; p.hold_L = L; p.hold_H = H; p.hold_h0 = G.h0; p.hold_nh = G.nh;
    p.hold_ng = ngroups; p.hold_gi = i;
    p.BH = B * G.nh; p.L = Ls; p.Dk = Dk; p.Dv = Dv; p.C = C; p.N = N;
    const OpsLayout ol = ops_layout((size_t)p.BH, N, CP, DKP, es);
    p.ops = carve_ops(ws + lay.gla[i], ol);
    p.Hs = ws + lay.gla[i] + ol.total;
    p.events = LaunchEvents{nullptr, 0};
  }
  if (dispatch_fwd_batches(dtype, DKP, CP, ps, ngroups, hs) != hipSuccess) return GLA_ERR_HIP;
  for (int i = 0; i < ngroups && ht; ++i) {
    const MsglaGroup& G = mp.grp[i];
    if (hipMemcpy2DAsync(ht + (size_t)G.h0 * Dk * Dv, (size_t)H * head_bytes, ws + lay.htg[i], G.nh * head_bytes,
                         G.nh * head_bytes, B, hipMemcpyDeviceToDevice, hs) != hipSuccess)
      return GLA_ERR_HIP;
  }
  return GLA_OK;
}

}  // extern "C"
