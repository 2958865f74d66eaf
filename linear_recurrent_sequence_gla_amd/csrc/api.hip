// api.hip -- the extern "C" entry points declared in include/gla.h: synchronous argument
// validation, workspace carving and kernel dispatch.  Nothing is enqueued unless every check
// passes, so a failing call leaves all outputs untouched.
#include <stdint.h>
#include <string.h>

#include <initializer_list>

#include "../../include/gla.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace gla;

namespace {

constexpr int kAbiVersion = 1;
constexpr size_t kAlign = 256;

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
  size_t qs, qst, kdt, a, gam, total;
};

OpsLayout ops_layout(size_t BH, size_t N, size_t CP, size_t DKP, size_t es, bool want_qst) {
  OpsLayout l{};
  size_t off = 0;
  l.qs = off;  off += align_up(BH * N * CP * DKP * es);
  l.qst = off; if (want_qst) off += align_up(BH * N * CP * DKP * es);
  l.kdt = off; off += align_up(BH * N * CP * DKP * es);
  l.a = off;   off += align_up(BH * N * CP * CP * es);
  l.gam = off; off += align_up(BH * N * DKP * 4);
  l.total = off;
  return l;
}

ChunkOps carve_ops(char* ws, const OpsLayout& l, bool want_qst) {
  ChunkOps o;
  o.Qs = ws + l.qs;
  o.QsT = want_qst ? ws + l.qst : nullptr;
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

hipError_t dispatch_bwd(int dtype, int DKP, int CP, const BwdParams& p, hipStream_t s) {
  if (dtype == GLA_BF16) GLA_DISPATCH_DKCP(launch_gla_bwd, bf16, DKP, CP, p, s);
  else GLA_DISPATCH_DKCP(launch_gla_bwd, float, DKP, CP, p, s);
  return hipErrorInvalidValue;
}

size_t fwd_ws_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  (void)Dv;
  const size_t BH = (size_t)B * H, CP = pad_c(C), DKP = pad_dk(Dk), N = (L + C - 1) / C;
  return ops_layout(BH, N, CP, DKP, esize_of(dtype), false).total;
}

struct BwdLayout {
  OpsLayout ops;
  size_t hs, dhs, carry, total;
};

BwdLayout bwd_layout(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  const size_t BH = (size_t)B * H, CP = pad_c(C), DKP = pad_dk(Dk), N = (L + C - 1) / C;
  const size_t es = esize_of(dtype), DVP = pad_dv(Dv), NT = DVP / kDvTile;
  BwdLayout l;
  l.ops = ops_layout(BH, N, CP, DKP, es, true);
  size_t off = l.ops.total;
  l.hs = off;    off += align_up(BH * N * DKP * DVP * es);
  l.dhs = off;   off += align_up(BH * N * DKP * DVP * es);
  l.carry = off; off += align_up(BH * N * NT * DKP * 4);
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
      return "GLA_ERR_UNSUPPORTED: C must be 16/32/64/128, Dk and m multiples of 16 up to 256, "
             "Dv a multiple of 16 up to 512, B*H <= 65535, 16-byte aligned tensors; tiles that "
             "exceed a CU's LDS are not supported (bf16: Dk > 128 with C = 128; fp32: C = 128, "
             "or Dk > 128 with C = 64)";
    case GLA_ERR_WORKSPACE: return "GLA_ERR_WORKSPACE: workspace NULL or smaller than the query returned";
    case GLA_ERR_ALIAS: return "GLA_ERR_ALIAS: an output overlaps an input, another output or the workspace";
    case GLA_ERR_HIP: return "GLA_ERR_HIP: a HIP kernel launch failed";
    default: return "unknown status";
  }
}

size_t gla_fwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  return fwd_ws_bytes(B, H, L, Dk, Dv, C, dtype);
}

size_t gla_bwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  if (!bwd_config_fits(esize_of(dtype), pad_dk(Dk), pad_c(C))) return 0;
  return bwd_layout(B, H, L, Dk, Dv, C, dtype).total;
}

}  // extern "C"

namespace {

int fwd_impl(const void* q, const void* k, const void* v, const void* g, const float* h0,
             void* o, float* ht, int B, int H, int L, int Dk, int Dv, int C, int dtype,
             void* workspace, size_t workspace_bytes, void* stream, LaunchEvents ev) {
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
  p.ops = carve_ops(static_cast<char*>(workspace), ops_layout(BH, N, CP, DKP, es, false), false);
  p.events = ev;
  if (dispatch_fwd(dtype, DKP, CP, p, static_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

int bwd_impl(const void* q, const void* k, const void* v, const void* g, const float* h0,
             const void* do_, const float* dht, void* dq, void* dk, void* dv, float* dg,
             float* dh0, int B, int H, int L, int Dk, int Dv, int C, int dtype,
             void* workspace, size_t workspace_bytes, void* stream, LaunchEvents ev) {
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
  p.ops = carve_ops(ws, lay.ops, true);
  p.Hs = ws + lay.hs;
  p.dHs = ws + lay.dhs;
  p.carry = reinterpret_cast<float*>(ws + lay.carry);
  p.events = ev;
  if (dispatch_bwd(dtype, DKP, CP, p, static_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
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

int gla_bwd_launch_count(int B, int H, int L, int Dk, int Dv, int C, int dtype) {
  if (check_dims(B, H, L, Dk, Dv, C, dtype) != GLA_OK) return 0;
  return bwd_launch_count(esize_of(dtype), pad_dk(Dk), pad_c(C));
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

}  // extern "C"
