// msgla.hip -- the multi-scale GLA (MS-GLA) front end's temporal pooling per head group.
// Each group's pooled sequence then runs through the GLA forward kernels unchanged (MS-GLA
// summary, section 3.4: static, non-overlapping pooling keeps each branch a contiguous,
// shorter GLA sequence), and the forward's output kernel writes the causal hold with the
// per-token fusion weights itself (FwdParams::hold_o).
//
//   pooling (section 3.1): block j of group scale s averages tokens j*s .. min(j*s+s, L) - 1
//       of q, k, g and v (a trailing partial block averages only its real tokens), for the
//       group's heads, into contiguous [B][heads][ceil(L/s)][D] tensors (scale 1 is the
//       identity: those heads are read in place, through a strided sequence view);
//   hold and fusion (section 3.3): token t takes the pooled output of block (t+1)/s - 1, the
//       latest block it has fully seen (zero before the first completes), times the caller's
//       weight w[b][t][group].
//
// The pooling is a plain HBM stream with 16-byte accesses and fp32 sums; nothing here
// contracts, so there is no matrix-core work.
#include "common.hpp"
#include "kernels.hpp"

namespace gla {

constexpr int kMsRowsPerBlock = 4;      // pooled rows per pooling workgroup
constexpr int kMsUnroll = 4;            // tokens whose loads are in flight together

// grid (ceil(max pooled length / kMsRowsPerBlock), B * pooled heads): only the groups with a
// scale above 1 are pooled; blocks past their group's pooled length return
template <typename T>
__global__ __launch_bounds__(256) void msgla_pool_kernel(MsglaParams p) {
  typedef typename V16<T>::type VT;
  constexpr int V = V16<T>::N;
  const int b = blockIdx.y / p.pooled_heads;
  int k = blockIdx.y - b * p.pooled_heads, gi = 0;
#pragma unroll 1
  for (; gi < p.ngroups; ++gi) {            // the k-th pooled head, in head order
    if (p.grp[gi].s == 1) continue;
    if (k < p.grp[gi].nh) break;
    k -= p.grp[gi].nh;
  }
  const MsglaGroup& G = p.grp[gi];
  const int s = G.s, Ls = (p.L + s - 1) / s, hl = k, h = G.h0 + hl, bh = b * p.H + h;
  const int j0 = blockIdx.x * kMsRowsPerBlock;
  if (j0 >= Ls) return;
  const int nk = p.Dk / V, nv = p.Dv / V, per_row = 3 * nk + nv;
  const size_t src_k = (size_t)bh * p.L * p.Dk, src_v = (size_t)bh * p.L * p.Dv;
  const size_t dst_row = (size_t)(b * G.nh + hl) * Ls;
  const int rows = min(kMsRowsPerBlock, Ls - j0);
  for (int idx = threadIdx.x; idx < rows * per_row; idx += 256) {
    const int r = idx / per_row, c = idx - r * per_row;
    const int j = j0 + r;
    const int t0 = j * s, cnt = min(s, p.L - t0);
    const T* src;
    T* dst;
    int col, D;
    if (c < 3 * nk) {
      const int which = c / nk;
      col = (c - which * nk) * V;
      D = p.Dk;
      src = reinterpret_cast<const T*>(which == 0 ? p.q : which == 1 ? p.k : p.g) + src_k;
      dst = reinterpret_cast<T*>(which == 0 ? G.qp : which == 1 ? G.kp : G.gp) + dst_row * p.Dk;
    } else {
      col = (c - 3 * nk) * V;
      D = p.Dv;
      src = reinterpret_cast<const T*>(p.v) + src_v;
      dst = reinterpret_cast<T*>(G.vp) + dst_row * p.Dv;
    }
    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.f;
    // kMsUnroll tokens' loads issued together, from rows clamped into the block
    for (int u0 = 0; u0 < cnt; u0 += kMsUnroll) {
      VT x[kMsUnroll];
#pragma unroll
      for (int u = 0; u < kMsUnroll; ++u)
        x[u] = *reinterpret_cast<const VT*>(src + (size_t)(t0 + min(u0 + u, cnt - 1)) * D + col);
#pragma unroll
      for (int u = 0; u < kMsUnroll; ++u) {
        if (u0 + u < cnt) {
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] += to_f32(x[u][e]);
        }
      }
    }
    const float inv = 1.f / (float)cnt;
    VT y;
#pragma unroll
    for (int e = 0; e < V; ++e) y[e] = from_f32<T>(cnt == 1 ? acc[e] : acc[e] * inv);
    *reinterpret_cast<VT*>(dst + (size_t)j * D + col) = y;
  }
}

template <typename T>
hipError_t launch_msgla_pool(const MsglaParams& p, hipStream_t s) {
  if (p.pooled_heads == 0) return hipSuccess;
  hipLaunchKernelGGL((msgla_pool_kernel<T>),
                     dim3((p.max_pooled_len + kMsRowsPerBlock - 1) / kMsRowsPerBlock, p.B * p.pooled_heads),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_msgla_pool<bf16>(const MsglaParams&, hipStream_t);
template hipError_t launch_msgla_pool<float>(const MsglaParams&, hipStream_t);

}  // namespace gla
