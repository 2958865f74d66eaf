/*
 * gla.h -- C ABI of the MI355X (gfx950) gated linear attention library, libgla_amd.so.
 *
 * Operations (all per batch row b and head h, tokens t = 0..L-1):
 *
 *   GLA  (gated linear attention; GLA visual companion "Gated Linear Attention for Efficient
 *         Long Sequences", cards "Core move" and "Step-by-step memory update"; MS-GLA summary,
 *         section 2.1 "Linear Attention and Gated Linear Attention (GLA)"):
 *         alpha_t = exp(g_t) per key channel (the forget gate scales the rows of the memory)
 *         S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t,   o_t = q_t S_t,   S_{-1} = h0 (or 0),
 *         ht = S_{L-1}.  Computed chunkwise (same section: sequential inter-chunk updates,
 *         parallel intra-chunk computation) with chunk size C; the result does not depend on C
 *         beyond rounding.
 *   GSA  (gated slot attention; "Gated Slot Attention for Efficient Linear-Time Sequence
 *         Modeling": abstract, and research-map summary "Approach"): m slots with per-slot
 *         forget gates alpha_t = exp(g_t), write weights w_t = 1 - alpha_t;
 *         pass 1 (slot keys):   S1_t = S1_{t-1} Diag(alpha_t) + k_t^T w_t,  z_t = q_t S1_t
 *         p_t = softmax(z_t) over the m slots (or an element-wise read-out, gsa_act)
 *         pass 2 (slot values): S2_t = Diag(alpha_t) S2_{t-1} + w_t^T v_t,  o_t = p_t S2_t
 *
 * Conventions shared by every entry point
 *   - Tensors are device pointers (HIP device memory of the current device), contiguous,
 *     row-major, last dimension fastest.  Shapes are given next to each argument.
 *   - dtype (gla_dtype) is the element type of q, k, v, g, o, do_, dq, dk, dv (all the same).
 *     States (h0, ht, state, hk*, hv*, dh*) and gate gradients dg are always float32.
 *     Internal accumulation is float32; bf16 operands feed bf16 matrix cores.
 *   - Ownership: the caller owns every buffer.  The library never allocates device memory;
 *     scratch space is the caller's `workspace` of at least the size the matching
 *     *_workspace_bytes() query returns (its contents on entry do not matter).  The one
 *     exception is gla_fwd_noalloc, whose scratch is a fixed 64 MiB array of the library's own
 *     device memory (one per device, created with the library's code object).
 *   - Synchrony: arguments are validated on the host before anything is enqueued.  On any
 *     error the call returns a non-zero gla_status and enqueues nothing, so no output is
 *     touched.  On success all work is enqueued on `stream` (a hipStream_t, NULL = the null
 *     stream) and the call returns at once; outputs are valid once the stream is synchronised.
 *   - Errors are reported only through the return value; the library never prints or aborts.
 *     GLA_ERR_HIP means a launch failed (hipGetLastError); faults inside kernels surface at
 *     the caller's next synchronisation.
 *   - Outputs must not overlap inputs or each other (GLA_ERR_ALIAS), except `state` of
 *     gla_decode_step, which is updated in place.
 *   - Supported sizes: B, H >= 1; L >= 1 (any value; the last chunk may be partial);
 *     C in {16, 32, 64, 128}; Dk and m multiples of 16 up to 256; Dv a multiple of 16 up to
 *     512; B*H <= 65535; every tensor 16-byte aligned.  The result does not depend on C, a
 *     tiling choice: where the requested C's chunk tiles do not fit a CU's LDS (bf16 with
 *     Dk > 128 and C = 128; float32 with Dk > 128 and C = 64, Dk > 64 and C = 128, and every
 *     backward with C = 128), the call runs with the largest smaller C whose tiles fit, the
 *     same for a saving forward and its backward, and the sizes queried follow it.  Other
 *     values return GLA_ERR_UNSUPPORTED (shape errors such as L < 1 return GLA_ERR_SHAPE);
 *     a *_workspace_bytes() query returns 0 for them.
 *   - Results are deterministic: no floating-point atomics are used, so two runs on the same
 *     inputs give bitwise-identical outputs.
 *   - The library is reentrant.  Its only global state, kept per device it has run on and
 *     read once, is the compute-unit count (it picks the state walks' tile height), how many
 *     chunk-gradient workgroups the device runs at once (the size of that kernel's persistent
 *     grid) and the address of gla_fwd_noalloc's scratch array (whose contents calls of that
 *     entry point share).
 */
#ifndef GLA_AMD_GLA_H
#define GLA_AMD_GLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_OK = 0,
  GLA_ERR_NULL_ARG = 1,    /* a required pointer is NULL                               */
  GLA_ERR_SHAPE = 2,       /* a size is < 1                                           */
  GLA_ERR_DTYPE = 3,       /* dtype is not a gla_dtype value                          */
  GLA_ERR_UNSUPPORTED = 4, /* C, Dk, Dv or m outside the supported set                */
  GLA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the query returned       */
  GLA_ERR_ALIAS = 6,       /* an output overlaps an input or another output           */
  GLA_ERR_HIP = 7,         /* a HIP launch failed                                     */
  GLA_ERR_SCRATCH = 8      /* gla_fwd_noalloc: the sizes need more than its fixed scratch */
} gla_status;

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype;

/* Read-out between GSA's two passes (argument `act` of the gsa_* entry points).  Softmax over
 * the slots is GSA's own; the GSA summary's ablations ("Measured effects") replace it with
 * Swish, ReLU or ReLU^2, or drop it.  The replacements act on each slot score z alone, with
 * no normalisation over the slots:  SWISH p = z sigmoid(z);  RELU p = max(z, 0);
 * RELU2 p = max(z, 0)^2;  NONE p = z.  Other values give GLA_ERR_UNSUPPORTED. */
typedef enum {
  GSA_ACT_SOFTMAX = 0,
  GSA_ACT_SWISH = 1,
  GSA_ACT_RELU = 2,
  GSA_ACT_RELU2 = 3,
  GSA_ACT_NONE = 4
} gsa_act;

/* Version of this ABI (incremented on any incompatible change). */
int gla_abi_version(void);

/* Static, human-readable text for a status code (unknown codes give "unknown status"). */
const char* gla_status_str(int status);

/* ---------------------------------------------------------------- GLA forward ----------
 * Bytes of workspace gla_fwd needs for these sizes (0 if the sizes are unsupported). */
size_t gla_fwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype);

/* Chunkwise GLA forward.
 *   q, k, g : [B,H,L,Dk] dtype  (g = log of the forget gate, any real; normally <= 0)
 *   v       : [B,H,L,Dv] dtype
 *   h0      : [B,H,Dk,Dv] float32 initial state, or NULL for zeros
 *   o       : [B,H,L,Dv] dtype   output
 *   ht      : [B,H,Dk,Dv] float32 final state, or NULL to skip it */
int gla_fwd(const void* q, const void* k, const void* v, const void* g, const float* h0,
            void* o, float* ht,
            int B, int H, int L, int Dk, int Dv, int C, int dtype,
            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- GLA forward, no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gla_fwd with the same arguments, results and errors,
 * minus the workspace.  Its scratch is a fixed buffer of gla_fwd_noalloc_max_workspace_bytes()
 * = 64 MiB in the library's own device memory, one per device the library runs on, held until
 * the process ends.  Sizes whose gla_fwd_workspace_bytes() exceeds it return GLA_ERR_SCRATCH
 * before anything is enqueued.  The call never allocates or frees device memory.
 *   - Every call on one device shares that device's buffer and leaves its contents behind;
 *     nothing in it needs clearing between calls.  Calls that overlap on one device (other
 *     streams, other host threads) race on it: order them, e.g. on one stream.
 *   - The first call on a device looks the buffer's address up (hipGetSymbolAddress, no
 *     allocation); make that first call outside graph capture. */
size_t gla_fwd_noalloc_max_workspace_bytes(void);
int gla_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const float* h0,
                    void* o, float* ht,
                    int B, int H, int L, int Dk, int Dv, int C, int dtype, void* stream);

/* ---------------------------------------------------------------- GLA backward ---------
 * Gradients of sum(o * do_) + sum(ht * dht).  gla_bwd recomputes what it needs from the
 * forward inputs (no saved activations).
 *   q, k, v, g, h0 : as in gla_fwd (h0 NULL = zeros)
 *   do_  : [B,H,L,Dv] dtype   gradient of o
 *   dht  : [B,H,Dk,Dv] float32 gradient of ht, or NULL for zero
 *   dq, dk : [B,H,L,Dk] dtype;  dv : [B,H,L,Dv] dtype
 *   dg   : [B,H,L,Dk] float32  gradient of the log gates
 *   dh0  : [B,H,Dk,Dv] float32 gradient of h0, or NULL to skip it */
size_t gla_bwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype);
int gla_bwd(const void* q, const void* k, const void* v, const void* g, const float* h0,
            const void* do_, const float* dht,
            void* dq, void* dk, void* dv, float* dg, float* dh0,
            int B, int H, int L, int Dk, int Dv, int C, int dtype,
            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- profiling ------------
 * Same as gla_fwd / gla_bwd, and additionally records caller-created hipEvent_t handles on
 * `stream` at kernel boundaries: events[0] before the first kernel, events[i] after the i-th
 * (gla_fwd launches 3 kernels: chunk preparation, state walk, chunk outputs, or 2 of them per
 * gla_fwd_launch_count(), events[2] and events[3] then both after the second; gla_bwd launches
 * gla_bwd_launch_count() kernels: chunk preparation, forward state walk, reverse state walk,
 * chunk gradients, and a value-gradient kernel when the key width is split).  nevents must
 * be at least 4 (forward) or 6 (backward), else GLA_ERR_NULL_ARG.  The events are owned by the caller and are only
 * recorded, never created, synchronised or destroyed.  Used to time individual kernels. */
int gla_fwd_profiled(const void* q, const void* k, const void* v, const void* g, const float* h0,
                     void* o, float* ht,
                     int B, int H, int L, int Dk, int Dv, int C, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream, void** events, int nevents);
int gla_bwd_profiled(const void* q, const void* k, const void* v, const void* g, const float* h0,
                     const void* do_, const float* dht,
                     void* dq, void* dk, void* dv, float* dg, float* dh0,
                     int B, int H, int L, int Dk, int Dv, int C, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream, void** events, int nevents);
/* Number of kernels gla_bwd launches for these sizes (0 if unsupported). */
int gla_bwd_launch_count(int B, int H, int L, int Dk, int Dv, int C, int dtype);
/* Kernel phases of gla_fwd (keep_states = 0) or gla_fwd_save (keep_states = 1) for these sizes
 * on the current device: 3 (chunk preparation, state walk, chunk outputs), or 2 where the state
 * walk and the chunk outputs run as one kernel (bf16, Dk in 65..128, C = 64, B*H*Dv/32 at
 * least the device's compute units, and Dv a multiple of 32, or of 64 with keep_states); 0 if
 * unsupported.  With 2, the profiled entry points record events[2] and events[3] both after
 * the fused kernel.  Pure host query: nothing is enqueued. */
int gla_fwd_launch_count(int B, int H, int L, int Dk, int Dv, int C, int dtype, int keep_states);

/* ---------------------------------------------------------------- GLA saved activations --
 * A training step runs the forward and then the backward on the same q, k, v, g, h0.  The
 * backward needs the per-chunk operands (decayed queries and keys, Gamma, the intra-chunk
 * scores) and the state at every chunk start; gla_bwd recomputes them (one preparation and
 * one forward state walk), which gla_fwd_save / gla_bwd_saved avoid by keeping them:
 *
 *   gla_fwd_save   computes exactly what gla_fwd computes (o, ht) and also leaves the chunk
 *                  operands and the chunk-start states H_n (the sequential inter-chunk state
 *                  of the chunkwise form, MS-GLA summary section 2.1) in `saved`.
 *   gla_bwd_saved  computes exactly what gla_bwd computes, reading them from `saved`.
 *
 * saved: device buffer of at least gla_saved_bytes() bytes, owned by the caller; its contents
 *   on entry to gla_fwd_save do not matter, and gla_bwd_saved only reads it.  It is valid
 *   for the q, k, g, h0, C and dtype of the gla_fwd_save call that filled it; passing other
 *   inputs to gla_bwd_saved gives undefined results (the library cannot check this).  The
 *   states take B*H*ceil(L/C)*pad(Dk)*pad(Dv) elements of dtype (pad(Dv) = Dv rounded up to
 *   64, pad(Dk) = 32, 64, 128 or 256), about 130 MB at B=8, H=4, L=2048, Dk=128, Dv=256.
 * workspace (gla_bwd_saved): at least gla_bwd_saved_workspace_bytes() bytes.
 * events / nevents: optional (NULL, 0) launch-boundary events as for gla_*_profiled:
 *   gla_fwd_save launches 3 kernels, or 2 per gla_fwd_launch_count(..., 1) (nevents >= 4 either
 *   way), gla_bwd_saved launches
 *   gla_bwd_launch_count() - 2 kernels (nevents >= 4).
 * Sizes, dtypes, alignment and errors as for gla_bwd (the saved path supports the sizes the
 * backward supports); `saved` must not overlap any input or output (GLA_ERR_ALIAS). */
size_t gla_saved_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype);
size_t gla_bwd_saved_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype);
int gla_fwd_save(const void* q, const void* k, const void* v, const void* g, const float* h0,
                 void* o, float* ht,
                 int B, int H, int L, int Dk, int Dv, int C, int dtype,
                 void* saved, size_t saved_bytes, void* stream, void** events, int nevents);
int gla_bwd_saved(const void* q, const void* k, const void* v, const void* g, const float* h0,
                  const void* do_, const float* dht,
                  void* dq, void* dk, void* dv, float* dg, float* dh0,
                  int B, int H, int L, int Dk, int Dv, int C, int dtype,
                  const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                  void* stream, void** events, int nevents);

/* ---------------------------------------------------------------- GLA decode -----------
 * One recurrent inference step per (batch, head): the O(1)-memory form of the recurrence
 * (MS-GLA summary, section 1; GSA abstract: efficient recurrent inference).
 *   q, k, g : [B,H,Dk] dtype;  v : [B,H,Dv] dtype
 *   state   : [B,H,Dk,Dv] float32, read and overwritten with Diag(exp g) state + k^T v
 *   o       : [B,H,Dv] dtype = q state (after the update)
 * Needs no workspace.  Dk up to 256 and Dv up to 512, multiples of 16. */
int gla_decode_step(const void* q, const void* k, const void* v, const void* g,
                    float* state, void* o,
                    int B, int H, int Dk, int Dv, int dtype, void* stream);

/* ---------------------------------------------------------------- GSA forward ----------
 * Supported: C in {16, 32, 64, 128}; m a multiple of 16 up to 128; Dk a multiple of 16 up to
 * 256; Dv a multiple of 16 up to 512 (others: GLA_ERR_UNSUPPORTED).  As for GLA, C is a tiling
 * choice: the GSA kernels tile chunks of at most 64 rows, and the backward (gsa_bwd,
 * gsa_fwd_save, gsa_bwd_saved) of at most 32 with m > 64 (and of float32 with m = 64), so a
 * larger C runs at the largest that fits.  float32 with m > 64 has a forward only.
 * act: a gsa_act value.
 *   q, k : [B,H,L,Dk] dtype;  v : [B,H,L,Dv] dtype;  g : [B,H,L,m] dtype slot log-gates
 *   hk0  : [B,H,Dk,m] float32 initial pass-1 state or NULL;  hv0 : [B,H,m,Dv] or NULL
 *   o    : [B,H,L,Dv] dtype
 *   hkt, hvt : final states (same shapes as hk0, hv0) or NULL to skip */
size_t gsa_fwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype);
int gsa_fwd(const void* q, const void* k, const void* v, const void* g,
            const float* hk0, const float* hv0,
            void* o, float* hkt, float* hvt,
            int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, int act,
            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- GSA backward ---------
 * Gradients of sum(o * do_) + sum(hkt * dhkt) + sum(hvt * dhvt).
 *   do_ : [B,H,L,Dv] dtype;  dhkt [B,H,Dk,m], dhvt [B,H,m,Dv] float32 or NULL (= zero)
 *   dq, dk : [B,H,L,Dk] dtype;  dv : [B,H,L,Dv] dtype;  dg : [B,H,L,m] float32
 *   dhk0, dhv0 : gradients of hk0, hv0 (float32) or NULL to skip */
size_t gsa_bwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype);
int gsa_bwd(const void* q, const void* k, const void* v, const void* g,
            const float* hk0, const float* hv0,
            const void* do_, const float* dhkt, const float* dhvt,
            void* dq, void* dk, void* dv, float* dg, float* dhk0, float* dhv0,
            int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, int act,
            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- GSA saved activations --
 * As for GLA: gsa_bwd recomputes the forward's intermediate tensors (the write weights
 * w = 1 - exp(g), the pass-1 chunk operands and chunk-start states, the read-out p and its
 * float32 copy, pass 2's chunk operands and chunk-start states), which gsa_fwd_save /
 * gsa_bwd_saved avoid by keeping them:
 *   gsa_fwd_save   computes exactly what gsa_fwd computes and also leaves them in `saved`;
 *   gsa_bwd_saved  computes exactly what gsa_bwd computes, reading them from `saved`.
 * saved: device buffer of at least gsa_saved_bytes() bytes, owned by the caller; its contents
 *   on entry to gsa_fwd_save do not matter, and gsa_bwd_saved only reads it.  It is valid for
 *   the q, k, g, hk0, hv0, C, dtype and act of the gsa_fwd_save call that filled it; passing
 *   other inputs to gsa_bwd_saved gives undefined results (the library cannot check this).
 *   NULL saved in gsa_bwd_saved: GLA_ERR_NULL_ARG.
 * workspace (gsa_bwd_saved): at least gsa_bwd_saved_workspace_bytes() bytes.
 * Sizes, dtypes, alignment and errors as for gsa_bwd (the saved path supports the sizes the
 * backward supports); `saved` must not overlap any input or output (GLA_ERR_ALIAS). */
size_t gsa_saved_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype);
size_t gsa_bwd_saved_workspace_bytes(int B, int H, int L, int Dk, int Dv, int m, int C, int dtype);
int gsa_fwd_save(const void* q, const void* k, const void* v, const void* g,
                 const float* hk0, const float* hv0,
                 void* o, float* hkt, float* hvt,
                 int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, int act,
                 void* saved, size_t saved_bytes, void* stream);
int gsa_bwd_saved(const void* q, const void* k, const void* v, const void* g,
                  const float* hk0, const float* hv0,
                  const void* do_, const float* dhkt, const float* dhvt,
                  void* dq, void* dk, void* dv, float* dg, float* dhk0, float* dhv0,
                  int B, int H, int L, int Dk, int Dv, int m, int C, int dtype, int act,
                  const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ---------------------------------------------------------------- GSA decode -----------
 * One recurrent inference step of gated slot attention per (batch, head): the fixed-size
 * slot memories are updated with the token and read through a softmax over the m slots
 * (GSA abstract: efficient recurrent inference; research-map summary, "Approach").
 *   q, k : [B,H,Dk] dtype;  v : [B,H,Dv] dtype;  g : [B,H,m] dtype slot log-gates
 *   hk   : [B,H,Dk,m] float32 slot keys (transposed), read and overwritten with
 *          hk Diag(exp g) + k^T (1 - exp g)
 *   hv   : [B,H,m,Dv] float32 slot values, read and overwritten with
 *          Diag(exp g) hv + (1 - exp g)^T v
 *   o    : [B,H,Dv] dtype = softmax(q hk) hv (after the update), or f(q hk) hv for the
 *          element-wise read-outs (act: a gsa_act value)
 * The memories have the layout of gsa_fwd's hkt and hvt, so a prefill by gsa_fwd can be
 * continued token by token.  Needs no workspace.  Dk up to 256, Dv up to 512 and m up to
 * 256, multiples of 16.  hk and hv must overlap neither each other nor q, k, v, g; o must
 * overlap nothing (GLA_ERR_ALIAS). */
int gsa_decode_step(const void* q, const void* k, const void* v, const void* g,
                    float* hk, float* hv, void* o,
                    int B, int H, int Dk, int Dv, int m, int dtype, int act, void* stream);

/* ---------------------------------------------------------------- MS-GLA front end -----
 * Multi-scale GLA over head groups (MS-GLA summary, sections 3.1 to 3.4).  Group i holds heads
 * heads[0] + ... + heads[i-1] .. + heads[i] - 1 (consecutive, sum(heads) = H) at temporal scale
 * scales[i]:
 *   pooling: non-overlapping averages of scales[i] tokens of q, k, g and v of those heads (the
 *            trailing partial block averages only its real tokens), ceil(L / scales[i]) pooled
 *            tokens;
 *   branch:  GLA (as gla_fwd, chunk size C) on the pooled sequence, from h0's slice;
 *   hold:    token t reads the pooled output of block (t + 1) / scales[i] - 1 (integer
 *            division), the latest block whose tokens it has all seen, and zeros before the
 *            first block completes;
 *   fusion:  o[b,h,t,:] = w[b,t,i] * held[b,h,t,:] for the group i of head h.
 *   q, k, g : [B,H,L,Dk] dtype;  v : [B,H,L,Dv] dtype
 *   h0      : [B,H,Dk,Dv] float32 initial state of every head's branch, or NULL (zeros)
 *   w       : [B,L,ngroups] float32 fusion weights (4-byte aligned), or NULL (all 1)
 *   o       : [B,H,L,Dv] dtype
 *   ht      : [B,H,Dk,Dv] float32, each branch's state after its last pooled token, or NULL
 *   ngroups : 1 .. 8;  scales, heads: HOST arrays of ngroups ints (1 <= scales[i] <= 65536,
 *             heads[i] >= 1)
 * Every group's pooled shape must be supported by gla_fwd (same C, Dk, Dv rules).  Bad group
 * arrays give GLA_ERR_SHAPE (counts) or GLA_ERR_UNSUPPORTED (ngroups, scales).
 * The groups' GLA forwards run together, each kernel launched once for all groups, each
 * group with its own workspace slice.  A scale-1 group reads q, k, v and g in place; other
 * groups read pooled copies in the workspace.  The branches' output kernel writes the held,
 * weighted tokens straight into o (no pooled output is stored). */
size_t msgla_fwd_workspace_bytes(int B, int H, int L, int Dk, int Dv, int C, int dtype,
                                 int ngroups, const int* scales, const int* heads);
int msgla_fwd(const void* q, const void* k, const void* v, const void* g,
              const float* h0, const float* w, void* o, float* ht,
              int B, int H, int L, int Dk, int Dv, int C, int dtype,
              int ngroups, const int* scales, const int* heads,
              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_AMD_GLA_H */
