/*
 * hybrid_attn.h -- C ABI of the MI355X (gfx950) Hybrid Linear-Softmax Attention
 * library: the gated linear layer, the gated softmax anchor and the 3:1 group
 * of SANA-Video 2.0 ("SANA-Video 2.0: Hybrid Linear Attention with Attention
 * Residuals for Efficient Video Generation": summary page, section 03; review
 * page, sections 1 and 3; news item, "Innovatie in aandachtmechanismen").
 *
 * The pages name the two layer kinds and the 3:1 ratio but print no formula.
 * This library computes, per batch item b and head h, over N tokens:
 *
 *   linear:  S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j),  phi(x) = max(x, 0)
 *            o_i = sigmoid(g_i) * (phi(q_i)^T S) / (phi(q_i) . z + HA_LINEAR_EPS)
 *   softmax: o_i = sigmoid(g_i) * sum_j softmax_j(q_i . k_j / sqrt(d)) v_j
 *
 * with sigmoid(x) = 1 / (1 + exp(-x)) and "*" elementwise (G has O's shape).
 * Attention is bidirectional: every query sees all N tokens of its own (b, h).
 *
 * Tensor layout: every Q, K, V, G, O is a dense row-major [B, H, N, d] array,
 * d fastest; a group takes stacked [4, B, H, N, d] arrays, layer l at element
 * offset l * B * H * N * d.  All five tensors of a call share one dtype.
 *
 * Ownership and ordering: the caller owns every buffer (device memory),
 * including the workspace.  The library allocates nothing, frees nothing and
 * keeps no state between calls, so calls are reentrant.  All work is enqueued
 * asynchronously on `stream` (0 = the null stream) of the current device; inputs
 * must stay alive and unmodified until the stream has passed the call.  No entry
 * point allocates, copies, clears memory or synchronises, so each can be
 * captured into a HIP graph on `stream` and replayed on the same buffers.
 *
 * Errors: every entry point validates its arguments on the host, in the order
 * listed under ha_status, and returns before any HIP call when they are invalid:
 * nothing is enqueued.  An empty problem (B, H or N equal to 0) returns HA_OK
 * and enqueues nothing, except hybrid_attn_kv_state, which still writes a zero
 * state when B * H > 0.  A failed kernel launch returns HA_EHIP; faults inside
 * a kernel surface at the caller's next synchronisation of the stream.  No C++
 * exception crosses this interface.
 *
 * Determinism: the split of the linear-state reduction over tokens is a pure
 * function of (B, H, N, d); partial states are summed in a fixed order without
 * atomics, so repeated calls on the same inputs give bitwise equal outputs.
 */
#ifndef HYBRID_ATTN_H
#define HYBRID_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HA_API __attribute__((visibility("default")))

/* Storage dtype of Q, K, V, G, O.  HA_BF16: bfloat16 I/O, bf16 MFMA products
 * with float32 accumulation, outputs rounded to nearest even.  HA_F32: float32
 * I/O and float32 arithmetic throughout. */
/* The two range markers make the enum as wide as int, so that any int a C
 * caller passes is a valid value of the type (and is rejected by the check
 * with HA_EUNSUPPORTED) rather than an out-of-range enum value. */
typedef enum ha_dtype {
  HA_BF16 = 0,
  HA_F32 = 1,
  HA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  HA_DTYPE_RANGE_MAX_ = 2147483647
} ha_dtype;

/* Status codes, in the order the checks run. */
typedef enum ha_status {
  HA_OK = 0,
  HA_EUNSUPPORTED = -2, /* d not 64 or 128, or unknown dtype                      */
  HA_EINVAL = -1,       /* negative or too large B/H/N, null pointer, output that
                           overlaps an input, workspace that overlaps a tensor of
                           the call, null kinds array                            */
  HA_EALIGN = -3,       /* a tensor or workspace pointer not 16-byte aligned      */
  HA_EWORKSPACE = -4,   /* workspace null or smaller than hybrid_attn_workspace_bytes */
  HA_EHIP = -5          /* a kernel launch or event record failed                 */
} ha_status;

/* eps of the linear layer's denominator phi(q).z + eps. */
#define HA_LINEAR_EPS 1e-6f

/* Size limits checked by every entry point (HA_EINVAL beyond them). */
#define HA_MAX_N (1LL << 23)   /* tokens per (b, h); byte offsets of one head fit 32 bits */
#define HA_MAX_BH (1LL << 20)  /* B * H              */

/* Text for a status code (static storage, never NULL). */
HA_API const char* hybrid_attn_strerror(int status);

/* Bytes of device workspace that hybrid_attn_linear, hybrid_attn_group and
 * hybrid_attn_kv_state need for these sizes.  Pure function of its arguments:
 * no device query.  Returns 0 for an empty or invalid problem. */
HA_API size_t hybrid_attn_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype);

/* Linear-attention state of every (b, h): S[b,h] = sum_j phi(k_j) v_j^T as a
 * row-major float32 [B, H, d, d] array (row = key feature, column = value
 * feature) and z[b,h] = sum_j phi(k_j) as float32 [B, H, d].  K, V: [B, H, N, d]
 * of `dtype`.  This is the first half of the linear layer on its own (its
 * state reduction); the layer below computes the same state in its workspace. */
HA_API int hybrid_attn_kv_state(const void* K, const void* V, float* S, float* z,
                                int B, int H, int64_t N, int d, ha_dtype dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One gated linear-attention layer (formula above).  Q, K, V, G in, O out, all
 * [B, H, N, d] of `dtype`.  O must not overlap any input. */
HA_API int hybrid_attn_linear(const void* Q, const void* K, const void* V, const void* G, void* O,
                              int B, int H, int64_t N, int d, ha_dtype dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* hybrid_attn_linear that also records four caller-created events on `stream`:
 * events[0] before pass 1 of the state reduction, events[1] after it,
 * events[2] after pass 2 and events[3] after the apply, so the caller can time
 * each kernel of the layer with hipEventElapsedTime.  HA_EINVAL for a NULL
 * array or entry; otherwise exactly hybrid_attn_linear (the same result). */
HA_API int hybrid_attn_linear_timed(const void* Q, const void* K, const void* V, const void* G, void* O,
                                    int B, int H, int64_t N, int d, ha_dtype dtype,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    hipEvent_t const events[4]);

/* One gated softmax anchor layer (formula above), logit scale 1/sqrt(d).  No
 * workspace.  O must not overlap any input. */
HA_API int hybrid_attn_softmax(const void* Q, const void* K, const void* V, const void* G, void* O,
                               int B, int H, int64_t N, int d, ha_dtype dtype, hipStream_t stream);

/* Block sizes of the block-sparse anchor's pattern: query block qb holds rows
 * qb*256 .. qb*256+255 and key block kb holds keys kb*64 .. kb*64+63 of each
 * (b, h); the last blocks of a sequence may be partial. */
#define HA_SPARSE_BLOCK_Q 256
#define HA_SPARSE_BLOCK_K 64

/* Block-sparse gated softmax anchor: the anchor above with each query attending
 * only to the keys of the key blocks its query block lists, i.e. the softmax is
 * taken over the union of those blocks' keys.  The SANA-Video 2.0 pages name
 * sparse attention only as one part of the Sol-Engine inference stack (summary
 * page, section 04; review page, section 1) without giving its pattern; the
 * block-structured sets this entry point takes are those of Long Video Sparse
 * Attention (LVSA explainer page, "LVSA: Training-Free Sparse Attention for
 * Long Video Diffusion", section 2, Method: each frame attends to a local
 * window of frames plus a rotating set of global frames under a frame budget)
 * and of LoSA's frozen per-query-block key-block sets (LoSA article).  The
 * pattern, shared by every batch item and head, is in CSR form in device
 * memory:
 *   block_offsets: int32 [ceil(N / HA_SPARSE_BLOCK_Q) + 1], non-decreasing,
 *                  block_offsets[0] = 0, last entry = num_indices;
 *   block_indices: int32 [num_indices]; query block qb lists the key blocks
 *                  block_indices[block_offsets[qb] .. block_offsets[qb+1]-1].
 * Indices must be distinct within a query block (any order); an index outside
 * [0, ceil(N / HA_SPARSE_BLOCK_K)) names no key and is ignored; offsets are
 * clamped to [0, num_indices].  A query block with no valid key writes O = 0.
 * The pattern is read, never written; it must not overlap O.  HA_EINVAL for a
 * NULL block_offsets, a NULL block_indices with num_indices > 0, or
 * num_indices outside [0, 2^30); HA_EALIGN for pattern arrays that are not
 * 4-byte aligned.  The full pattern (every key block for every query block)
 * gives the dense anchor's result. */
HA_API int hybrid_attn_softmax_blocksparse(const void* Q, const void* K, const void* V, const void* G,
                                           void* O, int B, int H, int64_t N, int d, ha_dtype dtype,
                                           const int32_t* block_offsets, const int32_t* block_indices,
                                           int64_t num_indices, hipStream_t stream);

/* One hybrid group: layers 0, 1, 2 gated linear, layer 3 the gated softmax
 * anchor (the 3:1 ratio of the pages, anchor last in the period).  Q4, K4, V4,
 * G4 in and O4 out are stacked [4, B, H, N, d] arrays; layer l of the output is
 * bitwise equal to the single-layer call on layer l of the inputs.  The three
 * linear layers reuse one workspace in turn. */
HA_API int hybrid_attn_group(const void* Q4, const void* K4, const void* V4, const void* G4, void* O4,
                             int B, int H, int64_t N, int d, ha_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* hybrid_attn_group for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid allocation): the same
 * computation with the same kernels (outputs bitwise equal to hybrid_attn_group),
 * its linear layers' workspace taken from a fixed array of
 * HA_NOALLOC_SCRATCH_BYTES in the library's device memory instead of a caller
 * buffer.  The library calls no hipMalloc or hipFree here.  Every device keeps
 * its own array from its first call until the process ends.  All calls on one
 * device share that device's array, so calls that overlap on one device (other
 * streams, other threads) race and must not be issued.  Returns HA_EWORKSPACE
 * when hybrid_attn_workspace_bytes(B, H, N, d, dtype) exceeds
 * HA_NOALLOC_SCRATCH_BYTES (at d = 128 that holds for B*H up to about 100),
 * HA_EHIP when the array's device address cannot be obtained, and otherwise
 * what hybrid_attn_group returns. */
#define HA_NOALLOC_SCRATCH_BYTES (64ull << 20)
HA_API int hybrid_attn_group_noalloc(const void* Q4, const void* K4, const void* V4, const void* G4, void* O4,
                                     int B, int H, int64_t N, int d, ha_dtype dtype, hipStream_t stream);

/* hybrid_attn_group that also records five caller-created events on `stream`:
 * events[0] before layer 0 and events[l + 1] after layer l, so the caller can
 * time each layer of the group with hipEventElapsedTime.  A NULL `events`
 * behaves exactly like hybrid_attn_group; otherwise all five must be valid
 * events of the stream's device (HA_EINVAL for a NULL entry). */
HA_API int hybrid_attn_group_timed(const void* Q4, const void* K4, const void* V4, const void* G4,
                                   void* O4, int B, int H, int64_t N, int d, ha_dtype dtype,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t const events[5]);

/* ---- Backward pass ----------------------------------------------------------
 * The model is trained from scratch (review page, section 3; news item,
 * "Prestaties"), so each layer has a backward pass: given dO = dL/dO it returns
 * dQ, dK, dV, dG (all [B, H, N, d] of `dtype`, the inputs' layout).  The
 * gradients follow the forward formulas above by the chain rule, with the
 * ReLU's derivative taken as 0 at 0; they are exact up to rounding (bf16
 * operands, float32 accumulation).  Outputs must not overlap any input or each
 * other.  Deterministic: fixed reduction orders, no atomics. */

/* Bytes of device workspace hybrid_attn_linear_backward needs (pure function;
 * 0 for an empty or invalid problem). */
HA_API size_t hybrid_attn_linear_backward_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype);

/* Backward pass of the gated linear layer.  Recomputes the state S, z from K, V
 * and streams every token four more times: dG, dn = sigmoid(g) dO / den and
 * dden = -(sigmoid(g) dO . a) / den per token; dS = sum phi(q)^T dn and
 * dz = sum dden phi(q) (deterministic split-N reduction); then
 * dQ = (dn S^T + dden z) [Q > 0], dV = phi(K) dS, dK = (V dS^T + dz) [K > 0]. */
HA_API int hybrid_attn_linear_backward(const void* Q, const void* K, const void* V, const void* G,
                                       const void* dO, void* dQ, void* dK, void* dV, void* dG,
                                       int B, int H, int64_t N, int d, ha_dtype dtype,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The gated softmax anchor (as hybrid_attn_softmax) that also writes, per query
 * row, lse[b, h, i] = ln sum_j exp(q_i . k_j / sqrt(d)) as float32 [B, H, N]:
 * the forward pass of a training step, whose O and lse the backward consumes.
 * lse must not overlap O. */
HA_API int hybrid_attn_softmax_lse(const void* Q, const void* K, const void* V, const void* G, void* O,
                                   float* lse, int B, int H, int64_t N, int d, ha_dtype dtype,
                                   hipStream_t stream);

/* Bytes of device workspace hybrid_attn_softmax_backward needs (da and D). */
HA_API size_t hybrid_attn_softmax_backward_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype);

/* Backward pass of the gated softmax anchor.  O and lse are the outputs of
 * hybrid_attn_softmax_lse on the same Q, K, V, G.  With s = sigmoid(G),
 * da = dO s, D_i = dO_i . O_i, P_ij = exp(q_i . k_j / sqrt(d) - lse_i) and
 * dS_ij = P_ij (da_i . v_j - D_i): dG = dO O (1 - s), dQ = dS K / sqrt(d),
 * dK = dS^T Q / sqrt(d), dV = P^T da.  Costs about 3.5 forward passes. */
HA_API int hybrid_attn_softmax_backward(const void* Q, const void* K, const void* V, const void* G,
                                        const void* O, const void* dO, const float* lse,
                                        void* dQ, void* dK, void* dV, void* dG,
                                        int B, int H, int64_t N, int d, ha_dtype dtype,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Attention block around the group --------------------------------------
 * The hybrid layers sit inside DiT blocks (review page, section 3: the compiled
 * DiT forward; summary page, section 03: the 3:1 interleave).  The block here is
 * four attention sub-layers on a residual stream x, a dense row-major
 * [B, N, C] array with C = H * d, sub-layer l of the group's kind l:
 *     [Q | K | V | G] = x W_in[l]^T            W_in[l]: row-major [4C, C]
 *     O = gated linear or softmax layer (Q, K, V, G)
 *     x = x + concat_h(O) W_out[l]^T           W_out[l]: row-major [C, C]
 * Weights are in the [output feature, input feature] layout.  Output feature
 * t*C + h*d + e of W_in's product is feature e of head h of tensor t (Q, K, V,
 * G in that order); column h*d + e of the concatenation is feature e of head h
 * of O.  Q, K, V, G, O are [B, H, N, d] as above.  The pages print neither the
 * projections nor the residual; this is the plainest reading.  Products are
 * taken on the MFMA in bf16 with float32 accumulation (float32 throughout for
 * HA_F32); results are rounded once, on store. */

/* Q, K, V, G = the four C-wide blocks of x W_in^T, split into heads.  x: [B, N, C],
 * W_in: [4C, C]; outputs [B, H, N, d], none overlapping another buffer. */
HA_API int hybrid_attn_proj_in(const void* x, const void* W_in, void* Q, void* K, void* V, void* G,
                               int B, int H, int64_t N, int d, ha_dtype dtype, hipStream_t stream);

/* x_out = x + concat_h(O) W_out^T.  O: [B, H, N, d], W_out: [C, C], x, x_out:
 * [B, N, C].  x_out may be x itself (in place); otherwise it must not overlap
 * any input. */
HA_API int hybrid_attn_proj_out(const void* O, const void* W_out, const void* x, void* x_out,
                                int B, int H, int64_t N, int d, ha_dtype dtype, hipStream_t stream);

/* Bytes of device workspace hybrid_attn_block needs: Q, K, V, G, O of one
 * sub-layer plus the linear layer's workspace.  0 for an empty or invalid problem. */
HA_API size_t hybrid_attn_block_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype);

/* The block: the four sub-layers in order on one stream.  W_in4: [4, 4C, C],
 * W_out4: [4, C, C].  x_out may be x (in place); the workspace must not overlap
 * x, x_out or the weights.  Each stage is the same kernel as the matching
 * single entry point, so the result is bitwise equal to calling
 * hybrid_attn_proj_in, the layer and hybrid_attn_proj_out in turn. */
HA_API int hybrid_attn_block(const void* x, const void* W_in4, const void* W_out4, void* x_out,
                             int B, int H, int64_t N, int d, ha_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Block attention residuals (AttnRes) ------------------------------------
 * Summaries of completed blocks are routed into later linear layers (summary
 * page, section 03; review page, sections 1 and 3; news item).  The pages give
 * no formula; the reading implemented here: a block is one hybrid group, its
 * summary is the stream after it, and each linear sub-layer of a later block
 * projects, instead of the stream x, the per-token softmax mixture
 *     h = sum_m softmax_m(w . v_m / rms(v_m) / sqrt(C)) v_m,
 *     rms(v) = sqrt(mean(v^2) + HA_RMS_EPS),
 * over the candidates v_0 .. v_{M-1} = the completed summaries and v_M = x,
 * with w a learned float32 routing vector of the sub-layer.  The anchor reads
 * x; every residual update still goes to x. */
#define HA_RMS_EPS 1e-6f
#define HA_ATTNRES_MAX_SUMMARIES 63

/* h = the mixture above.  summaries: M stacked [B, N, C] arrays (M in
 * [0, HA_ATTNRES_MAX_SUMMARIES]; may be NULL when M = 0), x, h: [B, N, C],
 * w: float32 [C].  h must not overlap any input. */
HA_API int hybrid_attn_attnres_mix(const void* summaries, int M, const void* x, const float* w, void* h,
                                   int B, int64_t N, int C, ha_dtype dtype, hipStream_t stream);

/* Bytes of device workspace hybrid_attn_block_routed needs: the block's and
 * one [B, N, C] mixture. */
HA_API size_t hybrid_attn_block_routed_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype);

/* hybrid_attn_block with AttnRes: sub-layer l, when linear, projects
 * hybrid_attn_attnres_mix(summaries, M, stream, w_route + l * C) instead of the
 * stream.  w_route: float32 [4, C] (the anchor's row is unused).  x_out may be
 * x; it must not overlap the summaries, so a stack of blocks can write block
 * k's output straight into slot k of its summaries array and pass slots
 * 0 .. k-1 as the next block's summaries. */
HA_API int hybrid_attn_block_routed(const void* x, const void* summaries, int M, const float* w_route,
                                    const void* W_in4, const void* W_out4, void* x_out,
                                    int B, int H, int64_t N, int d, ha_dtype dtype,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Writes the layer kinds of a group in order: 0 = gated linear, 1 = gated
 * softmax anchor; i.e. {0, 0, 0, 1}.  Returns HA_EINVAL for a NULL array. */
HA_API int hybrid_attn_group_schedule(int kinds[4]);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_ATTN_H */
